"""CPU float64 oracle for PSA self-attention (test infrastructure only).

Importable only from the test suite, the package smoke check and the
benchmark's CPU-baseline leg; the product path never reaches it.
"""
from .psa_oracle import (backward, backward_slice, forward, forward_backward,  # noqa: F401
                         forward_slice, max_rel_err, preprocess_D)
