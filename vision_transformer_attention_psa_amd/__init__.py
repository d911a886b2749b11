"""PSA self-attention (forward + backward) for AMD Instinct MI355X (gfx950).

``binding`` exposes the C ABI of libpsa_attn.so (``psa_attn_fwd``,
``psa_attn_bwd``, ...) plus torch conveniences ``fwd``/``bwd``; ``inputs``
draws the seeded synthetic workloads.  Importing the package loads nothing:
the library is opened on first use and its absence is an error, never a
fallback.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs", "binding"]
