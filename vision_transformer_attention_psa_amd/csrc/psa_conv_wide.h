// Launchers of the wide-tile convolution GEMMs (psa_conv_wide.hip, built as
// its own translation unit), called by the C ABI in psa_attn.hip.
#pragma once
#include <hip/hip_runtime.h>

#include "psa_conv_kernels.h"

namespace psa {

// The large-tile dx kernels (16-bit types; cin and cout multiples of 128),
// one workgroup per CU: for rows of N a multiple of 8, the direct-load
// pipeline with 256 x 256 or 128 x 256 (ci x n) tiles; otherwise the
// register-staged kernel with 256 x 256 (cin a multiple of 256) or 128 x 512
// tiles.  `none` when the problem has too few large tiles to fill the CUs
// (the caller then runs psa_conv_dx_kernel).
enum class DxLarge { none, pipe256, pipe128, staged256, staged128 };
DxLarge conv_dx_large_kind(int B, int cin, int N);
// dx = w^T dy per batch into the parts of dx with the chosen kernel.
// Enqueues one kernel; a launch error is left for the caller's
// hipGetLastError.
void conv_dx_large_launch(DxLarge kind, const void* w, const void* dy, const DxParts<bf16>& dx, int B, int cin,
                          int cout, int N, hipStream_t st);
void conv_dx_large_launch(DxLarge kind, const void* w, const void* dy, const DxParts<f16>& dx, int B, int cin,
                          int cout, int N, hipStream_t st);

}  // namespace psa
