// Launchers of the wide-tile convolution GEMMs (psa_conv_wide.hip, built as
// its own translation unit), called by the C ABI in psa_attn.hip.
#pragma once
#include <hip/hip_runtime.h>

#include "psa_conv_kernels.h"

namespace psa {

// The large-tile dx kernel (16-bit types; cin and cout multiples of 128;
// dy rows of ld tokens a multiple of 8: ld = N, or N rounded up to 8 with
// zero columns past N), one workgroup per CU: the direct-load pipeline with
// 256 x 256 or 128 x 256 (ci x n) tiles.  `none` for other ld, or when the
// problem has too few large tiles to fill the CUs (the caller then runs
// psa_conv_dx_kernel).
enum class DxLarge { none, pipe256, pipe128 };
DxLarge conv_dx_large_kind(int B, int cin, int N, int ld);
// dx = w^T dy per batch into the parts of dx (rows of N) with the chosen
// kernel.  Enqueues one kernel; a launch error is left for the caller's
// hipGetLastError.
void conv_dx_large_launch(DxLarge kind, const void* w, const void* dy, const DxParts<bf16>& dx, int B, int cin,
                          int cout, int N, int ld, hipStream_t st);
void conv_dx_large_launch(DxLarge kind, const void* w, const void* dy, const DxParts<f16>& dx, int B, int cin,
                          int cout, int N, int ld, hipStream_t st);

}  // namespace psa
