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

// The large-tile dw kernel (16-bit types; cin a multiple of 256, cout of
// 128; x and dy rows of ld tokens, a multiple of 8, zero past N): 128 x 256
// (co x ci) tiles, one workgroup per CU, the (b, token) sum cut into the
// returned number of ranges; 0 when the kernel does not apply or the
// problem has too few tiles to fill the CUs (the caller then runs
// psa_conv_dw_kernel).
int conv_dw_pipe_splits(int B, int cin, int cout, int ld, int cus);
// dw (S == 1) or the S fp32 partials part[s][co][ci] (S > 1) with that
// kernel.  Enqueues one kernel; a launch error is left for the caller.
void conv_dw_pipe_launch(const bf16* x, const bf16* dy, bf16* dw, float* part, int B, int cin, int cout, int ld,
                         int S, hipStream_t st);
void conv_dw_pipe_launch(const f16* x, const f16* dy, f16* dw, float* part, int B, int cin, int cout, int ld,
                         int S, hipStream_t st);

}  // namespace psa
