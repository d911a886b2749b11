// Launchers of the wide-tile convolution GEMMs (psa_conv_wide.hip, built as
// its own translation unit), called by the C ABI in psa_attn.hip.
#pragma once
#include <hip/hip_runtime.h>

#include "psa_conv_kernels.h"

namespace psa {

// 2 when cin is a multiple of 256: 256 x 256 workgroup tiles (the pipelined
// kernel for N a multiple of 8, else the register-staged one with 2 x 2
// waves); else 1: 128 x 512 tiles (register-staged, 1 x 4 waves).
int conv_dx_wide_wm(int cin);
// Workgroups the wide dx launch runs for a problem.
long long conv_dx_wide_blocks(int B, int cin, int N);
// dx = w^T dy per batch into the parts of dx (16-bit types; cin and cout
// multiples of 128).  Enqueues one kernel; a launch error is left for the
// caller's hipGetLastError.
void conv_dx_wide_launch(const void* w, const void* dy, const DxParts<bf16>& dx, int B, int cin, int cout, int N,
                         hipStream_t st);
void conv_dx_wide_launch(const void* w, const void* dy, const DxParts<f16>& dx, int B, int cin, int cout, int N,
                         hipStream_t st);

}  // namespace psa
