/* A plain C99 consumer of include/psa_attn.h: the header compiles as C, the
 * library links, and argument validation answers before any device work
 * (fake 16-byte aligned addresses; every call below must be rejected). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "psa_attn.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d, want %d (%s)\n", what, got, want, psa_last_error());
    ++failures;
  }
}

int main(void) {
  void* qkv = (void*)(uintptr_t)(1u << 20);
  void* o = (void*)(uintptr_t)(1u << 24);
  float* lse = (float*)(uintptr_t)(1u << 26);
  void* d = (void*)(uintptr_t)(1u << 28);
  void* parts[2] = {o, d};
  int chans[2] = {64, 32};

  expect("supported (64,64) bf16", psa_attn_supported(64, 64, PSA_BF16), 1);
  expect("supported (48,64) f32", psa_attn_supported(48, 64, PSA_F32), 0);
  if (psa_attn_version() < 100) ++failures;
  expect("fwd NULL", psa_attn_fwd(NULL, o, lse, 1, 1, 64, 64, 64, 0.125f, PSA_BF16, NULL), PSA_ERR_NULL);
  if (strlen(psa_last_error()) == 0) ++failures;
  expect("fwd N=0", psa_attn_fwd(qkv, o, lse, 1, 1, 0, 64, 64, 0.125f, PSA_BF16, NULL), PSA_ERR_SHAPE);
  expect("fwd bad scale", psa_attn_fwd(qkv, o, lse, 1, 1, 64, 64, 64, -1.f, PSA_BF16, NULL), PSA_ERR_SHAPE);
  expect("fwd no instance", psa_attn_fwd(qkv, o, lse, 1, 1, 64, 48, 64, 0.125f, PSA_F32, NULL),
         PSA_ERR_UNSUPPORTED);
  expect("fwd misaligned", psa_attn_fwd((char*)qkv + 2, o, lse, 1, 1, 64, 64, 64, 0.125f, PSA_BF16, NULL),
         PSA_ERR_ALIGN);
  expect("fwd alias", psa_attn_fwd(qkv, qkv, lse, 1, 1, 64, 64, 64, 0.125f, PSA_BF16, NULL), PSA_ERR_ALIAS);
  expect("bwd alias", psa_attn_bwd(qkv, o, lse, d, qkv, 1, 1, 64, 64, 64, 0.125f, PSA_BF16, NULL),
         PSA_ERR_ALIAS);
  expect("vslice past V", psa_attn_fwd_vslice(qkv, o, lse, 1, 1, 64, 32, 64, 48, 32, 0.2f, PSA_BF16, NULL),
         PSA_ERR_SHAPE);
  expect("merge alias", psa_merge_fwd(o, o, d, 1, 1, 64, 32, PSA_BF16, NULL), PSA_ERR_ALIAS);
  expect("cat range", psa_channel_cat_bwd(qkv, o, 1, 40, 64, 32, PSA_BF16, NULL), PSA_ERR_SHAPE);
  expect("conv channels", psa_qkv_conv_bwd(qkv, o, lse, d, (char*)d + (1 << 24), 1, 96, 128, 16, PSA_BF16, NULL),
         PSA_ERR_UNSUPPORTED);
  expect("conv parts sum", psa_qkv_conv_cat_bwd(qkv, o, lse, parts, chans, 2, (char*)d + (1 << 24), 1, 128, 128,
                                                16, PSA_BF16, NULL), PSA_ERR_SHAPE);
  expect("timing slots", PSA_TIMING_SLOTS, 9);
  if (failures == 0) printf("abi_check ok\n");
  return failures == 0 ? 0 : 1;
}
