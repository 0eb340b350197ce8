/*
 * Calls into libwide.so's C ABI from C, with enum arguments outside their
 * enumerators (legal C: an enum object holds any int value). Linked into the
 * host sanitizer driver; returns the number of wrong results.
 */
#include <stdint.h>
#include <string.h>

#include "wide.h"

int c_caller_bad_enums(void* p) {
  int fails = 0;
  const wide_status_t st = (wide_status_t)99;
  const wide_dtype_t dt = (wide_dtype_t)99;
  const wide_stage_t sg = (wide_stage_t)99;
  const wide_act_t ac = (wide_act_t)99;
  if (strcmp(wide_status_string(st), "unknown status") != 0) ++fails;
  if (wide_ffn_workspace_size(16, 64, 128, 64, dt) != 0) ++fails;
  if (wide_ffn_workspace_size_for(16, 64, 128, 64, dt, 1) != 0) ++fails;
  if (wide_ffn_forward(p, p, p, p, (const uint8_t*)p, 16, 64, 128, 64, dt, p, NULL, p, 1u << 30, 0,
                       NULL) != WIDE_ERR_DTYPE)
    ++fails;
  if (wide_gemm_k(p, p, (const uint8_t*)p, 16, 64, 128, 64, dt, p, p, 1u << 30, NULL) !=
      WIDE_ERR_DTYPE)
    ++fails;
  if (wide_gemm_mn(p, p, (const uint8_t*)p, 16, 128, 64, 64, dt, p, p, 1u << 30, NULL) !=
      WIDE_ERR_DTYPE)
    ++fails;
  if (wide_ffn_stage(sg, p, p, p, p, (const uint8_t*)p, 64, 64, 128, 64, WIDE_BF16, p, NULL, p,
                     1u << 30, 0, NULL) != WIDE_ERR_SHAPE)
    ++fails;
  if (wide_router_forward(p, p, p, 4, 64, 16, 2, ac, WIDE_BF16, (uint8_t*)p, NULL, p, 1u << 20,
                          NULL) != WIDE_ERR_SHAPE)
    ++fails;
  if (wide_router_forward(p, p, p, 4, 64, 16, 2, WIDE_ACT_SILU, dt, (uint8_t*)p, NULL, p, 1u << 20,
                          NULL) != WIDE_ERR_DTYPE)
    ++fails;
  if (wide_attention_prefill(p, p, p, (const uint8_t*)p, 4, 2, 1, 128, dt, p, 0, p, 1u << 30,
                             NULL) != WIDE_ERR_DTYPE)
    ++fails;
  if (wide_attention_decode(p, p, p, (const uint8_t*)p, 4, 2, 1, 128, dt, p, 0, p, 1u << 30,
                            NULL) != WIDE_ERR_DTYPE)
    ++fails;
  return fails;
}
