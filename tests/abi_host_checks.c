/*
 * Host-side argument checks of libflashcache's C ABI, driven from C: every
 * entry point is called with arguments its host code must reject (and with
 * size queries at edge values). Nothing here reaches a kernel, so it runs
 * without a GPU. Built with AddressSanitizer and UndefinedBehaviorSanitizer on
 * the library's host code by tests/test_abi.py; exits non-zero on the first
 * unexpected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "flashcache.h"

static int failures = 0;

#define FAKE ((void*)0x1000) /* non-null, never dereferenced by a rejected call */

static void expect(const char* what, fc_status_t got, fc_status_t want) {
  const char* msg = fc_last_error();
  if (got != want || msg == NULL || (want != FC_OK && msg[0] == 0)) {
    fprintf(stderr, "FAIL %s: status %d (want %d), message '%s'\n", what, (int)got, (int)want,
            msg ? msg : "(null)");
    ++failures;
  }
}

int main(void) {
  const int32_t* I = (const int32_t*)FAKE;
  for (int s = -1; s < 7; ++s)
    if (fc_status_string((fc_status_t)s) == NULL) { fprintf(stderr, "FAIL status string\n"); ++failures; }
  if (strncmp(fc_version(), "flashcache-gfx950", 17) != 0) { fprintf(stderr, "FAIL version\n"); ++failures; }

  /* projection */
  expect("qkv B=0", fc_qkv_rope_cache_write(FAKE, I, I, 0, 4, FAKE, 256, 2, 128, 1e4f, FAKE, FAKE, I, 4,
                                            16, FAKE, NULL, NULL, FAKE, 1 << 20, FC_DTYPE_BF16, NULL),
         FC_ERR_INVALID_VALUE);
  expect("qkv d != H*D", fc_qkv_rope_cache_write(FAKE, I, I, 1, 4, FAKE, 255, 2, 128, 1e4f, FAKE, FAKE, I,
                                                 4, 16, FAKE, NULL, NULL, FAKE, 1 << 20, FC_DTYPE_BF16,
                                                 NULL),
         FC_ERR_INVALID_VALUE);
  expect("qkv one cache", fc_qkv_rope_cache_write(FAKE, I, I, 1, 4, FAKE, 256, 2, 128, 1e4f, FAKE, NULL,
                                                  I, 4, 16, FAKE, NULL, NULL, FAKE, 1 << 20,
                                                  FC_DTYPE_BF16, NULL),
         FC_ERR_INVALID_VALUE);
  expect("qkv page 24", fc_qkv_rope_cache_write(FAKE, I, I, 1, 4, FAKE, 256, 2, 128, 1e4f, FAKE, FAKE, I,
                                                4, 24, FAKE, NULL, NULL, FAKE, 1 << 20, FC_DTYPE_BF16,
                                                NULL),
         FC_ERR_INVALID_VALUE);
  expect("qkv dtype", fc_qkv_rope_cache_write(FAKE, I, I, 1, 4, FAKE, 256, 2, 128, 1e4f, FAKE, FAKE, I, 4,
                                              16, FAKE, NULL, NULL, FAKE, 1 << 20, 9, NULL),
         FC_ERR_INVALID_VALUE);
  expect("qkv bf16 D=64", fc_qkv_rope_cache_write(FAKE, I, I, 1, 4, FAKE, 256, 4, 64, 1e4f, FAKE, FAKE,
                                                  I, 4, 16, FAKE, NULL, NULL, FAKE, 1 << 20,
                                                  FC_DTYPE_BF16, NULL),
         FC_ERR_UNSUPPORTED);
  expect("qkv no workspace", fc_qkv_rope_cache_write(FAKE, I, I, 1, 4, FAKE, 256, 2, 128, 1e4f, FAKE,
                                                     FAKE, I, 4, 16, FAKE, NULL, NULL, NULL, 0,
                                                     FC_DTYPE_BF16, NULL),
         FC_ERR_WORKSPACE);
  expect("qkv huge", fc_qkv_rope_cache_write(FAKE, I, I, 1, 1 << 30, FAKE, 4096, 32, 128, 1e4f, FAKE,
                                             FAKE, I, 4, 16, FAKE, NULL, NULL, FAKE, (size_t)-1,
                                             FC_DTYPE_BF16, NULL),
         FC_ERR_UNSUPPORTED);
  expect("qkv T_q=0", fc_qkv_rope_cache_write(NULL, NULL, NULL, 1, 0, NULL, 256, 2, 128, 1e4f, NULL,
                                              NULL, NULL, 0, 16, NULL, NULL, NULL, NULL, 0,
                                              FC_DTYPE_BF16, NULL),
         FC_OK);
  /* workspace queries at edge sizes: no overflow, monotone in T_q */
  {
    size_t a = fc_qkv_workspace_size(1, 4096, 128, FC_DTYPE_BF16);
    size_t b = fc_qkv_workspace_size(1 << 20, 4096, 128, FC_DTYPE_BF16);
    size_t c = fc_qkv_workspace_size(0x7fffffff, 256, 128, FC_DTYPE_BF16);
    if (!(a > 0 && b >= a && c >= b / 16)) { fprintf(stderr, "FAIL qkv workspace sizes\n"); ++failures; }
    if (fc_qkv_workspace_size(-5, 4096, 128, FC_DTYPE_BF16) != 0) { fprintf(stderr, "FAIL ws<0\n"); ++failures; }
    size_t w = fc_attention_workspace_size(0x7fffffff, 0x7fffffff, 0x7fffffff, 1 << 20, 128, 1, 64);
    if (w == 0) { fprintf(stderr, "FAIL attention workspace\n"); ++failures; }
    /* a request too large for any allocation saturates instead of wrapping */
    size_t w2 = fc_attention_workspace_size(4, 0x7fffffff, 0x7fffffff, 0x7fffffff, 128, 1, 0x7fffffff);
    if (w2 != (size_t)-1) { fprintf(stderr, "FAIL attention workspace saturation\n"); ++failures; }
    size_t w3 = fc_attention_workspace_size(4, 1024, 1000, 8, 128, 1, 300);   /* 2 extra row tiles */
    if (w3 < (size_t)2 * 8 * 1000 * 4) { fprintf(stderr, "FAIL attention row-tile workspace\n"); ++failures; }
  }

  /* attention */
  expect("attn B=0", fc_varlen_bidir_attention(FAKE, FAKE, FAKE, I, 4, 16, I, I, 0, 128, 100, 32, 128,
                                               0.088f, FAKE, NULL, 0, FAKE, 1 << 20, FC_DTYPE_BF16,
                                               NULL),
         FC_ERR_INVALID_VALUE);
  expect("attn scale", fc_varlen_bidir_attention(FAKE, FAKE, FAKE, I, 4, 16, I, I, 1, 128, 100, 32, 128,
                                                 0.f, FAKE, NULL, 0, FAKE, 1 << 20, FC_DTYPE_BF16,
                                                 NULL),
         FC_ERR_INVALID_VALUE);
  expect("attn page 3", fc_varlen_bidir_attention(FAKE, FAKE, FAKE, I, 4, 3, I, I, 1, 128, 100, 32, 128,
                                                  0.088f, FAKE, NULL, 0, FAKE, 1 << 20, FC_DTYPE_BF16,
                                                  NULL),
         FC_ERR_INVALID_VALUE);
  expect("attn null q", fc_varlen_bidir_attention(NULL, FAKE, FAKE, I, 4, 16, I, I, 1, 128, 100, 32,
                                                  128, 0.088f, FAKE, NULL, 0, FAKE, 1 << 20,
                                                  FC_DTYPE_BF16, NULL),
         FC_ERR_INVALID_VALUE);
  expect("attn workspace", fc_varlen_bidir_attention(FAKE, FAKE, FAKE, I, 4, 16, I, I, 1, 128, 100, 32,
                                                     128, 0.088f, FAKE, (float*)FAKE, 0, NULL, 0,
                                                     FC_DTYPE_BF16, NULL),
         FC_ERR_WORKSPACE);
  expect("attn bf16 D=64", fc_varlen_bidir_attention(FAKE, FAKE, FAKE, I, 4, 16, I, I, 1, 128, 100, 32,
                                                     64, 0.125f, FAKE, NULL, 0, FAKE, 1 << 20,
                                                     FC_DTYPE_BF16, NULL),
         FC_ERR_UNSUPPORTED);

  /* top-k */
  expect("topk k=0", fc_importance_topk((const float*)FAKE, I, 1, 10, 4, NULL, 0, (int32_t*)FAKE,
                                        (int32_t*)FAKE, NULL, NULL),
         FC_ERR_INVALID_VALUE);
  expect("topk null pos", fc_importance_topk((const float*)FAKE, I, 1, 10, 4, NULL, 3, NULL,
                                             (int32_t*)FAKE, NULL, NULL),
         FC_ERR_INVALID_VALUE);

  /* verify */
  expect("verify odd R", fv_verify_accept(FAKE, 100, I, 1, 3, I, 0.9f, (int32_t*)FAKE, (float*)FAKE,
                                          (uint8_t*)FAKE, NULL, NULL),
         FC_ERR_INVALID_VALUE);
  expect("verify tau", fv_verify_accept(FAKE, 100, I, 1, 4, I, 1.5f, (int32_t*)FAKE, (float*)FAKE,
                                        (uint8_t*)FAKE, NULL, NULL),
         FC_ERR_INVALID_VALUE);
  expect("verify vocab", fv_verify_accept(FAKE, 0, I, 1, 4, I, 0.9f, (int32_t*)FAKE, (float*)FAKE,
                                          (uint8_t*)FAKE, NULL, NULL),
         FC_ERR_INVALID_VALUE);
  expect("verify R=0", fv_verify_accept(NULL, 100, I, 1, 0, NULL, 0.9f, NULL, NULL, NULL, NULL, NULL),
         FC_OK);

  /* layer-stack helpers, assembly, validation */
  expect("linear K", fc_linear_residual(FAKE, FAKE, FAKE, 4, 128, 0, FC_DTYPE_BF16, NULL),
         FC_ERR_INVALID_VALUE);
  expect("rms N", fc_rms_row_scale(FAKE, 4, 0, 1e-5f, (float*)FAKE, FC_DTYPE_BF16, NULL),
         FC_ERR_INVALID_VALUE);
  expect("assemble B", fc_assemble_query(I, I, 4, I, I, 0, (int32_t*)FAKE, NULL), FC_ERR_INVALID_VALUE);
  expect("assemble k", fc_assemble_query(NULL, I, 4, I, I, 2, (int32_t*)FAKE, NULL),
         FC_ERR_INVALID_VALUE);
  expect("validate pages", fc_validate_step_inputs(I, I, I, 1, 4, 4, I, 1, 16, 0, NULL),
         FC_ERR_INVALID_VALUE);
  expect("validate ps", fc_validate_step_inputs(I, I, I, 1, 4, 4, I, 1, 12, 8, NULL),
         FC_ERR_INVALID_VALUE);

  /* verify side: confidence acceptance, views, commit, LM head, probes */
  expect("confidence tau", fv_confidence_accept(FAKE, 100, I, 1, 4, 0.f, 1, (int32_t*)FAKE,
                                                (float*)FAKE, (uint8_t*)FAKE, NULL),
         FC_ERR_INVALID_VALUE);
  expect("confidence R=0", fv_confidence_accept(NULL, 100, I, 1, 0, 0.9f, 1, NULL, NULL, NULL, NULL),
         FC_OK);
  expect("fork page ids", fv_fork_view_pages(FAKE, FAKE, I, 8, 16, I, I, 0x40000000, 4, 128,
                                             0x7ffffff0, 3, (int32_t*)FAKE, NULL),
         FC_ERR_INVALID_VALUE);
  expect("fork head_dim", fv_fork_view_pages(FAKE, FAKE, I, 8, 16, I, I, 2, 4, 64, 100, 3,
                                             (int32_t*)FAKE, NULL),
         FC_ERR_UNSUPPORTED);
  expect("commit none", fv_commit_accepted(FAKE, FAKE, I, I, 8, 16, I, I, 2, 0, NULL, 4, 128, NULL),
         FC_OK);
  expect("lmhead vocab", fv_lmhead_verify_accept(FAKE, FAKE, 512, 2000, I, 2, 8, I, 0.9f, FAKE, 1 << 20,
                                                 (int32_t*)FAKE, (float*)FAKE, (uint8_t*)FAKE,
                                                 (uint8_t*)FAKE, NULL),
         FC_ERR_UNSUPPORTED);
  expect("lmhead size", fv_lmhead_verify_accept(FAKE, FAKE, 0x7fffffc0, 0x7fffff00, I, 2, 8, I, 0.9f,
                                                FAKE, 1 << 20, (int32_t*)FAKE, (float*)FAKE,
                                                (uint8_t*)FAKE, (uint8_t*)FAKE, NULL),
         FC_ERR_UNSUPPORTED);
  if (fv_lmhead_workspace_size(0x7fffffff, 0x7fffffff) == 0) {
    fprintf(stderr, "FAIL lmhead workspace size\n");
    ++failures;
  }
  expect("probe passes", fc_probe_kv_stream(FAKE, FAKE, I, 8, 16, I, 2, 4, 128, 3, 0, FAKE, NULL),
         FC_ERR_INVALID_VALUE);
  expect("probe mfma", fc_probe_mfma_bf16(0, 10, FAKE, NULL), FC_ERR_INVALID_VALUE);

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("abi host checks ok\n");
  return 0;
}
