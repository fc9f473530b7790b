/* The C ABI's host-side validation under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with the host
 * pass of capi.cpp instrumented). Every call here fails validation, so no
 * call reaches the device: fake, well-separated addresses are never
 * dereferenced. Exits non-zero when a call returns another status than
 * expected. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/lcs.h"

#define EXPECT(call, status)                                                          \
  do {                                                                                \
    const int _s = (int)(call);                                                       \
    if (_s != (int)(status)) {                                                        \
      fprintf(stderr, "line %d: status %d, expected %d (%s)\n", __LINE__, _s, (int)(status), \
              lcs_last_error());                                                      \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

#define P(i) ((void*)(uintptr_t)(0x100000ull + ((uint64_t)(i) << 30)))

int main(void) {
  const int32_t B = 2, T = 1, L = 1000, K = 2048;
  /* indexer: null, misaligned, stride below L, outputs over every input */
  EXPECT(lcs_idx_score(NULL, P(1), P(2), P(3), P(4), L, P(5), B, T, L, P(6), NULL), LCS_ERR_NULL);
  EXPECT(lcs_idx_score((const uint8_t*)P(0) + 4, P(1), P(2), P(3), P(4), L, P(5), B, T, L, P(6),
                       NULL),
         LCS_ERR_SHAPE);
  EXPECT(lcs_idx_score(P(0), P(1), P(2), P(3), P(4), L - 1, P(5), B, T, L, P(6), NULL),
         LCS_ERR_SHAPE);
  EXPECT(lcs_idx_score(P(0), P(1), P(2), P(3), P(4), L, P(5), B, T, 1 << 30, P(6), NULL),
         LCS_ERR_SHAPE);
  for (int i = 0; i < 6; ++i) {
    void* in[6] = {P(0), P(1), P(2), P(3), P(4), P(5)};
    EXPECT(lcs_idx_score(in[0], in[1], in[2], in[3], in[4], L, in[5], B, T, L, in[i], NULL),
           LCS_ERR_SHAPE);
  }
  /* top-k and attention: workspace and outputs over inputs */
  const size_t tws = lcs_topk_workspace_bytes(B, T, L, K);
  EXPECT(lcs_topk_select(P(0), P(1), B, T, L, K, P(2), P(0), tws, NULL), LCS_ERR_SHAPE);
  EXPECT(lcs_topk_select(P(0), P(1), B, T, L, K, P(1), P(3), tws, NULL), LCS_ERR_SHAPE);
  EXPECT(lcs_topk_select(P(0), P(1), B, T, L, 0, P(2), P(3), tws, NULL), LCS_ERR_UNSUPPORTED);
  const size_t aws = lcs_attn_workspace_bytes(B, T, K);
  EXPECT(lcs_sparse_mla_attn(P(0), P(1), LCS_KV_FP8_E4M3, P(2), 5000, P(3), B, T, L, K, 1.f / 24,
                             (uint16_t*)P(1) + 5000 * 288, P(5), P(6), aws, NULL),
         LCS_ERR_SHAPE);
  EXPECT(lcs_sparse_mla_attn(P(0), P(1), LCS_KV_BF16, NULL, L, P(3), B, T, L, K, 1.f / 24, P(4),
                             P(4), P(6), aws, NULL),
         LCS_ERR_SHAPE);
  EXPECT(lcs_sparse_mla_attn(P(0), P(1), LCS_KV_BF16, NULL, L, P(3), B, T, L, K, 0.f, P(4), P(5),
                             P(6), aws, NULL),
         LCS_ERR_SHAPE);
  EXPECT(lcs_sparse_mla_attn_noalloc(P(0), P(1), LCS_KV_BF16, NULL, L, P(3), 255, T, L, K,
                                     1.f / 24, P(4), P(5), NULL),
         LCS_ERR_WORKSPACE);
  EXPECT(lcs_sparse_mla_attn_noalloc(P(0), P(1), LCS_KV_BF16, NULL, L, P(3), B, T, L, K, 1.f / 24,
                                     P(0), P(5), NULL),
         LCS_ERR_SHAPE);
  /* the composite over 78 layers: one output overlapping an input of another
   * layer, found among ~800 ranges; then a NULL deep in the list (the error
   * message keeps its cause) */
  static lcs_layer ly[78];
  for (int l = 0; l < 78; ++l) {
    const void* base[10];
    for (int f = 0; f < 10; ++f) base[f] = P(10 * l + f + 1);
    ly[l].q8 = base[0];
    ly[l].q_scale = base[1];
    ly[l].w = base[2];
    ly[l].k8 = base[3];
    ly[l].k_scale = base[4];
    ly[l].q = base[5];
    ly[l].kv = base[6];
    ly[l].kv_scale = base[7];
    ly[l].out = (uint16_t*)base[8];
    ly[l].lse = (float*)base[9];
  }
  const size_t iws = lcs_indexshare_workspace_bytes(B, T, L, K);
  ly[77].out = (uint16_t*)ly[3].kv;
  EXPECT(lcs_indexshare_forward(ly, 78, LCS_SCHED_GLM52, NULL, 0, LCS_KV_FP8_E4M3, P(900), B, T, L,
                                K, 1.f / 24, P(901), P(902), P(903), iws, NULL),
         LCS_ERR_SHAPE);
  if (!strstr(lcs_last_error(), "layer 77 out")) return 2;
  ly[77].out = (uint16_t*)P(999);
  ly[60].q = NULL;
  EXPECT(lcs_indexshare_forward(ly, 78, LCS_SCHED_GLM52, NULL, 0, LCS_KV_FP8_E4M3, P(900), B, T, L,
                                K, 1.f / 24, P(901), P(902), P(903), iws, NULL),
         LCS_ERR_NULL);
  if (strcmp(lcs_last_error(), "layer 60 attention: q is NULL") != 0) return 3;
  /* quantiser, append, context-parallel and paged calls */
  EXPECT(lcs_quantize_e4m3(P(0), 4, 128, (uint8_t*)P(0) + 16, P(2), NULL), LCS_ERR_SHAPE);
  EXPECT(lcs_cache_append(P(0), NULL, LCS_KV_BF16, P(1), B, T, L, (uint8_t*)P(0) + 128, P(3), NULL,
                          NULL, NULL),
         LCS_ERR_SHAPE);
  EXPECT(lcs_topk_candidates(P(0), P(1), B, T, L, K, 0, P(1), P(3), NULL), LCS_ERR_SHAPE);
  EXPECT(lcs_topk_merge(P(0), P(1), 17, B, T, K, K, P(2), NULL), LCS_ERR_UNSUPPORTED);
  EXPECT(lcs_idx_localize(P(0), B, T, K, 0, 10, P(0), NULL), LCS_ERR_SHAPE);
  EXPECT(lcs_lse_combine(P(0), P(1), 2, B, T, (uint16_t*)P(0) + 64, NULL, NULL), LCS_ERR_SHAPE);
  lcs_paged pg = {(const int32_t*)P(50), 16, 64, 100};
  EXPECT(lcs_idx_score_paged(P(0), P(1), P(2), P(3), P(4), &pg, P(5), B, T, L, P(3), NULL),
         LCS_ERR_SHAPE);
  pg.block_size = 96;
  EXPECT(lcs_sparse_mla_attn_paged(P(0), P(1), LCS_KV_BF16, NULL, &pg, P(3), B, T, L, K, 1.f / 24,
                                   P(4), NULL, P(6), aws, NULL),
         LCS_ERR_UNSUPPORTED);
  EXPECT(lcs_count_full_layers(LCS_SCHED_GLM52, 78, NULL, 0), 21);
  /* enum arguments outside their enumerators: a C caller may pass any int */
  for (int v = 2; v < 200; v += 97) {
    EXPECT(lcs_sparse_mla_attn(P(0), P(1), (lcs_kv_dtype)v, NULL, L, P(3), B, T, L, K, 1.f / 24,
                               P(4), P(5), P(6), aws, NULL),
           LCS_ERR_UNSUPPORTED);
    EXPECT(lcs_cache_append(P(0), NULL, (lcs_kv_dtype)v, P(1), B, T, L, P(2), P(3), NULL, NULL,
                            NULL),
           LCS_ERR_UNSUPPORTED);
    EXPECT(lcs_count_full_layers((lcs_sched)(v + 2), 78, NULL, 0), -1);
    EXPECT(lcs_indexshare_forward(ly, 78, (lcs_sched)(v + 2), NULL, 0, LCS_KV_FP8_E4M3, P(900), B,
                                  T, L, K, 1.f / 24, P(901), P(902), P(903), iws, NULL),
           LCS_ERR_UNSUPPORTED);
    if (strcmp(lcs_status_string((lcs_status)(v + 4)), "unknown status") != 0) return 4;
  }
  printf("capi sanitizer driver ok\n");
  return 0;
}
