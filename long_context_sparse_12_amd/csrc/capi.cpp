// capi.cpp -- the extern "C" boundary: host-side validation, workspace
// sizing, launches, and the IndexShare layer driver.
//
// Validation runs before any HIP call, so every error path can be exercised
// without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/lcs.h"
#include "common.h"

namespace {

thread_local char g_err[512];

lcs_status fail(lcs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

lcs_status ok() {
  g_err[0] = 0;
  return LCS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int32_t kMaxL = 1 << 30;

lcs_status check_dims(int32_t B, int32_t T, int32_t L) {
  if (B <= 0 || T <= 0 || L <= 0)
    return fail(LCS_ERR_SHAPE, "B, T and L must be positive (got %d, %d, %d)", B, T, L);
  if (L > kMaxL) return fail(LCS_ERR_SHAPE, "L = %d exceeds 2^30", L);
  if ((int64_t)B * T > (1LL << 31) - 1) return fail(LCS_ERR_SHAPE, "B*T too large");
  if ((int64_t)B * L > (1LL << 40)) return fail(LCS_ERR_SHAPE, "B*L too large");
  return LCS_OK;
}

lcs_status check_k(int32_t k) {
  if (k < 1 || k > LCS_MAX_TOPK)
    return fail(LCS_ERR_UNSUPPORTED, "k = %d outside [1, %d]", k, LCS_MAX_TOPK);
  return LCS_OK;
}

#define REQUIRE(ptr, name)                                                             \
  do {                                                                                 \
    if (!(ptr)) return fail(LCS_ERR_NULL, "%s is NULL", name);                        \
    if (!aligned16(ptr)) return fail(LCS_ERR_SHAPE, "%s is not 16-byte aligned", name); \
  } while (0)

#define TRY(expr)                     \
  do {                                \
    lcs_status _s = (expr);           \
    if (_s != LCS_OK) return _s;      \
  } while (0)

lcs_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LCS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return LCS_OK;
}

lcs_status validate_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                              const uint8_t* k8, const float* k_scale, const int32_t* vis_len,
                              int32_t B, int32_t T, int32_t L, const float* scores) {
  REQUIRE(q8, "q8");
  REQUIRE(q_scale, "q_scale");
  REQUIRE(w, "w");
  REQUIRE(k8, "k8");
  REQUIRE(k_scale, "k_scale");
  REQUIRE(vis_len, "vis_len");
  REQUIRE(scores, "scores");
  TRY(check_dims(B, T, L));
  return LCS_OK;
}

lcs_status validate_topk(const float* scores, const int32_t* vis_len, int32_t B, int32_t T,
                         int32_t L, int32_t k, const int32_t* idx, const void* ws,
                         size_t ws_bytes) {
  REQUIRE(scores, "scores");
  REQUIRE(vis_len, "vis_len");
  REQUIRE(idx, "idx");
  TRY(check_dims(B, T, L));
  TRY(check_k(k));
  const size_t need = lcs::topk_workspace_bytes((int64_t)B * T, L, k);
  if (!ws) return fail(LCS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(LCS_ERR_SHAPE, "workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(LCS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return LCS_OK;
}

lcs_status validate_attn(const uint16_t* q, const void* kv, int kv_dtype, const float* kv_scale,
                         const int32_t* idx, int32_t B, int32_t T, int32_t L, int32_t k,
                         float sm_scale, const uint16_t* out, const float* lse, const void* ws,
                         size_t ws_bytes) {
  REQUIRE(q, "q");
  REQUIRE(kv, "kv");
  REQUIRE(idx, "idx");
  REQUIRE(out, "out");
  if (lse && !aligned16(lse)) return fail(LCS_ERR_SHAPE, "lse is not 16-byte aligned");
  if (kv_dtype != LCS_KV_BF16 && kv_dtype != LCS_KV_FP8_E4M3)
    return fail(LCS_ERR_UNSUPPORTED, "unknown kv_dtype %d", kv_dtype);
  if (kv_dtype == LCS_KV_FP8_E4M3) {
    REQUIRE(kv_scale, "kv_scale");
  } else if (kv_scale) {
    return fail(LCS_ERR_SHAPE, "kv_scale must be NULL for bf16 kv");
  }
  TRY(check_dims(B, T, L));
  TRY(check_k(k));
  if (!(sm_scale > 0.f) || sm_scale != sm_scale || sm_scale > 1e30f)
    return fail(LCS_ERR_SHAPE, "sm_scale must be a finite positive number");
  const size_t need = lcs::attn_workspace_bytes((int64_t)B * T, k);
  if (need > 0) {
    if (!ws) return fail(LCS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned16(ws)) return fail(LCS_ERR_SHAPE, "workspace is not 16-byte aligned");
    if (ws_bytes < need)
      return fail(LCS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  }
  return LCS_OK;
}

lcs_status validate_append(const uint16_t* k_new, const uint16_t* kv_new, int kv_dtype,
                           const int32_t* pos, int32_t B, int32_t T, int32_t L,
                           const uint8_t* k8, const float* k_scale, const void* kv,
                           const float* kv_scale) {
  if (!k_new && !kv_new) return fail(LCS_ERR_NULL, "k_new and kv_new are both NULL");
  REQUIRE(pos, "pos");
  if (k_new) {
    REQUIRE(k_new, "k_new");
    REQUIRE(k8, "k8");
    REQUIRE(k_scale, "k_scale");
  } else if (k8 || k_scale) {
    return fail(LCS_ERR_SHAPE, "k8 and k_scale must be NULL when k_new is NULL");
  }
  if (kv_dtype != LCS_KV_BF16 && kv_dtype != LCS_KV_FP8_E4M3)
    return fail(LCS_ERR_UNSUPPORTED, "unknown kv_dtype %d", kv_dtype);
  if (kv_new) {
    REQUIRE(kv_new, "kv_new");
    REQUIRE(kv, "kv");
    if (kv_dtype == LCS_KV_FP8_E4M3) {
      REQUIRE(kv_scale, "kv_scale");
    } else if (kv_scale) {
      return fail(LCS_ERR_SHAPE, "kv_scale must be NULL for bf16 kv");
    }
  } else if (kv || kv_scale) {
    return fail(LCS_ERR_SHAPE, "kv and kv_scale must be NULL when kv_new is NULL");
  }
  TRY(check_dims(B, T, L));
  return LCS_OK;
}

// A paged layout: a table of int32 pool blocks, power-of-two blocks of at
// least 64 rows, L within the table, pool rows addressable in int32.
lcs_status validate_paged(const lcs_paged* pg, int32_t L, int* lbs) {
  if (!pg) return fail(LCS_ERR_NULL, "paged layout is NULL");
  REQUIRE(pg->block_table, "block_table");
  const int32_t bs = pg->block_size;
  if (bs < 64 || (bs & (bs - 1)) != 0)
    return fail(LCS_ERR_UNSUPPORTED, "block_size = %d is not a power of two >= 64", bs);
  if (pg->max_blocks <= 0 || pg->n_blocks <= 0)
    return fail(LCS_ERR_SHAPE, "max_blocks and n_blocks must be positive");
  if ((int64_t)pg->max_blocks * bs < L)
    return fail(LCS_ERR_SHAPE, "L = %d exceeds max_blocks * block_size = %lld", L,
                (long long)pg->max_blocks * bs);
  if ((int64_t)pg->n_blocks * bs > 0x7FFFFFFF)
    return fail(LCS_ERR_SHAPE, "n_blocks * block_size must stay below 2^31 rows");
  int l = 0;
  while ((1 << l) < bs) ++l;
  *lbs = l;
  return LCS_OK;
}

bool is_full_layer(lcs_sched sched, int32_t l, const uint8_t* mask) {
  switch (sched) {
    case LCS_SCHED_GROUP4:
      return l % 4 == 0;
    case LCS_SCHED_GLM52:
      return l < 2 || (l - 2) % 4 == 0;
    case LCS_SCHED_ALL_FULL:
      return true;
    case LCS_SCHED_MASK:
      return mask[l] != 0;
  }
  return false;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* lcs_status_string(lcs_status s) {
  switch (s) {
    case LCS_OK: return "ok";
    case LCS_ERR_NULL: return "null pointer";
    case LCS_ERR_SHAPE: return "invalid shape or alignment";
    case LCS_ERR_UNSUPPORTED: return "unsupported argument";
    case LCS_ERR_WORKSPACE: return "workspace missing or too small";
    case LCS_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* lcs_last_error(void) { return g_err; }

lcs_status lcs_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                         const uint8_t* k8, const float* k_scale, const int32_t* vis_len,
                         int32_t B, int32_t T, int32_t L, float* scores, hipStream_t stream) {
  TRY(validate_idx_score(q8, q_scale, w, k8, k_scale, vis_len, B, T, L, scores));
  TRY(hip_status(lcs::launch_idx_score(q8, q_scale, w, k8, k_scale, vis_len, B, T, L, scores,
                                       stream),
                 "idx_score launch"));
  return ok();
}

size_t lcs_topk_workspace_bytes(int32_t B, int32_t T, int32_t L, int32_t k) {
  if (B <= 0 || T <= 0 || L <= 0 || k < 1) return 0;
  return lcs::topk_workspace_bytes((int64_t)B * T, L, k);
}

lcs_status lcs_topk_select(const float* scores, const int32_t* vis_len, int32_t B, int32_t T,
                           int32_t L, int32_t k, int32_t* idx, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  TRY(validate_topk(scores, vis_len, B, T, L, k, idx, workspace, workspace_bytes));
  TRY(hip_status(lcs::launch_topk(scores, vis_len, B * T, L, k, idx, workspace, stream),
                 "topk launch"));
  return ok();
}

size_t lcs_attn_workspace_bytes(int32_t B, int32_t T, int32_t k) {
  if (B <= 0 || T <= 0 || k < 1) return 0;
  return lcs::attn_workspace_bytes((int64_t)B * T, k);
}

lcs_status lcs_sparse_mla_attn(const uint16_t* q, const void* kv, lcs_kv_dtype kv_dtype,
                               const float* kv_scale, const int32_t* idx, int32_t B, int32_t T,
                               int32_t L, int32_t k, float sm_scale, uint16_t* out, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  TRY(validate_attn(q, kv, (int)kv_dtype, kv_scale, idx, B, T, L, k, sm_scale, out, lse,
                    workspace, workspace_bytes));
  TRY(hip_status(lcs::launch_sparse_mla(q, kv, kv_dtype == LCS_KV_FP8_E4M3, kv_scale, idx, B, T,
                                        L, k, sm_scale, out, lse, workspace, stream),
                 "sparse_mla launch"));
  return ok();
}

lcs_status lcs_quantize_e4m3(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes,
                             float* scales, hipStream_t stream) {
  if (D != LCS_IDX_DIM && D != LCS_KV_DIM)
    return fail(LCS_ERR_UNSUPPORTED, "row width D = %d is not 128 or 576", D);
  if (rows < 0 || rows > (1LL << 40) / D)
    return fail(LCS_ERR_SHAPE, "rows = %lld outside [0, 2^40 / D]", (long long)rows);
  if (rows == 0) return ok();
  REQUIRE(x, "x");
  REQUIRE(codes, "codes");
  REQUIRE(scales, "scales");
  TRY(hip_status(lcs::launch_quantize_e4m3(x, rows, D, codes, scales, stream),
                 "quantize launch"));
  return ok();
}

lcs_status lcs_cache_append(const uint16_t* k_new, const uint16_t* kv_new, lcs_kv_dtype kv_dtype,
                            const int32_t* pos, int32_t B, int32_t T, int32_t L, uint8_t* k8,
                            float* k_scale, void* kv, float* kv_scale, hipStream_t stream) {
  TRY(validate_append(k_new, kv_new, (int)kv_dtype, pos, B, T, L, k8, k_scale, kv, kv_scale));
  TRY(hip_status(lcs::launch_cache_append(k_new, kv_new, kv_dtype == LCS_KV_FP8_E4M3, pos, B, T,
                                          L, k8, k_scale, kv, kv_scale, nullptr, 0, 0, 0, stream),
                 "cache_append launch"));
  return ok();
}

lcs_status lcs_topk_candidates(const float* scores, const int32_t* idx, int32_t B, int32_t T,
                               int32_t L, int32_t k, int32_t pos_base, float* cand_score,
                               int32_t* cand_idx, hipStream_t stream) {
  REQUIRE(scores, "scores");
  REQUIRE(idx, "idx");
  REQUIRE(cand_score, "cand_score");
  REQUIRE(cand_idx, "cand_idx");
  TRY(check_dims(B, T, L));
  TRY(check_k(k));
  if (pos_base < 0 || (int64_t)pos_base + L > 0x7FFFFFFF)
    return fail(LCS_ERR_SHAPE, "pos_base = %d: positions pos_base + [0, L) must fit in int32",
                pos_base);
  TRY(hip_status(lcs::launch_topk_candidates(scores, idx, (int64_t)B * T, L, k, pos_base,
                                             cand_score, cand_idx, stream),
                 "topk_candidates launch"));
  return ok();
}

lcs_status lcs_topk_merge(const float* cand_score, const int32_t* cand_idx, int32_t G, int32_t B,
                          int32_t T, int32_t k_in, int32_t k, int32_t* idx, hipStream_t stream) {
  REQUIRE(cand_score, "cand_score");
  REQUIRE(cand_idx, "cand_idx");
  REQUIRE(idx, "idx");
  if (G <= 0 || k_in <= 0) return fail(LCS_ERR_SHAPE, "G and k_in must be positive");
  if ((int64_t)G * k_in > LCS_MAX_MERGE_CANDIDATES)
    return fail(LCS_ERR_UNSUPPORTED, "G * k_in = %lld exceeds %d candidates per query",
                (long long)G * k_in, LCS_MAX_MERGE_CANDIDATES);
  TRY(check_dims(B, T, 1));
  TRY(check_k(k));
  TRY(hip_status(lcs::launch_topk_merge(cand_score, cand_idx, G, (int64_t)B * T, k_in, k, idx,
                                        stream),
                 "topk_merge launch"));
  return ok();
}

lcs_status lcs_idx_localize(const int32_t* idx, int32_t B, int32_t T, int32_t k, int32_t lo,
                            int32_t hi, int32_t* local, hipStream_t stream) {
  REQUIRE(idx, "idx");
  REQUIRE(local, "local");
  if (idx == local) return fail(LCS_ERR_SHAPE, "idx and local must not alias");
  TRY(check_dims(B, T, 1));
  TRY(check_k(k));
  if (lo < 0 || hi < lo) return fail(LCS_ERR_SHAPE, "need 0 <= lo <= hi (got %d, %d)", lo, hi);
  TRY(hip_status(lcs::launch_idx_localize(idx, (int64_t)B * T, k, lo, hi, local, stream),
                 "idx_localize launch"));
  return ok();
}

lcs_status lcs_lse_combine(const uint16_t* part_out, const float* part_lse, int32_t G, int32_t B,
                           int32_t T, uint16_t* out, float* lse, hipStream_t stream) {
  REQUIRE(part_out, "part_out");
  REQUIRE(part_lse, "part_lse");
  REQUIRE(out, "out");
  if (lse && !aligned16(lse)) return fail(LCS_ERR_SHAPE, "lse is not 16-byte aligned");
  if (G <= 0 || G > LCS_MAX_SHARDS)
    return fail(LCS_ERR_SHAPE, "G = %d outside [1, %d]", G, LCS_MAX_SHARDS);
  TRY(check_dims(B, T, 1));
  TRY(hip_status(lcs::launch_lse_combine(part_out, part_lse, G, (int64_t)B * T, out, lse, stream),
                 "lse_combine launch"));
  return ok();
}

lcs_status lcs_idx_score_paged(const uint8_t* q8, const float* q_scale, const float* w,
                               const uint8_t* k8_pool, const float* k_scale_pool,
                               const lcs_paged* paged, const int32_t* vis_len, int32_t B,
                               int32_t T, int32_t L, float* scores, hipStream_t stream) {
  TRY(validate_idx_score(q8, q_scale, w, k8_pool, k_scale_pool, vis_len, B, T, L, scores));
  int lbs = 0;
  TRY(validate_paged(paged, L, &lbs));
  TRY(hip_status(lcs::launch_idx_score_paged(q8, q_scale, w, k8_pool, k_scale_pool,
                                             paged->block_table, paged->max_blocks, lbs,
                                             paged->n_blocks, vis_len, B, T, L, scores, stream),
                 "idx_score launch"));
  return ok();
}

lcs_status lcs_sparse_mla_attn_paged(const uint16_t* q, const void* kv_pool,
                                     lcs_kv_dtype kv_dtype, const float* kv_scale_pool,
                                     const lcs_paged* paged, const int32_t* idx, int32_t B,
                                     int32_t T, int32_t L, int32_t k, float sm_scale,
                                     uint16_t* out, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  TRY(validate_attn(q, kv_pool, (int)kv_dtype, kv_scale_pool, idx, B, T, L, k, sm_scale, out, lse,
                    workspace, workspace_bytes));
  int lbs = 0;
  TRY(validate_paged(paged, L, &lbs));
  TRY(hip_status(lcs::launch_sparse_mla_paged(q, kv_pool, kv_dtype == LCS_KV_FP8_E4M3,
                                              kv_scale_pool, paged->block_table,
                                              paged->max_blocks, lbs, paged->n_blocks, idx, B, T,
                                              L, k, sm_scale, out, lse, workspace, stream),
                 "sparse_mla launch"));
  return ok();
}

lcs_status lcs_cache_append_paged(const uint16_t* k_new, const uint16_t* kv_new,
                                  lcs_kv_dtype kv_dtype, const int32_t* pos, int32_t B, int32_t T,
                                  int32_t L, const lcs_paged* paged, uint8_t* k8_pool,
                                  float* k_scale_pool, void* kv_pool, float* kv_scale_pool,
                                  hipStream_t stream) {
  TRY(validate_append(k_new, kv_new, (int)kv_dtype, pos, B, T, L, k8_pool, k_scale_pool, kv_pool,
                      kv_scale_pool));
  int lbs = 0;
  TRY(validate_paged(paged, L, &lbs));
  TRY(hip_status(lcs::launch_cache_append(k_new, kv_new, kv_dtype == LCS_KV_FP8_E4M3, pos, B, T, L,
                                          k8_pool, k_scale_pool, kv_pool, kv_scale_pool,
                                          paged->block_table, paged->max_blocks, lbs,
                                          paged->n_blocks, stream),
                 "cache_append launch"));
  return ok();
}

int32_t lcs_count_full_layers(lcs_sched sched, int32_t n_layers, const uint8_t* full_mask,
                              int32_t mtp_steps) {
  if (n_layers <= 0 || mtp_steps < 0) return -1;
  if (mtp_steps > 0) return mtp_steps == n_layers ? 1 : -1;
  if ((int)sched < 0 || (int)sched > 3) return -1;
  if (sched == LCS_SCHED_MASK && !full_mask) return -1;
  int32_t n = 0;
  for (int32_t l = 0; l < n_layers; ++l) n += is_full_layer(sched, l, full_mask) ? 1 : 0;
  return n;
}

size_t lcs_indexshare_workspace_bytes(int32_t B, int32_t T, int32_t L, int32_t k) {
  if (B <= 0 || T <= 0 || L <= 0 || k < 1) return 0;
  return align256(lcs::topk_workspace_bytes((int64_t)B * T, L, k)) +
         align256(lcs::attn_workspace_bytes((int64_t)B * T, k));
}

lcs_status lcs_indexshare_forward(const lcs_layer* layers, int32_t n_layers, lcs_sched sched,
                                  const uint8_t* full_mask, int32_t mtp_steps,
                                  lcs_kv_dtype kv_dtype, const int32_t* vis_len, int32_t B,
                                  int32_t T, int32_t L, int32_t k, float sm_scale,
                                  float* scores_scratch, int32_t* idx_out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (!layers) return fail(LCS_ERR_NULL, "layers is NULL");
  if (n_layers <= 0) return fail(LCS_ERR_SHAPE, "n_layers must be positive");
  if (mtp_steps < 0) return fail(LCS_ERR_SHAPE, "mtp_steps must be >= 0");
  if (mtp_steps > 0 && mtp_steps != n_layers)
    return fail(LCS_ERR_SHAPE, "mtp_steps (%d) must equal n_layers (%d)", mtp_steps, n_layers);
  if (mtp_steps == 0) {
    if ((int)sched < 0 || (int)sched > 3)
      return fail(LCS_ERR_UNSUPPORTED, "unknown schedule %d", (int)sched);
    if (sched == LCS_SCHED_MASK && !full_mask) return fail(LCS_ERR_NULL, "full_mask is NULL");
    if (!is_full_layer(sched, 0, full_mask))
      return fail(LCS_ERR_SHAPE, "layer 0 must run its own indexer");
  }
  REQUIRE(scores_scratch, "scores_scratch");
  REQUIRE(idx_out, "idx_out");
  REQUIRE(vis_len, "vis_len");
  TRY(check_dims(B, T, L));
  TRY(check_k(k));
  const size_t need = lcs_indexshare_workspace_bytes(B, T, L, k);
  if (!workspace) return fail(LCS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(workspace)) return fail(LCS_ERR_SHAPE, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(LCS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  char* ws_topk = (char*)workspace;
  char* ws_attn = ws_topk + align256(lcs::topk_workspace_bytes((int64_t)B * T, L, k));
  const size_t ws_attn_bytes = lcs::attn_workspace_bytes((int64_t)B * T, k);

  // validate every layer before launching anything
  for (int32_t l = 0; l < n_layers; ++l) {
    const lcs_layer& ly = layers[l];
    const bool full = mtp_steps > 0 ? l == 0 : is_full_layer(sched, l, full_mask);
    const lcs_layer& kvl = mtp_steps > 0 ? layers[0] : ly;
    lcs_status s;
    if (full) {
      s = validate_idx_score(ly.q8, ly.q_scale, ly.w, ly.k8, ly.k_scale, vis_len, B, T, L,
                             scores_scratch);
      if (s != LCS_OK) return fail(s, "layer %d indexer: %s", l, g_err);
    }
    s = validate_attn(ly.q, kvl.kv, (int)kv_dtype, kvl.kv_scale, idx_out, B, T, L, k, sm_scale,
                      ly.out, ly.lse, ws_attn, ws_attn_bytes);
    if (s != LCS_OK) return fail(s, "layer %d attention: %s", l, g_err);
  }

  const size_t per = (size_t)B * T * k;
  // One query per sequence: the indexer also builds the selection's first
  // histogram. The selection re-zeroes it, so one clear serves every full layer.
  const bool fused_hist = T == 1 && lcs::topk_takes_prebuilt_hist((int64_t)B * T, L);
  if (fused_hist)
    TRY(hip_status(lcs::launch_topk_clear(ws_topk, B * T, L, stream), "topk clear launch"));
  int32_t* cur = nullptr;
  int32_t nfull = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    const lcs_layer& ly = layers[l];
    const bool full = mtp_steps > 0 ? l == 0 : is_full_layer(sched, l, full_mask);
    if (full) {
      cur = idx_out + (size_t)nfull * per;
      ++nfull;
      if (fused_hist) {
        TRY(hip_status(lcs::launch_idx_score_hist(ly.q8, ly.q_scale, ly.w, ly.k8, ly.k_scale,
                                                  vis_len, B, L, scores_scratch,
                                                  lcs::topk_hist_area(ws_topk, B, L), stream),
                       "idx_score launch"));
        TRY(hip_status(lcs::launch_topk_prebuilt(scores_scratch, vis_len, B, L, k, cur, ws_topk,
                                                 stream),
                       "topk launch"));
      } else {
        TRY(hip_status(lcs::launch_idx_score(ly.q8, ly.q_scale, ly.w, ly.k8, ly.k_scale, vis_len,
                                             B, T, L, scores_scratch, stream),
                       "idx_score launch"));
        TRY(hip_status(lcs::launch_topk(scores_scratch, vis_len, B * T, L, k, cur, ws_topk, stream),
                       "topk launch"));
      }
    }
    // KV Share: every MTP draft step reads the first step's cache
    const lcs_layer& kvl = mtp_steps > 0 ? layers[0] : ly;
    TRY(hip_status(lcs::launch_sparse_mla(ly.q, kvl.kv, kv_dtype == LCS_KV_FP8_E4M3, kvl.kv_scale,
                                          cur, B, T, L, k, sm_scale, ly.out, ly.lse, ws_attn,
                                          stream),
                   "sparse_mla launch"));
  }
  return ok();
}

}  // extern "C"
