/*
 * oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU implementation of what the DSA +
 * IndexShare attention path computes, in double precision. It shares no code,
 * header, table or constant with the HIP library, and neither side includes or
 * links the other. Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load it; the product path never does.
 *
 * What is computed (sources are the five GLM-5.2 pages):
 *  - "一枚 Token，怎样穿过 78 层" (ailearn GLM-5.2 special edition), panel
 *    "MLA 压缩，DSA 精读": an indexer scans the whole history, then core
 *    attention reads only the Top-2,048; the architecture table gives 64
 *    attention heads, 32 indexer heads and a rank-512 joint KV compression.
 *  - "IndexShare：省掉3/4的索引计算" (Hygon DCU forum post): the indexer picks
 *    each query's most relevant top-k tokens, core attention drops from
 *    O(L^2) to O(Lk), the indexer itself stays O(L^2).
 *  - "IndexShare：四层共用一次搜索结果" (ailearn special edition): full
 *    indexers on 0-based layers 0, 1, 2, 6, 10, ..., 74; every other layer
 *    reuses the previous Top-2,048.
 *  - "MTP：同一位速记员，多猜几枚未来 Token" (same page) and "推理优化"
 *    (engineering-report wiki): the first draft step computes the top-k, later
 *    draft steps reuse those positions and the first step's KV.
 * The pages do not give the indexer formula, the number formats, the tie rule
 * or the order of the returned positions; the readings taken are stated at
 * each function.
 *
 * Every function returns 0 on success, nonzero on invalid input.
 */
#ifndef LCS_ORACLE_H
#define LCS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OCP FP8 E4M3 (bias 7, no infinities, 0x7F/0xFF are NaN) -> double */
double oracle_e4m3(uint8_t code);
/* bf16 bits -> double (exact) */
double oracle_bf16(uint16_t bits);
/* double -> bf16 bits, round to nearest even (finite inputs) */
uint16_t oracle_round_bf16(double x);

/* finite double -> E4M3 code: saturate to +-448, nearest code, ties to the
 * even code, sign kept (so -0.0 and small negatives give 0x80) */
uint8_t oracle_encode_e4m3(double v);

/* Row quantisation. x [rows][D] bf16 -> codes [rows][D] E4M3, scales [rows]
 * fp32: scale = fl32(max|x| / 448) (1 for an all-zero row), code =
 * oracle_encode_e4m3(fl32(x / scale)). Rows with a non-finite value are
 * rejected. */
int oracle_quantize_e4m3(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes,
                         float* scales);

/* Cache append. k_new [B][T][128] bf16 (nullable), kv_new [B][T][576] bf16
 * (nullable, not both NULL), pos [B][T]: token (b, t) goes to row pos[b,t] of
 * sequence b; positions outside [0, L) are skipped, repeated positions within
 * a sequence are rejected. Keys: k8 [B][L][128] codes + k_scale [B][L], by
 * oracle_quantize_e4m3. Latents: kv [B][L][576] bf16 copied as is (kv_fp8 = 0)
 * or quantised into codes + kv_scale [B][L] (kv_fp8 = 1). Rows not addressed
 * are left untouched. */
int oracle_cache_append(const uint16_t* k_new, const uint16_t* kv_new, int32_t kv_fp8,
                        const int32_t* pos, int32_t B, int32_t T, int32_t L,
                        uint8_t* k8, float* k_scale, void* kv, float* kv_scale);

/* Indexer scores.
 * q8 [B][T][32][128] e4m3 codes, q_scale [B][T][32], w [B][T][32],
 * k8 [B][L][128] e4m3 codes, k_scale [B][L], vis_len [B][T] (clamped to
 * [0, L]). scores [B][T][L] fp32: for s < vis_len,
 *   I = k_scale[s] * sum_j w[j] * q_scale[j] * relu(sum_i q8[j][i] * k8[s][i])
 * with decoded codes, evaluated in double and rounded once to fp32;
 * -inf for s >= vis_len. scores64 (nullable) receives the double values
 * (-inf likewise). */
int oracle_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                     const uint8_t* k8, const float* k_scale,
                     const int32_t* vis_len, int32_t B, int32_t T, int32_t L,
                     float* scores, double* scores64);

/* Top-k per (b, t): among s < vis_len, order by (score descending, s
 * ascending) and keep the first min(k, vis_len); return them in ascending
 * position order, padded with -1 up to k. idx [B][T][k]. NaN scores are
 * rejected. */
int oracle_topk(const float* scores, const int32_t* vis_len, int32_t B,
                int32_t T, int32_t L, int32_t k, int32_t* idx);

/* Sparse MLA attention, absorbed form.
 * q [B][T][64][576] bf16; kv [B][L][576] bf16 (kv_fp8 = 0) or e4m3 codes
 * with kv_scale [B][L] (kv_fp8 = 1); idx [B][T][k] (-1 = empty slot).
 * For each (b, t, h): z_i = sm_scale * q . kv[idx_i] over 576 dims;
 * out = softmax(z) . kv[idx_i][0:512]; lse = log sum exp z. No valid index:
 * out = 0, lse = -inf. out [B][T][64][512] bf16, lse [B][T][64] fp32;
 * out64 (nullable) receives the double outputs before rounding. */
int oracle_sparse_mla(const uint16_t* q, const void* kv, int32_t kv_fp8,
                      const float* kv_scale, const int32_t* idx, int32_t B,
                      int32_t T, int32_t L, int32_t k, double sm_scale,
                      uint16_t* out, float* lse, double* out64);

/* Context-parallel halves (a shard holds positions [lo, lo + L_shard)):
 * candidates of a shard's selection: (scores[q][idx], idx + pos_base), or
 * (-inf, -1) for an empty slot. scores [Q][L], idx [Q][k]. */
int oracle_topk_candidates(const float* scores, const int32_t* idx, int32_t Q, int32_t L,
                           int32_t k, int32_t pos_base, float* cand_score, int32_t* cand_idx);
/* selection from G shards' candidates cand_* [G][Q][k_in] (cand_idx < 0 =
 * none): order by (score desc, position asc), keep min(k, count), ascending,
 * -1 padded, idx [Q][k]. Repeated positions and NaN scores are rejected. */
int oracle_topk_merge(const float* cand_score, const int32_t* cand_idx, int32_t G, int32_t Q,
                      int32_t k_in, int32_t k, int32_t* idx);
/* entries of each ascending list idx [Q][k] in [lo, hi), minus lo, then -1 */
int oracle_idx_localize(const int32_t* idx, int32_t Q, int32_t k, int32_t lo, int32_t hi,
                        int32_t* local);
/* out = sum_g w_g out_g / sum_g w_g, w_g = exp(lse_g - max lse), lse = max +
 * log sum w, in double. part_out [G][Q][64][512] bf16, part_lse [G][Q][64];
 * out [Q][64][512] bf16, lse [Q][64] (nullable), out64 (nullable). */
int oracle_lse_combine(const uint16_t* part_out, const float* part_lse, int32_t G, int32_t Q,
                       uint16_t* out, float* lse, double* out64);

/* IndexShare layer schedules */
enum { ORACLE_SCHED_GROUP4 = 0, ORACLE_SCHED_GLM52 = 1, ORACLE_SCHED_ALL_FULL = 2,
       ORACLE_SCHED_MASK = 3 };
/* 1 if layer l runs its own indexer under the schedule, 0 if it reuses */
int oracle_is_full_layer(int32_t sched, int32_t l, const uint8_t* mask);

typedef struct {
  const uint8_t* q8;
  const float* q_scale;
  const float* w;
  const uint8_t* k8;
  const float* k_scale;
  const uint16_t* q;
  const void* kv;
  const float* kv_scale;
  uint16_t* out;
  float* lse;
} oracle_layer;

/* One decode/prefill pass over n_layers layers. Full layers score, select
 * and attend; the other layers attend with the latest full layer's idx.
 * mtp_steps > 0: layers[] are mtp_steps draft steps of one shared layer;
 * step 0 runs the indexer, every step attends with step 0's idx over step
 * 0's kv/kv_scale (the layers' own q). idx_out [n_full][B][T][k] receives
 * each full layer's selection in order. */
int oracle_indexshare(const oracle_layer* layers, int32_t n_layers,
                      int32_t sched, const uint8_t* mask, int32_t mtp_steps,
                      int32_t kv_fp8, const int32_t* vis_len, int32_t B,
                      int32_t T, int32_t L, int32_t k, double sm_scale,
                      int32_t* idx_out);

#ifdef __cplusplus
}
#endif

#endif
