/*
 * lcs.h -- C ABI of the MI355X (gfx950) DSA + IndexShare attention path.
 *
 * Three stages, as the GLM-5.2 pages describe the attention of one layer
 * ("一枚 Token，怎样穿过 78 层", panel "MLA 压缩，DSA 精读", ailearn GLM-5.2
 * special edition; and "IndexShare：省掉3/4的索引计算", Hygon DCU forum post):
 * a light indexer scores every cached position for each query, a Top-2,048
 * selection keeps the best positions, and core attention reads only those
 * latent-KV rows. IndexShare ("IndexShare：四层共用一次搜索结果", same special
 * edition) runs the indexer on some layers and lets the following layers reuse
 * the selection; the MTP draft steps reuse it too ("MTP：同一位速记员，多猜几枚
 * 未来 Token": IndexShare and KV Share).
 *
 * Fixed shapes: 32 indexer heads x 128 dims (the pages give the 32 heads;
 * 128 is a reading), 64 attention heads ("Attention 64 Heads"), latent KV rows
 * of 512 latent dims ("KV 低秩联合压缩 Rank 512") plus 64 rope dims (a reading
 * of the absorbed MLA form), so 576 dims per cached row.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *    row-major in the order given, and 16-byte aligned; the key and latent
 *    caches of lcs_idx_score and lcs_sparse_mla_attn may instead place the
 *    sequences a batch stride apart (a view of a larger cache). bf16 values are
 *    passed as uint16_t bit patterns. FP8 values are OCP E4M3 codes (bias 7,
 *    max 448).
 *  - Outputs (and workspaces) must not overlap any other buffer of the call;
 *    inputs may share memory. A call whose byte ranges break this returns
 *    LCS_ERR_SHAPE naming the two buffers.
 *  - Calls are asynchronous on `stream` (NULL = the default stream). The
 *    library never allocates, frees or synchronises, and keeps no state
 *    between calls except inside caller-provided workspaces.
 *  - Arguments are validated on the host before any launch. On failure the
 *    call returns a nonzero lcs_status, launches nothing, and lcs_last_error()
 *    gives a thread-local description. Launch failures return LCS_ERR_HIP.
 *    Device faults surface at the caller's next synchronisation.
 *  - vis_len values are read on the device and clamped to [0, L].
 *  - Workspaces are scratch device memory of at least the queried size, with
 *    any content: each call initialises what it uses. One allocation serves
 *    any number of calls and shapes up to its size. Calls that share a
 *    workspace must not overlap in time (use one stream, or one workspace per
 *    stream).
 */
#ifndef LCS_H
#define LCS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
  LCS_OK = 0,
  LCS_ERR_NULL = 1,        /* a required pointer is NULL */
  LCS_ERR_SHAPE = 2,       /* a size is out of range, a pointer misaligned, or an output
                              overlaps another buffer */
  LCS_ERR_UNSUPPORTED = 3, /* k outside [1, 2048], an unknown enum value */
  LCS_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
  LCS_ERR_HIP = 5          /* a HIP launch or runtime call failed */
} lcs_status;

typedef enum { LCS_KV_BF16 = 0, LCS_KV_FP8_E4M3 = 1 } lcs_kv_dtype;

#define LCS_IDX_HEADS 32
#define LCS_IDX_DIM 128
#define LCS_ATT_HEADS 64
#define LCS_KV_LATENT 512
#define LCS_KV_ROPE 64
#define LCS_KV_DIM 576
#define LCS_MAX_TOPK 2048
#define LCS_MAX_MERGE_CANDIDATES 32768 /* G * k_in of lcs_topk_merge */
#define LCS_MAX_SHARDS 1024            /* G of lcs_lse_combine */

/* Indexer scores ("Indexer 先扫历史": every cached position is scored).
 * q8      [B][T][32][128] E4M3 query codes
 * q_scale [B][T][32]      fp32 dequantisation scale per (query, head), > 0
 * w       [B][T][32]      fp32 head weights
 * k8      [B][L][128]     E4M3 key codes;  k_scale [B][L] fp32 per-key scale;
 *                         sequence b's rows start at row b * k_batch_stride of
 *                         both (k_batch_stride >= L; L for a dense cache), so
 *                         a cache of more positions can be scored on its
 *                         first L
 * vis_len [B][T]          int32 visible prefix length of each query (L < 2^30)
 * scores  [B][T][L]       fp32 output:
 *   scores[b,t,s] = k_scale[s] * sum_j w[j]*q_scale[j] * relu(q8[j] . k8[s])
 *   for s < vis_len[b,t], -inf otherwise.
 * T < 16 uses a key-streaming kernel (one pass over the keys per group of
 * up to 6 queries, the 32 heads as the FP8 MFMA M dimension); T >= 16 uses a
 * tiled FP8 MFMA kernel. */
lcs_status lcs_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                         const uint8_t* k8, const float* k_scale, int64_t k_batch_stride,
                         const int32_t* vis_len, int32_t B, int32_t T, int32_t L,
                         float* scores, hipStream_t stream);

/* Workspace bytes needed by lcs_topk_select for these sizes. */
size_t lcs_topk_workspace_bytes(int32_t B, int32_t T, int32_t L, int32_t k);

/* Top-k selection ("核心 Attention 只精看 Top-2,048").
 * scores [B][T][L] fp32 (no NaN), vis_len [B][T] -> idx [B][T][k] int32:
 * the min(k, vis_len) positions s < vis_len with the largest scores, equal
 * scores broken by the lower position, listed in ascending position order and
 * padded with -1. k in [1, 2048]. Exact (radix select on the fp32 bit
 * patterns; -0.0 counts as +0.0). */
lcs_status lcs_topk_select(const float* scores, const int32_t* vis_len, int32_t B,
                           int32_t T, int32_t L, int32_t k, int32_t* idx,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Workspace bytes needed by lcs_sparse_mla_attn for these sizes. */
size_t lcs_attn_workspace_bytes(int32_t B, int32_t T, int32_t k);

/* Sparse MLA attention over the selected rows, absorbed form.
 * q   [B][T][64][576] bf16
 * kv  [B][L][576] bf16 (LCS_KV_BF16), or E4M3 codes with kv_scale [B][L]
 *     fp32 (LCS_KV_FP8_E4M3; kv_scale must be NULL for bf16); sequence b's
 *     rows start at row b * kv_batch_stride of both (kv_batch_stride >= L; L
 *     for a dense cache)
 * idx [B][T][k] int32 positions in [0, L), or -1 for an empty slot
 * out [B][T][64][512] bf16 = softmax_i(sm_scale * q . kv[idx_i]) . kv[idx_i][0:512]
 * lse [B][T][64] fp32 natural-log sum of exp of the scaled logits (nullable);
 * a query with no valid index gets out = 0 and lse = -inf.
 * The kernels gather the sequence's position 0 for each -1 slot and weight it
 * zero: position 0 of a sequence with any valid index must hold finite
 * values (the first token's row always does); a query with no valid index
 * outputs zeros whatever that row holds.
 * Positions outside [-1, L) are a caller error (not checked on the device). */
lcs_status lcs_sparse_mla_attn(const uint16_t* q, const void* kv,
                               lcs_kv_dtype kv_dtype, const float* kv_scale,
                               int64_t kv_batch_stride, const int32_t* idx, int32_t B,
                               int32_t T, int32_t L,
                               int32_t k, float sm_scale, uint16_t* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* lcs_sparse_mla_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid hipMalloc). When the selection is split over several workgroups
 * (fewer queries than the GPU has compute units), the partial outputs go to a
 * static device array of 20 MiB that the library holds on every GPU it runs
 * on until the process ends; that covers any B * T with k <= 2048 whose
 * lcs_attn_workspace_bytes(B, T, k) is at most 20 MiB (for example 32 decode
 * queries, or 1 - 16), and larger needs return LCS_ERR_WORKSPACE. The call
 * allocates nothing and needs no clearing (each call writes every partial it
 * reads). Calls on one GPU share the array: two of them in flight at once on
 * different streams race, so a caller runs them on one stream (or otherwise
 * one after the other). Otherwise the same as lcs_sparse_mla_attn. */
lcs_status lcs_sparse_mla_attn_noalloc(const uint16_t* q, const void* kv,
                                       lcs_kv_dtype kv_dtype, const float* kv_scale,
                                       int64_t kv_batch_stride, const int32_t* idx, int32_t B,
                                       int32_t T, int32_t L, int32_t k, float sm_scale,
                                       uint16_t* out, float* lse, hipStream_t stream);

/* One layer of the composite call. The indexer fields are read only on
 * layers that run their own indexer; q/kv/out are used on every layer. */
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
} lcs_layer;

/* Which layers run their own indexer ("IndexShare：四层共用一次搜索结果").
 *  GROUP4   : layer l is full iff l % 4 == 0 (one computing layer and three
 *             reusing layers per group of four)
 *  GLM52    : layers 0 and 1, then 2, 6, 10, ... (every fourth from 2); for
 *             78 layers that is 21 full and 57 reusing layers
 *  ALL_FULL : every layer (IndexShare off)
 *  MASK     : full_mask[l] != 0 (host array of n_layers bytes)
 * Layer 0 must be full. */
typedef enum {
  LCS_SCHED_GROUP4 = 0,
  LCS_SCHED_GLM52 = 1,
  LCS_SCHED_ALL_FULL = 2,
  LCS_SCHED_MASK = 3
} lcs_sched;

/* Number of layers that run their own indexer (the leading dimension of
 * idx_out), or -1 for invalid arguments. mtp_steps > 0 gives 1. */
int32_t lcs_count_full_layers(lcs_sched sched, int32_t n_layers,
                              const uint8_t* full_mask, int32_t mtp_steps);

/* Workspace bytes needed by lcs_indexshare_forward for these sizes. */
size_t lcs_indexshare_workspace_bytes(int32_t B, int32_t T, int32_t L, int32_t k);

/* The whole path over n_layers layers (layers is a HOST array). For each
 * layer in order: a full layer runs lcs_idx_score into scores_scratch
 * [B][T][L] and lcs_topk_select into the next slot of idx_out
 * [n_full][B][T][k]; every layer then runs lcs_sparse_mla_attn with the
 * latest full layer's selection. mtp_steps > 0 (MTP draft reuse): layers[]
 * holds mtp_steps draft steps of one layer; step 0 runs the indexer, and
 * every step attends with step 0's selection over step 0's kv/kv_scale (KV
 * Share), each with its own q, out and lse. With LCS_ROCTX=1 in the
 * environment each layer's launches sit in a roctx range ("lcs layer 6
 * shared", "lcs layer 2 full") for rocprofv3 --marker-trace; the roctx
 * library is loaded at run time, and is not needed otherwise. */
lcs_status lcs_indexshare_forward(const lcs_layer* layers, int32_t n_layers,
                                  lcs_sched sched, const uint8_t* full_mask,
                                  int32_t mtp_steps, lcs_kv_dtype kv_dtype,
                                  const int32_t* vis_len, int32_t B, int32_t T,
                                  int32_t L, int32_t k, float sm_scale,
                                  float* scores_scratch, int32_t* idx_out,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Per-row FP8 quantisation. The pages keep the KV cache in FP8 (training
 * section of "GLM-5.2 — 1M上下文开放权重的长程任务旗舰"; the `fp8_ds_mla` cache
 * type of the vLLM launch in "IndexShare：省掉3/4的索引计算", Hygon DCU forum
 * post) and name E4M3 as the release's FP8 format; the row scaling is a
 * reading:
 * x      [rows][D] bf16, finite values (other rows get unspecified bytes)
 * codes  [rows][D] E4M3 output, scales [rows] fp32 output:
 *   scale = fl32(max|x| / 448), or 1 for an all-zero row;
 *   code  = E4M3(fl32(x / scale)), saturated at +-448, nearest, ties to the
 *           even code, sign kept (so -0.0 gives 0x80).
 * D is 128 (indexer keys; indexer queries, one row per (token, head)) or 576
 * (latent KV rows). rows = 0 launches nothing. Decoding code * scale gives
 * back x to within half an E4M3 step. */
lcs_status lcs_quantize_e4m3(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes,
                             float* scales, hipStream_t stream);

/* Cache append: the T new tokens of each sequence enter the caches the
 * indexer and attention read (same passages as lcs_quantize_e4m3).
 * k_new  [B][T][128] bf16 indexer keys, or NULL for a layer that keeps no key
 *        cache (an IndexShare layer that reuses another layer's selection);
 *        k8 [B][L][128] and k_scale [B][L] receive the quantised rows (both
 *        NULL when k_new is NULL)
 * kv_new [B][T][576] bf16 latent rows, or NULL; kv [B][L][576] receives them
 *        as bf16 (LCS_KV_BF16, kv_scale NULL) or as E4M3 codes with kv_scale
 *        [B][L] (LCS_KV_FP8_E4M3), quantised as in lcs_quantize_e4m3
 * pos    [B][T] int32 device array: token (b, t) goes to row pos[b,t] of
 *        sequence b (a decode step at length n passes n; a prefill chunk or
 *        an accepted draft run passes consecutive positions). Positions
 *        outside [0, L) are skipped, so -1 marks a token not to store. Two
 *        tokens of one sequence with the same position race (caller error,
 *        not checked on the device).
 * At least one of k_new and kv_new is given. Rows not addressed by pos are
 * left as they are. */
lcs_status lcs_cache_append(const uint16_t* k_new, const uint16_t* kv_new, lcs_kv_dtype kv_dtype,
                            const int32_t* pos, int32_t B, int32_t T, int32_t L, uint8_t* k8,
                            float* k_scale, void* kv, float* kv_scale, hipStream_t stream);

/* Context parallelism: the single-device halves. Context parallelism splits
 * the KV pool over devices (panel "CP · EP · P/D · HiCache", ailearn GLM-5.2
 * special edition); the pages do not say how the selection and the attention
 * are put back together. A shard holds positions [lo, lo + L_shard) of every
 * sequence (its own k8/kv of L = L_shard rows, vis_len clamped to the shard)
 * and runs lcs_idx_score + lcs_topk_select on them. The whole sequence's
 * top-k lies inside the union of the shards' top-k's, so:
 *   1. lcs_topk_candidates turns each shard's selection into (score, global
 *      position) pairs;
 *   2. the pairs of all G shards are gathered (on one device: written side by
 *      side; across devices: an all-gather) as cand_* [G][B][T][k_in];
 *   3. lcs_topk_merge selects from them exactly what lcs_topk_select would
 *      have selected over the whole sequence;
 *   4. lcs_idx_localize gives each shard its share of the merged list;
 *      each shard runs lcs_sparse_mla_attn with it over its own rows;
 *   5. lcs_lse_combine merges the G shard outputs [G][B][T][...] (gathered
 *      likewise) into the attention over all selected rows. */

/* Candidates of one shard's selection.
 * scores [B][T][L] fp32 (the shard's lcs_idx_score output), idx [B][T][k]
 * (its lcs_topk_select output) -> cand_score [B][T][k] fp32 and cand_idx
 * [B][T][k] int32: (scores[b,t,idx], idx + pos_base) per slot; an empty slot
 * (idx outside [0, L)) gives (-inf, -1). pos_base = the shard's first
 * position, with pos_base + L <= 2^31 - 1. */
lcs_status lcs_topk_candidates(const float* scores, const int32_t* idx, int32_t B, int32_t T,
                               int32_t L, int32_t k, int32_t pos_base, float* cand_score,
                               int32_t* cand_idx, hipStream_t stream);

/* Selection from the candidates of G shards.
 * cand_score/cand_idx [G][B][T][k_in] (cand_idx < 0 = no candidate) ->
 * idx [B][T][k]: the min(k, count) candidates with the largest scores, equal
 * scores broken by the lower position and -0.0 equal to +0.0 (the order of
 * lcs_topk_select), listed in ascending position order and padded with -1.
 * Exact. G * k_in <= LCS_MAX_MERGE_CANDIDATES, k in [1, 2048]. A position
 * offered twice for one query is a caller error (the output stays within
 * idx, its content is then unspecified); scores must not be NaN. */
lcs_status lcs_topk_merge(const float* cand_score, const int32_t* cand_idx, int32_t G, int32_t B,
                          int32_t T, int32_t k_in, int32_t k, int32_t* idx, hipStream_t stream);

/* A shard's share of a selection: local [B][T][k] = the entries of idx
 * [B][T][k] in [lo, hi), in list order, minus lo, then -1 (so an ascending
 * list gives an ascending local list, ready for lcs_sparse_mla_attn over the
 * shard's rows). idx and local must not alias. */
lcs_status lcs_idx_localize(const int32_t* idx, int32_t B, int32_t T, int32_t k, int32_t lo,
                            int32_t hi, int32_t* local, hipStream_t stream);

/* Attention from shard outputs.
 * part_out [G][B][T][64][512] bf16 and part_lse [G][B][T][64] fp32 (natural
 * log; -inf for a shard with no selected row), as lcs_sparse_mla_attn writes
 * them per shard -> out [B][T][64][512] bf16 and lse [B][T][64] (nullable):
 *   out = sum_g e^(lse_g - M) out_g / sum_g e^(lse_g - M), M = max_g lse_g,
 *   lse = M + log sum_g e^(lse_g - M);
 * all shards empty: out = 0, lse = -inf. G in [1, LCS_MAX_SHARDS]. */
lcs_status lcs_lse_combine(const uint16_t* part_out, const float* part_lse, int32_t G, int32_t B,
                           int32_t T, uint16_t* out, float* lse, hipStream_t stream);

/* Paged KV. The pages credit finer-grained management of KV-cache memory
 * (LayerSplit) with raising the cache's capacity (section "推理优化" of
 * "GLM-5.2 — 1M上下文开放权重的长程任务旗舰"; the agents-report article makes
 * the same point) and do not describe it; the layout here is a reading: caches live in pools of fixed-size blocks, and each sequence maps
 * its position blocks to pool blocks through a table. Position p of sequence
 * b is pool row block_table[b * max_blocks + p / block_size] * block_size +
 * p % block_size; one table serves the key pool and the latent pool of a
 * layer. Pools: k8 [n_blocks][block_size][128] E4M3 + k_scale
 * [n_blocks][block_size] fp32; kv [n_blocks][block_size][576] (bf16, or E4M3
 * + kv_scale [n_blocks][block_size]). Results equal those of the contiguous
 * calls on the same logical cache, bit for bit. */
typedef struct {
  const int32_t* block_table; /* [B][max_blocks] int32, DEVICE memory */
  int32_t max_blocks;         /* table entries per sequence; L <= max_blocks * block_size */
  int32_t block_size;         /* rows per block: a power of two >= 64 */
  int32_t n_blocks;           /* blocks in each pool; n_blocks * block_size < 2^31.
                               * Table entries are clamped to [0, n_blocks) on the
                               * device, so a bad entry reads or writes a wrong row
                               * of the pool, never memory outside it. */
} lcs_paged;

/* lcs_idx_score over paged keys (paged is a HOST pointer). */
lcs_status lcs_idx_score_paged(const uint8_t* q8, const float* q_scale, const float* w,
                               const uint8_t* k8_pool, const float* k_scale_pool,
                               const lcs_paged* paged, const int32_t* vis_len, int32_t B,
                               int32_t T, int32_t L, float* scores, hipStream_t stream);

/* lcs_sparse_mla_attn over a paged latent cache; workspace as
 * lcs_attn_workspace_bytes(B, T, k). Pools may exceed 4 GB. -1 slots gather
 * position 0 through the sequence's first table entry, never an unmapped
 * block. */
lcs_status lcs_sparse_mla_attn_paged(const uint16_t* q, const void* kv_pool,
                                     lcs_kv_dtype kv_dtype, const float* kv_scale_pool,
                                     const lcs_paged* paged, const int32_t* idx, int32_t B,
                                     int32_t T, int32_t L, int32_t k, float sm_scale,
                                     uint16_t* out, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* lcs_cache_append into paged caches: token (b, t) goes to the pool row of
 * position pos[b,t] (positions outside [0, L) are skipped). */
lcs_status lcs_cache_append_paged(const uint16_t* k_new, const uint16_t* kv_new,
                                  lcs_kv_dtype kv_dtype, const int32_t* pos, int32_t B, int32_t T,
                                  int32_t L, const lcs_paged* paged, uint8_t* k8_pool,
                                  float* k_scale_pool, void* kv_pool, float* kv_scale_pool,
                                  hipStream_t stream);

/* Static description of a status code. */
const char* lcs_status_string(lcs_status s);
/* Thread-local detail of this thread's last failed call ("" if none). */
const char* lcs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif
