/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY: plain CPU oracle of the DSA +
 * IndexShare attention path (see oracle.h for what is computed and which page
 * passage each part follows). Single-threaded, double precision, no blocking
 * or reordering beyond the definitions. Not used by the product path.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define IDX_HEADS 32 /* "32 个 Indexer Heads" (architecture panel) */
#define IDX_DIM 128  /* indexer key/query width: a reading, not on the pages */
#define ATT_HEADS 64 /* "Attention 64 Heads" (architecture panel) */
#define KV_LATENT 512 /* "KV 低秩联合压缩 Rank 512" (kv_lora_rank) */
#define KV_ROPE 64    /* decoupled rope part of each cached row: a reading */
#define KV_DIM (KV_LATENT + KV_ROPE)

/* OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * exponent field 0: subnormal (m/8) * 2^-6; S.1111.111: NaN; else
 * (1 + m/8) * 2^(e-7). Largest finite value 448. */
double oracle_e4m3(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* (m/8) * 2^-6 */
  else
    v = ldexp(8.0 + (double)m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* bf16 is the top half of an IEEE binary32 */
double oracle_bf16(uint16_t bits) {
  union { uint32_t u; float f; } c;
  c.u = (uint32_t)bits << 16;
  return (double)c.f;
}

/* Round a finite double to the nearest bf16 (8 significant bits), ties to
 * even, directly from the double (no intermediate fp32 rounding). */
uint16_t oracle_round_bf16(double x) {
  uint16_t sign = 0;
  if (signbit(x)) { sign = 0x8000; x = -x; }
  if (x == 0.0) return sign;
  if (isinf(x)) return (uint16_t)(sign | 0x7F80);
  int e;
  double fr = frexp(x, &e); /* x = fr * 2^e, fr in [0.5, 1) */
  /* binary32 normal range: exponent of the leading bit e-1 >= -126 */
  int lead = e - 1;
  double q;
  if (lead < -126) {
    /* subnormal bf16: step 2^-133 */
    q = rint(ldexp(x, 133));
    union { uint32_t u; float f; } c;
    c.f = (float)ldexp(q, -133); /* exact: q < 2^7 times a power of two */
    return (uint16_t)(sign | (c.u >> 16));
  }
  q = rint(ldexp(fr, 8)); /* 8 significant bits: in [128, 256] */
  double v = ldexp(q, e - 8);
  if (v > 3.3895313892515355e38) return (uint16_t)(sign | 0x7F80); /* above the largest bf16 */
  union { uint32_t u; float f; } c;
  c.f = (float)v; /* exact: v has 8 significant bits and is in range */
  return (uint16_t)(sign | (c.u >> 16));
}

/* double -> E4M3 code. The FP8 release of the model stores E4M3 (the weight
 * file table under "40B Active，为什么仍要装下 0.465～1.507 TB 权重", ailearn
 * GLM-5.2 special edition), but no page gives a rounding rule; the reading is saturation to +-448, then the
 * nearest finite code, ties to the even code (the code whose last mantissa
 * bit is 0), with the sign kept for zero results. Written as a search over
 * all 127 finite non-negative codes so that it can be checked by eye. */
uint8_t oracle_encode_e4m3(double v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) { /* values increase strictly with c */
    double d = fabs(oracle_e4m3((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best_d = d;
      best = c;
    }
  }
  return (uint8_t)(best | (neg << 7));
}

/* One row of D bf16 values -> D codes and one fp32 scale. The pages keep the
 * KV cache in FP8 (the closing line of the training section of "GLM-5.2 — 1M
 * 上下文开放权重的长程任务旗舰"; the `fp8_ds_mla` cache type in the vLLM launch
 * of the Hygon DCU forum post) without saying how a row is scaled. Reading:
 * amax = max |x|, scale = fl32(amax / 448) (1 when amax = 0), and
 * code_i = encode(fl32(x_i / scale)); the quotient is taken in binary32, so
 * the code a value gets is decided in binary32. Non-finite values: rejected. */
static int quantize_row(const uint16_t* x, int32_t D, uint8_t* codes, float* scale_out) {
  float amax = 0.0f;
  for (int32_t i = 0; i < D; ++i) {
    double v = oracle_bf16(x[i]);
    if (!isfinite(v)) return 1;
    float a = (float)fabs(v); /* exact: a bf16 value is a binary32 value */
    if (a > amax) amax = a;
  }
  float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int32_t i = 0; i < D; ++i) {
    float q = (float)oracle_bf16(x[i]) / scale; /* binary32 division */
    codes[i] = oracle_encode_e4m3((double)q);
  }
  *scale_out = scale;
  return 0;
}

int oracle_quantize_e4m3(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes,
                         float* scales) {
  if (!x || !codes || !scales || rows < 0 || D <= 0) return 1;
  for (int64_t r = 0; r < rows; ++r)
    if (quantize_row(x + r * D, D, codes + r * D, scales + r)) return 1;
  return 0;
}

/* New tokens enter the caches at their positions: the indexer key row is
 * quantised (one scale per key), the latent row is copied (bf16 cache) or
 * quantised (FP8 cache, one scale per row). Tokens whose position lies
 * outside [0, L) are not written; two tokens of one sequence with the same
 * position are rejected. */
int oracle_cache_append(const uint16_t* k_new, const uint16_t* kv_new, int32_t kv_fp8,
                        const int32_t* pos, int32_t B, int32_t T, int32_t L,
                        uint8_t* k8, float* k_scale, void* kv, float* kv_scale) {
  if (!pos || B <= 0 || T <= 0 || L <= 0 || (!k_new && !kv_new)) return 1;
  if (k_new && (!k8 || !k_scale)) return 1;
  if (kv_new && (!kv || (kv_fp8 && !kv_scale))) return 1;
  unsigned char* seen = calloc((size_t)L, 1);
  if (!seen) return 1;
  int rc = 0;
  for (int32_t b = 0; b < B && !rc; ++b) {
    memset(seen, 0, (size_t)L);
    for (int32_t t = 0; t < T && !rc; ++t) {
      int64_t tok = (int64_t)b * T + t;
      int32_t p = pos[tok];
      if (p < 0 || p >= L) continue;
      if (seen[p]) { rc = 1; break; }
      seen[p] = 1;
      int64_t row = (int64_t)b * L + p;
      if (k_new)
        rc |= quantize_row(k_new + tok * IDX_DIM, IDX_DIM, k8 + row * IDX_DIM, k_scale + row);
      if (kv_new) {
        if (kv_fp8)
          rc |= quantize_row(kv_new + tok * KV_DIM, KV_DIM, (uint8_t*)kv + row * KV_DIM,
                             kv_scale + row);
        else
          memcpy((uint16_t*)kv + row * KV_DIM, kv_new + tok * KV_DIM, KV_DIM * sizeof(uint16_t));
      }
    }
  }
  free(seen);
  return rc;
}

static int clamp_vis(int32_t v, int32_t L) {
  if (v < 0) return 0;
  if (v > L) return L;
  return v;
}

int oracle_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                     const uint8_t* k8, const float* k_scale,
                     const int32_t* vis_len, int32_t B, int32_t T, int32_t L,
                     float* scores, double* scores64) {
  if (!q8 || !q_scale || !w || !k8 || !k_scale || !vis_len || !scores) return 1;
  if (B < 0 || T < 0 || L < 0) return 2;
  double qd[IDX_HEADS][IDX_DIM];
  double wq[IDX_HEADS];
  double kd[IDX_DIM];
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t t = 0; t < T; ++t) {
      const size_t bt = (size_t)b * T + t;
      for (int j = 0; j < IDX_HEADS; ++j) {
        for (int i = 0; i < IDX_DIM; ++i) {
          qd[j][i] = oracle_e4m3(q8[(bt * IDX_HEADS + j) * IDX_DIM + i]);
          if (isnan(qd[j][i])) return 3;
        }
        /* the head weight and the query's dequantisation scale are both
         * positive per-head factors; their product is exact in double */
        wq[j] = (double)w[bt * IDX_HEADS + j] * (double)q_scale[bt * IDX_HEADS + j];
      }
      const int vis = clamp_vis(vis_len[bt], L);
      float* srow = scores + bt * (size_t)L;
      double* s64 = scores64 ? scores64 + bt * (size_t)L : NULL;
      for (int32_t s = 0; s < L; ++s) {
        if (s >= vis) {
          srow[s] = -INFINITY;
          if (s64) s64[s] = -INFINITY;
          continue;
        }
        for (int i = 0; i < IDX_DIM; ++i) {
          kd[i] = oracle_e4m3(k8[((size_t)b * L + s) * IDX_DIM + i]);
          if (isnan(kd[i])) return 3;
        }
        double sum = 0.0;
        for (int j = 0; j < IDX_HEADS; ++j) {
          double d = 0.0; /* exact: see the exactness pin in the tests */
          for (int i = 0; i < IDX_DIM; ++i) d += qd[j][i] * kd[i];
          double r = d > 0.0 ? d : 0.0; /* ReLU */
          sum += wq[j] * r;
        }
        double I = (double)k_scale[(size_t)b * L + s] * sum;
        srow[s] = (float)I;
        if (s64) s64[s] = I;
      }
    }
  }
  return 0;
}

typedef struct {
  float score;
  int32_t pos;
} scored_pos;

/* strict total order: higher score first, then lower position */
static int cmp_rank(const void* a, const void* b) {
  const scored_pos* x = (const scored_pos*)a;
  const scored_pos* y = (const scored_pos*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_int(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int oracle_topk(const float* scores, const int32_t* vis_len, int32_t B,
                int32_t T, int32_t L, int32_t k, int32_t* idx) {
  if (!scores || !vis_len || !idx) return 1;
  if (B < 0 || T < 0 || L < 0 || k <= 0) return 2;
  scored_pos* buf = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(L > 0 ? L : 1));
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  if (!buf || !sel) { free(buf); free(sel); return 4; }
  for (size_t bt = 0; bt < (size_t)B * T; ++bt) {
    const int vis = clamp_vis(vis_len[bt], L);
    const float* srow = scores + bt * (size_t)L;
    for (int s = 0; s < vis; ++s) {
      if (isnan(srow[s])) { free(buf); free(sel); return 3; }
      buf[s].score = srow[s];
      buf[s].pos = s;
    }
    qsort(buf, (size_t)vis, sizeof(scored_pos), cmp_rank);
    const int m = vis < k ? vis : k;
    for (int i = 0; i < m; ++i) sel[i] = buf[i].pos;
    qsort(sel, (size_t)m, sizeof(int32_t), cmp_int);
    int32_t* out = idx + bt * (size_t)k;
    for (int i = 0; i < k; ++i) out[i] = i < m ? sel[i] : -1;
  }
  free(buf);
  free(sel);
  return 0;
}

/* ---- context-parallel halves of the selection and the attention ----
 * Context parallelism splits the KV pool over devices (panel "CP · EP · P/D ·
 * HiCache", ailearn special edition). Each shard holds the positions
 * [lo, lo + L_shard) of every sequence and selects its own top-k; the
 * definitions below turn those local selections into the selection over the
 * whole sequence, and shard attention outputs into the whole attention. */

/* A shard's selection as (score, global position) candidates: for each
 * (query, slot) with idx >= 0, (scores[q][idx], idx + pos_base); empty slots
 * give (-inf, -1). scores [Q][L], idx/cand_idx [Q][k], cand_score [Q][k]. */
int oracle_topk_candidates(const float* scores, const int32_t* idx, int32_t Q, int32_t L,
                           int32_t k, int32_t pos_base, float* cand_score, int32_t* cand_idx) {
  if (!scores || !idx || !cand_score || !cand_idx || Q < 0 || L <= 0 || k <= 0) return 1;
  for (int64_t q = 0; q < Q; ++q)
    for (int32_t i = 0; i < k; ++i) {
      int32_t p = idx[q * k + i];
      if (p >= L) return 2;
      cand_score[q * k + i] = p >= 0 ? scores[q * L + p] : -INFINITY;
      cand_idx[q * k + i] = p >= 0 ? p + pos_base : -1;
    }
  return 0;
}

/* Selection from candidates: per query, the candidates with cand_idx >= 0
 * ordered by (score descending, position ascending) -- the order of
 * oracle_topk -- keep the first min(k, count), list them in ascending
 * position order, pad with -1. cand_* [G][Q][k_in] (shard-major, as gathered
 * from G shards); idx [Q][k]. Repeated positions or NaN scores: rejected. */
int oracle_topk_merge(const float* cand_score, const int32_t* cand_idx, int32_t G, int32_t Q,
                      int32_t k_in, int32_t k, int32_t* idx) {
  if (!cand_score || !cand_idx || !idx || G <= 0 || Q < 0 || k_in <= 0 || k <= 0) return 1;
  const size_t n = (size_t)G * k_in;
  scored_pos* buf = (scored_pos*)malloc(sizeof(scored_pos) * n);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (n > (size_t)k ? n : (size_t)k));
  if (!buf || !sel) { free(buf); free(sel); return 4; }
  int rc = 0;
  for (int64_t q = 0; q < Q && !rc; ++q) {
    size_t m = 0;
    for (int32_t g = 0; g < G; ++g)
      for (int32_t i = 0; i < k_in; ++i) {
        size_t at = ((size_t)g * Q + (size_t)q) * k_in + i;
        if (cand_idx[at] < 0) continue;
        if (isnan(cand_score[at])) rc = 3;
        buf[m].score = cand_score[at];
        buf[m].pos = cand_idx[at];
        ++m;
      }
    for (size_t i = 0; i < m; ++i) sel[i] = buf[i].pos; /* repeated positions? */
    qsort(sel, m, sizeof(int32_t), cmp_int);
    for (size_t i = 1; i < m; ++i)
      if (sel[i] == sel[i - 1]) rc = 5;
    qsort(buf, m, sizeof(scored_pos), cmp_rank);
    const size_t take = m < (size_t)k ? m : (size_t)k;
    for (size_t i = 0; i < take; ++i) sel[i] = buf[i].pos;
    qsort(sel, take, sizeof(int32_t), cmp_int);
    for (int32_t i = 0; i < k; ++i) idx[q * k + i] = (size_t)i < take ? sel[i] : -1;
  }
  free(buf);
  free(sel);
  return rc;
}

/* A shard's share of an ascending selection: the entries in [lo, hi), in
 * list order, minus lo, then -1. idx/local [Q][k]. */
int oracle_idx_localize(const int32_t* idx, int32_t Q, int32_t k, int32_t lo, int32_t hi,
                        int32_t* local) {
  if (!idx || !local || Q < 0 || k <= 0 || lo < 0 || hi < lo) return 1;
  for (int64_t q = 0; q < Q; ++q) {
    int32_t m = 0;
    for (int32_t i = 0; i < k; ++i) {
      int32_t p = idx[q * k + i];
      if (p >= lo && p < hi) local[q * k + m++] = p - lo;
    }
    for (; m < k; ++m) local[q * k + m] = -1;
  }
  return 0;
}

/* Attention from shard outputs. Shard g attended over the selected rows it
 * holds, giving out_g (bf16) and lse_g = log sum_{i in g} exp(z_i). Over all
 * rows, sum_i e^{z_i} v_i / sum_i e^{z_i} = sum_g e^{lse_g} out_g / sum_g
 * e^{lse_g}: with M = max_g lse_g and w_g = exp(lse_g - M),
 * out = sum_g w_g out_g / sum_g w_g and lse = M + log sum_g w_g, in double;
 * shards with lse = -inf weigh nothing; all -inf gives out = 0, lse = -inf.
 * part_out [G][Q][64][512] bf16, part_lse [G][Q][64] -> out [Q][64][512]
 * bf16 (RNE), lse [Q][64] fp32; out64 (nullable) gets the unrounded out. */
int oracle_lse_combine(const uint16_t* part_out, const float* part_lse, int32_t G, int32_t Q,
                       uint16_t* out, float* lse, double* out64) {
  if (!part_out || !part_lse || !out || G <= 0 || Q < 0) return 1;
  const size_t per = (size_t)ATT_HEADS * KV_LATENT;
  for (size_t q = 0; q < (size_t)Q; ++q)
    for (int h = 0; h < ATT_HEADS; ++h) {
      double M = -INFINITY;
      for (int32_t g = 0; g < G; ++g) {
        double l = part_lse[((size_t)g * Q + q) * ATT_HEADS + h];
        if (isnan(l) || l == INFINITY) return 3;
        if (l > M) M = l;
      }
      double wsum = 0.0;
      for (int v = 0; v < KV_LATENT; ++v) {
        double acc = 0.0;
        wsum = 0.0;
        for (int32_t g = 0; g < G; ++g) {
          double l = part_lse[((size_t)g * Q + q) * ATT_HEADS + h];
          if (l == -INFINITY) continue;
          double w = exp(l - M);
          wsum += w;
          acc += w * oracle_bf16(part_out[((size_t)g * Q + q) * per + (size_t)h * KV_LATENT + v]);
        }
        double o = wsum > 0.0 ? acc / wsum : 0.0;
        out[q * per + (size_t)h * KV_LATENT + v] = oracle_round_bf16(o);
        if (out64) out64[q * per + (size_t)h * KV_LATENT + v] = o;
      }
      if (lse) lse[q * ATT_HEADS + h] = M == -INFINITY ? -INFINITY : (float)(M + log(wsum));
    }
  return 0;
}

int oracle_sparse_mla(const uint16_t* q, const void* kv, int32_t kv_fp8,
                      const float* kv_scale, const int32_t* idx, int32_t B,
                      int32_t T, int32_t L, int32_t k, double sm_scale,
                      uint16_t* out, float* lse, double* out64) {
  if (!q || !kv || !idx || !out || !lse) return 1;
  if (kv_fp8 && !kv_scale) return 1;
  if (B < 0 || T < 0 || L < 0 || k <= 0) return 2;
  double* rows = (double*)malloc(sizeof(double) * (size_t)k * KV_DIM);
  double* z = (double*)malloc(sizeof(double) * (size_t)k);
  if (!rows || !z) { free(rows); free(z); return 4; }
  const uint16_t* kv16 = (const uint16_t*)kv;
  const uint8_t* kv8 = (const uint8_t*)kv;
  int rc = 0;
  for (int32_t b = 0; b < B && !rc; ++b) {
    for (int32_t t = 0; t < T && !rc; ++t) {
      const size_t bt = (size_t)b * T + t;
      const int32_t* sel = idx + bt * (size_t)k;
      /* gather the selected rows, decoded exactly */
      int n = 0;
      for (int i = 0; i < k; ++i) {
        const int32_t s = sel[i];
        if (s == -1) continue;
        if (s < 0 || s >= L) { rc = 2; break; }
        const size_t base = ((size_t)b * L + s) * KV_DIM;
        for (int d = 0; d < KV_DIM; ++d) {
          double v;
          if (kv_fp8) {
            v = oracle_e4m3(kv8[base + d]);
            if (isnan(v)) { rc = 3; break; }
            v *= (double)kv_scale[(size_t)b * L + s]; /* exact */
          } else {
            v = oracle_bf16(kv16[base + d]);
          }
          rows[(size_t)n * KV_DIM + d] = v;
        }
        ++n;
      }
      if (rc) break;
      for (int h = 0; h < ATT_HEADS; ++h) {
        const uint16_t* qh = q + (bt * ATT_HEADS + h) * KV_DIM;
        uint16_t* oh = out + (bt * ATT_HEADS + h) * KV_LATENT;
        double* o64 = out64 ? out64 + (bt * ATT_HEADS + h) * KV_LATENT : NULL;
        if (n == 0) {
          for (int v = 0; v < KV_LATENT; ++v) {
            oh[v] = 0;
            if (o64) o64[v] = 0.0;
          }
          lse[bt * ATT_HEADS + h] = -INFINITY;
          continue;
        }
        double mu = -INFINITY;
        for (int i = 0; i < n; ++i) {
          double dot = 0.0;
          for (int d = 0; d < KV_DIM; ++d) dot += oracle_bf16(qh[d]) * rows[(size_t)i * KV_DIM + d];
          z[i] = sm_scale * dot;
          if (z[i] > mu) mu = z[i];
        }
        double denom = 0.0;
        for (int i = 0; i < n; ++i) {
          z[i] = exp(z[i] - mu); /* z now holds e_i */
          denom += z[i];
        }
        for (int v = 0; v < KV_LATENT; ++v) {
          double acc = 0.0;
          for (int i = 0; i < n; ++i) acc += z[i] * rows[(size_t)i * KV_DIM + v];
          const double o = acc / denom;
          oh[v] = oracle_round_bf16(o);
          if (o64) o64[v] = o;
        }
        lse[bt * ATT_HEADS + h] = (float)(mu + log(denom));
      }
    }
  }
  free(rows);
  free(z);
  return rc;
}

/* "IndexShare：四层共用一次搜索结果": layers 0 and 1 have their own indexer;
 * from layer 2 on every fourth layer (2, 6, 10, ..., 74) has one and passes
 * its Top-k to the three layers after it. GROUP4 is the plain "first layer of
 * every four" wording of the engineering-report wiki. */
int oracle_is_full_layer(int32_t sched, int32_t l, const uint8_t* mask) {
  if (l < 0) return 0;
  switch (sched) {
    case ORACLE_SCHED_GROUP4:
      return l % 4 == 0;
    case ORACLE_SCHED_GLM52:
      if (l == 0 || l == 1) return 1;
      return (l - 2) % 4 == 0;
    case ORACLE_SCHED_ALL_FULL:
      return 1;
    case ORACLE_SCHED_MASK:
      return mask ? mask[l] != 0 : 0;
    default:
      return 0;
  }
}

int oracle_indexshare(const oracle_layer* layers, int32_t n_layers,
                      int32_t sched, const uint8_t* mask, int32_t mtp_steps,
                      int32_t kv_fp8, const int32_t* vis_len, int32_t B,
                      int32_t T, int32_t L, int32_t k, double sm_scale,
                      int32_t* idx_out) {
  if (!layers || !vis_len || !idx_out || n_layers <= 0) return 1;
  if (mtp_steps < 0 || (mtp_steps > 0 && mtp_steps != n_layers)) return 2;
  const size_t per = (size_t)B * T * k;
  float* scores = (float*)malloc(sizeof(float) * (size_t)B * T * (size_t)(L > 0 ? L : 1));
  if (!scores) return 4;
  const int32_t* cur = NULL;
  int32_t nfull = 0;
  int rc = 0;
  for (int32_t l = 0; l < n_layers && !rc; ++l) {
    const oracle_layer* ly = &layers[l];
    const int full = mtp_steps > 0 ? (l == 0) : oracle_is_full_layer(sched, l, mask);
    if (full) {
      int32_t* dst = idx_out + (size_t)nfull * per;
      rc = oracle_idx_score(ly->q8, ly->q_scale, ly->w, ly->k8, ly->k_scale, vis_len, B, T, L,
                            scores, NULL);
      if (!rc) rc = oracle_topk(scores, vis_len, B, T, L, k, dst);
      cur = dst;
      ++nfull;
    } else if (!cur) {
      rc = 2; /* a shared layer with no earlier full layer */
    }
    if (rc) break;
    /* KV Share: every draft step reads the first step's cache */
    const oracle_layer* kvl = mtp_steps > 0 ? &layers[0] : ly;
    rc = oracle_sparse_mla(ly->q, kvl->kv, kv_fp8, kvl->kv_scale, cur, B, T, L, k, sm_scale,
                           ly->out, ly->lse, NULL);
  }
  free(scores);
  return rc;
}
