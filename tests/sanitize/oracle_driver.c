/* Every oracle function on small seeded inputs, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py (test infrastructure:
 * it links the oracle, which only tests may). Exits non-zero on a failed
 * check; the sanitizers abort on an out-of-bounds access or undefined
 * behaviour. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return (uint32_t)(g_state >> 11);
}
static double next_unit(void) { return (next_u32() & 0xFFFFFF) / 16777216.0; }
static uint8_t finite_code(void) {
  uint8_t c = (uint8_t)(next_u32() % 254);
  return c < 0x7F ? c : (uint8_t)(c + 1);
}
static uint16_t bf16_of(double x) { return oracle_round_bf16(x); }

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

int main(void) {
  enum { B = 2, T = 3, L = 300, K = 64, H = 32, D = 128, AH = 64, KV = 576, LAT = 512 };
  /* scalar conversions over every code and a few doubles */
  for (int c = 0; c < 256; ++c) {
    const double v = oracle_e4m3((uint8_t)c);
    if (!isnan(v)) CHECK(oracle_encode_e4m3(v) == (uint8_t)c || v == 0.0);
  }
  CHECK(oracle_encode_e4m3(1e30) == 0x7E && oracle_encode_e4m3(-1e30) == 0xFE);
  for (int i = 0; i < 1000; ++i) (void)oracle_bf16(bf16_of(next_unit() * 8 - 4));

  /* indexer, top-k */
  uint8_t* q8 = xmalloc((size_t)B * T * H * D);
  float* qs = xmalloc(sizeof(float) * B * T * H);
  float* w = xmalloc(sizeof(float) * B * T * H);
  uint8_t* k8 = xmalloc((size_t)B * L * D);
  float* ks = xmalloc(sizeof(float) * B * L);
  int32_t vis[B * T];
  for (size_t i = 0; i < (size_t)B * T * H * D; ++i) q8[i] = finite_code();
  for (size_t i = 0; i < (size_t)B * L * D; ++i) k8[i] = finite_code();
  for (int i = 0; i < B * T * H; ++i) {
    qs[i] = (float)(0.01 + next_unit());
    w[i] = (float)next_unit();
  }
  for (int i = 0; i < B * L; ++i) ks[i] = (float)(0.01 + next_unit());
  for (int i = 0; i < B * T; ++i) vis[i] = (int32_t)(next_u32() % (L + 20)) - 10;
  vis[0] = L;
  vis[1] = K - 1;
  float* sc = xmalloc(sizeof(float) * B * T * L);
  double* sc64 = xmalloc(sizeof(double) * B * T * L);
  CHECK(oracle_idx_score(q8, qs, w, k8, ks, vis, B, T, L, sc, sc64) == 0);
  int32_t* idx = xmalloc(sizeof(int32_t) * B * T * K);
  CHECK(oracle_topk(sc, vis, B, T, L, K, idx) == 0);
  for (int r = 0; r < B * T; ++r) {
    const int32_t* row = idx + (size_t)r * K;
    for (int i = 1; i < K; ++i)
      if (row[i] >= 0) CHECK(row[i] > row[i - 1]);
  }

  /* sparse attention, bf16 and FP8 latent rows */
  uint16_t* q = xmalloc(sizeof(uint16_t) * B * T * AH * KV);
  uint16_t* kvb = xmalloc(sizeof(uint16_t) * B * L * KV);
  uint8_t* kv8 = xmalloc((size_t)B * L * KV);
  float* kvs = xmalloc(sizeof(float) * B * L);
  for (size_t i = 0; i < (size_t)B * T * AH * KV; ++i) q[i] = bf16_of(next_unit() * 2 - 1);
  for (size_t i = 0; i < (size_t)B * L * KV; ++i) {
    kvb[i] = bf16_of(next_unit() * 2 - 1);
    kv8[i] = finite_code();
  }
  for (int i = 0; i < B * L; ++i) kvs[i] = (float)(0.001 + 0.01 * next_unit());
  uint16_t* out = xmalloc(sizeof(uint16_t) * B * T * AH * LAT);
  float* lse = xmalloc(sizeof(float) * B * T * AH);
  double* out64 = xmalloc(sizeof(double) * B * T * AH * LAT);
  CHECK(oracle_sparse_mla(q, kvb, 0, NULL, idx, B, T, L, K, 1.0 / 24, out, lse, out64) == 0);
  CHECK(oracle_sparse_mla(q, kv8, 1, kvs, idx, B, T, L, K, 1.0 / 24, out, lse, NULL) == 0);

  /* quantisation and cache append (one duplicate position is rejected) */
  uint16_t* x = xmalloc(sizeof(uint16_t) * 7 * KV);
  for (int i = 0; i < 7 * KV; ++i) x[i] = bf16_of(next_unit() * 100 - 50);
  for (int i = 0; i < KV; ++i) x[3 * KV + i] = 0;
  uint8_t* codes = xmalloc(7 * KV);
  float* qsc = xmalloc(sizeof(float) * (7 * KV / D));
  CHECK(oracle_quantize_e4m3(x, 7, KV, codes, qsc) == 0);
  CHECK(oracle_quantize_e4m3(x, 7 * KV / D, D, codes, qsc) == 0);  /* the same bytes as 128-wide rows */
  int32_t pos[B * T];
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t) pos[b * T + t] = t == 2 ? -1 : (b + 3 * t) % L;
  uint16_t* k_new = xmalloc(sizeof(uint16_t) * B * T * D);
  for (int i = 0; i < B * T * D; ++i) k_new[i] = bf16_of(next_unit() - 0.5);
  CHECK(oracle_cache_append(k_new, x, 1, pos, B, T, L, k8, ks, kv8, kvs) == 0);
  CHECK(oracle_cache_append(k_new, x, 0, pos, B, T, L, k8, ks, kvb, NULL) == 0);
  pos[1] = pos[0];
  CHECK(oracle_cache_append(k_new, NULL, 0, pos, B, T, L, k8, ks, NULL, NULL) != 0);

  /* context-parallel halves over G = 3 shards of the first row set */
  enum { G = 3 };
  float* cs = xmalloc(sizeof(float) * G * B * T * K);
  int32_t* ci = xmalloc(sizeof(int32_t) * G * B * T * K);
  for (int g = 0; g < G; ++g)
    CHECK(oracle_topk_candidates(sc, idx, B * T, L, K, g * L, cs + (size_t)g * B * T * K,
                                 ci + (size_t)g * B * T * K) == 0);
  int32_t* merged = xmalloc(sizeof(int32_t) * B * T * K);
  CHECK(oracle_topk_merge(cs, ci, G, B * T, K, K, merged) == 0);
  int32_t* local = xmalloc(sizeof(int32_t) * B * T * K);
  CHECK(oracle_idx_localize(merged, B * T, K, L, 2 * L, local) == 0);
  uint16_t* po = xmalloc(sizeof(uint16_t) * G * B * T * AH * LAT);
  float* pl = xmalloc(sizeof(float) * G * B * T * AH);
  for (size_t i = 0; i < (size_t)G * B * T * AH * LAT; ++i) po[i] = bf16_of(next_unit());
  for (int i = 0; i < G * B * T * AH; ++i) pl[i] = i % 5 == 0 ? -INFINITY : (float)next_unit();
  CHECK(oracle_lse_combine(po, pl, G, B * T, out, lse, out64) == 0);

  /* IndexShare over 6 layers (GLM-5.2 schedule) and an MTP round of 3 steps */
  oracle_layer ly[6];
  memset(ly, 0, sizeof(ly));
  for (int l = 0; l < 6; ++l) {
    ly[l].q8 = q8;
    ly[l].q_scale = qs;
    ly[l].w = w;
    ly[l].k8 = k8;
    ly[l].k_scale = ks;
    ly[l].q = q;
    ly[l].kv = kv8;
    ly[l].kv_scale = kvs;
    ly[l].out = xmalloc(sizeof(uint16_t) * B * T * AH * LAT);
    ly[l].lse = xmalloc(sizeof(float) * B * T * AH);
  }
  int32_t n_full = 0;
  for (int l = 0; l < 6; ++l) n_full += oracle_is_full_layer(ORACLE_SCHED_GLM52, l, NULL);
  CHECK(n_full == 3);  /* layers 0, 1, 2 of the GLM-5.2 list */
  int32_t* idx_out = xmalloc(sizeof(int32_t) * (size_t)n_full * B * T * K);
  CHECK(oracle_indexshare(ly, 6, ORACLE_SCHED_GLM52, NULL, 0, 1, vis, B, T, L, K, 1.0 / 24,
                          idx_out) == 0);
  CHECK(oracle_indexshare(ly, 3, ORACLE_SCHED_GROUP4, NULL, 3, 1, vis, B, T, L, K, 1.0 / 24,
                          idx_out) == 0);
  for (int l = 0; l < 6; ++l) {
    free(ly[l].out);
    free(ly[l].lse);
  }
  free(idx_out); free(po); free(pl); free(local); free(merged); free(cs); free(ci);
  free(k_new); free(qsc); free(codes); free(x); free(out64); free(lse); free(out);
  free(kvs); free(kv8); free(kvb); free(q); free(idx); free(sc64); free(sc);
  free(ks); free(k8); free(w); free(qs); free(q8);
  printf("oracle sanitizer driver ok\n");
  return 0;
}
