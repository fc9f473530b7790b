/*
 * synth.h -- counter-based generator of the seeded synthetic inputs.
 *
 * This module only makes inputs. It holds none of the arithmetic of the
 * indexer, the top-k or the attention. The same definitions are compiled for
 * the host (synth_host.c, plain C) and for the device (synth_dev.hip), so a
 * tensor filled on the GPU is bit-identical to the same tensor filled on the
 * CPU. The including file defines SYN_FN before including this header.
 *
 * Definitions
 *   mix(x)     SplitMix64 output function (Steele, Lea and Flood, "Fast
 *              splittable pseudorandom number generators", OOPSLA 2014) applied
 *              to x + 0x9E3779B97F4A7C15.
 *   row key    mix chained over (seed, tensor id, layer, batch, row).
 *   draw j     mix(rowkey + 3*d + j) for element d, j = 0, 1, 2.
 *   normal     Irwin-Hall sum of twelve 16-bit uniforms taken from the three
 *              draws, minus its mean 6*65536, times 2^-16. Mean 0, variance
 *              1 (up to the 16-bit discretisation), support [-6, 6). The sum is
 *              an integer below 2^19, so the value is exact in fp32 and the
 *              result does not depend on the platform's float arithmetic.
 *   uniform    top 24 bits of draw 0 times 2^-24, in [0, 1), exact in fp32.
 *   bf16       round to nearest even of the fp32 value (bit arithmetic).
 *   e4m3       OCP FP8 E4M3 (bias 7, max 448, no infinities), round to nearest
 *              even, saturating at +-448; built with frexp/ldexp/rint on
 *              doubles, which are exact or IEEE-rounded on both sides.
 *   quantised row: amax = max |x|; scale = (float)(amax / 448.0) in double,
 *              or 1 when amax = 0; code_i = e4m3(x_i / scale) in double.
 *   planted rows: in a row set of size R, n = round(R * permyriad / 10000)
 *              rows are planted: r is planted iff (a*r + c) mod R < n, where
 *              a (coprime to R) and c come from the key. The map r -> a*r+c mod
 *              R is a bijection, so exactly n rows are planted. A planted
 *              row's pre-quantisation values are shifted by +3.0 (3 sigma).
 */
#ifndef LCS_SYNTH_H
#define LCS_SYNTH_H

#include <stdint.h>

#ifndef SYN_FN
#error "define SYN_FN (function qualifiers) before including synth.h"
#endif

/* tensor ids: every synthetic tensor has its own stream */
enum {
  SYN_T_IDX_KEY = 1,  /* indexer keys            [B][L][128]  fp8 + scale */
  SYN_T_IDX_Q = 2,    /* indexer queries         [B][T*32][128] fp8 + scale */
  SYN_T_IDX_W = 3,    /* indexer head weights    [B][T][32]   U(0,1)       */
  SYN_T_ATT_Q = 4,    /* attention queries       [B][T*64][576] bf16       */
  SYN_T_KV = 5,       /* latent KV               [B][L][576]  bf16 or fp8  */
  SYN_T_PLANT = 6     /* planted-row selection (per batch)                 */
};

#define SYN_GOLDEN 0x9E3779B97F4A7C15ull

SYN_FN uint64_t syn_mix(uint64_t x) {
  uint64_t z = x + SYN_GOLDEN;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

SYN_FN uint64_t syn_rowkey(uint64_t seed, uint32_t tensor, uint32_t layer,
                           uint32_t b, uint64_t row) {
  uint64_t h = syn_mix(seed);
  h = syn_mix(h ^ (uint64_t)tensor);
  h = syn_mix(h ^ (uint64_t)layer);
  h = syn_mix(h ^ (uint64_t)b);
  h = syn_mix(h ^ row);
  return h;
}

/* approximately N(0,1), exact multiple of 2^-16 */
SYN_FN float syn_normal(uint64_t rowkey, uint32_t d) {
  int32_t s = 0;
  for (uint32_t j = 0; j < 3; ++j) {
    uint64_t r = syn_mix(rowkey + 3ull * d + j);
    s += (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
         (int32_t)((r >> 32) & 0xFFFF) + (int32_t)(r >> 48);
  }
  s -= 6 * 65536;
  return (float)s * (1.0f / 65536.0f);
}

SYN_FN float syn_uniform(uint64_t rowkey, uint32_t d) {
  uint64_t r = syn_mix(rowkey + 3ull * d);
  return (float)(uint32_t)(r >> 40) * (1.0f / 16777216.0f);
}

SYN_FN uint32_t syn_f2u(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}
SYN_FN float syn_u2f(uint32_t u) {
  union { float f; uint32_t u; } c;
  c.u = u;
  return c.f;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite) */
SYN_FN uint16_t syn_bf16(float f) {
  uint32_t u = syn_f2u(f);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}
SYN_FN float syn_bf16_to_f32(uint16_t h) { return syn_u2f((uint32_t)h << 16); }

/* one generated element as it enters quantisation: bf16 value as float */
SYN_FN float syn_value(uint64_t rowkey, uint32_t d, int planted) {
  float x = syn_normal(rowkey, d);
  if (planted) x += 3.0f; /* exact: both terms are multiples of 2^-16 below 2^4 */
  return syn_bf16_to_f32(syn_bf16(x));
}

/* double -> OCP E4M3 code, round to nearest even, saturate at 448 */
SYN_FN uint8_t syn_e4m3(double v) {
  uint8_t sign = 0;
  if (v < 0.0) { sign = 0x80; v = -v; }
  if (!(v < 448.0)) return (uint8_t)(sign | 0x7E); /* saturate (and +-448) */
  if (v < 0.015625) { /* below 2^-6: subnormal grid of step 2^-9 */
    double m = rint(v * 512.0); /* 0..8; 8 is the smallest normal 2^-6 */
    return (uint8_t)(sign | (uint8_t)m);
  }
  int e;
  double fr = frexp(v, &e); /* v = fr * 2^e, fr in [0.5, 1) */
  /* v = (1 + f) * 2^(e-1); mantissa 3 bits: round fr*16 to an integer */
  double q = rint(ldexp(fr, 4)); /* in [8, 16] */
  int ex = e - 1;
  if (q >= 16.0) { q = 8.0; ex += 1; }
  int biased = ex + 7; /* 1..15 */
  uint32_t mant = (uint32_t)q - 8u;
  uint32_t code = ((uint32_t)biased << 3) | mant;
  if (code > 0x7E) code = 0x7E; /* 480 or more rounds down to 448 */
  return (uint8_t)(sign | code);
}

SYN_FN uint64_t syn_gcd(uint64_t a, uint64_t b) {
  while (b) { uint64_t t = a % b; a = b; b = t; }
  return a;
}

/* number of planted rows among R: round(R * permyriad / 10000) */
SYN_FN uint64_t syn_n_plant(uint64_t R, uint32_t permyriad) {
  return (R * (uint64_t)permyriad + 5000ull) / 10000ull;
}

/* exact-count planted-row test (see header) */
SYN_FN int syn_planted(uint64_t seed, uint32_t layer, uint32_t b, uint64_t r,
                       uint64_t R, uint32_t permyriad) {
  if (permyriad == 0 || R == 0) return 0;
  uint64_t key = syn_rowkey(seed, SYN_T_PLANT, layer, b, 0);
  uint64_t a = (syn_mix(key) % R) | 1ull;
  while (syn_gcd(a, R) != 1ull) a += 2ull; /* terminates: R and 1 are coprime */
  uint64_t c = syn_mix(key + 1ull) % R;
  uint64_t p = ((a % R) * (r % R) + c) % R; /* a, r < 2^31 in every use */
  return p < syn_n_plant(R, permyriad);
}

#endif
