/*
 * synth_host.c -- host fill routines of the synthetic-input generator.
 * Every routine fills a dense block of rows [b0, b0+nb) x [r0, r0+nr) of a
 * logical tensor [B][R][D]; the element values depend only on
 * (seed, tensor, layer, b, r, d), never on the block shape, so any sub-block
 * equals the same slice of the full tensor (and of the device fill).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define SYN_FN static inline
#include "synth.h"

#define SYN_MAX_D 1024

/* quantised rows: codes [nb][nr][D], scales [nb][nr] */
int synth_host_fp8_rows(uint64_t seed, uint32_t tensor, uint32_t layer,
                        int64_t R, int32_t D, uint32_t plant_permyriad,
                        int32_t b0, int32_t nb, int64_t r0, int64_t nr,
                        uint8_t* codes, float* scales) {
  if (D <= 0 || D > SYN_MAX_D || nb < 0 || nr < 0) return 1;
  float x[SYN_MAX_D];
  for (int32_t bi = 0; bi < nb; ++bi) {
    uint32_t b = (uint32_t)(b0 + bi);
    for (int64_t ri = 0; ri < nr; ++ri) {
      uint64_t r = (uint64_t)(r0 + ri);
      uint64_t key = syn_rowkey(seed, tensor, layer, b, r);
      int planted = syn_planted(seed, layer, b, r, (uint64_t)R, plant_permyriad);
      float amax = 0.0f;
      for (int32_t d = 0; d < D; ++d) {
        x[d] = syn_value(key, (uint32_t)d, planted);
        float a = fabsf(x[d]);
        if (a > amax) amax = a;
      }
      float scale = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
      size_t row = (size_t)bi * (size_t)nr + (size_t)ri;
      for (int32_t d = 0; d < D; ++d)
        codes[row * (size_t)D + (size_t)d] = syn_e4m3((double)x[d] / (double)scale);
      scales[row] = scale;
    }
  }
  return 0;
}

/* bf16 rows [nb][nr][D] */
int synth_host_bf16_rows(uint64_t seed, uint32_t tensor, uint32_t layer,
                         int32_t D, int32_t b0, int32_t nb, int64_t r0,
                         int64_t nr, uint16_t* out) {
  if (D <= 0 || nb < 0 || nr < 0) return 1;
  for (int32_t bi = 0; bi < nb; ++bi)
    for (int64_t ri = 0; ri < nr; ++ri) {
      uint64_t key = syn_rowkey(seed, tensor, layer, (uint32_t)(b0 + bi),
                                (uint64_t)(r0 + ri));
      size_t row = (size_t)bi * (size_t)nr + (size_t)ri;
      for (int32_t d = 0; d < D; ++d)
        out[row * (size_t)D + (size_t)d] = syn_bf16(syn_normal(key, (uint32_t)d));
    }
  return 0;
}

/* U(0,1) fp32 rows [nb][nr][D] */
int synth_host_uniform_rows(uint64_t seed, uint32_t tensor, uint32_t layer,
                            int32_t D, int32_t b0, int32_t nb, int64_t r0,
                            int64_t nr, float* out) {
  if (D <= 0 || nb < 0 || nr < 0) return 1;
  for (int32_t bi = 0; bi < nb; ++bi)
    for (int64_t ri = 0; ri < nr; ++ri) {
      uint64_t key = syn_rowkey(seed, tensor, layer, (uint32_t)(b0 + bi),
                                (uint64_t)(r0 + ri));
      size_t row = (size_t)bi * (size_t)nr + (size_t)ri;
      for (int32_t d = 0; d < D; ++d)
        out[row * (size_t)D + (size_t)d] = syn_uniform(key, (uint32_t)d);
    }
  return 0;
}

/* planted flags for rows [r0, r0+nr) of batch b (1 = planted) */
int synth_host_planted(uint64_t seed, uint32_t layer, int32_t b, int64_t R,
                       uint32_t plant_permyriad, int64_t r0, int64_t nr,
                       uint8_t* out) {
  for (int64_t i = 0; i < nr; ++i)
    out[i] = (uint8_t)syn_planted(seed, layer, (uint32_t)b, (uint64_t)(r0 + i),
                                  (uint64_t)R, plant_permyriad);
  return 0;
}

/* e4m3 encoder exposed for the input-preparation tests */
uint8_t synth_host_e4m3(double v) { return syn_e4m3(v); }
uint16_t synth_host_bf16(float f) { return syn_bf16(f); }
