// cache.hip -- per-row FP8 (OCP E4M3) quantisation and the cache append of new
// tokens, the step that feeds the indexer and attention caches each decode step.
//
// The pages keep the KV cache in FP8 (the closing line of the training section
// of "GLM-5.2 — 1M上下文开放权重的长程任务旗舰"; the `fp8_ds_mla` cache type in
// the vLLM launch of the Hygon DCU forum post "IndexShare：省掉3/4的索引计算")
// and name E4M3 as the FP8 format of the release (weight-file table under
// "40B Active，为什么仍要装下 0.465～1.507 TB 权重", ailearn special edition).
// How a row is scaled is not on the pages; the reading implemented here is one
// fp32 scale per row, scale = fl32(max|x| / 448) (1 for an all-zero row), and
// code = E4M3(fl32(x / scale)) with saturation at 448 and round-to-nearest,
// ties to the even code (the OCP OFP8 conversion rule).
//
// Layout and mapping: rows of 128 values (indexer keys and queries) take 16
// lanes each, 8 bf16 per lane (one 16-byte load, one 8-byte code store), so a
// wave quantises 4 rows; rows of 576 values (latent KV) take a whole wave, 8
// values per lane for dims 0..511 plus one rope value per lane for 512..575.
// The row maximum is a shuffle reduction inside the row's lanes. One launch
// serves both row widths: the first blocks take the 128-wide rows, the rest
// the 576-wide rows. The work is pure data movement (read 2 bytes, write 1 per
// value), so the kernel is bound by HBM bandwidth and, at decode sizes, by
// launch latency.
#include "common.h"

namespace lcs {
namespace {

constexpr int kThreads = 256;
constexpr int kRows128PerBlock = 16;  // 4 waves x 4 rows
constexpr int kRows576PerBlock = 4;   // 4 waves x 1 row

// One set of rows to process. Row r of src goes to destination row
//   r                              (dst_pos == nullptr), or
//   (r / T) * L + dst_pos[r]       (cache append; skipped when dst_pos[r]
//                                   is outside [0, L)), or, with a block
//   table (paged caches), pool row (blk << lbs) + (p & (2^lbs - 1)) with
//   blk = btab[(r / T) * max_blocks + (p >> lbs)] clamped to the pool.
// codes != nullptr: quantise into codes/scales; else copy the bf16 row to copy
// (576-wide rows only: a bf16 latent cache takes the new rows as they are).
struct RowJob {
  const uint16_t* src;
  int64_t rows;
  const int32_t* dst_pos;
  int T;
  int L;
  uint8_t* codes;
  float* scales;
  uint16_t* copy;
  const int32_t* btab;
  int max_blocks, lbs, n_blocks;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Magnitude code of a binary32 value a in [0, 448].
//  below 2^-6 (E4M3 subnormals, step 2^-9): the nearest multiple of 2^-9, ties
//  to even, is rint(a * 512), exact because the scaling is by a power of two;
//  a result of 8 is the code of 2^-6 itself.
//  otherwise: round the binary32 significand to 3 bits, ties to even, by adding
//  just under half a step plus the kept last bit; a carry moves into the
//  exponent as it should. E4M3's exponent bias is 7, binary32's 127.
__device__ __forceinline__ uint32_t e4m3_magnitude(float a) {
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  return (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
}

// binary32 quotient -> E4M3 code, saturating at +-448, sign kept (also for 0)
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  return sign | e4m3_magnitude(fminf(fabsf(q), 448.0f));
}

__device__ __forceinline__ int64_t dst_row(const RowJob& j, int64_t r, bool& valid) {
  if (r >= j.rows) {
    valid = false;
    return 0;
  }
  if (!j.dst_pos) {
    valid = true;
    return r;
  }
  const int p = j.dst_pos[r];
  valid = p >= 0 && p < j.L;
  if (!j.btab) return (r / j.T) * (int64_t)j.L + p;
  const int blk = valid ? j.btab[(r / j.T) * (int64_t)j.max_blocks + (p >> j.lbs)] : 0;
  return ((int64_t)min(max(blk, 0), j.n_blocks - 1) << j.lbs) + (p & ((1 << j.lbs) - 1));
}

// 8 values -> 8 codes packed little-endian into two words
__device__ __forceinline__ uint2 encode8(const uint4 v, float scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = e4m3_code(bf16_lo(w[i]) / scale);
    const uint32_t hi = e4m3_code(bf16_hi(w[i]) / scale);
    out[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
  }
  return make_uint2(out[0], out[1]);
}

__device__ __forceinline__ float amax8(const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  return m;
}

__device__ __forceinline__ float row_scale(float amax) {
  return amax > 0.0f ? amax / 448.0f : 1.0f;  // correctly rounded binary32 division
}

// 16 lanes per 128-value row, 4 rows per wave
__device__ void rows128(const RowJob& j, int64_t block) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15;
  const int64_t r = block * kRows128PerBlock + (threadIdx.x >> 6) * 4 + (lane >> 4);
  bool valid;
  const int64_t d = dst_row(j, r, valid);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (valid) v = *(const uint4*)(j.src + r * kIdxDim + sub * 8);
  float m = amax8(v);
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (!valid) return;
  const float scale = row_scale(m);
  *(uint2*)(j.codes + d * kIdxDim + sub * 8) = encode8(v, scale);
  if (sub == 0) j.scales[d] = scale;
}

// one wave per 576-value row
__device__ void rows576(const RowJob& j, int64_t block) {
  const int lane = threadIdx.x & 63;
  const int64_t r = block * kRows576PerBlock + (threadIdx.x >> 6);
  bool valid;
  const int64_t d = dst_row(j, r, valid);  // uniform across the wave
  if (!valid) return;
  const uint16_t* src = j.src + r * kKvDim;
  const uint4 v = *(const uint4*)(src + lane * 8);
  const uint16_t t = src[kLatent + lane];
  if (!j.codes) {
    *(uint4*)(j.copy + d * kKvDim + lane * 8) = v;
    j.copy[d * kKvDim + kLatent + lane] = t;
    return;
  }
  const float tv = __uint_as_float((uint32_t)t << 16);
  float m = fmaxf(amax8(v), fabsf(tv));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float scale = row_scale(m);
  *(uint2*)(j.codes + d * kKvDim + lane * 8) = encode8(v, scale);
  j.codes[d * kKvDim + kLatent + lane] = (uint8_t)e4m3_code(tv / scale);
  if (lane == 0) j.scales[d] = scale;
}

__global__ __launch_bounds__(kThreads) void quant_rows_kernel(RowJob j128, RowJob j576,
                                                              int64_t blocks128) {
  const int64_t b = blockIdx.x;
  if (b < blocks128)
    rows128(j128, b);
  else
    rows576(j576, b - blocks128);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t launch_jobs(const RowJob& j128, const RowJob& j576, hipStream_t stream) {
  const int64_t b128 = ceil_div(j128.rows, kRows128PerBlock);
  const int64_t b576 = ceil_div(j576.rows, kRows576PerBlock);
  const int64_t blocks = b128 + b576;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch_kernel(quant_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, j128,
                       j576, b128);
}

}  // namespace

hipError_t launch_quantize_e4m3(const uint16_t* x, int64_t rows, int D, uint8_t* codes,
                                float* scales, hipStream_t stream) {
  RowJob none{};
  RowJob job{x, rows, nullptr, 1, 0, codes, scales, nullptr, nullptr, 0, 0, 0};
  return D == kIdxDim ? launch_jobs(job, none, stream) : launch_jobs(none, job, stream);
}

hipError_t launch_cache_append(const uint16_t* k_new, const uint16_t* kv_new, bool kv_fp8,
                               const int32_t* pos, int B, int T, int L, uint8_t* k8,
                               float* k_scale, void* kv, float* kv_scale,
                               const int32_t* block_table, int max_blocks, int lbs, int n_blocks,
                               hipStream_t stream) {
  const int64_t tokens = (int64_t)B * T;
  RowJob keys{};
  RowJob lat{};
  if (k_new)
    keys = RowJob{k_new, tokens, pos, T, L, k8, k_scale, nullptr, block_table, max_blocks, lbs,
                  n_blocks};
  if (kv_new)
    lat = kv_fp8 ? RowJob{kv_new, tokens, pos, T, L, (uint8_t*)kv, kv_scale, nullptr, block_table,
                          max_blocks, lbs, n_blocks}
                 : RowJob{kv_new, tokens, pos, T, L, nullptr, nullptr, (uint16_t*)kv, block_table,
                          max_blocks, lbs, n_blocks};
  return launch_jobs(keys, lat, stream);
}

}  // namespace lcs
