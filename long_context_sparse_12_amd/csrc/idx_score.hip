// idx_score.hip -- indexer scores on gfx950.
//
// The pages say a light indexer with 32 heads scans the whole history of each
// query ("一枚 Token，怎样穿过 78 层", panel "MLA 压缩，DSA 精读") and that the
// indexer stays O(L^2) ("IndexShare：省掉3/4的索引计算"). The score is the DSA
// lightning-indexer form I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) with FP8
// queries and keys, each with a per-row dequantisation scale.
//
// Decode (T <= 4): every key is read once from HBM; each wave runs the 32
// heads of a query as the M dimension of v_mfma_f32_16x16x128_f8f6f4 (two
// 16-head halves) against 16 keys as N, K = the whole 128-dim row, then folds
// ReLU * (w * q_scale) over its heads, sums across the four lane groups and
// scales by the key's scale. 132 bytes of HBM traffic per key, no reuse, so
// the kernel is bound by HBM bandwidth; MFMA keeps the 8192 MACs per key off
// the vector ALU.
#include "common.h"

namespace lcs {
namespace {

#ifndef LCS_IDX_TARGET_WGS
#define LCS_IDX_TARGET_WGS 1024
#endif
#ifndef LCS_IDX_MAX_ITERS
#define LCS_IDX_MAX_ITERS 16
#endif

constexpr int kWaves = 4;
constexpr int kSuper = 64;  // keys per wave iteration (4 MFMA column tiles of 16)

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  v4f c = {0.f, 0.f, 0.f, 0.f};
  // format codes 0/0 = FP8 E4M3 for A and B; zero scale operands select the
  // unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int TQ>
__global__ void __launch_bounds__(256) idx_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, const int32_t* __restrict__ vis_len, int T,
    int t0, int L, int keys_per_wg, float* __restrict__ scores) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;  // lane group: K slice of the operands, head quad of the result
  const int n = lane & 15;

  // A operands: the 32 heads of each query, two 16-head halves
  v8i a0[TQ], a1[TQ];
  float wq0[TQ][4], wq1[TQ][4];
  int vis[TQ];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    const int64_t bt = (int64_t)b * T + t0 + t;
    const uint8_t* qrow = q8 + bt * (kIdxHeads * kIdxDim);
    a0[t] = *(const v8i*)(qrow + n * kIdxDim + 32 * g);
    a1[t] = *(const v8i*)(qrow + (16 + n) * kIdxDim + 32 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h0 = 4 * g + i, h1 = 16 + 4 * g + i;
      wq0[t][i] = w[bt * kIdxHeads + h0] * q_scale[bt * kIdxHeads + h0];
      wq1[t][i] = w[bt * kIdxHeads + h1] * q_scale[bt * kIdxHeads + h1];
    }
    vis[t] = clamp_vis(vis_len[bt], L);
  }

  const int64_t key_base_b = (int64_t)b * L;
  const int wg_begin = blockIdx.x * keys_per_wg;
  const int wg_end = min(L, wg_begin + keys_per_wg);

  int base = wg_begin + wave * kSuper;
  if (base >= wg_end) return;

  auto load_tile = [&](int tile_base, v8i (&bv)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int key = tile_base + 16 * j + n;
      key = key < L ? key : L - 1;
      bv[j] = *(const v8i*)(k8 + (key_base_b + key) * kIdxDim + 32 * g);
    }
  };

  v8i cur[4], nxt[4];
  load_tile(base, cur);
  for (; base < wg_end; base += kWaves * kSuper) {
    const int next_base = base + kWaves * kSuper;
    if (next_base < wg_end) load_tile(next_base, nxt);
    const int my_key = base + lane;
    const float ks = k_scale[key_base_b + (my_key < L ? my_key : L - 1)];
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
      float res = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f d0 = mfma_fp8_16x16x128(a0[t], cur[j]);
        const v4f d1 = mfma_fp8_16x16x128(a1[t], cur[j]);
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p = fmaf(wq0[t][i], fmaxf(d0[i], 0.f), p);
          p = fmaf(wq1[t][i], fmaxf(d1[i], 0.f), p);
        }
        p += __shfl_xor(p, 16, 64);
        p += __shfl_xor(p, 32, 64);
        res = (g == j) ? p : res;  // lane 16g+n keeps column tile g: key base + lane
      }
      if (my_key < wg_end) {
        const int64_t bt = (int64_t)b * T + t0 + t;
        scores[bt * L + my_key] = my_key < vis[t] ? res * ks : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
  }
}

}  // namespace

hipError_t launch_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                            const uint8_t* k8, const float* k_scale, const int32_t* vis_len,
                            int B, int T, int L, float* scores, hipStream_t stream) {
  // keys per workgroup: a multiple of 4 waves x 64 keys, sized for enough WGs
  const int64_t total_keys = (int64_t)B * L;
  int64_t iters = total_keys / ((int64_t)LCS_IDX_TARGET_WGS * kWaves * kSuper);
  if (iters < 1) iters = 1;
  if (iters > LCS_IDX_MAX_ITERS) iters = LCS_IDX_MAX_ITERS;
  const int kpw = (int)(iters * kWaves * kSuper);
  dim3 grid((unsigned)((L + kpw - 1) / kpw), (unsigned)B);
  for (int t0 = 0; t0 < T; t0 += 4) {
    const int tq = T - t0 < 4 ? T - t0 : 4;
    hipError_t e;
    switch (tq) {
      case 1:
        e = launch_kernel(idx_decode_kernel<1>, grid, dim3(256), 0, stream, q8, q_scale, w, k8,
                          k_scale, vis_len, T, t0, L, kpw, scores);
        break;
      case 2:
        e = launch_kernel(idx_decode_kernel<2>, grid, dim3(256), 0, stream, q8, q_scale, w, k8,
                          k_scale, vis_len, T, t0, L, kpw, scores);
        break;
      case 3:
        e = launch_kernel(idx_decode_kernel<3>, grid, dim3(256), 0, stream, q8, q_scale, w, k8,
                          k_scale, vis_len, T, t0, L, kpw, scores);
        break;
      default:
        e = launch_kernel(idx_decode_kernel<4>, grid, dim3(256), 0, stream, q8, q_scale, w, k8,
                          k_scale, vis_len, T, t0, L, kpw, scores);
        break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lcs
