// sparse_mla.hip -- sparse MLA attention over the selected latent-KV rows.
//
// Core attention reads only the Top-2,048 positions picked by the indexer
// ("一枚 Token，怎样穿过 78 层", panel "MLA 压缩，DSA 精读"), for 64 heads
// (architecture panel) over rows of the rank-512 joint KV compression
// ("KV 低秩联合压缩 Rank 512"). In the absorbed form every head's query is a
// 576-dim vector (512 latent + 64 rope) and the values are the 512 latent dims
// of the same rows, so one gathered row serves all 64 heads.
//
// One workgroup = one query and a slice of its selected rows (split-K over
// the selection for decode), 4 waves x 16 heads. Per tile of 32 rows:
//   gather 32 rows into LDS (FP8 rows are widened to bf16 on the way; their
//   per-row scale is applied to the logits and folded into P), then per wave
//   S^T[32 rows x 16 heads] = KV_tile . Q^T   (bf16 MFMA 16x16x32, K = 576)
//   online softmax per head (a head is one lane column, so its running max and
//   sum stay in the lane)
//   O^T[512 x 16] += V_tile^T . P^T            (bf16 MFMA 16x16x32, K = 32 rows)
// The K order inside each P.V MFMA is a fixed permutation of the 32 rows,
// chosen so that P^T comes straight out of the S^T accumulators.
// With more than one split, normalised partial outputs and their log-sum-exp
// are combined by a second kernel.
#include "common.h"

namespace lcs {
namespace {

constexpr int kTileRows = 32;
constexpr int kRowStrideH = 580;  // LDS row stride in bf16 elements (1160 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SplitPlan {
  int splits;
  int rows_per_split;  // multiple of kTileRows
};

__host__ __device__ inline SplitPlan plan_splits(int64_t queries, int k) {
  SplitPlan p;
  int64_t s = (256 + queries - 1) / queries;  // ~one workgroup per CU
  const int64_t max_s = (k + kTileRows - 1) / kTileRows;
  if (s > max_s) s = max_s;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  int64_t r = (k + s - 1) / s;
  r = (r + kTileRows - 1) / kTileRows * kTileRows;
  p.rows_per_split = (int)r;
  p.splits = (int)((k + r - 1) / r);
  return p;
}

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(const v4i& x) {
  union { v4i i; v8bf b; } u;
  u.i = x;
  return u.b;
}

template <bool FP8>
__global__ void __launch_bounds__(256) sparse_mla_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv,
    const float* __restrict__ kv_scale, const int32_t* __restrict__ idx, int T, int L, int k,
    int rows_per_split, float sm_scale, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) uint16_t s_kv[2][kTileRows * kRowStrideH];
  __shared__ float s_rscale[2][kTileRows];  // per-row logit factor (scale * sm * log2 e)
  __shared__ float s_pscale[2][kTileRows];  // per-row factor folded into P (scale)
  __shared__ float s_mask[2][kTileRows];    // 0 or -inf

  const int qi = blockIdx.y;  // flattened (b, t)
  const int sp = blockIdx.x;
  const int splits = gridDim.x;
  const int b = qi / T;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;

  const int row_begin = sp * rows_per_split;
  const int row_end = min(k, row_begin + rows_per_split);
  const int n_tiles = (row_end - row_begin + kTileRows - 1) / kTileRows;
  const int32_t* qidx = idx + (int64_t)qi * k;
  const float c_log = sm_scale * kLog2e;

  // Q^T as the B operand: lane holds head (16*wave + n), dims 32*ks + 8g .. +8
  v8bf qT[18];
  {
    const uint16_t* qh = q + ((int64_t)qi * kAttHeads + 16 * wave + n) * kKvDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qT[ks] = as_v8bf(*(const v4i*)(qh + 32 * ks));
  }

  // tile loader: 32 rows x 72 granules (16 B of bf16, or 8 FP8 codes), 9 per thread
  v4i pre[9];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int c = tid + 256 * i;
      const int r = c / 72, col = c - r * 72;
      const int j = row_begin + tile * kTileRows + r;
      const int32_t s = (j < row_end) ? qidx[j] : -1;
      if (s >= 0) {
        const int64_t rowoff = (int64_t)b * L + s;
        if (FP8) {
          const v2i x = *(const v2i*)((const uint8_t*)kv + rowoff * kKvDim + 8 * col);
          pre[i] = v4i{x[0], x[1], 0, 0};
        } else {
          pre[i] = *(const v4i*)((const uint16_t*)kv + rowoff * kKvDim + 8 * col);
        }
      } else {
        pre[i] = v4i{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf, int tile) {
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int c = tid + 256 * i;
      const int r = c / 72, col = c - r * 72;
      v4i v = pre[i];
      if (FP8) {
        // E4M3 -> bf16 is exact: widen through fp32 and keep the high halves
        const v2f f0 = __builtin_amdgcn_cvt_pk_f32_fp8(v[0], false);
        const v2f f1 = __builtin_amdgcn_cvt_pk_f32_fp8(v[0], true);
        const v2f f2 = __builtin_amdgcn_cvt_pk_f32_fp8(v[1], false);
        const v2f f3 = __builtin_amdgcn_cvt_pk_f32_fp8(v[1], true);
        auto hi2 = [](v2f f) {
          return (int)((__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u));
        };
        v = v4i{hi2(f0), hi2(f1), hi2(f2), hi2(f3)};
      }
      uint16_t* dst = &s_kv[buf][r * kRowStrideH + 8 * col];
      *(v2i*)dst = v2i{v[0], v[1]};
      *(v2i*)(dst + 4) = v2i{v[2], v[3]};
    }
    if (tid < kTileRows) {
      const int j = row_begin + tile * kTileRows + tid;
      const int32_t s = (j < row_end) ? qidx[j] : -1;
      float sc = 1.f;
      if (FP8 && s >= 0) sc = kv_scale[(int64_t)b * L + s];
      s_rscale[buf][tid] = sc * c_log;
      s_pscale[buf][tid] = sc;
      s_mask[buf][tid] = s >= 0 ? 0.f : -INFINITY;
    }
  };

  v4f acc[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) acc[d] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of the log2-domain logits of this lane's head
  float l_run = 0.f;        // this lane's share of the running sum

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0, 0);
  }
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) load_tile(tile + 1);
    const uint16_t* kvb = s_kv[buf];

    // S^T: rows (2 M-tiles of 16) x 16 heads
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const uint16_t* a0p = kvb + n * kRowStrideH + 32 * ks + 8 * g;
      const uint16_t* a1p = a0p + 16 * kRowStrideH;
      const v2i x0 = *(const v2i*)a0p, y0 = *(const v2i*)(a0p + 4);
      const v2i x1 = *(const v2i*)a1p, y1 = *(const v2i*)(a1p + 4);
      s0 = mfma_bf16(as_v8bf(v4i{x0[0], x0[1], y0[0], y0[1]}), qT[ks], s0);
      s1 = mfma_bf16(as_v8bf(v4i{x1[0], x1[1], y1[0], y1[1]}), qT[ks], s1);
    }
    // log2-domain logits with row scale and mask; rows 4g+i and 16+4g+i
    float t[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = 4 * g + i, r1 = 16 + 4 * g + i;
      t[i] = s0[i] * s_rscale[buf][r0] + s_mask[buf][r0];
      t[4 + i] = s1[i] * s_rscale[buf][r1] + s_mask[buf][r1];
    }
    float mx = t[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, t[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = (t[i] == -INFINITY) ? 0.f : exp2f(t[i] - m_new);
      psum += p[i];
    }
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int d = 0; d < 32; ++d) acc[d] *= alpha;
    }
    m_run = m_new;
    // P^T (B operand): k-slots 0-3 = rows 4g..4g+3, 4-7 = rows 16+4g..16+4g+3,
    // each weighted by its row's dequantisation scale
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r0 = 4 * g + 2 * i, r1 = 16 + 4 * g + 2 * i;
      pk[i] = pack_bf16x2(p[2 * i] * s_pscale[buf][r0], p[2 * i + 1] * s_pscale[buf][r0 + 1]);
      pk[2 + i] = pack_bf16x2(p[4 + 2 * i] * s_pscale[buf][r1], p[5 + 2 * i] * s_pscale[buf][r1 + 1]);
    }
    const v8bf pT = as_v8bf(v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});
    // O^T += V^T . P^T ; A operand: lane holds dim (16*dt + n) for the same 8 rows
    const uint16_t* vrow0 = kvb + (4 * g) * kRowStrideH + n;
    const uint16_t* vrow1 = kvb + (16 + 4 * g) * kRowStrideH + n;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const int d = 16 * dt;
      const uint32_t e0 = vrow0[d], e1 = vrow0[kRowStrideH + d];
      const uint32_t e2 = vrow0[2 * kRowStrideH + d], e3 = vrow0[3 * kRowStrideH + d];
      const uint32_t e4 = vrow1[d], e5 = vrow1[kRowStrideH + d];
      const uint32_t e6 = vrow1[2 * kRowStrideH + d], e7 = vrow1[3 * kRowStrideH + d];
      const v4i a = v4i{(int)(e0 | (e1 << 16)), (int)(e2 | (e3 << 16)), (int)(e4 | (e5 << 16)),
                        (int)(e6 | (e7 << 16))};
      acc[dt] = mfma_bf16(as_v8bf(a), pT, acc[dt]);
    }
    if (tile + 1 < n_tiles) store_tile(buf ^ 1, tile + 1);
    __syncthreads();
  }

  // per-head totals: the four lane groups hold disjoint row subsets
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int head = 16 * wave + n;
  const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;  // log2 domain
  if (splits == 1) {
    uint16_t* orow = out + ((int64_t)qi * kAttHeads + head) * kLatent + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const uint32_t lo = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      const uint32_t hi = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *(v2i*)(orow + 16 * dt) = v2i{(int)lo, (int)hi};
    }
    if (lse && g == 0) lse[(int64_t)qi * kAttHeads + head] = lse2 * kLn2;
  } else {
    float* prow = part_o + (((int64_t)qi * splits + sp) * kAttHeads + head) * kLatent + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *(v4f*)(prow + 16 * dt) = acc[dt] * inv;
    if (g == 0) part_lse[((int64_t)qi * splits + sp) * kAttHeads + head] = lse2;
  }
}

// out[q][h][:] = sum_s w_s * o_s / sum_s w_s with w_s = 2^(lse_s - max lse)
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      int splits, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  const int qi = blockIdx.x;
  const int tid = threadIdx.x;
  // 64 heads x 512 dims; thread handles head (tid / 4) and 128 dims
  const int head = tid >> 2;
  const int d0 = (tid & 3) * 128;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s)
    mx = fmaxf(mx, part_lse[((int64_t)qi * splits + s) * kAttHeads + head]);
  float wsum = 0.f;
  float wts[16];
  for (int s = 0; s < splits; ++s) {
    const float l = part_lse[((int64_t)qi * splits + s) * kAttHeads + head];
    const float wgt = (l == -INFINITY) ? 0.f : exp2f(l - mx);
    wts[s] = wgt;
    wsum += wgt;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* orow = out + ((int64_t)qi * kAttHeads + head) * kLatent + d0;
  for (int d = 0; d < 128; d += 4) {
    v4f a = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
      const v4f o = *(const v4f*)(part_o + (((int64_t)qi * splits + s) * kAttHeads + head) * kLatent + d0 + d);
      a += o * wts[s];
    }
    a *= inv;
    *(v2i*)(orow + d) = v2i{(int)pack_bf16x2(a[0], a[1]), (int)pack_bf16x2(a[2], a[3])};
  }
  if (lse && (tid & 3) == 0)
    lse[(int64_t)qi * kAttHeads + head] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
}

}  // namespace

size_t attn_workspace_bytes(int64_t queries, int k) {
  const SplitPlan p = plan_splits(queries, k);
  if (p.splits <= 1) return 0;
  size_t o = (size_t)queries * p.splits * kAttHeads * kLatent * sizeof(float);
  size_t l = (size_t)queries * p.splits * kAttHeads * sizeof(float);
  return o + l;
}

hipError_t launch_sparse_mla(const uint16_t* q, const void* kv, bool kv_fp8,
                             const float* kv_scale, const int32_t* idx, int B, int T, int L,
                             int k, float sm_scale, uint16_t* out, float* lse,
                             void* workspace, hipStream_t stream) {
  const int64_t queries = (int64_t)B * T;
  const SplitPlan p = plan_splits(queries, k);
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (p.splits > 1) {
    part_o = (float*)workspace;
    part_lse = part_o + (size_t)queries * p.splits * kAttHeads * kLatent;
  }
  dim3 grid((unsigned)p.splits, (unsigned)queries);
  hipError_t e;
  if (kv_fp8)
    e = launch_kernel(sparse_mla_kernel<true>, grid, dim3(256), 0, stream, q, kv, kv_scale, idx, T,
                      L, k, p.rows_per_split, sm_scale, out, lse, part_o, part_lse);
  else
    e = launch_kernel(sparse_mla_kernel<false>, grid, dim3(256), 0, stream, q, kv, kv_scale, idx,
                      T, L, k, p.rows_per_split, sm_scale, out, lse, part_o, part_lse);
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_kernel(combine_kernel, dim3((unsigned)queries), dim3(256), 0, stream, part_o,
                       part_lse, p.splits, out, lse);
}

}  // namespace lcs
