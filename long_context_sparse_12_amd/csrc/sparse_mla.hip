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

// LDS tile of 32 rows x 1152 bytes (576 bf16), row-major without padding.
// The 16-byte granule c of row r sits at position c ^ swz(r); swz(r) takes the
// values 0,2,4,6,1,3,5,7 over r = 0..7 (and repeats), so both operand reads
// below hit 32 distinct banks per 128-byte phase:
//   S operand : 16 rows x the same granule  (ds_read_b128)
//   V^T       : 4 rows x 32 consecutive bytes (ds_read_b64_tr_b16)
constexpr int kRowBytes = kKvDim * 2;             // 1152
constexpr int kTileBytes = kTileRows * kRowBytes;  // 36864
constexpr int kStages = 4;
constexpr int kMaxSplitRows = 2048;

__device__ __forceinline__ int swz(int r) { return (((r & 3) << 1) | ((r >> 2) & 1)) & 7; }

__device__ __forceinline__ uint32_t tile_off(int r, int c) { return r * kRowBytes + 16 * (c ^ swz(r)); }

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4s lds_read_tr16(const uint8_t* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4s __attribute__((address_space(3)))*)((__attribute__((address_space(3))) uint8_t*)base + off));
}

__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)gsrc,
                                   (void __attribute__((address_space(3)))*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most `ahead` tiles of `per` loads each are still in flight
template <int PER>
__device__ __forceinline__ void wait_tiles(int ahead) {
  switch (ahead) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<PER>(); break;
    case 2: wait_vm<2 * PER>(); break;
    default: wait_vm<3 * PER>(); break;
  }
}

// Workgroup barrier for the tile pipeline. A workgroup fence would drain every
// in-flight global->LDS load (they count as LDS writes), including those of
// later tiles, so instead: each wave has already waited for its own loads of
// the tile (vmcnt), waits here for its LDS writes (lgkmcnt), and the empty asm
// statements keep the compiler from moving memory accesses across s_barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-workgroup state of the attention loop. The four stage buffers are
// distinct LDS arrays, and every access names its stage at compile time: the
// compiler can then tell a load into one stage from a read of another and does
// not stall reads on the loads that are still in flight for later tiles.
template <bool FP8>
struct AttnCtx {
  static constexpr int kStageBytes = FP8 ? kTileRows * kKvDim : kTileBytes;
  static constexpr int kGranPerRow = FP8 ? kKvDim / 16 : kRowBytes / 16;  // 36 or 72
  static constexpr int kInstr = kTileRows * kGranPerRow / 64;               // 18 or 36
  static constexpr int kPerLo = kInstr / 4, kPerHi = (kInstr + 3) / 4;
  uint8_t* st[kStages];
  uint8_t* cvt;
  const int32_t* s_idx;
  const float* s_scl;
  const uint8_t* kv8;
  int64_t kv_b;
  int n_tiles;
  int wave, lane, g, n;
  float c_log;
  v8bf qT[18];
  v4f acc[32];
  float m_run, l_run;
};

template <bool FP8, int S>
__device__ __forceinline__ void issue_tile(AttnCtx<FP8>& c, int tile) {
  uint8_t* dst = c.st[S];
#pragma unroll
  for (int i = 0; i < AttnCtx<FP8>::kPerHi; ++i) {
    const int j = c.wave + 4 * i;
    if (j < AttnCtx<FP8>::kInstr) {
      const int gi = j * 64 + c.lane;  // granule index in the tile
      const int r = gi / AttnCtx<FP8>::kGranPerRow;
      const int pos = gi - r * AttnCtx<FP8>::kGranPerRow;
      int32_t s = c.s_idx[tile * kTileRows + r];
      s = s >= 0 ? s : 0;  // padding rows load row 0 (finite data, masked below)
      const int gran = FP8 ? pos : (pos ^ swz(r));
      dma16(c.kv8 + (c.kv_b + s) * (int64_t)(FP8 ? kKvDim : kRowBytes) + 16 * gran,
            dst + j * 1024);
    }
  }
}

template <bool FP8, int S>
__device__ __forceinline__ void tile_step(AttnCtx<FP8>& c, int tile, int tid) {
  using C = AttnCtx<FP8>;
  // tile's loads are complete once at most `ahead` later tiles are in flight
  const int ahead = min(kStages - 2, c.n_tiles - 1 - tile);
  if (C::kInstr % 4 == 0 || c.wave >= C::kInstr % 4)
    wait_tiles<C::kPerLo>(ahead);
  else
    wait_tiles<C::kPerHi>(ahead);
  lds_barrier();  // tile visible to all waves; stage S-1 (tile-1) is free
  if (tile + kStages - 1 < c.n_tiles) issue_tile<FP8, (S + kStages - 1) % kStages>(c, tile + kStages - 1);
  const uint8_t* tb = c.st[S];
  if (FP8) {
    // widen 32 rows of E4M3 codes to bf16 (exact) into the swizzled layout
    for (int gi = tid; gi < kTileRows * 36; gi += 256) {
      const int r = gi / 36, c8 = gi - r * 36;
      const v4i x = *(const v4i*)(tb + r * kKvDim + 16 * c8);
      auto hi2 = [](v2f f) {
        return (int)((__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u));
      };
      const v4i lo = v4i{hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[0], false)),
                         hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[0], true)),
                         hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[1], false)),
                         hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[1], true))};
      const v4i hi = v4i{hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[2], false)),
                         hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[2], true)),
                         hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[3], false)),
                         hi2(__builtin_amdgcn_cvt_pk_f32_fp8(x[3], true))};
      *(v4i*)(c.cvt + tile_off(r, 2 * c8)) = lo;
      *(v4i*)(c.cvt + tile_off(r, 2 * c8 + 1)) = hi;
    }
    lds_barrier();
    tb = c.cvt;
  }
  const int g = c.g, n = c.n;
  const int rbase = tile * kTileRows;

  // S^T: rows (2 M-tiles of 16) x 16 heads
  v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    const v4i a0 = *(const v4i*)(tb + tile_off(n, 4 * ks + g));
    const v4i a1 = *(const v4i*)(tb + tile_off(16 + n, 4 * ks + g));
    s0 = mfma_bf16(as_v8bf(a0), c.qT[ks], s0);
    s1 = mfma_bf16(as_v8bf(a1), c.qT[ks], s1);
  }
  // log2-domain logits with row scale and mask; rows 4g+i and 16+4g+i
  float t[8], psc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r0 = 4 * g + i, r1 = 16 + 4 * g + i;
    const bool v0 = c.s_idx[rbase + r0] >= 0, v1 = c.s_idx[rbase + r1] >= 0;
    const float f0 = FP8 ? c.s_scl[rbase + r0] : 1.f, f1 = FP8 ? c.s_scl[rbase + r1] : 1.f;
    psc[i] = f0;
    psc[4 + i] = f1;
    t[i] = v0 ? s0[i] * (f0 * c.c_log) : -INFINITY;
    t[4 + i] = v1 ? s1[i] * (f1 * c.c_log) : -INFINITY;
  }
  float mx = t[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, t[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_new = fmaxf(c.m_run, mx);
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = (t[i] == -INFINITY) ? 0.f : exp2f(t[i] - m_new);
    psum += p[i];
  }
  const float alpha = (c.m_run == -INFINITY) ? 0.f : exp2f(c.m_run - m_new);
  c.l_run = c.l_run * alpha + psum;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int d = 0; d < 32; ++d) c.acc[d] *= alpha;
  }
  c.m_run = m_new;
  // P^T (B operand): k-slots 0-3 = rows 4g..4g+3, 4-7 = rows 16+4g..16+4g+3,
  // each weighted by its row's dequantisation scale
  const v8bf pT = as_v8bf(v4i{(int)pack_bf16x2(p[0] * psc[0], p[1] * psc[1]),
                              (int)pack_bf16x2(p[2] * psc[2], p[3] * psc[3]),
                              (int)pack_bf16x2(p[4] * psc[4], p[5] * psc[5]),
                              (int)pack_bf16x2(p[6] * psc[6], p[7] * psc[7])});
  // O^T += V^T . P^T. The A operand (dims x the same 8 rows) comes from two
  // transposing reads: address lane 4j+q of each 16-lane group points at row
  // (4g+j) [then 16+4g+j], dims 16dt+4q..+3; lane i receives dim 16dt+i.
  const int jr = n >> 2, qd = n & 3;
  const int ra = 4 * g + jr, rb = 16 + 4 * g + jr;
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) {
    const int gc = 2 * dt + (qd >> 1);
    const uint32_t half = 8u * (qd & 1);
    union { v4s h[2]; v8bf b; } u;
    u.h[0] = lds_read_tr16(tb, tile_off(ra, gc) + half);
    u.h[1] = lds_read_tr16(tb, tile_off(rb, gc) + half);
    c.acc[dt] = mfma_bf16(u.b, pT, c.acc[dt]);
  }
}

template <bool FP8>
__global__ void __launch_bounds__(256) sparse_mla_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv,
    const float* __restrict__ kv_scale, const int32_t* __restrict__ idx, int T, int L, int k,
    int rows_per_split, float sm_scale, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  using C = AttnCtx<FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t s_st0[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st1[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st2[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st3[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_cvt[FP8 ? kTileBytes : 16];
  __shared__ int32_t s_idx[kMaxSplitRows];
  __shared__ float s_scl[FP8 ? kMaxSplitRows : 1];

  const int qi = blockIdx.y;  // flattened (b, t)
  const int sp = blockIdx.x;
  const int splits = gridDim.x;
  const int b = qi / T;
  const int tid = threadIdx.x;

  C c;
  c.st[0] = s_st0;
  c.st[1] = s_st1;
  c.st[2] = s_st2;
  c.st[3] = s_st3;
  c.cvt = s_cvt;
  c.s_idx = s_idx;
  c.s_scl = s_scl;
  c.kv8 = (const uint8_t*)kv;
  c.kv_b = (int64_t)b * L;
  c.lane = tid & 63;
  c.wave = tid >> 6;
  c.g = c.lane >> 4;
  c.n = c.lane & 15;
  c.c_log = sm_scale * kLog2e;
  c.m_run = -INFINITY;  // running max of the log2-domain logits of this lane's head
  c.l_run = 0.f;        // this lane's share of the running sum

  const int row_begin = sp * rows_per_split;
  const int row_end = min(k, row_begin + rows_per_split);
  const int n_rows = row_end - row_begin;
  c.n_tiles = (n_rows + kTileRows - 1) / kTileRows;

  // selected positions (and FP8 row scales) of this split; -1 for padding
  for (int i = tid; i < c.n_tiles * kTileRows; i += 256) {
    const int32_t s = i < n_rows ? idx[(int64_t)qi * k + row_begin + i] : -1;
    s_idx[i] = s;
    if (FP8) s_scl[i] = s >= 0 ? kv_scale[(int64_t)b * L + s] : 0.f;
  }
  // Q^T as the B operand: lane holds head (16*wave + n), dims 32*ks + 8g .. +8
  {
    const uint16_t* qh = q + ((int64_t)qi * kAttHeads + 16 * c.wave + c.n) * kKvDim + 8 * c.g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) c.qT[ks] = as_v8bf(*(const v4i*)(qh + 32 * ks));
  }
#pragma unroll
  for (int d = 0; d < 32; ++d) c.acc[d] = v4f{0.f, 0.f, 0.f, 0.f};
  wait_vm<0>();
  __syncthreads();

  if (c.n_tiles > 0) issue_tile<FP8, 0>(c, 0);
  if (c.n_tiles > 1) issue_tile<FP8, 1>(c, 1);
  if (c.n_tiles > 2) issue_tile<FP8, 2>(c, 2);
  for (int tile = 0; tile < c.n_tiles; tile += kStages) {
    tile_step<FP8, 0>(c, tile, tid);
    if (tile + 1 < c.n_tiles) tile_step<FP8, 1>(c, tile + 1, tid);
    if (tile + 2 < c.n_tiles) tile_step<FP8, 2>(c, tile + 2, tid);
    if (tile + 3 < c.n_tiles) tile_step<FP8, 3>(c, tile + 3, tid);
  }

  // per-head totals: the four lane groups hold disjoint row subsets
  float l_tot = c.l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int head = 16 * c.wave + c.n;
  const int g = c.g;
  const float lse2 = l_tot > 0.f ? c.m_run + log2f(l_tot) : -INFINITY;  // log2 domain
  if (splits == 1) {
    uint16_t* orow = out + ((int64_t)qi * kAttHeads + head) * kLatent + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const uint32_t lo = pack_bf16x2(c.acc[dt][0] * inv, c.acc[dt][1] * inv);
      const uint32_t hi = pack_bf16x2(c.acc[dt][2] * inv, c.acc[dt][3] * inv);
      *(v2i*)(orow + 16 * dt) = v2i{(int)lo, (int)hi};
    }
    if (lse && g == 0) lse[(int64_t)qi * kAttHeads + head] = lse2 * kLn2;
  } else {
    float* prow = part_o + (((int64_t)qi * splits + sp) * kAttHeads + head) * kLatent + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *(v4f*)(prow + 16 * dt) = c.acc[dt] * inv;
    if (g == 0) part_lse[((int64_t)qi * splits + sp) * kAttHeads + head] = lse2;
  }
}

// out[q][h][:] = sum_s w_s * o_s / sum_s w_s with w_s = 2^(lse_s - max lse);
// one workgroup per query, consecutive threads on consecutive output dims
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      int splits, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  __shared__ float s_w[kAttHeads][16];
  const int qi = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < kAttHeads) {
    const int head = tid;
    float mx = -INFINITY;
    for (int s = 0; s < splits; ++s)
      mx = fmaxf(mx, part_lse[((int64_t)qi * splits + s) * kAttHeads + head]);
    float wts[16];
    float wsum = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float l = part_lse[((int64_t)qi * splits + s) * kAttHeads + head];
      wts[s] = (l == -INFINITY) ? 0.f : exp2f(l - mx);
      wsum += wts[s];
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    for (int s = 0; s < splits; ++s) s_w[head][s] = wts[s] * inv;
    if (lse) lse[(int64_t)qi * kAttHeads + head] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const int64_t per_split = (int64_t)kAttHeads * kLatent;
  const float* base = part_o + (int64_t)qi * splits * per_split;
  uint16_t* obase = out + (int64_t)qi * per_split;
  for (int i = tid; i < kAttHeads * kLatent / 4; i += 256) {
    const int e = 4 * i;
    const int head = e / kLatent;
    v4f a = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) a += *(const v4f*)(base + s * per_split + e) * s_w[head][s];
    *(v2i*)(obase + e) = v2i{(int)pack_bf16x2(a[0], a[1]), (int)pack_bf16x2(a[2], a[3])};
  }
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
