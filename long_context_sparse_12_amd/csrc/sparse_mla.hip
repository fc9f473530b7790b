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
// With more than one split, normalised partial outputs (bf16: the final output
// is bf16 too, and rounding the partials adds at most 2^-8 relative error) and
// their log-sum-exp (fp32) are combined by a second kernel.
#include <mutex>

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

#ifndef LCS_ATTN_TARGET_WGS
#define LCS_ATTN_TARGET_WGS 256  // about one workgroup per CU
#endif
#ifndef LCS_ATTN_MAX_SPLITS
#define LCS_ATTN_MAX_SPLITS 32
#endif

__host__ __device__ inline SplitPlan plan_splits(int64_t queries, int k) {
  SplitPlan p;
  int64_t s = (LCS_ATTN_TARGET_WGS + queries - 1) / queries;
  const int64_t max_s = (k + kTileRows - 1) / kTileRows;
  if (s > max_s) s = max_s;
  if (s > LCS_ATTN_MAX_SPLITS) s = LCS_ATTN_MAX_SPLITS;
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

__device__ __forceinline__ v16f mfma32_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(const v4i& x) {
  union { v4i i; v8bf b; } u;
  u.i = x;
  return u.b;
}

// LDS tile of 32 rows x 1152 bytes (576 bf16), row-major without padding.
// The 16-byte granule c of row r sits at position c ^ (r & 7). Measured with
// the LDS bank-conflict counter, this makes both operand reads below
// conflict-free (the unswizzled layout stalls 3 of every 4 LDS cycles):
//   S operand : 16 rows x the same granule  (ds_read_b128)
//   V^T       : 4 rows x 32 consecutive bytes (ds_read_b64_tr_b16)
constexpr int kRowBytes = kKvDim * 2;             // 1152
constexpr int kTileBytes = kTileRows * kRowBytes;  // 36864
constexpr int kStages = 3;
constexpr int kMaxSplitRows = 2048;
constexpr float kRescaleSlack = 8.f;
#ifndef LCS_ATTN_SBATCH
#define LCS_ATTN_SBATCH 6
#endif
constexpr int kSBatch = LCS_ATTN_SBATCH;  // S-operand reads in flight per batch

__device__ __forceinline__ int swz(int r) { return r & 7; }

__device__ __forceinline__ uint32_t tile_off(int r, int c) { return r * kRowBytes + 16 * (c ^ swz(r)); }

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4s lds_read_tr16(const uint8_t* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4s __attribute__((address_space(3)))*)((__attribute__((address_space(3))) uint8_t*)base + off));
}

__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)gsrc,
                                   (void __attribute__((address_space(3)))*)lds_base, 16, 0, 0);
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

// Per-workgroup state of the attention loop. Eight waves: wave w serves head
// group hg = w & 1 (32 heads) and dim quarter dq = w >> 1. It computes the
// partial S over dims [144 dq, 144 dq + 144) and the output dims
// [128 dq, 128 dq + 128). The three stage buffers are distinct LDS arrays and
// every access names its stage at compile time, so the compiler can tell a
// load into one stage from a read of another and does not stall reads on the
// loads still in flight for later tiles.
constexpr int kWavesA = 8;
constexpr int kThreadsA = 64 * kWavesA;

template <bool FP8>
struct AttnCtx {
  static constexpr int kStageBytes = FP8 ? kTileRows * kKvDim : kTileBytes;
  static constexpr int kGranPerRow = FP8 ? kKvDim / 16 : kRowBytes / 16;  // 36 or 72
  static constexpr int kInstr = kTileRows * kGranPerRow / 64;               // 18 or 36
  static constexpr int kPerLo = kInstr / kWavesA, kPerHi = (kInstr + kWavesA - 1) / kWavesA;
  uint8_t* st[kStages];
  uint8_t* cvt;
  float* xch;  // partial S of every wave
  const int32_t* s_idx;
  const float* s_scl;
  const uint8_t* kv8;
  int64_t kv_b;
  int n_tiles;
  int wave, lane;
  int hg, dq;
  float c_log;
  v8bf qT[9];   // Q^T B operand: head 32hg + (lane&31), dims 144dq + 16ks + 8(lane>>5) .. +8
  v16f acc[4];  // O^T: dims 128dq + 32mt + (row of the 32x32 tile), heads as columns
  float m_run, l_run;
};

template <bool FP8, int S>
__device__ __forceinline__ void issue_tile(AttnCtx<FP8>& c, int tile) {
  using C = AttnCtx<FP8>;
  uint8_t* dst = c.st[S];
  // all row positions first (independent LDS reads), then the loads
  int32_t rows[C::kPerHi];
  int gran[C::kPerHi];
#pragma unroll
  for (int i = 0; i < C::kPerHi; ++i) {
    const int j = c.wave + kWavesA * i;
    const int gi = (j < C::kInstr ? j : 0) * 64 + c.lane;  // granule index in the tile
    const int r = gi / C::kGranPerRow;
    const int pos = gi - r * C::kGranPerRow;
    gran[i] = FP8 ? pos : (pos ^ swz(r));
    rows[i] = c.s_idx[tile * kTileRows + r];
  }
#pragma unroll
  for (int i = 0; i < C::kPerHi; ++i) {
    const int j = c.wave + kWavesA * i;
    if (j < C::kInstr) {
      // padding rows load the sequence's first row (weighted zero below)
      const int32_t s = rows[i] >= 0 ? rows[i] : 0;
      dma16(c.kv8 + (c.kv_b + s) * (int64_t)(FP8 ? kKvDim : kRowBytes) + 16 * gran[i],
            dst + j * 1024);
    }
  }
}

template <bool FP8, int S>
__device__ __forceinline__ void tile_step(AttnCtx<FP8>& c, int tile, int tid) {
  using C = AttnCtx<FP8>;
  // tile's loads are complete once at most `ahead` later tiles are in flight
  const int ahead = min(kStages - 2, c.n_tiles - 1 - tile);
  if (C::kInstr % kWavesA == 0 || c.wave >= C::kInstr % kWavesA)
    wait_tiles<C::kPerLo>(ahead);
  else
    wait_tiles<C::kPerHi>(ahead);
  lds_barrier();  // tile visible to all waves; stage S-1 (tile-1) is free
  if (tile + kStages - 1 < c.n_tiles) issue_tile<FP8, (S + kStages - 1) % kStages>(c, tile + kStages - 1);
  const uint8_t* tb = c.st[S];
  if (FP8) {
    // widen 32 rows of E4M3 codes to bf16 (exact) into the swizzled layout
    for (int gi = tid; gi < kTileRows * 36; gi += kThreadsA) {
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
  const int lane = c.lane, ln = lane & 31, h = lane >> 5;
  const int rbase = tile * kTileRows;

  // Partial S^T[32 rows x 32 heads] over this wave's 144 dims (9 steps of
  // v_mfma_f32_32x32x16_bf16). A operand: lane holds row (lane&31), dims
  // 16ks+8h..+8, i.e. granule 2ks+h, at 8(ks/4) + ((2(ks&3)+h) ^ (row&7)):
  // four base addresses plus immediate offsets of 128(ks/4) bytes.
  const uint8_t* sb[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) sb[m] = tb + ln * kRowBytes + 16 * ((2 * m + h) ^ swz(ln));
  v4i a[9];
  const int ks0 = 9 * c.dq;
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int ks = ks0 + i;
    a[i] = *(const v4i*)(sb[ks & 3] + 128 * (ks >> 2));
  }
  v16f se, so;
#pragma unroll
  for (int i = 0; i < 16; ++i) { se[i] = 0.f; so[i] = 0.f; }
#pragma unroll
  for (int i = 0; i < 9; i += 2) {
    se = mfma32_bf16(as_v8bf(a[i]), c.qT[i], se);
    if (i + 1 < 9) so = mfma32_bf16(as_v8bf(a[i + 1]), c.qT[i + 1], so);
  }
  // full S: the four partials of the head group, summed in a fixed order so
  // that all four waves hold bit-identical values
  float sfull[16];
  {
    float* mine = c.xch + (c.wave * 16) * 64 + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) mine[i * 64] = se[i] + so[i];
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* col = c.xch + (c.hg * 16 + i) * 64 + lane;  // wave hg + 2k at 2k*16*64
      sfull[i] = ((col[0] + col[2 * 16 * 64]) + col[4 * 16 * 64]) + col[6 * 16 * 64];
    }
  }
  // lane holds head (lane&31) for rows 8(i/4) + 4h + (i&3), i = 0..15
  float t[16], psc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + 4 * h + (i & 3);
    const bool v = c.s_idx[rbase + r] >= 0;
    const float f = FP8 ? c.s_scl[rbase + r] : 1.f;
    psc[i] = f;
    t[i] = v ? sfull[i] * (f * c.c_log) : -INFINITY;
  }
  float mx = t[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, t[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  // Lazy rescaling: the exponent offset m_run only moves when the tile max
  // exceeds it by more than kRescaleSlack (log2 units), so P stays below
  // 2^kRescaleSlack and the accumulators are rescaled rarely. The final O / l
  // and lse = m_run + log2 l are exact for any offset. Before the first valid
  // row the accumulators are zero, so moving the offset needs no rescale.
  const bool first = c.m_run == -INFINITY;
  const float m_new = (first || mx > c.m_run + kRescaleSlack) ? mx : c.m_run;
  float p[16];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p[i] = (t[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(t[i] - m_new);
    psum += p[i];
  }
  if (__ballot(!first && m_new != c.m_run)) {
    const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(c.m_run - m_new);
    c.l_run *= alpha;
#pragma unroll
    for (int d = 0; d < 4; ++d) c.acc[d] *= alpha;
  }
  c.l_run += psum;
  c.m_run = m_new;
  // P^T B operand of the two 16-row K-steps: k-slot s of K-step ks is row
  // 16ks + 8(s/4) + 4h + (s&3), i.e. accumulator element 8ks + s; each
  // weighted by its row's dequantisation scale
  v8bf pT[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int o = 8 * ks;
    pT[ks] = as_v8bf(v4i{(int)pack_bf16x2(p[o + 0] * psc[o + 0], p[o + 1] * psc[o + 1]),
                         (int)pack_bf16x2(p[o + 2] * psc[o + 2], p[o + 3] * psc[o + 3]),
                         (int)pack_bf16x2(p[o + 4] * psc[o + 4], p[o + 5] * psc[o + 5]),
                         (int)pack_bf16x2(p[o + 6] * psc[o + 6], p[o + 7] * psc[o + 7])});
  }
  // O^T[dims x heads] += V^T . P^T, 4 M-tiles of 32 dims x 2 K-steps. The A
  // operand (lane: dim 32mt + (lane&31), the same 8 rows as its P^T k-slots)
  // comes from two transposing reads per MFMA: in each 16-lane group, address
  // lane 4j+q points at row 16ks + 4h + j (then + 8), dims base + 4q .. +3, and
  // lane i receives dim base + i. Row r's swizzle r & 7 = 4h + j for all of
  // these rows, so each M-tile parity needs one base address.
  const int a16 = lane & 15, jr = a16 >> 2, qd = a16 & 3, mh = (lane >> 4) & 1;
  const int r0 = 4 * h + jr;
  const uint8_t* vb[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int lo3 = (4 * par + 2 * mh + (qd >> 1)) ^ swz(r0);
    vb[par] = tb + r0 * kRowBytes + 16 * (16 * c.dq + lo3) + 8 * (qd & 1);
  }
  v8bf va[8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int off = 16 * ks * kRowBytes + 128 * (mt >> 1);
      union { v4s h4[2]; v8bf b; } u;
      u.h4[0] = lds_read_tr16(vb[mt & 1], off);
      u.h4[1] = lds_read_tr16(vb[mt & 1], off + 8 * kRowBytes);
      va[2 * mt + ks] = u.b;
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    c.acc[mt] = mfma32_bf16(va[2 * mt], pT[0], c.acc[mt]);
    c.acc[mt] = mfma32_bf16(va[2 * mt + 1], pT[1], c.acc[mt]);
  }
}

template <bool FP8>
__global__ void __launch_bounds__(kThreadsA) sparse_mla_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv,
    const float* __restrict__ kv_scale, int64_t kv_stride, const int32_t* __restrict__ idx, int T,
    int L, int k, int rows_per_split, float sm_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  using C = AttnCtx<FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t s_st0[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st1[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st2[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_cvt[FP8 ? kTileBytes : 16];
  __shared__ int32_t s_idx[kMaxSplitRows];
  __shared__ float s_scl[FP8 ? kMaxSplitRows : 1];
  __shared__ float s_xch[kWavesA * 16 * 64];

  const int qi = blockIdx.y;  // flattened (b, t)
  const int sp = blockIdx.x;
  const int splits = gridDim.x;
  const int b = qi / T;
  const int tid = threadIdx.x;

  C c;
  c.st[0] = s_st0;
  c.st[1] = s_st1;
  c.st[2] = s_st2;
  c.cvt = s_cvt;
  c.xch = s_xch;
  c.s_idx = s_idx;
  c.s_scl = s_scl;
  c.kv8 = (const uint8_t*)kv;
  c.kv_b = (int64_t)b * kv_stride;  // this sequence's first row
  c.lane = tid & 63;
  c.wave = tid >> 6;
  c.hg = c.wave & 1;
  c.dq = c.wave >> 1;
  c.c_log = sm_scale * kLog2e;
  c.m_run = -INFINITY;  // exponent offset (log2 domain) of this lane's head
  c.l_run = 0.f;        // this lane's share of the running sum

  const int row_begin = sp * rows_per_split;
  const int row_end = min(k, row_begin + rows_per_split);
  const int n_rows = row_end - row_begin;
  c.n_tiles = (n_rows + kTileRows - 1) / kTileRows;

  // selected positions of this split; -1 for padding
  for (int i = tid; i < c.n_tiles * kTileRows; i += kThreadsA)
    s_idx[i] = i < n_rows ? idx[(int64_t)qi * k + row_begin + i] : -1;
  // Q^T as the B operand: lane holds head 32hg + (lane&31), dims 144dq + 16ks + 8(lane>>5) .. +8
  {
    const uint16_t* qh = q + ((int64_t)qi * kAttHeads + 32 * c.hg + (c.lane & 31)) * kKvDim +
                         144 * c.dq + 8 * (c.lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) c.qT[ks] = as_v8bf(*(const v4i*)(qh + 16 * ks));
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) c.acc[d][i] = 0.f;
  wait_vm<0>();
  __syncthreads();

  static_assert(kStages == 3, "the loop below is unrolled for three stages");
  // FP8 row scales: their loads depend on the positions just published, so
  // they go out together with the first two tiles' gathers (one memory
  // latency for both) and reach LDS before the first tile step's barrier
  constexpr int kSclPer = kMaxSplitRows / kThreadsA;
  float scl[FP8 ? kSclPer : 1];
  if (FP8) {
#pragma unroll
    for (int u = 0; u < kSclPer; ++u) {
      const int i = tid + kThreadsA * u;
      const int32_t s = i < c.n_tiles * kTileRows ? s_idx[i] : -1;
      scl[u] = s >= 0 ? kv_scale[c.kv_b + s] : 0.f;
    }
  }
  if (c.n_tiles > 0) issue_tile<FP8, 0>(c, 0);
  if (c.n_tiles > 1) issue_tile<FP8, 1>(c, 1);
  if (FP8) {
#pragma unroll
    for (int u = 0; u < kSclPer; ++u) {
      const int i = tid + kThreadsA * u;
      if (i < c.n_tiles * kTileRows) s_scl[i] = scl[u];
    }
  }
  for (int tile = 0; tile < c.n_tiles; tile += kStages) {
    tile_step<FP8, 0>(c, tile, tid);
    if (tile + 1 < c.n_tiles) tile_step<FP8, 1>(c, tile + 1, tid);
    if (tile + 2 < c.n_tiles) tile_step<FP8, 2>(c, tile + 2, tid);
  }

  // per-head totals: the two lane halves hold disjoint row subsets; all waves
  // of a head group hold identical softmax state
  float l_tot = c.l_run;
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int h = c.lane >> 5;
  const int head = 32 * c.hg + (c.lane & 31);
  const float lse2 = l_tot > 0.f ? c.m_run + log2f(l_tot) : -INFINITY;  // log2 domain
  // lane holds dims 128dq + 32mt + 8(i/4) + 4h + (i&3) of its head; the
  // normalised output goes to `out` (one split) or to this split's partial
  // output (bf16, same layout), whose log-sum-exp the combine needs. As in
  // the split-role kernel below, each wave transposes its [32 heads][128
  // dims] block through LDS (rows 272 bytes apart; with FP8 rows two waves
  // per stage buffer and the last two in the conversion buffer, with bf16
  // rows four per stage buffer) and stores whole 256-byte rows, four per
  // instruction.
  constexpr int kEpiRow = 272, kEpiWave = 32 * kEpiRow;
  static_assert(2 * kEpiWave <= C::kStageBytes && 4 * kEpiWave <= kTileBytes, "epilogue staging");
  __syncthreads();  // every wave is done with the stage and conversion buffers
  // (constant indices into c.st: a runtime index would put the context in scratch)
  const int eslot = FP8 ? c.wave >> 1 : c.wave >> 2;
  uint8_t* ebuf = eslot == 0 ? c.st[0] : eslot == 1 ? c.st[1] : eslot == 2 ? c.st[2] : c.cvt;
  uint8_t* eb = ebuf + (FP8 ? (c.wave & 1) : (c.wave & 3)) * kEpiWave;
  const int ln = c.lane & 31;
  // a head with no visible row writes zeros, whatever its padding rows held
  // (0 x NaN is not 0). All heads of a query share its rows, so this is rare
  // and, for finite logits, the same for the whole wave: a scalar branch.
  if (!__all(l_tot > 0.f)) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) c.acc[mt][i] = l_tot > 0.f ? c.acc[mt][i] : 0.f;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const v16f& a = c.acc[mt];
      const uint32_t lo = pack_bf16x2(a[4 * i4] * inv, a[4 * i4 + 1] * inv);
      const uint32_t hi = pack_bf16x2(a[4 * i4 + 2] * inv, a[4 * i4 + 3] * inv);
      *(v2i*)(eb + ln * kEpiRow + 2 * (32 * mt + 8 * i4 + 4 * h)) = v2i{(int)lo, (int)hi};
    }
  uint16_t* obase = (splits == 1 ? out + ((int64_t)qi * kAttHeads + 32 * c.hg) * kLatent
                                 : part_o + (((int64_t)qi * splits + sp) * kAttHeads + 32 * c.hg) * kLatent) +
                    128 * c.dq;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int hl = 4 * it + (c.lane >> 4);  // head within the group
    const v4i x = *(const v4i*)(eb + hl * kEpiRow + 16 * (c.lane & 15));
    *(v4i*)(obase + hl * kLatent + 8 * (c.lane & 15)) = x;
  }
  if (c.dq == 0 && h == 0) {
    if (splits > 1)
      part_lse[((int64_t)qi * splits + sp) * kAttHeads + head] = lse2;
    else if (lse)
      lse[(int64_t)qi * kAttHeads + head] = lse2 * kLn2;
  }
}

// ---------------------------------------------------------------------------
// bf16 latent KV: split roles. The 64 x 32 logits of a 32-row tile need K =
// 576 per output element, so splitting the dims over waves (as above) costs
// an exchange of partial logits per tile. Here two "S waves" (one per head
// group of 32) each hold their group's whole Q^T (36 K-steps, 144 VGPRs) and
// compute the full S^T[32 rows x 32 heads] of a tile alone, then the online
// softmax, and hand P^T (bf16, 2 KB per head group) and the rescale factor to
// four "PV waves" through LDS. PV wave (hg, dh) owns O^T for 256 output dims
// of its head group (8 accumulators, 128 VGPRs). Two "gather waves" issue the
// row gathers. Waves land on SIMD (wave & 3): the S waves (0, 1) share their
// SIMDs only with the gather waves (4, 5), which use no MFMA, and the PV waves
// (2, 3, 6, 7) fill SIMDs 2 and 3, so each SIMD's matrix core gets 36 (S) or
// 2 x 16 (PV) MFMAs per tile. The roles work on consecutive tiles at the same
// time (S waves on tile j+1 while PV waves finish tile j), with one barrier
// per tile; four stage buffers give every gather two tiles of lead time.
constexpr int kWavesB = 8;
constexpr int kThreadsB = 64 * kWavesB;
constexpr int kStagesB = 4;
constexpr int kGatherWaves = 2;
constexpr int kDmaPerB = kTileBytes / 1024 / kGatherWaves;  // 18 gathers per lane per tile

enum Role { kRoleS, kRolePV, kRoleGather };
__device__ __forceinline__ Role role_of(int wave) {
  return wave < 2 ? kRoleS : (wave == 4 || wave == 5) ? kRoleGather : kRolePV;
}

#ifndef LCS_ATTN_S_AHEAD
#define LCS_ATTN_S_AHEAD 8
#endif
#ifndef LCS_ATTN_B_TARGET_WGS
#define LCS_ATTN_B_TARGET_WGS 256
#endif
#ifndef LCS_ATTN_B_MAX_SPLITS
#define LCS_ATTN_B_MAX_SPLITS 16  // fewer, longer splits pipeline better than a wider combine
#endif

// Splits per query: as many as fit one round of workgroups (one per CU), so
// no launch ends with a partial second round: 192 verify queries take one
// split each (192 workgroups, no combine) rather than two (384 workgroups,
// the second round on half the CUs, and a combine).
__host__ __device__ inline SplitPlan plan_splits_b(int64_t queries, int k) {
  SplitPlan p;
  int64_t s = LCS_ATTN_B_TARGET_WGS / queries;
  const int64_t max_s = (k + kTileRows - 1) / kTileRows;
  if (s > max_s) s = max_s;
  if (s > LCS_ATTN_B_MAX_SPLITS) s = LCS_ATTN_B_MAX_SPLITS;
  if (s < 1) s = 1;
  int64_t r = (k + s - 1) / s;
  r = (r + kTileRows - 1) / kTileRows * kTileRows;
  p.rows_per_split = (int)r;
  p.splits = (int)((k + r - 1) / r);
  return p;
}

// LDS layout of a bf16 tile in this kernel: granule c of row r sits at
// (c & ~7) | ((c & 7) ^ swz_b(r)) with swz_b(r) = 4 * bit1(r) + bits 3..2 (r).
// The LDS serves 256 bytes per cycle: 16 lanes of a 16-byte read or 32 lanes
// of an 8-byte one. For the S operand (16 lanes = rows 0..15 or 16..31 at one
// granule) swz_b is a bijection on the even and on the odd rows; for the
// transposing V reads (32 lanes = 4 rows x 4 granules of an aligned group)
// rows r and r + 2 differ in bit 2 of the swizzle. Both are then free of bank
// conflicts (row 8 apart: swz_b(r + 8) = swz_b(r) ^ 2; 16 apart: equal).
__device__ __forceinline__ int swz_b(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// byte offset of bf16 granule cg (8 dims) of row r in a stage
__device__ __forceinline__ int stage_off_b(int r, int cg) {
  return r * kRowBytes + 16 * ((cg & ~7) | ((cg & 7) ^ swz_b(r)));
}

// state shared by both roles
struct AttnB {
  uint8_t* st[kStagesB];
  uint8_t* p_buf;   // [2 parity][2 hg][64 lanes][32 B]  P^T B operands
  float* alpha;     // [2 parity][2 hg][32 heads]
  int* flag;        // [2 parity][2 hg]
  int32_t* ring;    // [4 slots][32 rows]  positions of the tiles t with t & 3 = slot
  float* sring;     // [4 slots][32 rows]  FP8 row scales of the same tiles
  const float* kscale;   // FP8 row scales of this sequence (kv_scale + b * stride), or
                         // of the whole pool (paged)
  const int32_t* idx_q;  // this split's selected positions (global memory)
  const int32_t* btab;   // paged: this sequence's block table row
  int lbs, nblk;         // paged: log2 rows per block, blocks in the pool
  int n_rows, n_tiles;
  int wave, lane, hg;
  uint32_t pad_row;  // the row padding entries load: the sequence's position 0 (paged: its pool row)
};

// A split may hold all k selected rows, so its positions do not sit in LDS
// at once: S wave 0 streams them, one tile per pipeline step, into a ring of
// four 32-entry slots (tile t in slot t & 3, -1 for padding and for rows past
// the split's end). Only that wave loads positions into registers; the gather
// waves read them from the ring and issue nothing but global->LDS copies, so
// their waits count copies alone (loads into registers in flight beside the
// copies would make the compiler wait for all of them before any use).
constexpr int kPosSlots = 4;
__device__ __forceinline__ int32_t* pos_slot(const AttnB& c, int tile) {
  return c.ring + (tile & (kPosSlots - 1)) * kTileRows;
}

// position of row (lane & 31) of `tile` (rows past the end read the split's
// last entry, a valid address; ring_put masks them)
__device__ __forceinline__ int32_t load_pos(const AttnB& c, int tile) {
  return c.idx_q[min(tile * kTileRows + (c.lane & 31), c.n_rows - 1)];
}

__device__ __forceinline__ void ring_put(const AttnB& c, int tile, int32_t p) {
  const int r = tile * kTileRows + (c.lane & 31);
  if (c.lane < kTileRows) pos_slot(c, tile)[c.lane] = r < c.n_rows ? p : -1;
}

// Paged KV: a sequence's position p lives in pool block btab[p >> lbs] at row
// p & (bs - 1). S wave 0 then streams pool rows instead of positions into the
// ring, one pipeline step later than the positions (the block loads need the
// positions): positions two steps ahead, blocks one step ahead. Block ids are
// clamped to the pool; -1 (no row) stays -1.
__device__ __forceinline__ int32_t load_blk(const AttnB& c, int32_t p) {
  return c.btab[(p >= 0 ? p : 0) >> c.lbs];
}
__device__ __forceinline__ int32_t pool_row(const AttnB& c, int32_t p, int32_t blk) {
  const int32_t bk = min(max(blk, 0), c.nblk - 1);
  return p >= 0 ? (bk << c.lbs) | (p & ((1 << c.lbs) - 1)) : -1;
}

// FP8 KV: the row scales follow the positions one step later (their loads
// need the positions): tile t's scales go into slot t & 3 of the scale ring
// in step t-3 and are read by the S waves in step t-1.
__device__ __forceinline__ float load_scale(const AttnB& c, int32_t p) {
  return c.kscale[p >= 0 ? p : 0];  // padding rows: replaced by 1 in s_phase
}
__device__ __forceinline__ void scale_put(const AttnB& c, int tile, float v) {
  if (c.lane < kTileRows) c.sring[(tile & (kPosSlots - 1)) * kTileRows + c.lane] = v;
}

struct SWave {
  v8bf qT[36];  // Q^T: head 32hg + (lane&31), dims 16ks + 8(lane>>5) .. +8
  float c_log;
  float m_run, l_run;
  int32_t pn;  // S wave 0: positions of the next tile to enter the ring
  float sn;    // S wave 0, FP8: scales of the next tile to enter the scale ring
  int32_t bn;  // S wave 0, paged: pool blocks of the positions pn
  int32_t pn2; // S wave 0, paged: positions of the tile after pn's
};

struct PWave {
  v16f acc[8];  // O^T: dims 256dh + 32mt + (row of the 32x32 tile), heads as columns
  int dh;
};

struct GWave {
  int g;                // 0 or 1 (wave-uniform)
  const uint8_t* kvb;   // this sequence's rows: kv + b * stride * (1152 or 576); paged: the pool
  int dma_row[kDmaPerB];  // row inside the tile of each gather
  int dma_off[kDmaPerB];  // byte offset inside the row (swizzled granule)
};

// FP8 KV: a tile is 32 rows x 36 granules of 16 E4M3 codes. Gather lane (g, l)
// carries granules 64 (g + 2 i) + l, i < 9: it loads them into registers one
// step ahead, then widens each to two bf16 granules (exact) and writes them
// into the stage in the bf16 kernel's swizzled layout. These waves issue only
// register loads, a fixed nine per step, so the compiler's own waits before
// the widening leave the next tile's loads in flight.
constexpr int kFp8Per = kTileRows * (kKvDim / 16) / (64 * kGatherWaves);  // 9
struct GWave8 {
  int g;
  const uint8_t* kvb;     // kv + b * stride * 576; paged: the pool
  int row[kFp8Per];       // tile row of each granule
  int src[kFp8Per];       // byte offset inside the 576-byte row
  int dst[kFp8Per];       // stage byte offset of its first bf16 granule
  int dst2[kFp8Per];      // ... and of its second
  v4i fr[2][kFp8Per];     // loaded codes, by tile parity
};

__device__ __forceinline__ int stage_off_b(int r, int cg);

template <int B, bool PAGED>
__device__ __forceinline__ void fetch_fp8(const AttnB& c, GWave8& w, int tile) {
  const int32_t* slot = pos_slot(c, tile);
  int32_t rows[kFp8Per];
#pragma unroll
  for (int i = 0; i < kFp8Per; ++i) rows[i] = slot[w.row[i]];
#pragma unroll
  for (int i = 0; i < kFp8Per; ++i) {
    // padding rows load the sequence's first row (position 0; paged: its first
    // table entry's pool row), weighted zero
    const uint32_t s = rows[i] >= 0 ? (uint32_t)rows[i] : c.pad_row;
    if (PAGED)  // pool row: a 64-bit offset (pools may exceed 4 GB)
      w.fr[B][i] = *(const v4i*)(w.kvb + ((uint64_t)s * kKvDim + (uint32_t)w.src[i]));
    else  // 32-bit offset from the sequence base (the launcher keeps L * 576 < 2^32)
      w.fr[B][i] = *(const v4i*)(w.kvb + (s * (uint32_t)kKvDim + (uint32_t)w.src[i]));
  }
}

__device__ __forceinline__ int widen2(v2f f) {
  return (int)((__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u));
}

template <int S, int B>
__device__ __forceinline__ void store_fp8(const AttnB& c, const GWave8& w) {
#pragma unroll
  for (int i = 0; i < kFp8Per; ++i) {
    const v4i x = w.fr[B][i];
    const v4i lo = v4i{widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[0], false)),
                       widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[0], true)),
                       widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[1], false)),
                       widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[1], true))};
    const v4i hi = v4i{widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[2], false)),
                       widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[2], true)),
                       widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[3], false)),
                       widen2(__builtin_amdgcn_cvt_pk_f32_fp8(x[3], true))};
    *(v4i*)(c.st[S] + w.dst[i]) = lo;
    *(v4i*)(c.st[S] + w.dst2[i]) = hi;
  }
}

// gathers of `tile` into stage S: gather-wave lane (g, l), gather i covers
// LDS bytes [1024 (g + 2 i), +1024) of the stage, 16 bytes per lane
template <int S, bool PAGED>
__device__ __forceinline__ void issue_tile_b(const AttnB& c, const GWave& w, int tile) {
  int32_t rows[kDmaPerB];
#pragma unroll
  for (int i = 0; i < kDmaPerB; ++i) rows[i] = pos_slot(c, tile)[w.dma_row[i]];
#pragma unroll
  for (int i = 0; i < kDmaPerB; ++i) {
    // padding rows load the sequence's first row (position 0; paged: its first
    // table entry's pool row), weighted zero
    const uint32_t s = rows[i] >= 0 ? (uint32_t)rows[i] : c.pad_row;
    if (PAGED)  // pool row: a 64-bit offset (pools may exceed 4 GB)
      dma16(w.kvb + ((uint64_t)s * kRowBytes + (uint32_t)w.dma_off[i]),
            c.st[S] + 1024 * (w.g + kGatherWaves * i));
    else  // 32-bit offset from the sequence base (the launcher keeps L * 1152 < 2^32)
      dma16(w.kvb + (s * (uint32_t)kRowBytes + (uint32_t)w.dma_off[i]),
            c.st[S] + 1024 * (w.g + kGatherWaves * i));
  }
}

// S^T of one tile and its softmax (S waves); P^T, alpha and the rescale flag
// go to parity buffer `par`
template <int S, bool FP8, bool PAGED>
__device__ __forceinline__ void s_phase(const AttnB& c, SWave& w, int tile, int par) {
  const int lane = c.lane, ln = lane & 31, h = lane >> 5;
  const uint8_t* tb = c.st[S];
  const uint8_t* sb[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) sb[m] = tb + ln * kRowBytes + 16 * ((2 * m + h) ^ swz_b(ln));
  // A operand of K-step ks: lane holds row (lane&31), dims 16ks + 8h .. +8
  // (granule 2ks + h). The reads run LCS_ATTN_S_AHEAD K-steps ahead of the
  // MFMAs, so the LDS latency is paid once per tile, not once per K-step.
  // (paged FP8 KV: one K-step less, for the two registers of the block
  // lookups that S wave 0 carries between steps; 256 VGPRs otherwise spill)
  constexpr int kAhead = (FP8 && PAGED) ? LCS_ATTN_S_AHEAD - 1 : LCS_ATTN_S_AHEAD;
  v4i a[kAhead];
#pragma unroll
  for (int ks = 0; ks < kAhead; ++ks) a[ks] = *(const v4i*)(sb[ks & 3] + 128 * (ks >> 2));
  v16f se, so;
#pragma unroll
  for (int i = 0; i < 16; ++i) { se[i] = 0.f; so[i] = 0.f; }
  // scheduling barriers keep each read kAhead K-steps before its MFMA (the
  // scheduler would otherwise sink the reads next to their uses)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 36; ks += 2) {
    se = mfma32_bf16(as_v8bf(a[ks % kAhead]), w.qT[ks], se);
    so = mfma32_bf16(as_v8bf(a[(ks + 1) % kAhead]), w.qT[ks + 1], so);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int nk = ks + e + kAhead;
      if (nk < 36) a[(ks + e) % kAhead] = *(const v4i*)(sb[nk & 3] + 128 * (nk >> 2));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // validity of the tile's rows as a wave-uniform bit mask (bit r: row r has
  // a position); a tile without padding skips the masking
  const uint32_t valid = (uint32_t)__ballot(pos_slot(c, tile)[ln] >= 0);
  // lane holds head 32hg + (lane&31) for rows 8(i/4) + 4h + (i&3); raw dot
  // products here, the scale enters through the exponent's FMA below
  // FP8: dequantisation scales of this lane's 16 rows 8(i/4) + 4h + (i&3)
  // (read after the MFMAs, so that they hold no registers during them)
  float psc[16];
  if (FP8) {
    const float* sc = c.sring + (tile & (kPosSlots - 1)) * kTileRows + 4 * h;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const v4f v = *(const v4f*)(sc + 8 * q4);
      psc[4 * q4] = v[0];
      psc[4 * q4 + 1] = v[1];
      psc[4 * q4 + 2] = v[2];
      psc[4 * q4 + 3] = v[3];
    }
  }
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = FP8 ? (se[i] + so[i]) * psc[i] : se[i] + so[i];
  const bool all_valid = valid == 0xFFFFFFFFu;
  if (!all_valid) {
    // padding rows: no logit, and scale 1 (their P entry is 0, and the scale
    // loaded for them, of row 0, need not be finite)
    const uint32_t mine = valid >> (4 * h);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!((mine >> (8 * (i >> 2) + (i & 3))) & 1u)) {
        t[i] = -INFINITY;
        if (FP8) psc[i] = 1.f;
      }
  }
  float mx = t[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, t[i]);
  {
    // the other lane half holds the same head's other 16 rows
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * w.c_log;  // log2 domain
  }
  // lazy rescaling, as in the split-dims kernel above
  const bool first = w.m_run == -INFINITY;
  const float m_new = (first || mx > w.m_run + kRescaleSlack) ? mx : w.m_run;
  float p[16];
  float psum = 0.f;
  if (all_valid) {
    // m_new is finite: exp2(x * c - m) of every row
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(t[i], w.c_log, -m_new));
      psum += p[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = (t[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(fmaf(t[i], w.c_log, -m_new));
      psum += p[i];
    }
  }
  const bool rescale = __ballot(!first && m_new != w.m_run) != 0;
  if (rescale) {
    const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(w.m_run - m_new);
    w.l_run *= alpha;
    if (h == 0) c.alpha[(par * 2 + c.hg) * 32 + ln] = alpha;
  }
  w.l_run += psum;
  w.m_run = m_new;
  if (lane == 0) c.flag[par * 2 + c.hg] = rescale ? 1 : 0;
  uint8_t* pb = c.p_buf + ((par * 2 + c.hg) * 64 + lane) * 32;
  // FP8: the stage holds the unscaled codes (widened), so each row's scale
  // also weights its P entry: sum_r p_r (code_r * scale_r) = sum_r (p_r scale_r) code_r
  if (FP8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] *= psc[i];
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int o = 8 * ks;
    *(v4i*)(pb + 16 * ks) = v4i{(int)pack_bf16x2(p[o + 0], p[o + 1]), (int)pack_bf16x2(p[o + 2], p[o + 3]),
                                (int)pack_bf16x2(p[o + 4], p[o + 5]), (int)pack_bf16x2(p[o + 6], p[o + 7])};
  }
}

// O^T += V^T . P^T for one tile (PV waves), P^T from parity buffer `par`
template <int S>
__device__ __forceinline__ void pv_phase(const AttnB& c, PWave& w, int par) {
  const int lane = c.lane, h = lane >> 5;
  const uint8_t* tb = c.st[S];
  const uint8_t* pb = c.p_buf + ((par * 2 + c.hg) * 64 + lane) * 32;
  v8bf pT[2];
  pT[0] = as_v8bf(*(const v4i*)(pb));
  pT[1] = as_v8bf(*(const v4i*)(pb + 16));
  if (c.flag[par * 2 + c.hg]) {
    const float alpha = c.alpha[(par * 2 + c.hg) * 32 + (lane & 31)];
#pragma unroll
    for (int d = 0; d < 8; ++d) w.acc[d] *= alpha;
  }
  // as in the split-dims kernel: address lane 4j+q of each 16-lane group points
  // at row 4h + j (then + 8, + 16, + 24), dims base + 4q .. +3
  const int a16 = lane & 15, jr = a16 >> 2, qd = a16 & 3, mh = (lane >> 4) & 1;
  const int r0 = 4 * h + jr;
  // base addresses for rows r0 (+16) and r0 + 8 (+16), per granule-group parity
  const uint8_t* vb[2][2];
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int lo3 = (4 * pr + 2 * mh + (qd >> 1)) ^ swz_b(r0 + 8 * e);
      vb[pr][e] = tb + (r0 + 8 * e) * kRowBytes + 16 * (32 * w.dh + lo3) + 8 * (qd & 1);
    }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    v8bf va[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int off = 16 * ks * kRowBytes + 128 * (mt >> 1);
      union { v4s h4[2]; v8bf b; } u;
      u.h4[0] = lds_read_tr16(vb[mt & 1][0], off);
      u.h4[1] = lds_read_tr16(vb[mt & 1][1], off);
      va[ks] = u.b;
    }
    w.acc[mt] = mfma32_bf16(va[0], pT[0], w.acc[mt]);
    w.acc[mt] = mfma32_bf16(va[1], pT[1], w.acc[mt]);
  }
}

// PV side of pipeline step j: accumulate tile j (stage SJ)
template <int SJ>
__device__ __forceinline__ void pv_step(const AttnB& c, PWave& w, int j) {
  if (j >= 0) pv_phase<SJ>(c, w, j & 1);
  lds_barrier();
}

template <int SJ, bool PAGED>
__device__ __forceinline__ void g_step(const AttnB& c, const GWave& w, int j) {
  const bool more = j + 3 < c.n_tiles;
  if (more) issue_tile_b<(SJ + 3) % kStagesB, PAGED>(c, w, j + 3);
  if (j + 2 < c.n_tiles) {
    if (more) wait_vm<kDmaPerB>();
    else wait_vm<0>();
  }
  lds_barrier();
}

// FP8 gather side of pipeline step j: load tile j+3's codes (positions from
// the ring slot written in step j-1), then widen tile j+2's (loaded in step
// j-1) into stage (SJ+2)%4, which held tile j-2, finished before this step.
// Every step loads and widens, past the split's end too (valid addresses;
// the stage is not read again): loads whose only use sat under a branch
// would be moved into it by the compiler, next to the widening. For the same
// reason the gather waves run their steps in groups of four without a
// branch; a step past the last tile (j >= n_tiles) skips only the barrier,
// which the other roles do not have for it (they are done with every stage
// by then, and the final barrier orders these writes before the epilogue's).
template <int SJ, bool PAGED>
__device__ __forceinline__ void g_step8(const AttnB& c, GWave8& w, int j) {
  fetch_fp8<(SJ + 3) & 1, PAGED>(c, w, j + 3);
  __builtin_amdgcn_sched_barrier(0);  // the loads go out before the widening
  store_fp8<(SJ + 2) % kStagesB, SJ & 1>(c, w);
  if (j < c.n_tiles) lds_barrier();
}

// S side of pipeline step j: S wave 0 puts tile j+4's positions (loaded one
// step earlier) into the ring slot of tile j (read for the last time in step
// j-1) and loads tile j+5's; with FP8 KV it also puts tile j+3's row scales
// (loaded one step earlier) into the scale ring and loads tile j+4's. Then
// score tile j+1 (stage (SJ+1)%4). The gather waves read tile j+4's slot in
// step j+1, after this step's barrier. Paged: tile j+4's pool rows come from
// its positions (loaded two steps earlier) and blocks (loaded one step
// earlier); this step loads tile j+5's blocks and tile j+6's positions.
template <int SJ, bool FP8, bool PAGED>
__device__ __forceinline__ void s_step(const AttnB& c, SWave& w, int j) {
  if (c.wave == 0) {
    if (PAGED) {
      const int32_t r4 = pool_row(c, w.pn, w.bn);
      ring_put(c, j + 4, r4);
      if (FP8) {
        scale_put(c, j + 3, w.sn);
        w.sn = load_scale(c, r4);
      }
      w.bn = load_blk(c, w.pn2);
      w.pn = w.pn2;
      w.pn2 = load_pos(c, j + 6);
    } else {
      ring_put(c, j + 4, w.pn);
      if (FP8) {
        scale_put(c, j + 3, w.sn);
        w.sn = load_scale(c, w.pn);
      }
      w.pn = load_pos(c, j + 5);
    }
  }
  if (j + 1 < c.n_tiles) s_phase<(SJ + 1) % kStagesB, FP8, PAGED>(c, w, j + 1, (j + 1) & 1);
  lds_barrier();
}

// (kv without __restrict__: the FP8 gathers load it into registers, and a
// restrict-qualified load may be moved across the barriers' memory clobbers,
// away from the step that is meant to issue it)
// Paged KV (PAGED): kv and kv_scale are pools of blocks of 2^lbs rows,
// block_table [B][max_blocks] maps sequence blocks to pool blocks.
template <bool FP8, bool PAGED>
__global__ void __launch_bounds__(kThreadsB) sparse_mla_b_kernel(
    const uint16_t* __restrict__ q, const void* kv, const float* __restrict__ kv_scale,
    int64_t kv_stride, const int32_t* __restrict__ idx, int T, int L, int k, int rows_per_split,
    float sm_scale,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_lse, const int32_t* __restrict__ block_table, int max_blocks,
    int lbs, int n_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t s_st0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st2[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_st3[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[2 * 2 * 64 * 32];
  __shared__ float s_alpha[2 * 2 * 32];
  __shared__ int s_flag[2 * 2];
  __shared__ int32_t s_ring[kPosSlots * kTileRows];
  __shared__ __attribute__((aligned(16))) float s_sring[FP8 ? kPosSlots * kTileRows : 4];
  __shared__ float s_ml[2 * 2 * 32];

  const int qi = blockIdx.y;  // flattened (b, t)
  const int sp = blockIdx.x;
  const int splits = gridDim.x;
  const int b = qi / T;
  const int tid = threadIdx.x;

  AttnB c;
  c.st[0] = s_st0;
  c.st[1] = s_st1;
  c.st[2] = s_st2;
  c.st[3] = s_st3;
  c.p_buf = s_p;
  c.alpha = s_alpha;
  c.flag = s_flag;
  c.ring = s_ring;
  c.sring = s_sring;
  c.kscale = FP8 ? (PAGED ? kv_scale : kv_scale + (int64_t)b * kv_stride) : nullptr;
  c.btab = PAGED ? block_table + (int64_t)b * max_blocks : nullptr;
  c.lbs = lbs;
  c.nblk = n_blocks;
  c.pad_row = PAGED ? (uint32_t)min(max(c.btab[0], 0), n_blocks - 1) << lbs : 0u;
  c.lane = tid & 63;
  c.wave = tid >> 6;
  const Role role = role_of(c.wave);
  const int pw = (c.wave & 3) - 2 + 2 * (c.wave >> 2);  // PV index 0..3 for waves 2, 3, 6, 7
  c.hg = role == kRoleS ? c.wave : (pw & 1);

  const int row_begin = sp * rows_per_split;
  const int row_end = min(k, row_begin + rows_per_split);
  c.n_rows = row_end - row_begin;
  c.n_tiles = (c.n_rows + kTileRows - 1) / kTileRows;
  c.idx_q = idx + (int64_t)qi * k + row_begin;

  // The roles run separate code with the same sequence of barriers: one
  // after setup, one after the prologue, one per pipeline step j = -1 ..
  // n_tiles - 1, one before the epilogue.
  if (role == kRoleS) {
    SWave w;
    w.c_log = sm_scale * kLog2e;
    w.m_run = -INFINITY;
    w.l_run = 0.f;
    // The selected positions go out first and are published as soon as they
    // land: the gathers wait on them. The query (36 KB per wave) is needed
    // only from the first tile step on, so its loads stay in flight across
    // the setup barrier, behind the positions (the memory counter completes
    // in issue order, so waiting for a position does not wait for the query).
    int32_t p0 = 0, p1 = 0, p2 = 0, b0 = 0, b1 = 0, b2 = 0;
    if (c.wave == 0) {
      // tiles 0..2 into the ring before the gathers start; tile 3 goes in at step -1
      p0 = load_pos(c, 0);
      p1 = load_pos(c, 1);
      p2 = load_pos(c, 2);
      w.pn = load_pos(c, 3);
      if (PAGED) {
        // blocks of tiles 0..2; tile 3's blocks and tile 4's positions for step -1
        w.pn2 = load_pos(c, 4);
        b0 = load_blk(c, p0);
        b1 = load_blk(c, p1);
        b2 = load_blk(c, p2);
        w.bn = load_blk(c, w.pn);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the query loads issue after these
    const uint16_t* qh = q + ((int64_t)qi * kAttHeads + 32 * c.hg + (c.lane & 31)) * kKvDim +
                         8 * (c.lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) w.qT[ks] = as_v8bf(*(const v4i*)(qh + 16 * ks));
    __builtin_amdgcn_sched_barrier(0);
    if (c.wave == 0) {
      if (PAGED) {
        p0 = pool_row(c, p0, b0);
        p1 = pool_row(c, p1, b1);
        p2 = pool_row(c, p2, b2);
      }
      ring_put(c, 0, p0);
      ring_put(c, 1, p1);
      ring_put(c, 2, p2);
    }
    lds_barrier();  // setup: the ring holds tiles 0..2 (the query may still be loading)
    if (FP8 && c.wave == 0) {
      // scales of tiles 0 and 1 (they need the positions) land while the
      // gather waves fetch tile 0; tile 2's go in at step -1
      const float s0 = load_scale(c, p0), s1 = load_scale(c, p1);
      w.sn = load_scale(c, p2);
      scale_put(c, 0, s0);
      scale_put(c, 1, s1);
    }
    lds_barrier();  // prologue (tile 0 landed)
    // The query has landed by now (tile 0's logits need all of it). Waiting
    // for it here, before the steps, also tells the compiler so: otherwise it
    // keeps the query loads pending through the step loop and waits with
    // vmcnt(0) before the last logit MFMA of every step, which also waits for
    // the position load S wave 0 issued in that step for the next one.
    wait_vm<0>();
    s_step<3, FP8, PAGED>(c, w, -1);  // scores tile 0 from stage 0
    for (int j = 0; j < c.n_tiles; j += kStagesB) {
      s_step<0, FP8, PAGED>(c, w, j);
      if (j + 1 < c.n_tiles) s_step<1, FP8, PAGED>(c, w, j + 1);
      if (j + 2 < c.n_tiles) s_step<2, FP8, PAGED>(c, w, j + 2);
      if (j + 3 < c.n_tiles) s_step<3, FP8, PAGED>(c, w, j + 3);
    }
    // publish each head's exponent offset and sum
    float l_tot = w.l_run;
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (c.lane < 32) {
      s_ml[(0 * 2 + c.hg) * 32 + c.lane] = w.m_run;
      s_ml[(1 * 2 + c.hg) * 32 + c.lane] = l_tot;
    }
    __syncthreads();
    return;
  }
  if (FP8 && role == kRoleGather) {
    GWave8 w;
    w.g = __builtin_amdgcn_readfirstlane(c.wave - 4);
    w.kvb = (const uint8_t*)kv + (PAGED ? 0 : (int64_t)b * kv_stride * kKvDim);
#pragma unroll
    for (int i = 0; i < kFp8Per; ++i) {
      const int gi = 64 * (w.g + kGatherWaves * i) + c.lane;  // FP8 granule of the tile
      const int r = gi / (kKvDim / 16), c8 = gi - r * (kKvDim / 16);
      w.row[i] = r;
      w.src[i] = 16 * c8;
      w.dst[i] = stage_off_b(r, 2 * c8);
      w.dst2[i] = stage_off_b(r, 2 * c8 + 1);
    }
    __syncthreads();
    // prologue: tiles 0 and 1 loaded, tile 0 widened into stage 0
    fetch_fp8<0, PAGED>(c, w, 0);
    fetch_fp8<1, PAGED>(c, w, 1);
    __builtin_amdgcn_sched_barrier(0);
    store_fp8<0, 0>(c, w);
    lds_barrier();
    g_step8<3, PAGED>(c, w, -1);  // loads tile 2, widens tile 1 into stage 1
    for (int j = 0; j < c.n_tiles; j += kStagesB) {
      g_step8<0, PAGED>(c, w, j);
      g_step8<1, PAGED>(c, w, j + 1);
      g_step8<2, PAGED>(c, w, j + 2);
      g_step8<3, PAGED>(c, w, j + 3);
    }
    wait_vm<0>();  // loads past the split's end are still in flight
    __syncthreads();
    return;
  }
  if (!FP8 && role == kRoleGather) {
    GWave w;
    w.g = __builtin_amdgcn_readfirstlane(c.wave - 4);
    w.kvb = (const uint8_t*)kv + (PAGED ? 0 : (int64_t)b * kv_stride * kRowBytes);
#pragma unroll
    for (int i = 0; i < kDmaPerB; ++i) {
      const int o = 1024 * (w.g + kGatherWaves * i) + 16 * c.lane;  // LDS byte in the stage
      const int r = o / kRowBytes;
      const int pos = (o - r * kRowBytes) / 16;
      w.dma_row[i] = r;
      w.dma_off[i] = 16 * (pos ^ swz_b(r));
    }
    __syncthreads();
    // prologue: tiles 0 and 1 in flight, wait for tile 0
    issue_tile_b<0, PAGED>(c, w, 0);
    if (c.n_tiles > 1) {
      issue_tile_b<1, PAGED>(c, w, 1);
      wait_vm<kDmaPerB>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();
    g_step<3, PAGED>(c, w, -1);  // issues tile 2 into stage 2, waits for tile 1
    for (int j = 0; j < c.n_tiles; j += kStagesB) {
      g_step<0, PAGED>(c, w, j);
      if (j + 1 < c.n_tiles) g_step<1, PAGED>(c, w, j + 1);
      if (j + 2 < c.n_tiles) g_step<2, PAGED>(c, w, j + 2);
      if (j + 3 < c.n_tiles) g_step<3, PAGED>(c, w, j + 3);
    }
    __syncthreads();
    return;
  }

  PWave w;
  w.dh = pw >> 1;
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.acc[d][i] = 0.f;
  __syncthreads();
  lds_barrier();  // prologue
  pv_step<3>(c, w, -1);
  for (int j = 0; j < c.n_tiles; j += kStagesB) {
    pv_step<0>(c, w, j);
    if (j + 1 < c.n_tiles) pv_step<1>(c, w, j + 1);
    if (j + 2 < c.n_tiles) pv_step<2>(c, w, j + 2);
    if (j + 3 < c.n_tiles) pv_step<3>(c, w, j + 3);
  }
  __syncthreads();

  const int ln = c.lane & 31, h = c.lane >> 5;
  const float m_run = s_ml[(0 * 2 + c.hg) * 32 + ln];
  const float l_tot = s_ml[(1 * 2 + c.hg) * 32 + ln];
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int head = 32 * c.hg + ln;
  const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;  // log2 domain
  // lane holds dims 256dh + 32mt + 8(i/4) + 4h + (i&3) of its head. The
  // normalised output goes to `out` (one split) or to this split's partial
  // output (bf16, same layout). Stored lane-per-head, a store instruction
  // would write 16 bytes into each of 32 rows; instead each PV wave first
  // transposes its [32 heads][256 dims] block through its own stage buffer
  // (idle now: every gather has landed and been read), rows 528 bytes apart,
  // and then stores two whole 512-byte rows per instruction. A wave's LDS
  // accesses complete in order, so it reads back its own writes unsynchronised.
  constexpr int kEpiRow = 528;
  static_assert(32 * kEpiRow <= kTileBytes, "epilogue staging");
  uint8_t* eb = pw == 0 ? c.st[0] : pw == 1 ? c.st[1] : pw == 2 ? c.st[2] : c.st[3];  // not c.st[pw]: scratch
  // a head with no visible row writes zeros, whatever its padding rows held
  // (0 x NaN is not 0). All heads of a query share its rows, so this is rare
  // and, for finite logits, the same for the whole wave: a scalar branch.
  if (!__all(l_tot > 0.f)) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) w.acc[mt][i] = l_tot > 0.f ? w.acc[mt][i] : 0.f;
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const v16f& a = w.acc[mt];
      const uint32_t lo = pack_bf16x2(a[4 * i4] * inv, a[4 * i4 + 1] * inv);
      const uint32_t hi = pack_bf16x2(a[4 * i4 + 2] * inv, a[4 * i4 + 3] * inv);
      *(v2i*)(eb + ln * kEpiRow + 2 * (32 * mt + 8 * i4 + 4 * h)) = v2i{(int)lo, (int)hi};
    }
  uint16_t* obase = (splits == 1 ? out + ((int64_t)qi * kAttHeads + 32 * c.hg) * kLatent
                                 : part_o + (((int64_t)qi * splits + sp) * kAttHeads + 32 * c.hg) * kLatent) +
                    256 * w.dh;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int hl = 2 * it + h;  // head within the group
    const v4i x = *(const v4i*)(eb + hl * kEpiRow + 16 * ln);
    *(v4i*)(obase + hl * kLatent + 8 * ln) = x;
  }
  if (w.dh == 0 && h == 0) {
    if (splits > 1)
      part_lse[((int64_t)qi * splits + sp) * kAttHeads + head] = lse2;
    else if (lse)
      lse[(int64_t)qi * kAttHeads + head] = lse2 * kLn2;
  }
}

// out[q][h][:] = sum_s w_s * o_s / sum_s w_s with w_s = 2^(lse_s - max lse)
// (log2 domain; partial lse values are multiplied by l_mul on loading: 1 for
// the attention kernels' own log2 partials, log2(e) for natural-log lse).
// Partial s of query q sits at part_o + q * o_q + s * o_s (elements) and
// part_lse + q * l_q + s * l_s: query-major for the splits of one launch,
// shard-major for outputs gathered from several devices. 256 threads per
// workgroup = G split groups x 256/G columns of E output elements (E = 4 or
// 8: one 8- or 16-byte load per split); a workgroup covers 256 E / G
// consecutive elements of a query's [64 heads][512] output, so a query
// spreads over 128 G / E workgroups. Group g folds splits g, g + G, g + 2G,
// ... with a running maximum, the loads of up to eight of its splits in
// flight at a time; with G > 1 the groups' partial states then merge through
// LDS. G = 1 serves up to eight splits in one memory latency per thread,
// G = 4 up to 32.
constexpr int kCombBatch = 8;
template <int E>
struct BfVec;
template <>
struct BfVec<4> { using T = v2i; };
template <>
struct BfVec<8> { using T = v4i; };

template <int G, int E>
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      int splits, int64_t o_q, int64_t o_s,
                                                      int64_t l_q, int64_t l_s, float l_mul,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  using Vec = typename BfVec<E>::T;
  constexpr int kCols = 256 / G;
  constexpr int kWords = E / 2;  // bf16 pairs per thread
  __shared__ float s_acc[G > 1 ? G - 1 : 1][E][kCols];
  __shared__ float s_m[G], s_w[G];
  const int qi = blockIdx.y;
  const int tid = threadIdx.x, grp = tid / kCols, col = tid % kCols;
  const int64_t per_split = (int64_t)kAttHeads * kLatent;
  const int e = blockIdx.x * (E * kCols) + E * col;  // element within a split's output
  const int head = e / kLatent;
  const uint16_t* base = part_o + (int64_t)qi * o_q + e;
  const float* lbase = part_lse + (int64_t)qi * l_q + head;
  float m = -INFINITY, wsum = 0.f;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  for (int s0 = grp; s0 < splits; s0 += G * kCombBatch) {
    const int nb = min(kCombBatch, (splits - s0 + G - 1) / G);  // this group's splits in the batch
    float l[kCombBatch];
    Vec x[kCombBatch];
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      l[j] = -INFINITY;
      if (j < nb) {
        const int64_t sp = s0 + G * j;
        l[j] = lbase[sp * l_s] * l_mul;
        x[j] = *(const Vec*)(base + sp * o_s);  // E bf16
      }
    }
    float m_new = m;
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) m_new = fmaxf(m_new, l[j]);
    if (m_new == -INFINITY) continue;  // no valid row in these splits yet
    const float sc = m == -INFINITY ? 0.f : exp2f(m - m_new);
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= sc;
    wsum *= sc;
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      if (j >= nb) continue;
      const float w = l[j] == -INFINITY ? 0.f : exp2f(l[j] - m_new);
#pragma unroll
      for (int i = 0; i < kWords; ++i) {
        const uint32_t u = (uint32_t)x[j][i];
        acc[2 * i] += __uint_as_float(u << 16) * w;
        acc[2 * i + 1] += __uint_as_float(u & 0xFFFF0000u) * w;
      }
      wsum += w;
    }
    m = m_new;
  }
  float mx = m, wt = wsum;
  float o[E];
#pragma unroll
  for (int i = 0; i < E; ++i) o[i] = acc[i];
  if (G > 1) {
    // the threads of a group that serve one head hold the same m and wsum
    // (they depend on that head's lse values only); a workgroup spans whole heads
    if (grp > 0) {
#pragma unroll
      for (int i = 0; i < E; ++i) s_acc[grp > 0 ? grp - 1 : 0][i][col] = acc[i];
    }
    if (col == 0) {
      s_m[grp] = m;
      s_w[grp] = wsum;
    }
    __syncthreads();
    if (grp != 0) return;
    mx = s_m[0];
#pragma unroll
    for (int g = 1; g < G; ++g) mx = fmaxf(mx, s_m[g]);
    const float f0 = s_m[0] == -INFINITY ? 0.f : exp2f(s_m[0] - mx);
    wt = s_w[0] * f0;
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = acc[i] * f0;
#pragma unroll
    for (int g = 1; g < G; ++g) {
      const float mg = s_m[g];
      const float f = mg == -INFINITY ? 0.f : exp2f(mg - mx);
      wt += s_w[g] * f;
#pragma unroll
      for (int i = 0; i < E; ++i) o[i] += s_acc[g - 1][i][col] * f;
    }
  }
  const float inv = wt > 0.f ? 1.f / wt : 0.f;
  Vec y;
#pragma unroll
  for (int i = 0; i < kWords; ++i) y[i] = (int)pack_bf16x2(o[2 * i] * inv, o[2 * i + 1] * inv);
  *(Vec*)(out + (int64_t)qi * per_split + e) = y;
  if (lse && (e & (kLatent - 1)) == 0)
    lse[(int64_t)qi * kAttHeads + head] = wt > 0.f ? (mx + log2f(wt)) * kLn2 : -INFINITY;
}

}  // namespace

// Static scratch of lcs_sparse_mla_attn_noalloc: the split partials of one
// call (bf16 outputs + fp32 lse of every split), for callers that cannot
// allocate. Every GPU the library runs on holds one copy until the process
// ends; calls on one GPU share it. In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device is current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t attn_workspace_bytes(int64_t queries, int k) {
  // the larger of the two kernels' split plans (the size query has no KV type)
  const SplitPlan pa = plan_splits(queries, k);
  const SplitPlan pb = plan_splits_b(queries, k);
  const int splits = pa.splits > pb.splits ? pa.splits : pb.splits;
  if (splits <= 1) return 0;
  size_t o = (size_t)queries * splits * kAttHeads * kLatent * sizeof(uint16_t);
  size_t l = (size_t)queries * splits * kAttHeads * sizeof(float);
  return o + l;
}

hipError_t launch_sparse_mla(const uint16_t* q, const void* kv, bool kv_fp8,
                             const float* kv_scale, int64_t kv_stride, const int32_t* idx, int B,
                             int T, int L,
                             int k, float sm_scale, uint16_t* out, float* lse,
                             void* workspace, hipStream_t stream) {
  const int64_t queries = (int64_t)B * T;
  // the split-role kernel addresses a sequence's rows with 32-bit offsets
  const bool role_kernel = (int64_t)L * (kv_fp8 ? kKvDim : kRowBytes) < ((int64_t)1 << 32);
  const SplitPlan p = role_kernel ? plan_splits_b(queries, k) : plan_splits(queries, k);
  uint16_t* part_o = nullptr;
  float* part_lse = nullptr;
  if (p.splits > 1) {
    part_o = (uint16_t*)workspace;
    part_lse = (float*)(part_o + (size_t)queries * p.splits * kAttHeads * kLatent);
  }
  dim3 grid((unsigned)p.splits, (unsigned)queries);
  hipError_t e;
  const int32_t* no_tab = nullptr;
  if (role_kernel && kv_fp8)
    e = launch_kernel(sparse_mla_b_kernel<true, false>, grid, dim3(kThreadsB), 0, stream, q, kv,
                      kv_scale, kv_stride, idx, T, L, k, p.rows_per_split, sm_scale, out, lse,
                      part_o, part_lse, no_tab, 0, 0, 0);
  else if (role_kernel)
    e = launch_kernel(sparse_mla_b_kernel<false, false>, grid, dim3(kThreadsB), 0, stream, q, kv,
                      (const float*)nullptr, kv_stride, idx, T, L, k, p.rows_per_split, sm_scale,
                      out, lse, part_o, part_lse, no_tab, 0, 0, 0);
  else if (kv_fp8)
    e = launch_kernel(sparse_mla_kernel<true>, grid, dim3(kThreadsA), 0, stream, q, kv, kv_scale,
                      kv_stride, idx, T, L, k, p.rows_per_split, sm_scale, out, lse, part_o,
                      part_lse);
  else
    e = launch_kernel(sparse_mla_kernel<false>, grid, dim3(kThreadsA), 0, stream, q, kv, kv_scale,
                      kv_stride, idx, T, L, k, p.rows_per_split, sm_scale, out, lse, part_o,
                      part_lse);
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_split_combine(part_o, part_lse, p.splits, queries, out, lse, stream);
}

hipError_t launch_sparse_mla_paged(const uint16_t* q, const void* kv, bool kv_fp8,
                                   const float* kv_scale, const int32_t* block_table,
                                   int max_blocks, int lbs, int n_blocks, const int32_t* idx,
                                   int B, int T, int L, int k, float sm_scale, uint16_t* out,
                                   float* lse, void* workspace, hipStream_t stream) {
  // the split-role kernel with pool rows (64-bit gather offsets: no size limit)
  const int64_t queries = (int64_t)B * T;
  const SplitPlan p = plan_splits_b(queries, k);
  uint16_t* part_o = nullptr;
  float* part_lse = nullptr;
  if (p.splits > 1) {
    part_o = (uint16_t*)workspace;
    part_lse = (float*)(part_o + (size_t)queries * p.splits * kAttHeads * kLatent);
  }
  dim3 grid((unsigned)p.splits, (unsigned)queries);
  hipError_t e;
  if (kv_fp8)
    e = launch_kernel(sparse_mla_b_kernel<true, true>, grid, dim3(kThreadsB), 0, stream, q, kv,
                      kv_scale, (int64_t)0, idx, T, L, k, p.rows_per_split, sm_scale, out, lse,
                      part_o, part_lse, block_table, max_blocks, lbs, n_blocks);
  else
    e = launch_kernel(sparse_mla_b_kernel<false, true>, grid, dim3(kThreadsB), 0, stream, q, kv,
                      (const float*)nullptr, (int64_t)0, idx, T, L, k, p.rows_per_split, sm_scale,
                      out, lse, part_o, part_lse, block_table, max_blocks, lbs, n_blocks);
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_split_combine(part_o, part_lse, p.splits, queries, out, lse, stream);
}

// output elements per combine thread: 16-byte loads where one group folds
// every split (32 queries x 8 splits: 4.9 against 5.5 us per launch; 192 x 8:
// 22.0 against 25.9), 8-byte loads for the four-group kernel, whose few
// queries need the workgroups (2 x 16 splits: 4.5 against 4.4 us)
constexpr int kCombE1 = 8, kCombE4 = 4;

hipError_t launch_split_combine(const uint16_t* part_o, const float* part_lse, int splits,
                                int64_t queries, uint16_t* out, float* lse, hipStream_t stream) {
  const SplitPlan p{splits, 0};
  const int64_t per = (int64_t)kAttHeads * kLatent;
  if (p.splits <= kCombBatch)
    return launch_kernel(combine_kernel<1, kCombE1>, dim3(128 / kCombE1, (unsigned)queries), dim3(256), 0, stream,
                         part_o, part_lse, p.splits, p.splits * per, per,
                         (int64_t)p.splits * kAttHeads, (int64_t)kAttHeads, 1.0f, out, lse);
  return launch_kernel(combine_kernel<4, kCombE4>, dim3(128 * 4 / kCombE4, (unsigned)queries), dim3(256), 0, stream,
                       part_o, part_lse, p.splits, p.splits * per, per,
                       (int64_t)p.splits * kAttHeads, (int64_t)kAttHeads, 1.0f, out, lse);
}

hipError_t launch_lse_combine(const uint16_t* part_out, const float* part_lse, int G,
                              int64_t queries, uint16_t* out, float* lse, hipStream_t stream) {
  // shard-major [G][queries]; natural-log lse
  const int64_t per = (int64_t)kAttHeads * kLatent;
  if (queries == 0) return hipSuccess;
  if (G <= kCombBatch)
    return launch_kernel(combine_kernel<1, kCombE1>, dim3(128 / kCombE1, (unsigned)queries), dim3(256), 0, stream,
                         part_out, part_lse, G, per, queries * per, (int64_t)kAttHeads,
                         queries * kAttHeads, kLog2e, out, lse);
  return launch_kernel(combine_kernel<4, kCombE4>, dim3(128 * 4 / kCombE4, (unsigned)queries), dim3(256), 0, stream,
                       part_out, part_lse, G, per, queries * per, (int64_t)kAttHeads,
                       queries * kAttHeads, kLog2e, out, lse);
}

}  // namespace lcs

