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

#ifndef LCS_ATTN_TARGET_WGS
#define LCS_ATTN_TARGET_WGS 256  // about one workgroup per CU
#endif

__host__ __device__ inline SplitPlan plan_splits(int64_t queries, int k) {
  SplitPlan p;
  int64_t s = (LCS_ATTN_TARGET_WGS + queries - 1) / queries;
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
      const int32_t s = rows[i] >= 0 ? rows[i] : 0;  // padding rows load row 0 (masked below)
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
    const float* __restrict__ kv_scale, const int32_t* __restrict__ idx, int T, int L, int k,
    int rows_per_split, float sm_scale, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
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
  c.kv_b = (int64_t)b * L;
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

  // selected positions (and FP8 row scales) of this split; -1 for padding
  for (int i = tid; i < c.n_tiles * kTileRows; i += kThreadsA) {
    const int32_t s = i < n_rows ? idx[(int64_t)qi * k + row_begin + i] : -1;
    s_idx[i] = s;
    if (FP8) s_scl[i] = s >= 0 ? kv_scale[(int64_t)b * L + s] : 0.f;
  }
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
  if (c.n_tiles > 0) issue_tile<FP8, 0>(c, 0);
  if (c.n_tiles > 1) issue_tile<FP8, 1>(c, 1);
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
  // lane holds dims 128dq + 32mt + 8(i/4) + 4h + (i&3) of its head
  if (splits == 1) {
    uint16_t* orow = out + ((int64_t)qi * kAttHeads + head) * kLatent + 128 * c.dq + 4 * h;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v16f& a = c.acc[mt];
        const uint32_t lo = pack_bf16x2(a[4 * i4] * inv, a[4 * i4 + 1] * inv);
        const uint32_t hi = pack_bf16x2(a[4 * i4 + 2] * inv, a[4 * i4 + 3] * inv);
        *(v2i*)(orow + 32 * mt + 8 * i4) = v2i{(int)lo, (int)hi};
      }
    if (lse && c.dq == 0 && h == 0) lse[(int64_t)qi * kAttHeads + head] = lse2 * kLn2;
  } else {
    float* prow = part_o + (((int64_t)qi * splits + sp) * kAttHeads + head) * kLatent + 128 * c.dq +
                  4 * h;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const v16f& a = c.acc[mt];
        *(v4f*)(prow + 32 * mt + 8 * i4) =
            v4f{a[4 * i4] * inv, a[4 * i4 + 1] * inv, a[4 * i4 + 2] * inv, a[4 * i4 + 3] * inv};
      }
    if (c.dq == 0 && h == 0) part_lse[((int64_t)qi * splits + sp) * kAttHeads + head] = lse2;
  }
}

// out[q][h][:] = sum_s w_s * o_s / sum_s w_s with w_s = 2^(lse_s - max lse);
// one workgroup per (query, group of 4 heads), consecutive threads on
// consecutive output dims
constexpr int kCombHeads = 4;
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      int splits, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  __shared__ float s_w[kCombHeads][16];
  const int qi = blockIdx.y;
  const int h0 = blockIdx.x * kCombHeads;
  const int tid = threadIdx.x;
  if (tid < kCombHeads) {
    const int head = h0 + tid;
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
    for (int s = 0; s < splits; ++s) s_w[tid][s] = wts[s] * inv;
    if (lse) lse[(int64_t)qi * kAttHeads + head] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const int64_t per_split = (int64_t)kAttHeads * kLatent;
  const float* base = part_o + (int64_t)qi * splits * per_split + (int64_t)h0 * kLatent;
  uint16_t* obase = out + (int64_t)qi * per_split + (int64_t)h0 * kLatent;
  for (int i = tid; i < kCombHeads * kLatent / 4; i += 256) {
    const int e = 4 * i;
    const int hl = e / kLatent;
    v4f a = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) a += *(const v4f*)(base + s * per_split + e) * s_w[hl][s];
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
    e = launch_kernel(sparse_mla_kernel<true>, grid, dim3(kThreadsA), 0, stream, q, kv, kv_scale, idx, T,
                      L, k, p.rows_per_split, sm_scale, out, lse, part_o, part_lse);
  else
    e = launch_kernel(sparse_mla_kernel<false>, grid, dim3(kThreadsA), 0, stream, q, kv, kv_scale, idx,
                      T, L, k, p.rows_per_split, sm_scale, out, lse, part_o, part_lse);
  if (e != hipSuccess || p.splits <= 1) return e;
  return launch_kernel(combine_kernel, dim3(kAttHeads / kCombHeads, (unsigned)queries), dim3(256), 0,
                       stream, part_o,
                       part_lse, p.splits, out, lse);
}

}  // namespace lcs
