// idx_score.hip -- indexer scores on gfx950.
//
// The pages say a light indexer with 32 heads scans the whole history of each
// query ("一枚 Token，怎样穿过 78 层", panel "MLA 压缩，DSA 精读") and that the
// indexer stays O(L^2) ("IndexShare：省掉3/4的索引计算"). The score is the DSA
// lightning-indexer form I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) with FP8
// queries and keys, each with a per-row dequantisation scale.
//
// Decode (T < 16, up to 6 queries per pass over the keys): every key is read
// once from HBM per pass; each wave runs the 32
// heads of a query as the M dimension of v_mfma_f32_32x32x64_f8f6f4 against
// 32 keys as N, then folds ReLU * (w * q_scale) over its heads and scales by
// the key's scale. 132 bytes of HBM traffic per key, no reuse, so the kernel
// is bound by HBM bandwidth; MFMA keeps the 8192 MACs per key off the vector
// ALU.
#include "common.h"

namespace lcs {
namespace {

#ifndef LCS_IDX_TARGET_WGS
#define LCS_IDX_TARGET_WGS 512
#endif
#ifndef LCS_IDX_PREFILL_MIN_T
#define LCS_IDX_PREFILL_MIN_T 16
#endif
#ifndef LCS_IDX_MAX_ITERS
#define LCS_IDX_MAX_ITERS 16
#endif

constexpr int kWaves = 4;
constexpr int kSuper = 64;  // keys per wave iteration (2 MFMA column blocks of 32)

__device__ __forceinline__ v16f mfma_fp8_32x32x64(const v8i& a, const v8i& b) {
  v16f c;
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = 0.f;
  // format codes 0/0 = FP8 E4M3 for A and B; zero scale operands select the
  // unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_fp8_32x32x64_acc(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// max(x, 0) as one v_med3_f32. fmaxf would add a canonicalising max on the
// MFMA result (NaN quieting), i.e. two VALU ops per element instead of one.
// The dot products are bounded by 128 * 448^2, so the median of (x, 0, 3e38)
// is max(x, 0) (an infinite bound would be folded back into a max).
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.0e38f); }

// sum of a value across the two 32-lane halves (lane l and l^32), VALU only
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// For two per-lane partial sums x, y over the lane halves' heads: lanes
// 0..31 get x(l) + x(l + 32), lanes 32..63 get y(l - 32) + y(l), i.e. the
// full head sums of block x in the low half and of block y in the high half,
// with one v_permlane32_swap (it swaps the high half of x with the low half
// of y) and one add.
__device__ __forceinline__ float sum_pair(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One wave = 64 keys per step, as two 32-key column blocks of
// v_mfma_f32_32x32x64_f8f6f4 (the 32 heads are the M dimension, K = 128 in two
// halves). Operand layout (A and B alike): lane l holds row/column l&31 and
// the 32 bytes [64kh + 32(l>>5), +32) of the 128-byte row for K half kh. The
// result holds, in lane l, key l&31 of the block and heads 8(i/4) + 4(l>>5) +
// (i&3) for i = 0..15, so the head sum is 16 in-lane FMAs and one exchange
// between the lane halves.
//
// Paged keys (PAGED): k8 and k_scale are pools of blocks of 2^lbs >= 64 rows
// and block_table [B][max_blocks] maps a sequence's blocks to pool blocks. A
// 64-key tile starts at a multiple of 64, so it lies in one block; the
// workgroup's slice of the table (at most 65 entries) sits in LDS.
constexpr int kMaxWgKeys = LCS_IDX_MAX_ITERS * kWaves * kSuper;  // keys per workgroup, at most
constexpr int kMaxWgBlocks = kMaxWgKeys / 64 + 1;
// Up to kMaxTq queries share each key tile, so a multi-token verify of up to
// 6 tokens reads the keys once. Past 4 queries the combined head weights
// (w * q_scale, 16 per lane and query) move from registers to LDS, which the
// registers of the queries' MFMA operands would otherwise overrun.
constexpr int kMaxTq = 6;
// HIST (one query per sequence, T = 1): the kernel also counts its visible
// scores by their top 12 key bits (the first radix digit of the top-k
// selection) in an LDS histogram and adds it into hist[b][4096] at the end,
// so the selection needs no pass of its own over the scores to build it.
constexpr int kHistBins = 4096;
template <int TQ, bool PAGED, bool HIST = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TQ == 1 ? 4 : 2))) idx_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, int64_t key_stride, const int32_t* __restrict__ vis_len,
    int T, int t0, int L, int keys_per_wg, float* __restrict__ scores,
    const int32_t* __restrict__ block_table, int max_blocks, int lbs, int n_blocks,
    uint32_t* __restrict__ hist) {
  static_assert(!HIST || (TQ == 1 && !PAGED), "the fused histogram is built for T = 1 only");
  constexpr bool kWqLds = TQ > 4;
  // One query per launch: the workgroup's scores (at most 4096, 16 KB) are
  // kept in LDS and written in one burst at its end. Stores spread through
  // the key stream cost more than their 3 % of the bytes (measured: 109.1 ->
  // 106.5 us per 128K decode launch, 53.7 -> 51.8 us at 1M).
  constexpr bool kSBuf = TQ == 1;
  __shared__ float s_sc[kSBuf ? kMaxWgKeys : 1];
  __shared__ int32_t s_blk[PAGED ? kMaxWgBlocks : 1];
  // [query][lane half][16]: the weights of the 16 heads a lane half holds
  __shared__ __attribute__((aligned(16))) float s_wq[kWqLds ? TQ * 2 * 16 : 1];
  __shared__ uint32_t s_hist[HIST ? kHistBins : 1];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  // uniform, so a scalar register: nothing per lane is held across the key loop
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int ln = lane & 31, hh = lane >> 5;
  if (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) s_hist[i] = 0u;
    __syncthreads();
  }

  v8i aq[TQ][2];
  float wq[kWqLds ? 1 : TQ][16];
  int vis[TQ];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    const int64_t bt = (int64_t)b * T + t0 + t;
    const uint8_t* qrow = q8 + (bt * kIdxHeads + ln) * kIdxDim + 32 * hh;
    aq[t][0] = *(const v8i*)(qrow);
    aq[t][1] = *(const v8i*)(qrow + 64);
    if (!kWqLds) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hd = 8 * (i >> 2) + 4 * hh + (i & 3);
        wq[t][i] = w[bt * kIdxHeads + hd] * q_scale[bt * kIdxHeads + hd];
      }
    }
    vis[t] = clamp_vis(vis_len[bt], L);
  }
  if (kWqLds) {
    if ((int)threadIdx.x < TQ * 32) {
      const int t = threadIdx.x >> 5, h2 = (threadIdx.x >> 4) & 1, i = threadIdx.x & 15;
      const int hd = 8 * (i >> 2) + 4 * h2 + (i & 3);
      const int64_t o = ((int64_t)b * T + t0 + t) * kIdxHeads + hd;
      s_wq[(t * 2 + h2) * 16 + i] = w[o] * q_scale[o];
    }
    __syncthreads();
  }

  const int64_t key_base_b = (int64_t)b * key_stride;  // this sequence's first key row
  const int wg_begin = blockIdx.x * keys_per_wg;
  const int wg_end = min(L, wg_begin + keys_per_wg);
  const int blk0 = wg_begin >> lbs;
  if (PAGED) {
    const int nb = ((wg_end - 1) >> lbs) - blk0 + 1;
    if ((int)threadIdx.x < nb)
      s_blk[threadIdx.x] =
          min(max(block_table[(int64_t)b * max_blocks + blk0 + threadIdx.x], 0), n_blocks - 1);
    __syncthreads();
  }

  int base = wg_begin + wave * kSuper;
  if (!HIST && !kSBuf && base >= wg_end) return;

  // keys [tile_base + 32 blk + ln], K halves 0 and 1, and the scale of key
  // tile_base + lane
  auto load_tile = [&](int tile_base, v8i (&bv)[4], float& ks) {
    if (PAGED) {
      // the tile's pool rows: one block, so the keys past L are pool rows too
      const int64_t prow = ((int64_t)s_blk[(tile_base >> lbs) - blk0] << lbs) +
                           (tile_base & ((1 << lbs) - 1));
      ks = k_scale[prow + lane];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const uint8_t* row = k8 + (prow + 32 * blk + ln) * kIdxDim + 32 * hh;
        bv[2 * blk] = *(const v8i*)(row);
        bv[2 * blk + 1] = *(const v8i*)(row + 64);
      }
      return;
    }
    const int sk = tile_base + lane;
    ks = k_scale[key_base_b + (sk < L ? sk : L - 1)];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      int key = tile_base + 32 * blk + ln;
      key = key < L ? key : L - 1;
      const uint8_t* row = k8 + (key_base_b + key) * kIdxDim + 32 * hh;
      bv[2 * blk] = *(const v8i*)(row);
      bv[2 * blk + 1] = *(const v8i*)(row + 64);
    }
  };

  auto score_tile = [&](const v8i (&bv)[4], float ks, int tile_base) {
    const int my_key = tile_base + lane;
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
      float r[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        v16f d = mfma_fp8_32x32x64(aq[t][0], bv[2 * blk]);
        d = mfma_fp8_32x32x64_acc(aq[t][1], bv[2 * blk + 1], d);
        float p = 0.f;
        if (kWqLds) {
          const v4f* wl = (const v4f*)(s_wq + (t * 2 + hh) * 16);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const v4f wv = wl[m];
#pragma unroll
            for (int e = 0; e < 4; ++e) p = fmaf(wv[e], relu(d[4 * m + e]), p);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) p = fmaf(wq[kWqLds ? 0 : t][i], relu(d[i]), p);
        }
        r[blk] = sum_halves(p);
      }
      const float res = hh ? r[1] : r[0];  // lane l holds key tile_base + l
      if (my_key < wg_end) {
        const int64_t bt = (int64_t)b * T + t0 + t;
        const float v = res * ks;
        if (kSBuf)
          s_sc[my_key - wg_begin] = my_key < vis[t] ? v : -INFINITY;
        else
          scores[bt * L + my_key] = my_key < vis[t] ? v : -INFINITY;
        if (HIST && my_key < vis[t]) atomicAdd(&s_hist[score_key(v) >> 20], 1u);
      }
      // past 4 queries, one query's MFMA results at a time (the scheduler
      // would otherwise hold every query's in registers at once)
      if (kWqLds) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two register buffers in turn, the next tile always in flight while the
  // current one is scored. The prefetch is unconditional so that the wait
  // before scoring only covers the older tile: past the end of the range it
  // re-reads the tile being scored, which the caches hold.
  constexpr int kStride = kWaves * kSuper;
  v8i ta[4], tb[4];
  float ka, kb;
  if (base < wg_end) {
    load_tile(base, ta, ka);
    for (;;) {
      load_tile(base + kStride < wg_end ? base + kStride : base, tb, kb);
      score_tile(ta, ka, base);
      base += kStride;
      if (base >= wg_end) break;
      load_tile(base + kStride < wg_end ? base + kStride : base, ta, ka);
      score_tile(tb, kb, base);
      base += kStride;
      if (base >= wg_end) break;
    }
  }
  if (HIST || kSBuf) {
    __syncthreads();
    // the thread index rebuilt from the wave index (uniform) and the lane
    // count, so that no register holds it across the key loop
    const int tid = (wave << 6) +
                    (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    if (kSBuf) {
      float* row = scores + ((int64_t)b * T + t0) * L + wg_begin;  // TQ = 1: query t0
      for (int i = tid; i < wg_end - wg_begin; i += 256) row[i] = s_sc[i];
    }
  }
  if (HIST) {
    uint32_t* rh = hist + (size_t)b * kHistBins;
    const int tid = (wave << 6) +
                    (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    for (int i = tid; i < kHistBins; i += 256) {
      const uint32_t c = s_hist[i];
      if (c) atomicAdd(&rh[i], c);
    }
  }
}

// Prefill (many queries per sequence): a dense FP8 contraction of the query
// heads [T*32 x 128] with the keys [128 x L], each product passed through the
// ReLU-weighted head sum. Eight waves per workgroup; each wave keeps 128 keys
// (four 32-key MFMA column blocks, both K halves) in registers for the whole
// launch, so the workgroup covers 1024 keys, and the workgroup's queries
// stream through LDS in chunks of 8 (32 KB of codes + the 8 x 32 combined head
// weights w * q_scale), double-buffered: the global loads of chunk c+1 are in
// registers while chunk c is scored, and are written to LDS before the one
// barrier per chunk. Query rows (128 B) sit in LDS with their 16-byte
// granules XOR-swizzled by (row >> 1) & 7: 16 lanes reading 16 consecutive
// rows then cover all 64 banks, so the MFMA operand reads are free of bank
// conflicts. Per (query, 32 keys): two MFMAs (8192 MACs per pair) and, per
// lane, 16 max + 16 FMA for its 16 heads plus one lane-half exchange.
constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
#ifndef LCS_PF_KB
#define LCS_PF_KB 4
#endif
constexpr int kPfKB = LCS_PF_KB;  // 32-key MFMA column blocks per wave
constexpr int kPfKeysPerWave = 32 * kPfKB;
constexpr int kPfKeysPerWg = kPfWaves * kPfKeysPerWave;
constexpr int kPfChunk = 8;                              // queries per LDS chunk
constexpr int kPfQBytes = kPfChunk * kIdxHeads * kIdxDim;  // 32768
constexpr int kPfWBytes = kPfChunk * kIdxHeads * 4;        // 1024
constexpr int kPfBufBytes = kPfQBytes + kPfWBytes;
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 (gfx9): 32-bit data format

template <bool PAGED>
__global__ void __launch_bounds__(kPfThreads) idx_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, int64_t key_stride, const int32_t* __restrict__ vis_len,
    int T, int L, int queries_per_wg, float* __restrict__ scores,
    const int32_t* __restrict__ block_table,
    int max_blocks, int lbs, int n_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[2][kPfBufBytes];

  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31, hh = lane >> 5;
  const int t_begin = blockIdx.y * queries_per_wg;
  const int t_end = min(T, t_begin + queries_per_wg);
  if (t_begin >= t_end) return;

  const int64_t key_base_b = (int64_t)b * key_stride;
  const int kw0 = blockIdx.x * kPfKeysPerWg + wave * kPfKeysPerWave;

  // row of a key (clamped to L - 1): b * L + key, or its pool row (paged)
  auto key_row = [&](int key) -> int64_t {
    key = key < L ? key : L - 1;
    if (!PAGED) return key_base_b + key;
    const int blk = min(max(block_table[(int64_t)b * max_blocks + (key >> lbs)], 0), n_blocks - 1);
    return ((int64_t)blk << lbs) + (key & ((1 << lbs) - 1));
  };
  // this wave's keys: block kb holds keys kw0 + 32 kb + (lane & 31)
  v8i kreg[kPfKB][2];
#pragma unroll
  for (int kb = 0; kb < kPfKB; ++kb) {
    const uint8_t* row = k8 + key_row(kw0 + 32 * kb + ln) * kIdxDim + 32 * hh;
    kreg[kb][0] = *(const v8i*)(row);
    kreg[kb][1] = *(const v8i*)(row + 64);
  }
  // scales of the keys this lane stores: kw0 + 64 c + lane
  float ks[kPfKB / 2];
#pragma unroll
  for (int c = 0; c < kPfKB / 2; ++c) ks[c] = k_scale[key_row(kw0 + 64 * c + lane)];
  // Wait for the keys here: left pending, the compiler would wait with
  // vmcnt(0) at their first use inside the chunk loop, which also waits for
  // the next chunk's loads in flight.
  wait_vm<0>();

  // chunk loads: thread tid carries granules tid + 512 r (r < 4) of the
  // chunk's 2048 16-byte query granules, and (tid < 256) one combined weight
  v4i gq[4];
  float gw = 0.f, gs = 0.f;
  int gv = 0, vis_cur = 0;  // lanes 0..7: visible lengths of the chunk's queries
  auto load_chunk = [&](int c0) {
    {
      int t = c0 + (lane & 7);
      t = t < T ? t : T - 1;
      gv = vis_len[(int64_t)b * T + t];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = tid + kPfThreads * r;
      int t = c0 + (g >> 8);
      t = t < T ? t : T - 1;
      gq[r] = *(const v4i*)(q8 + (((int64_t)b * T + t) * kIdxHeads * kIdxDim) + 16 * (g & 255));
    }
    if (tid < kPfChunk * kIdxHeads) {
      int t = c0 + (tid >> 5);
      t = t < T ? t : T - 1;
      const int i = tid & 15, h2 = (tid >> 4) & 1;
      const int head = 8 * (i >> 2) + 4 * h2 + (i & 3);
      const int64_t o = ((int64_t)b * T + t) * kIdxHeads + head;
      gw = w[o];
      gs = q_scale[o];
    }
  };
  auto store_chunk = [&](uint8_t* buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = tid + kPfThreads * r;
      const int row = g >> 3, c = g & 7;  // row = query * 32 + head
      *(v4i*)(buf + row * kIdxDim + 16 * (c ^ ((row >> 1) & 7))) = gq[r];
    }
    // weights as [query][lane half][16]: the 16 heads a lane half holds
    if (tid < kPfChunk * kIdxHeads) ((float*)(buf + kPfQBytes))[tid] = gw * gs;
    vis_cur = gv;
  };

  // All 8 queries of a chunk are scored, with the same instruction stream
  // whatever the query or key range: a query past the range or a key past L
  // is dropped by the buffer store's range check. So each chunk issues a
  // fixed number of stores and the waits for the next chunk's loads never
  // have to cover them.
  //
  // The 32 (query, key block) units of a chunk run as a software pipeline:
  // unit u issues the two MFMAs of unit u + 2 and then the epilogue of unit
  // u, whose MFMAs have finished by then, so the epilogue never waits on the
  // matrix core. Query qi + 1's operands are read from LDS at qi's first unit.
  // A scheduling barrier after each unit keeps this order.
  auto lds_query = [&](const uint8_t* buf, int qi, v8i (&a)[2], float (&wq)[16]) {
    const uint8_t* qrow = buf + qi * (kIdxHeads * kIdxDim) + ln * kIdxDim;
    const int sw = (ln >> 1) & 7;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int c = 2 * hh + 4 * kh;
      const v4i lo = *(const v4i*)(qrow + 16 * (c ^ sw));
      const v4i hi = *(const v4i*)(qrow + 16 * ((c + 1) ^ sw));
      a[kh] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    const float* wrow = (const float*)(buf + kPfQBytes) + qi * kIdxHeads + 16 * hh;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const v4f v = *(const v4f*)(wrow + 4 * m);
      wq[4 * m] = v[0];
      wq[4 * m + 1] = v[1];
      wq[4 * m + 2] = v[2];
      wq[4 * m + 3] = v[3];
    }
  };

  auto score_chunk = [&](const uint8_t* buf, int c0) {
    v8i A[2][2];
    float W[2][16];
    v16f D[3];
    float P[2];
    lds_query(buf, 0, A[0], W[0]);
    auto mma = [&](int u) {
      const int qi = u / kPfKB, kb = u % kPfKB;
      D[u % 3] = mfma_fp8_32x32x64(A[qi & 1][0], kreg[kb][0]);
      D[u % 3] = mfma_fp8_32x32x64_acc(A[qi & 1][1], kreg[kb][1], D[u % 3]);
    };
    mma(0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kUnits = kPfKB * kPfChunk;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int qi = u / kPfKB, kb = u % kPfKB;
      if (kb == 0 && qi + 1 < kPfChunk) lds_query(buf, qi + 1, A[(qi + 1) & 1], W[(qi + 1) & 1]);
      if (u + 2 < kUnits) mma(u + 2);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = fmaf(W[qi & 1][i], relu(D[u % 3][i]), acc);
      P[kb & 1] = acc;
      if (kb & 1) {
        const int c = kb >> 1;
        const int t = c0 + qi;
        const int64_t bt = (int64_t)b * T + (t < t_end ? t : t_end - 1);
        // the row's byte range and each key's byte offset are unsigned 32-bit
        // values (L < 2^30 keeps 4 L below 2^32)
        const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
            scores + bt * L, 0, t < t_end ? (int)(4u * (uint32_t)L) : 0, kBufferWord3);
        const int vis = clamp_vis(__builtin_amdgcn_readlane(vis_cur, qi), L);
        // lane l: key kw0 + 64 c + l (blocks 2c and 2c+1 by lane half)
        const float res = sum_pair(P[0], P[1]) * ks[c];
        const int key = kw0 + 64 * c + lane;
        const float v = key < vis ? res : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out, (int)(4u * (uint32_t)key), 0,
                                              0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load_chunk(t_begin);
  store_chunk(s_buf[0]);
  lds_barrier();
  for (int c0 = t_begin;;) {
    const int c1 = c0 + kPfChunk;
    if (c1 < t_end) load_chunk(c1);
    score_chunk(s_buf[0], c0);
    if (c1 >= t_end) break;
    store_chunk(s_buf[1]);
    lds_barrier();
    c0 = c1;
    const int c2 = c0 + kPfChunk;
    if (c2 < t_end) load_chunk(c2);
    score_chunk(s_buf[1], c0);
    if (c2 >= t_end) break;
    store_chunk(s_buf[0]);
    lds_barrier();
    c0 = c2;
  }
}

}  // namespace

namespace {

template <bool PAGED>
hipError_t launch_idx_impl(const uint8_t* q8, const float* q_scale, const float* w,
                           const uint8_t* k8, const float* k_scale, int64_t kstride,
                           const int32_t* vis_len, int B,
                           int T, int L, float* scores, const int32_t* btab, int max_blocks,
                           int lbs, int n_blocks, uint32_t* hist, hipStream_t stream) {
  if (T >= LCS_IDX_PREFILL_MIN_T) {
    // workgroups: key blocks of 1024 x query ranges x batch, the query ranges
    // (multiples of the 8-query chunk) sized for about 4 workgroups per CU
    const int gx = (L + kPfKeysPerWg - 1) / kPfKeysPerWg;
    const int chunks = (T + kPfChunk - 1) / kPfChunk;
    int64_t want = (1024 + (int64_t)gx * B - 1) / ((int64_t)gx * B);
    if (want < 1) want = 1;
    if (want > chunks) want = chunks;
    const int per = (int)((chunks + want - 1) / want) * kPfChunk;
    const int gy = (T + per - 1) / per;
    return launch_kernel(idx_prefill_kernel<PAGED>, dim3(gx, gy, B), dim3(kPfThreads), 0, stream,
                         q8, q_scale, w, k8, k_scale, kstride, vis_len, T, L, per, scores, btab,
                         max_blocks, lbs, n_blocks);
  }
  // keys per workgroup: a multiple of 4 waves x 64 keys, sized for enough WGs
  const int64_t total_keys = (int64_t)B * L;
  int64_t iters = total_keys / ((int64_t)LCS_IDX_TARGET_WGS * kWaves * kSuper);
  if (iters < 1) iters = 1;
  if (iters > LCS_IDX_MAX_ITERS) iters = LCS_IDX_MAX_ITERS;
  const int kpw = (int)(iters * kWaves * kSuper);
  dim3 grid((unsigned)((L + kpw - 1) / kpw), (unsigned)B);
  if (hist) {
    if (PAGED || T != 1) return hipErrorInvalidValue;
    return launch_kernel(idx_decode_kernel<1, false, true>, grid, dim3(256), 0, stream, q8,
                         q_scale, w, k8, k_scale, kstride, vis_len, T, 0, L, kpw, scores, btab, max_blocks,
                         lbs, n_blocks, hist);
  }
  for (int t0 = 0; t0 < T; t0 += kMaxTq) {
    const int tq = T - t0 < kMaxTq ? T - t0 : kMaxTq;
    hipError_t e;
#define LCS_DECODE_CASE(N)                                                                      \
  case N:                                                                                       \
    e = launch_kernel(idx_decode_kernel<N, PAGED>, grid, dim3(256), 0, stream, q8, q_scale, w, k8, \
                      k_scale, kstride, vis_len, T, t0, L, kpw, scores, btab, max_blocks, lbs,     \
                      n_blocks,                                                                  \
                      nullptr);                                                                  \
    break;
    switch (tq) {
      LCS_DECODE_CASE(1)
      LCS_DECODE_CASE(2)
      LCS_DECODE_CASE(3)
      LCS_DECODE_CASE(4)
      LCS_DECODE_CASE(5)
      default:
        e = launch_kernel(idx_decode_kernel<kMaxTq, PAGED>, grid, dim3(256), 0, stream, q8, q_scale,
                          w, k8, k_scale, kstride, vis_len, T, t0, L, kpw, scores, btab, max_blocks, lbs,
                          n_blocks, nullptr);
        break;
    }
#undef LCS_DECODE_CASE
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                            const uint8_t* k8, const float* k_scale, int64_t kstride,
                            const int32_t* vis_len, int B, int T, int L, float* scores,
                            hipStream_t stream) {
  return launch_idx_impl<false>(q8, q_scale, w, k8, k_scale, kstride, vis_len, B, T, L, scores,
                                nullptr, 0, 0, 0, nullptr, stream);
}

hipError_t launch_idx_score_hist(const uint8_t* q8, const float* q_scale, const float* w,
                                 const uint8_t* k8, const float* k_scale, const int32_t* vis_len,
                                 int B, int L, float* scores, uint32_t* hist, hipStream_t stream) {
  return launch_idx_impl<false>(q8, q_scale, w, k8, k_scale, (int64_t)L, vis_len, B, 1, L, scores,
                                nullptr, 0, 0, 0, hist, stream);
}

hipError_t launch_idx_score_paged(const uint8_t* q8, const float* q_scale, const float* w,
                                  const uint8_t* k8, const float* k_scale,
                                  const int32_t* block_table, int max_blocks, int lbs,
                                  int n_blocks, const int32_t* vis_len, int B, int T, int L,
                                  float* scores, hipStream_t stream) {
  return launch_idx_impl<true>(q8, q_scale, w, k8, k_scale, 0, vis_len, B, T, L, scores,
                               block_table, max_blocks, lbs, n_blocks, nullptr, stream);
}

}  // namespace lcs
