// topk.hip -- exact top-k selection per query row on gfx950.
//
// "核心 Attention 只精看 Top-2,048" (ailearn GLM-5.2 special edition, "一枚
// Token，怎样穿过 78 层"): each query keeps the k best-scored positions. The
// pages give no tie rule or output order; here equal scores go to the lower
// position and the kept positions are listed in ascending order, padded with
// -1, which makes the result unique.
//
// Radix select on order-preserving uint32 keys, split over many workgroups
// per row so that a few long rows (decode at 128K-1M positions) still fill the
// chip. Four launches, with no device-scope fences (on this multi-XCD part a
// fence writes back and invalidates the whole L2, so cross-workgroup hand-offs
// go through launch boundaries instead):
//   clear : zero the row histograms (only when a row spans several chunks)
//   hist  : every (row, chunk) workgroup builds an LDS histogram of the top 12
//           key bits and adds it to the row histogram
//   filter: every (row, chunk) workgroup derives from the row histogram the
//           bucket b1 holding the k-th largest key, then writes, in position
//           order, the (position, key) pairs whose bucket is above b1 ("sure")
//           or equal to b1 ("candidate") into its slice of the row's list
//   final : one workgroup per row loads the row's entries into registers (32
//           consecutive entries per thread, up to 16384; longer lists are
//           re-read from global memory per pass), resolves the candidates with
//           two more digits (12 + 8 bits), which fixes the exact threshold key
//           tau and how many keys equal to tau are kept (the lowest positions),
//           then writes each thread's selected entries at its block prefix of
//           selection counts, i.e. in position order.
// The chunked launches read the scores twice; the lists carry the keys, so no
// score is gathered. The row kernel (below) reads them once in the common case.
#include "common.h"

namespace lcs {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesTk = kThreads / 64;
constexpr int kBins1 = 4096;  // key bits 31..20
constexpr int kBins2 = 4096;  // key bits 19..8
constexpr int kBins3 = 256;   // key bits 7..0
constexpr int kMinChunk = 2048;
// Fewest positions a chunk is given where the workgroup target alone would cut
// rows finer: 2 rows of 2^20 in 256 chunks of 4096 rather than 512 of 2048
// (each chunk's workgroup also reads the row's 16 KB histogram) took 23.8
// against 28.2 us per lcs_topk_select; the other decode shapes are unchanged.
constexpr int kMinChunkAim = 4096;
#ifndef LCS_TOPK_MAX_CHUNK
#define LCS_TOPK_MAX_CHUNK 8192
#endif
constexpr int64_t kMaxChunkAim = LCS_TOPK_MAX_CHUNK;
constexpr uint32_t kAll = 0xFFFFFFFFu;  // state.b1 marker: keep every visible position
constexpr uint32_t kSure = 0x80000000u;

struct RowState {
  uint32_t b1;       // bucket of the k-th largest key, or kAll
  uint32_t n_above;  // keys in buckets above b1
  uint32_t pad0, pad1;
};

// Many rows of moderate length take one workgroup per row (topk_row_kernel);
// the others the chunked launches. Two row workgroups share a CU, so up to 512
// rows run at once and the row kernel's time hardly depends on their number
// (about 19 us + 0.24 ns per position of a row), while the chunked launches'
// grows with rows x L (about 26 us + 2.1 ps per score): measured, the row
// kernel wins from about 100 rows of 2^17 positions (192 rows: 57 against
// 78 us) and loses below (32 rows: 54 against 35 us, and the decode composite
// also builds the chunked launches' histogram inside the indexer).
constexpr int kRowMaxL = 1 << 18;
#ifndef LCS_TOPK_ROW_MIN_ROWS
#define LCS_TOPK_ROW_MIN_ROWS 128
#endif
constexpr int kRowMinRows = LCS_TOPK_ROW_MIN_ROWS;
__host__ __device__ inline bool uses_row_kernel(int64_t rows, int L) {
  return L <= kRowMaxL && rows >= kRowMinRows;
}

struct Layout {
  int chunks;
  int chunk;  // elements per chunk, multiple of kMinChunk
  size_t off_hist, off_counts, off_lists, total;
};

__host__ __device__ inline Layout make_layout(int64_t rows, int L) {
  Layout ly;
  // aim for >= ~1024 workgroups per launch, and chunks of at most
  // kMaxChunkAim positions where that gives more, but of at least
  // kMinChunkAim positions
  int64_t want = (1024 + rows - 1) / rows;
  const int64_t by_len = (L + kMaxChunkAim - 1) / kMaxChunkAim;
  if (by_len > want) want = by_len;
  int64_t max_chunks = (L + kMinChunkAim - 1) / kMinChunkAim;
  if (want > max_chunks) want = max_chunks;
  if (want > 1024) want = 1024;
  if (want < 1) want = 1;
  int64_t c = (L + want - 1) / want;
  c = (c + kMinChunk - 1) / kMinChunk * kMinChunk;
  ly.chunk = (int)c;
  ly.chunks = (int)((L + c - 1) / c);
  if (ly.chunks < 1) ly.chunks = 1;
  size_t off = (size_t)rows * sizeof(RowState);
  off = (off + 255) & ~(size_t)255;
  ly.off_hist = off;
  off += (size_t)rows * kBins1 * sizeof(uint32_t);
  ly.off_counts = off;
  off += (size_t)rows * ly.chunks * sizeof(uint32_t);
  off = (off + 255) & ~(size_t)255;
  // list slots: (entry, key) pairs for the chunked launches, positions only
  // (the row kernel's spills) otherwise
  ly.off_lists = off;
  off += (size_t)rows * ly.chunks * (size_t)ly.chunk *
         (uses_row_kernel(rows, L) ? sizeof(uint32_t) : sizeof(uint2));
  ly.total = off;
  return ly;
}

// Exclusive prefix over the lanes of a wave of small counts c in [0, 7].
__device__ __forceinline__ uint32_t wave_prefix_small(uint32_t c, uint32_t& wave_total) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t m0 = __ballot(c & 1u), m1 = __ballot(c & 2u), m2 = __ballot(c & 4u);
  wave_total = (uint32_t)(__popcll(m0) + 2 * __popcll(m1) + 4 * __popcll(m2));
  return (uint32_t)(__popcll(m0 & lt) + 2 * __popcll(m1 & lt) + 4 * __popcll(m2 & lt));
}

// Block-wide exclusive prefix of small per-thread counts. s_wave holds
// 2 x kWavesTk slots; `parity` alternates between calls so one barrier
// suffices per call.
__device__ __forceinline__ uint32_t block_prefix_small(uint32_t c, uint32_t* s_wave, int parity,
                                                       uint32_t& block_total) {
  const int wave = threadIdx.x >> 6;
  uint32_t wt;
  const uint32_t wp = wave_prefix_small(c, wt);
  uint32_t* slot = s_wave + parity * kWavesTk;
  if ((threadIdx.x & 63) == 0) slot[wave] = wt;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWavesTk; ++i) {
    const uint32_t v = slot[i];
    before += (i < wave) ? v : 0u;
    tot += v;
  }
  block_total = tot;
  return before + wp;
}

// Block-wide exclusive prefix of one uint32 per thread: an inclusive scan
// inside each wave (shuffles), then the wave totals through LDS (s_tmp holds
// kWavesTk entries). Returns the exclusive prefix; total in `tot`.
__device__ uint32_t block_prefix(uint32_t v, uint32_t* s_tmp, uint32_t& tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t up = __shfl_up(incl, off, 64);
    if (lane >= off) incl += up;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < kWavesTk; ++i) {
    const uint32_t t = s_tmp[i];
    before += i < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();
  return before + incl - v;
}

// Find bucket b of hist[nb] (LDS) with  above(b) < need <= above(b) + hist[b],
// where above(b) = sum of hist over buckets > b. Result in s_out[0] (bucket),
// s_out[1] (above) and s_out[2] (hist[b]). Requires sum(hist) >= need >= 1. Thread t sums buckets
// [t BPT, (t + 1) BPT); a block prefix of those sums (shuffles in each wave,
// the wave totals through LDS) gives every thread the count above its range.
template <int NB>
__device__ void select_bucket(const uint32_t* hist, uint32_t need, uint32_t* s_scan,
                              uint32_t* s_out) {
  constexpr int BPT = NB / kThreads > 0 ? NB / kThreads : 1;
  constexpr int ACTIVE = NB / BPT;
  const int tid = threadIdx.x;
  uint32_t local = 0;
  if (tid < ACTIVE) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) local += hist[tid * BPT + i];
  }
  uint32_t tot;
  const uint32_t before = block_prefix(local, s_scan, tot);
  const uint32_t above = tot - before - local;
  if (tid < ACTIVE && above < need && need <= above + local) {
    uint32_t run = above;
    for (int i = BPT - 1; i >= 0; --i) {
      const int bin = tid * BPT + i;
      const uint32_t h = hist[bin];
      if (run + h >= need) {
        s_out[0] = (uint32_t)bin;
        s_out[1] = run;
        s_out[2] = h;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kThreads) topk_hist_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ vis_len, int L, int k,
    int chunks, int chunk, uint32_t* __restrict__ ghist) {
  __shared__ uint32_t hist[kBins1];
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int vis = clamp_vis(vis_len[row], L);
  const int begin = blockIdx.x * chunk;
  const int end = min(vis, begin + chunk);
  if (vis <= k || begin >= end) return;
  uint32_t* rh = ghist + (size_t)row * kBins1;
  for (int i = tid; i < kBins1; i += kThreads) hist[i] = 0;
  __syncthreads();
  const float* srow = scores + (size_t)row * L;
  // kHistPer loads of a thread in flight together, then their atomics (a
  // load per iteration would wait one memory latency per element)
  constexpr int kHistPer = kMinChunk * 2 / kThreads;  // 8
  for (int base = begin; base < end; base += kThreads * kHistPer) {
    float v[kHistPer];
#pragma unroll
    for (int j = 0; j < kHistPer; ++j) {
      const int s = base + kThreads * j + tid;
      v[j] = s < end ? srow[s] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kHistPer; ++j)
      if (base + kThreads * j + tid < end) atomicAdd(&hist[score_key(v[j]) >> 20], 1u);
  }
  __syncthreads();
  for (int i = tid; i < kBins1; i += kThreads) {
    const uint32_t c = hist[i];
    if (chunks == 1)
      rh[i] = c;
    else if (c)
      atomicAdd(&rh[i], c);
  }
}

__global__ void __launch_bounds__(kThreads) topk_filter_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ vis_len, int L, int k,
    int chunks, int chunk, RowState* __restrict__ state, const uint32_t* __restrict__ ghist,
    uint32_t* __restrict__ counts, uint2* __restrict__ lists, int32_t* __restrict__ idx) {
  __shared__ uint32_t s_wave[2 * kWavesTk];
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t s_scan[kThreads + kWavesTk];
  __shared__ uint32_t s_out[3];
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int vis = clamp_vis(vis_len[row], L);
  const int begin = blockIdx.x * chunk;
  const int end = min(vis, begin + chunk);
  int32_t* out = idx + (size_t)row * k;
  if (vis <= k) {
    // every visible position is kept: positions in order, then -1 padding
    for (int s = begin + tid; s < end; s += kThreads) out[s] = s;
    if (blockIdx.x == 0) {
      for (int i = vis + tid; i < k; i += kThreads) out[i] = -1;
      if (tid == 0) state[row] = RowState{kAll, 0u, 0u, 0u};
    }
    return;
  }
  // bucket of the k-th largest key from the row histogram
  const uint32_t* rh = ghist + (size_t)row * kBins1;
  for (int i = tid; i < kBins1; i += kThreads) hist[i] = rh[i];
  __syncthreads();
  select_bucket<kBins1>(hist, (uint32_t)k, s_scan, s_out);
  const uint32_t b1 = s_out[0];
  if (blockIdx.x == 0 && tid == 0) state[row] = RowState{b1, s_out[1], 0u, 0u};
  // ordered compaction of sure / candidate positions of this chunk
  const float* srow = scores + (size_t)row * L;
  uint2* my = lists + ((size_t)row * chunks + blockIdx.x) * (size_t)chunk;
  uint32_t written = 0;
  int parity = 0;
  // the next block's four scores per thread are loaded before this block's
  // scan barrier, so that their latency overlaps it
  float nv[4];
  auto load4 = [&](int base) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = base + 4 * tid + j;
      nv[j] = s < end ? srow[s] : 0.f;
    }
  };
  load4(begin);
  for (int base = begin; base < end; base += 4 * kThreads) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = nv[j];
    if (base + 4 * kThreads < end) load4(base + 4 * kThreads);
    uint32_t e[4], key[4];
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = base + 4 * tid + j;
      e[j] = 0;
      key[j] = score_key(v[j]);
      if (s < end) {
        const uint32_t d = key[j] >> 20;
        if (d >= b1) {
          e[j] = (uint32_t)s | (d > b1 ? kSure : 0u) | 0x40000000u;  // bit 30: valid
          ++c;
        }
      }
    }
    uint32_t tot;
    uint32_t pos = written + block_prefix_small(c, s_wave, parity, tot);
    parity ^= 1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e[j]) my[pos++] = uint2{e[j] & ~0x40000000u, key[j]};
    written += tot;
  }
  if (tid == 0) counts[(size_t)row * chunks + blockIdx.x] = written;
}



// Entries a row keeps in registers on the fast path of the final kernel:
// up to kStagePer per thread.
constexpr int kStagePer = 32;
constexpr int kStage = kThreads * kStagePer;  // 16384

// The list entries of a row are the chunks' lists concatenated in chunk
// (= position) order; entry e of the row is slot e - pref[c] of chunk c, the
// last chunk with pref[c] <= e.
__device__ __forceinline__ int chunk_of(const uint32_t* pref, int chunks, uint32_t e) {
  int lo = 0, hi = chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kThreads) topk_final_kernel(
    int k, int chunks, int chunk, const RowState* __restrict__ state,
    const uint32_t* __restrict__ counts, const uint2* __restrict__ lists,
    int32_t* __restrict__ idx, uint32_t* __restrict__ ghist) {
  __shared__ uint32_t hist[kBins2];
  __shared__ uint32_t s_scan[kThreads + kWavesTk];
  __shared__ uint32_t s_out[3];
  __shared__ uint32_t s_pref[1024 + 1];
  __shared__ uint32_t s_src[kStage];  // list slot of each entry (fast path)
  __shared__ uint32_t s_wtot[2][kWavesTk];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  // The filter launch has read the row histogram: leave it zero for the next
  // selection, whose histogram may be accumulated by the indexer launch.
  {
    uint4* h = (uint4*)(ghist + (size_t)row * kBins1);
    for (int i = tid; i < kBins1 / 4; i += kThreads) h[i] = uint4{0u, 0u, 0u, 0u};
  }
  for (int i = tid; i < kBins2; i += kThreads) hist[i] = 0;
  const RowState st = state[row];
  if (st.b1 == kAll) return;
  const uint32_t b1 = st.b1;
  int32_t* out = idx + (size_t)row * k;
  const uint2* list = lists + (size_t)row * chunks * (size_t)chunk;
  // chunk offsets in the concatenated entry list (chunks <= 2 * kThreads)
  {
    const int c0 = 2 * tid;
    const uint32_t v0 = c0 < chunks ? counts[(size_t)row * chunks + c0] : 0u;
    const uint32_t v1 = c0 + 1 < chunks ? counts[(size_t)row * chunks + c0 + 1] : 0u;
    uint32_t tot;
    const uint32_t ex = block_prefix(v0 + v1, s_scan, tot);
    if (c0 < chunks) s_pref[c0] = ex;
    if (c0 + 1 < chunks) s_pref[c0 + 1] = ex + v0;
    if (tid == 0) s_pref[chunks] = tot;
    __syncthreads();
  }
  const uint32_t n_ent = s_pref[chunks];
  const uint32_t need1 = (uint32_t)k - st.n_above;

  if (n_ent <= (uint32_t)kStage) {
    // Fast path: wave w holds entries [w 64 R, (w + 1) 64 R), lane l those
    // with e = w 64 R + 64 j + l (j < R <= kStagePer), with their keys, in
    // registers. Consecutive entries of a chunk are consecutive in memory, so
    // the loads are coalesced; their sources come from an LDS table.
    for (int c = tid; c < chunks; c += kThreads) {
      const uint32_t p0 = s_pref[c], n = s_pref[c + 1] - p0;
      for (uint32_t i = 0; i < n; ++i) s_src[p0 + i] = (uint32_t)c * chunk + i;
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    const uint32_t R = (n_ent + kThreads - 1) / kThreads;
    const uint32_t wbase = (uint32_t)wave * 64u * R;
    // (the loaded values are not touched here, so that no wait separates
    // the loads; bit j of vmask says whether slot j holds an entry)
    uint32_t ent[kStagePer], key[kStagePer], vmask = 0;
#pragma unroll
    for (int j = 0; j < kStagePer; ++j) {
      const uint32_t e = wbase + 64u * j + lane;
      ent[j] = 0u;
      key[j] = 0u;
      if ((uint32_t)j < R && e < n_ent) {
        const uint2 v = list[s_src[e]];
        ent[j] = v.x;
        key[j] = v.y;
        vmask |= 1u << j;
      }
    }
    auto cand = [&](int j) { return ((vmask >> j) & 1u) && !(ent[j] & kSure); };
    // digit 2 (key bits 19..8) over the candidates
#pragma unroll
    for (int j = 0; j < kStagePer; ++j)
      if (cand(j)) atomicAdd(&hist[(key[j] >> 8) & 0xFFFu], 1u);
    __syncthreads();
    select_bucket<kBins2>(hist, need1, s_scan, s_out);
    const uint32_t b2 = s_out[0];
    const uint32_t above2 = s_out[1];
    const uint32_t need2 = need1 - above2;
    const uint32_t pre12 = (b1 << 12) | b2;
    // tau: the smallest kept key; keys equal to tau past the first need_tie
    // are dropped, which needs tie ranks only when some are dropped
    uint32_t tau, need_tie;
    bool rank_ties;
    if (s_out[2] == need2) {
      // every candidate of bucket b2 is kept: no third digit
      tau = pre12 << 8;
      need_tie = 0;
      rank_ties = false;
    } else {
      for (int i = tid; i < kBins3; i += kThreads) hist[i] = 0;
      __syncthreads();
      // digit 3 (key bits 7..0) over the candidates inside bucket b2
#pragma unroll
      for (int j = 0; j < kStagePer; ++j)
        if (cand(j) && (key[j] >> 8) == pre12)
          atomicAdd(&hist[key[j] & 0xFFu], 1u);
      __syncthreads();
      select_bucket<kBins3>(hist, need2, s_scan, s_out);
      tau = (pre12 << 8) | s_out[0];
      need_tie = need2 - s_out[1];
      rank_ties = need_tie < s_out[2];
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // entries of this wave before this one (in entry order) that are ties
    uint32_t tie_run = 0;
    if (rank_ties) {
      uint32_t wt = 0;
#pragma unroll
      for (int j = 0; j < kStagePer; ++j)
        if ((uint32_t)j < R)
          wt += (uint32_t)__popcll(__ballot(cand(j) && key[j] == tau));
      if (lane == 0) s_wtot[0][wave] = wt;
      __syncthreads();
      for (int i = 0; i < wave; ++i) tie_run += s_wtot[0][i];
    }
    // keep flags, in entry order
    uint32_t sel = 0, wsel = 0;
#pragma unroll
    for (int j = 0; j < kStagePer; ++j) {
      if ((uint32_t)j >= R) continue;
      const bool valid = (vmask >> j) & 1u;
      const bool sure = valid && (ent[j] & kSure);
      const bool tie = valid && !sure && key[j] == tau;
      bool keep = valid && (sure || key[j] > tau);
      if (rank_ties) {
        const uint64_t tm = __ballot(tie);
        if (tie) keep = tie_run + (uint32_t)__popcll(tm & lt) < need_tie;
        tie_run += (uint32_t)__popcll(tm);
      } else if (tie) {
        keep = true;
      }
      sel |= (keep ? 1u : 0u) << j;
      wsel += (uint32_t)__popcll(__ballot(keep));
    }
    // this wave's output offset: the selections of the waves before it
    if (lane == 0) s_wtot[1][wave] = wsel;
    __syncthreads();
    uint32_t pos = 0;
    for (int i = 0; i < wave; ++i) pos += s_wtot[1][i];
#pragma unroll
    for (int j = 0; j < kStagePer; ++j) {
      if ((uint32_t)j >= R) continue;
      const bool keep = (sel >> j) & 1u;
      const uint64_t km = __ballot(keep);
      const uint32_t p = pos + (uint32_t)__popcll(km & lt);
      if (keep && p < (uint32_t)k) out[p] = (int32_t)(ent[j] & ~kSure);
      pos += (uint32_t)__popcll(km);
    }
    return;
  }

  // Slow path (more entries than the registers hold): every pass reads the
  // entries from the lists again.
  auto entry = [&](uint32_t e) -> uint2 {
    const int c = chunk_of(s_pref, chunks, e);
    return list[(size_t)c * chunk + (e - s_pref[c])];
  };
  for (uint32_t e = tid; e < n_ent; e += kThreads) {
    const uint2 v = entry(e);
    if (!(v.x & kSure)) atomicAdd(&hist[(v.y >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  select_bucket<kBins2>(hist, need1, s_scan, s_out);
  const uint32_t b2 = s_out[0];
  const uint32_t above2 = s_out[1];
  for (int i = tid; i < kBins3; i += kThreads) hist[i] = 0;
  __syncthreads();
  const uint32_t pre12 = (b1 << 12) | b2;
  for (uint32_t e = tid; e < n_ent; e += kThreads) {
    const uint2 v = entry(e);
    if (!(v.x & kSure) && (v.y >> 8) == pre12) atomicAdd(&hist[v.y & 0xFFu], 1u);
  }
  __syncthreads();
  const uint32_t need2 = need1 - above2;
  select_bucket<kBins3>(hist, need2, s_scan, s_out);
  const uint32_t b3 = s_out[0];
  const uint32_t tau = (pre12 << 8) | b3;
  const uint32_t need_tie = need2 - s_out[1];
  // ordered emission, one entry per thread per round
  uint32_t ties_before = 0, sel_before = 0;
  for (uint32_t base = 0; base < n_ent; base += kThreads) {
    const uint32_t e = base + tid;
    uint2 v = uint2{0u, 0u};
    if (e < n_ent) v = entry(e);
    const bool valid = e < n_ent;
    const bool tie = valid && !(v.x & kSure) && v.y == tau;
    uint32_t tie_tot;
    const uint32_t tie_rank = ties_before + block_prefix(tie ? 1u : 0u, s_scan, tie_tot);
    const bool keep = valid && ((v.x & kSure) || (!tie && v.y > tau) || (tie && tie_rank < need_tie));
    uint32_t sel_tot;
    const uint32_t pos = sel_before + block_prefix(keep ? 1u : 0u, s_scan, sel_tot);
    if (keep && pos < (uint32_t)k) out[pos] = (int32_t)(v.x & ~kSure);
    ties_before += tie_tot;
    sel_before += sel_tot;
  }
}

// ---------------------------------------------------------------------------
// One workgroup per row, for rows of at most kRowMaxL positions: the four
// launches above in one, with the candidate lists in LDS, and the row's
// scores read once in the common case. Every wave walks its own contiguous
// eighth of the row in position order (coalesced loads, two steps in flight).
// The waves' first steps (8 x 1024 positions) form a sample: their histogram
// of the top 12 key bits gives a bucket b_est below which the k-th largest key
// almost surely does not lie (the sample's rank 1.5x the expected share of the
// k best, plus 32; the exact bucket when the sample is the whole row).
// The pass compacts every position whose bucket is at least b_est into the
// wave's LDS list (kRowCap entries: position and key; entries past kRowCap go
// to the wave's slice of `spill`, positions only, their keys re-read from the
// scores), with no histogram atomics. If the lists hold at least k keys, the
// k-th largest lies in a bucket >= b_est, where the lists' histogram is the
// row's, so the threshold bucket b1 and the count above it come from the
// listed keys alone (keys below b1 are passed over later). Otherwise the
// sample over-estimated, and the row is read twice more: a histogram pass for
// b1, then a compaction with b1. Two more digits
// (12 + 8 bits) over the bucket-b1 entries fix the threshold key tau and how
// many keys equal to tau are kept, and the lists are emitted in wave order
// (= position order): the keys above tau and the first ties. A single
// workgroup keeps at most ~64 KB of loads in flight, so the row kernel pays
// only where many rows fill the chip (chunked prefill); a few long rows
// (decode) use the chunked launches, which spread each row over many CUs.
// LDS list entries per wave (8 waves: 10240): positions as 16-bit offsets in
// the wave's segment (at most kRowMaxL / 8 = 32768 positions) and 32-bit keys,
// so that the workgroup's LDS stays under half of the CU's and two workgroups
// share a CU (one's list phases overlap the other's pass over its row)
constexpr int kRowCap = 1280;
constexpr int kRowBufWord3 = 0x00020000;  // buffer resource word 3 (gfx9): 32-bit data format
#ifndef LCS_ROW_PER2
#define LCS_ROW_PER2 16  // scores per lane per step
#endif

// (four waves per SIMD: two workgroups of eight waves per CU)
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) topk_row_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ vis_len, int L, int k,
    int spill_stride, uint32_t* __restrict__ spill, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint16_t s_off[kWavesTk][kRowCap];
  __shared__ uint32_t s_key[kWavesTk][kRowCap];
  __shared__ uint32_t s_scan[kThreads + kWavesTk];
  __shared__ uint32_t s_out[3];
  __shared__ uint32_t s_cnt[kWavesTk], s_tie[kWavesTk], s_sel[kWavesTk];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vis = clamp_vis(vis_len[row], L);
  int32_t* out = idx + (size_t)row * k;
  if (vis <= k) {
    // every visible position is kept: positions in order, then -1 padding
    for (int i = tid; i < k; i += kThreads) out[i] = i < vis ? i : -1;
    return;
  }
  const float* srow = scores + (size_t)row * L;
  for (int i = tid; i < kBins1; i += kThreads) hist[i] = 0;
  __syncthreads();

  // wave w walks positions [w seg, (w+1) seg) in steps of kStep positions
  const int seg = (vis + kWavesTk - 1) / kWavesTk;
  const int seg_cap = spill_stride / kWavesTk;  // >= seg: spill_stride >= L, a multiple of 8
  const int p0 = wave * seg, p1 = min(vis, p0 + seg);
  uint32_t* my_spill = spill + (size_t)row * spill_stride + (size_t)wave * seg_cap;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t cnt = 0;
  // kPer loads of a lane per step, in two register buffers used in turn: the
  // next step's loads are issued before this step's atomics and ballots. The
  // loads are unconditional buffer loads over the row's vis scores (one
  // offset register; positions past the row read 0 and positions past the
  // segment are neither counted nor kept), so the wait before a step covers
  // that step's loads only.
  constexpr int kPer = LCS_ROW_PER2;
  constexpr int kStep = 64 * kPer;
  const __amdgpu_buffer_rsrc_t rrow = __builtin_amdgcn_make_buffer_rsrc(
      (void*)srow, 0, (int)(4u * (uint32_t)vis), kRowBufWord3);
  float va[kPer], vb[kPer];
  auto load = [&](float (&v)[kPer], int base) {
    const int off = 4 * (base + lane);  // < 4 (vis + 2 kStep) < 2^31
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rrow, off + 256 * j, 0, 0));
  };
  // histogram (count) and/or ordered compaction of the keys in buckets >= bmin
  auto step = [&](const float (&v)[kPer], int base, bool count, bool keep, uint32_t bmin) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = base + 64 * j + lane;
      const uint32_t key = score_key(v[j]);
      const bool valid = p < p1;
      if (count && valid) atomicAdd(&hist[key >> 20], 1u);
      if (keep) {
        const bool q = valid && (key >> 20) >= bmin;
        const uint64_t m = __ballot(q);
        if (q) {
          const uint32_t slot = cnt + (uint32_t)__popcll(m & lt);
          if (slot < (uint32_t)kRowCap) {
            s_off[wave][slot] = (uint16_t)(p - p0);
            s_key[wave][slot] = key;
          } else {
            my_spill[slot] = (uint32_t)p;
          }
        }
        cnt += (uint32_t)__popcll(m);
      }
    }
  };

  // ---- the sample: every wave's first step ----
  load(va, p0);
  load(vb, p0 + kStep);
  step(va, p0, true, false, 0u);
  __syncthreads();
  uint32_t sample = 0;
#pragma unroll
  for (int w = 0; w < kWavesTk; ++w) sample += (uint32_t)max(0, min(kStep, min(vis, w * seg + seg) - w * seg));
  uint32_t need_est = (uint32_t)k;
  if (sample < (uint32_t)vis) {
    const uint64_t share = ((uint64_t)k * sample + (uint64_t)vis - 1) / (uint64_t)vis;
    need_est = (uint32_t)min<uint64_t>((uint64_t)sample, (3 * share + 1) / 2 + 32);
  }
  select_bucket<kBins1>(hist, need_est, s_scan, s_out);
  const uint32_t b_est = s_out[0];

  // ---- the rest of the pass: compaction above b_est (no histogram) ----
  step(va, p0, false, true, b_est);
  for (int base = p0 + kStep; base < p1;) {
    load(va, base + kStep);
    step(vb, base, false, true, b_est);
    base += kStep;
    if (base >= p1) break;
    load(vb, base + kStep);
    step(va, base, false, true, b_est);
    base += kStep;
  }
  if (lane == 0) s_cnt[wave] = cnt;
  __syncthreads();
  uint32_t listed = 0;
#pragma unroll
  for (int w = 0; w < kWavesTk; ++w) listed += s_cnt[w];
  for (int i = tid; i < kBins1; i += kThreads) hist[i] = 0;
  __syncthreads();
  if (listed >= (uint32_t)k) {
    // at least k keys lie in buckets >= b_est, so the k-th largest does too,
    // and the lists' histogram of those buckets is the row's: b1 and the count
    // above it follow from the listed keys alone
    for (uint32_t e = lane; e < cnt; e += 64) {
      uint32_t key;
      if (e < (uint32_t)kRowCap) {
        key = s_key[wave][e];
      } else {
        key = score_key(srow[my_spill[e]]);
      }
      atomicAdd(&hist[key >> 20], 1u);
    }
  } else {
    // the sample over-estimated the threshold: histogram of the whole row,
    // then (below) a compaction with the exact bucket
    load(va, p0);
    for (int base = p0;;) {
      load(vb, base + kStep);
      step(va, base, true, false, 0u);
      base += kStep;
      if (base >= p1) break;
      load(va, base + kStep);
      step(vb, base, true, false, 0u);
      base += kStep;
      if (base >= p1) break;
    }
  }
  __syncthreads();
  select_bucket<kBins1>(hist, (uint32_t)k, s_scan, s_out);
  const uint32_t b1 = s_out[0];
  const uint32_t n_above = s_out[1];
  if (listed < (uint32_t)k) {
    cnt = 0;
    load(va, p0);
    for (int base = p0;;) {
      load(vb, base + kStep);
      step(va, base, false, true, b1);
      base += kStep;
      if (base >= p1) break;
      load(va, base + kStep);
      step(vb, base, false, true, b1);
      base += kStep;
      if (base >= p1) break;
    }
    if (lane == 0) s_cnt[wave] = cnt;
    __syncthreads();
  }

  // entry e of wave w's list: its position, and its key (re-read for spills)
  auto get = [&](int w, uint32_t e, uint32_t& key) -> uint32_t {
    if (e < (uint32_t)kRowCap) {
      key = s_key[w][e];
      return (uint32_t)(w * seg) + s_off[w][e];
    }
    const uint32_t p = spill[(size_t)row * spill_stride + (size_t)w * seg_cap + e];
    key = score_key(srow[p]);
    return p;
  };
  const uint32_t my_n = cnt;

  // ---- digit 2 (bits 19..8), then digit 3 (bits 7..0), over bucket b1 ----
  const uint32_t need1 = (uint32_t)k - n_above;
  for (int i = tid; i < kBins2; i += kThreads) hist[i] = 0;
  __syncthreads();
  for (uint32_t e = lane; e < my_n; e += 64) {
    uint32_t key;
    get(wave, e, key);
    if ((key >> 20) == b1) atomicAdd(&hist[(key >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  select_bucket<kBins2>(hist, need1, s_scan, s_out);
  const uint32_t b2 = s_out[0];
  const uint32_t above2 = s_out[1];
  const uint32_t need2 = need1 - above2;
  const uint32_t pre12 = (b1 << 12) | b2;
  uint32_t tau, need_tie;  // the smallest kept key; how many keys equal to it are kept
  if (s_out[2] == need2) {
    // every key of bucket b2 is kept: no third digit
    tau = pre12 << 8;
    need_tie = 0xFFFFFFFFu;
  } else {
    __syncthreads();
    for (int i = tid; i < kBins3; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (uint32_t e = lane; e < my_n; e += 64) {
      uint32_t key;
      get(wave, e, key);
      if ((key >> 8) == pre12) atomicAdd(&hist[key & 0xFFu], 1u);
    }
    __syncthreads();
    select_bucket<kBins3>(hist, need2, s_scan, s_out);
    tau = (pre12 << 8) | s_out[0];
    need_tie = need2 - s_out[1];
  }

  // ---- emission in position order (wave order, then list order) ----
  // kept: every key above tau, and the first need_tie keys equal to tau
  // (entries below bucket b1 are above no kept key and are passed over)
  uint32_t my_ties = 0;
  for (uint32_t e0 = 0; e0 < my_n; e0 += 64) {
    const uint32_t e = e0 + lane;
    uint32_t key = 0;
    if (e < my_n) get(wave, e, key);
    my_ties += (uint32_t)__popcll(__ballot(e < my_n && key == tau));
  }
  if (lane == 0) s_tie[wave] = my_ties;
  __syncthreads();
  uint32_t ties_before = 0;
  for (int w = 0; w < wave; ++w) ties_before += s_tie[w];
  auto walk = [&](bool write, uint32_t out_base) -> uint32_t {
    uint32_t tie_rank = ties_before, kept = 0;
    for (uint32_t e0 = 0; e0 < my_n; e0 += 64) {
      const uint32_t e = e0 + lane;
      uint32_t key = 0, p = 0;
      const bool in = e < my_n;
      if (in) p = get(wave, e, key);
      const bool tie = in && key == tau;
      const uint64_t tm = __ballot(tie);
      const uint32_t my_rank = tie_rank + (uint32_t)__popcll(tm & lt);
      const bool sel = (in && key > tau) || (tie && my_rank < need_tie);
      const uint64_t sm = __ballot(sel);
      if (write && sel) {
        const uint32_t at = out_base + kept + (uint32_t)__popcll(sm & lt);
        if (at < (uint32_t)k) out[at] = (int32_t)p;
      }
      tie_rank += (uint32_t)__popcll(tm);
      kept += (uint32_t)__popcll(sm);
    }
    return kept;
  };
  const uint32_t my_kept = walk(false, 0);
  if (lane == 0) s_sel[wave] = my_kept;
  __syncthreads();
  uint32_t kept_before = 0, kept_total = 0;
  for (int w = 0; w < kWavesTk; ++w) {
    kept_before += w < wave ? s_sel[w] : 0u;
    kept_total += s_sel[w];
  }
  walk(true, kept_before);
  for (int i = (int)kept_total + tid; i < k; i += kThreads) out[i] = -1;
}

// zero the row histograms (rows that span several chunks accumulate into them)
__global__ void __launch_bounds__(256) topk_clear_kernel(uint32_t* __restrict__ ghist) {
  uint4* h = (uint4*)(ghist + (size_t)blockIdx.x * kBins1);
  for (int i = threadIdx.x; i < kBins1 / 4; i += blockDim.x) h[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int L, int /*k*/) {
  return make_layout(rows, L).total;
}

namespace {


// the chunked launches after the row histograms are complete
hipError_t launch_filter_final(const float* scores, const int32_t* vis_len, int rows, int L, int k,
                               int32_t* idx, char* ws, const Layout& ly, hipStream_t stream) {
  RowState* state = (RowState*)ws;
  uint32_t* ghist = (uint32_t*)(ws + ly.off_hist);
  uint32_t* counts = (uint32_t*)(ws + ly.off_counts);
  uint2* lists = (uint2*)(ws + ly.off_lists);
  dim3 grid((unsigned)ly.chunks, (unsigned)rows);
  hipError_t e = launch_kernel(topk_filter_kernel, grid, dim3(kThreads), 0, stream, scores,
                               vis_len, L, k, ly.chunks, ly.chunk, state, ghist, counts, lists,
                               idx);
  if (e != hipSuccess) return e;
  return launch_kernel(topk_final_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, k,
                       ly.chunks, ly.chunk, state, counts, lists, idx, ghist);
}

}  // namespace

hipError_t launch_topk(const float* scores, const int32_t* vis_len, int rows, int L, int k,
                       int32_t* idx, void* workspace, hipStream_t stream) {
  const Layout ly = make_layout(rows, L);
  char* ws = (char*)workspace;
  uint32_t* ghist = (uint32_t*)(ws + ly.off_hist);
  uint32_t* lists = (uint32_t*)(ws + ly.off_lists);
  if (uses_row_kernel(rows, L))  // one workgroup per row; spills in the list area
    return launch_kernel(topk_row_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, scores,
                         vis_len, L, k, ly.chunks * ly.chunk, lists, idx);
  dim3 grid((unsigned)ly.chunks, (unsigned)rows);
  hipError_t e = hipSuccess;
  if (ly.chunks > 1) {
    e = launch_kernel(topk_clear_kernel, dim3((unsigned)rows), dim3(256), 0, stream, ghist);
    if (e != hipSuccess) return e;
  }
  e = launch_kernel(topk_hist_kernel, grid, dim3(kThreads), 0, stream, scores, vis_len, L, k,
                    ly.chunks, ly.chunk, ghist);
  if (e != hipSuccess) return e;
  return launch_filter_final(scores, vis_len, rows, L, k, idx, ws, ly, stream);
}

bool topk_takes_prebuilt_hist(int64_t rows, int L) { return !uses_row_kernel(rows, L); }

uint32_t* topk_hist_area(void* workspace, int64_t rows, int L) {
  return (uint32_t*)((char*)workspace + make_layout(rows, L).off_hist);
}

hipError_t launch_topk_clear(void* workspace, int rows, int L, hipStream_t stream) {
  return launch_kernel(topk_clear_kernel, dim3((unsigned)rows), dim3(256), 0, stream,
                       topk_hist_area(workspace, rows, L));
}

hipError_t launch_topk_prebuilt(const float* scores, const int32_t* vis_len, int rows, int L,
                                int k, int32_t* idx, void* workspace, hipStream_t stream) {
  if (!topk_takes_prebuilt_hist(rows, L)) return hipErrorInvalidValue;
  return launch_filter_final(scores, vis_len, rows, L, k, idx, (char*)workspace,
                             make_layout(rows, L), stream);
}

}  // namespace lcs
