// cp.hip -- the single-device halves of context parallelism for the selection:
// a shard's top-k as (score, global position) candidates, the top-k of all
// shards' candidates, and a shard's share of the merged list.
//
// Context parallelism splits the KV pool over devices (panel "CP · EP · P/D ·
// HiCache" of the ailearn GLM-5.2 special edition). With a shard holding
// positions [lo, lo + L_shard) of every sequence, the whole sequence's top-k
// lies inside the union of the shards' own top-k's (anything outside a shard's
// top-k is beaten by k positions of that shard), so one exchange of G x k
// (score, position) pairs per query and a merge under the same order as the
// one-device selection -- score descending, lower position first, -0.0 equal
// to +0.0 -- reproduce the one-device selection exactly.
//
// Merge: one 1024-thread workgroup per query holds its <= 32768 candidates in
// registers as 64-bit keys (order-preserving score bits above the inverted
// position, so a larger key ranks higher and keys are distinct), finds the
// k-th largest key with 8-bit radix passes over an LDS histogram and keeps
// the keys at or above it. When the candidates' positions ascend in list
// order -- shards gathered in position order, each shard's selection
// ascending, as lcs_topk_select writes it -- the kept positions are written
// in list order, already sorted; otherwise a bitonic sort in LDS orders
// them. The leading digits of real scores take few values (sign and
// exponent), so most lanes of a wave would add to one counter and the LDS
// atomics would serialise: the histogram has 16 copies, lane l adding to copy
// l % 16, with a row stride of 257 words so that one digit's counters of the
// 16 copies sit in 16 different banks. The passes stop once the threshold
// bucket is taken whole (for distinct scores: after the score bytes).
#include "common.h"

namespace lcs {
namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergePer = 32;  // candidates per thread: up to 32768 per query
constexpr int kLocThreads = 256;
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;  // words per copy: consecutive copies shift banks by one

__global__ void __launch_bounds__(256) candidates_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ idx,
                                                         int64_t n, int L, int k, int pos_base,
                                                         float* __restrict__ cand_score,
                                                         int32_t* __restrict__ cand_idx) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t q = i / k;
  const int p = idx[i];
  const bool ok = p >= 0 && p < L;  // anything else is an empty slot
  cand_score[i] = ok ? scores[q * L + p] : -INFINITY;
  cand_idx[i] = ok ? p + pos_base : -1;
}

__device__ __forceinline__ uint32_t wave_scan_add(uint32_t v) {  // inclusive, lane order
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ __forceinline__ int wave_scan_max(int v) {  // inclusive, lane order
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v = max(v, u);
  }
  return v;
}

// A key is held as two 32-bit registers so that vector loads land in place:
// hi = order-preserving score bits, lo = 0x7FFFFFFF - position; an empty slot
// has hi = lo = 0 (a valid hi is at least score_key(-inf) > 0).
__device__ __forceinline__ bool key_matches(uint32_t hi, uint32_t lo, uint64_t mask,
                                            uint64_t prefix) {
  return (hi & (uint32_t)(mask >> 32)) == (uint32_t)(prefix >> 32) &&
         (lo & (uint32_t)mask) == (uint32_t)prefix;
}
__device__ __forceinline__ bool key_at_least(uint32_t hi, uint32_t lo, uint64_t t) {
  return hi != 0 && (((uint64_t)hi << 32) | lo) >= t;
}

// Thread t owns candidates [32 t, 32 t + 32) of the query's list (shard g's
// k_in slots after shard g - 1's), so the list order is (thread, register).
__global__ void __launch_bounds__(kMergeThreads) topk_merge_kernel(
    const float* __restrict__ cand_score, const int32_t* __restrict__ cand_idx, int G,
    int64_t Q, int k_in, int k, int32_t* __restrict__ idx) {
  constexpr int kW = kMergeThreads / 64;
  __shared__ uint32_t s_hist[2][kHistCopies * kHistStride];
  __shared__ uint32_t s_sel[kMaxTopk];
  __shared__ uint32_t s_tot[4];
  __shared__ __attribute__((aligned(16))) uint32_t s_wsum[kW];
  __shared__ __attribute__((aligned(16))) int s_wmax[kW];
  __shared__ __attribute__((aligned(16))) uint32_t s_wok[kW];
  __shared__ uint32_t s_digit, s_need, s_full, s_total;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.x;
  const int n = G * k_in;

  for (int i = tid; i < 2 * kHistCopies * kHistStride; i += kMergeThreads) (&s_hist[0][0])[i] = 0;

  // ---- load (all loads issued before any use) ----
  uint32_t khi[kMergePer], klo[kMergePer];
  const int j0 = tid * kMergePer;
  if (k_in % kMergePer == 0) {
    // the thread's 32 candidates are 32 consecutive slots of one shard
    const int jc = min(j0, n - kMergePer);
    const int g = jc / k_in;
    const int64_t at = ((int64_t)g * Q + q) * k_in + (jc - g * k_in);
    const float4* sp = (const float4*)(cand_score + at);
    const int4* ip = (const int4*)(cand_idx + at);
#pragma unroll
    for (int v = 0; v < kMergePer / 4; ++v) {
      const float4 a = sp[v];
      const int4 b = ip[v];
      khi[4 * v + 0] = __float_as_uint(a.x);
      khi[4 * v + 1] = __float_as_uint(a.y);
      khi[4 * v + 2] = __float_as_uint(a.z);
      khi[4 * v + 3] = __float_as_uint(a.w);
      klo[4 * v + 0] = (uint32_t)b.x;
      klo[4 * v + 1] = (uint32_t)b.y;
      klo[4 * v + 2] = (uint32_t)b.z;
      klo[4 * v + 3] = (uint32_t)b.w;
    }
    if (j0 >= n)
#pragma unroll
      for (int r = 0; r < kMergePer; ++r) klo[r] = 0xFFFFFFFFu;
  } else {
    int g = min(j0, n - 1) / k_in, slot = min(j0, n - 1) - g * k_in;
#pragma unroll
    for (int r = 0; r < kMergePer; ++r) {
      const int64_t at = ((int64_t)g * Q + q) * k_in + slot;
      khi[r] = __float_as_uint(cand_score[at]);
      klo[r] = j0 + r < n ? (uint32_t)cand_idx[at] : 0xFFFFFFFFu;
      if (j0 + r + 1 < n && ++slot == k_in) {
        slot = 0;
        ++g;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kMergePer; ++r) {
    const int p = (int)klo[r];
    khi[r] = p >= 0 ? score_key(__uint_as_float(khi[r])) : 0u;
    klo[r] = p >= 0 ? 0x7FFFFFFFu - (uint32_t)p : 0u;
  }
  __syncthreads();  // histograms cleared

  // ---- radix select of the k-th largest key (8-bit digits, top first) ----
  // Pass p adds into s_hist[p & 1] and clears s_hist[(p + 1) & 1] (last read
  // before the previous pass's final barrier). Thread t < 256 owns digit
  // 255 - t; the first pass also counts every valid key.
  uint64_t prefix = 0, mask = 0, thresh = 1;
  uint32_t need = (uint32_t)k;
  for (int pass = 0, shift = 56; shift >= 0; ++pass, shift -= 8) {
    uint32_t* cur = s_hist[pass & 1];
    uint32_t* nxt = s_hist[(pass + 1) & 1];
    uint32_t* my_hist = cur + (tid & (kHistCopies - 1)) * kHistStride;
#pragma unroll
    for (int r = 0; r < kMergePer; ++r)
      if (khi[r] != 0 && key_matches(khi[r], klo[r], mask, prefix)) {
        const uint32_t d = shift >= 32 ? khi[r] >> (shift - 32) : klo[r] >> shift;
        atomicAdd(&my_hist[d & 255u], 1u);
      }
    for (int i = tid; i < kHistCopies * kHistStride; i += kMergeThreads) nxt[i] = 0;
    __syncthreads();
    uint32_t c = 0, incl = 0;
    if (tid < 256) {
#pragma unroll
      for (int cp = 0; cp < kHistCopies; ++cp) c += cur[cp * kHistStride + 255 - tid];
      incl = wave_scan_add(c);
      if (lane == 63) s_tot[wv] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wv; ++w) incl += s_tot[w];
      if (pass == 0 && tid == 255) s_total = incl;
      if (incl >= need && incl - c < need) {
        s_digit = 255 - tid;
        s_need = need - (incl - c);
        s_full = need - (incl - c) == c;  // the whole bucket is taken
      }
    }
    __syncthreads();
    if (pass == 0 && s_total <= (uint32_t)k) break;  // every valid key is kept
    prefix |= (uint64_t)s_digit << shift;
    mask |= (uint64_t)255 << shift;
    need = s_need;
    thresh = prefix;
    // every key matching the prefix is kept: keys >= prefix (lower digits
    // zero) are exactly the keys to keep
    if (s_full) break;
  }

  // ---- keep the keys >= thresh, in list order ----
  uint32_t mine = 0;
  int first = -1, last = -1;
  bool asc = true;
#pragma unroll
  for (int r = 0; r < kMergePer; ++r) {
    const int p = khi[r] != 0 ? (int)(0x7FFFFFFFu - klo[r]) : -1;
    if (p >= 0) {
      asc = asc && p > last;
      first = first < 0 ? p : first;
      last = p;
    }
    mine += key_at_least(khi[r], klo[r], thresh) ? 1u : 0u;
  }
  // exclusive sum of the kept counts (output slots) and the largest position
  // before this thread (is the list ascending across threads?)
  const uint32_t ws = wave_scan_add(mine);
  const int wm = wave_scan_max(last);
  if (lane == 63) {
    s_wsum[wv] = ws;
    s_wmax[wv] = wm;
  }
  __syncthreads();
  uint32_t before = 0, cnt = 0;
  int mx_before = -1;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const uint32_t a = s_wsum[w];
    const int b = s_wmax[w];
    cnt += a;
    if (w < wv) {
      before += a;
      mx_before = max(mx_before, b);
    }
  }
  const int prev_lane_max = __shfl_up(wm, 1);
  if (lane > 0) mx_before = max(mx_before, prev_lane_max);
  before += ws - mine;
  const bool ok = asc && (first < 0 || first > mx_before);
  const uint64_t bad = __ballot(!ok);
  if (lane == 0) s_wok[wv] = bad == 0 ? 1u : 0u;
  __syncthreads();
  bool all_ok = true;
#pragma unroll
  for (int w = 0; w < kW; ++w) all_ok = all_ok && s_wok[w] != 0;
  const int total = min((int)cnt, k);
  int32_t* out = idx + q * k;
  if (all_ok) {
    // positions ascend in list order: the kept keys are already sorted
    uint32_t at = before;
#pragma unroll
    for (int r = 0; r < kMergePer; ++r)
      if (key_at_least(khi[r], klo[r], thresh)) {
        if (at < (uint32_t)k) out[at] = (int32_t)(0x7FFFFFFFu - klo[r]);
        ++at;
      }
    for (int i = total + tid; i < k; i += kMergeThreads) out[i] = -1;
    return;
  }
  uint32_t at = before;
#pragma unroll
  for (int r = 0; r < kMergePer; ++r)
    if (key_at_least(khi[r], klo[r], thresh)) {
      if (at < (uint32_t)k) s_sel[at] = 0x7FFFFFFFu - klo[r];
      ++at;
    }
  int P = 1;
  while (P < total) P <<= 1;
  for (int i = total + tid; i < P; i += kMergeThreads) s_sel[i] = 0xFFFFFFFFu;
  // Bitonic sort of s_sel[0, P) ascending; thread t compares pair t of each
  // stage (P / 2 <= 1024 pairs). With a stride of at most 64, the 64 pairs of
  // a wave lie in its own 128 elements [128 w, 128 w + 128), so such a stage
  // only waits for the wave's own LDS writes; a stage that reads across waves
  // (stride >= 128), and the first stage after one, waits at a workgroup
  // barrier.
  int prev = 1 << 30;  // before the first stage: s_sel was written by any thread
  for (int size = 2, lsize = 1; size <= P; size <<= 1, ++lsize)
    for (int stride = size >> 1, ls = lsize - 1; stride > 0; stride >>= 1, --ls) {
      if (stride >= 128 || prev >= 128) {
        __syncthreads();
      } else {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
        asm volatile("" ::: "memory");
      }
      prev = stride;
      if (tid < P / 2) {
        const int i = ((tid >> ls) << (ls + 1)) + (tid & (stride - 1));
        const int j = i + stride;
        const uint32_t a = s_sel[i], b = s_sel[j];
        const bool up = (i & size) == 0;
        if ((a > b) == up) {
          s_sel[i] = b;
          s_sel[j] = a;
        }
      }
    }
  __syncthreads();
  for (int i = tid; i < k; i += kMergeThreads) out[i] = i < total ? (int32_t)s_sel[i] : -1;
}

// One workgroup per query: thread t takes entries [t*c, (t+1)*c) of the list;
// an exclusive scan of the in-range counts gives each in-range entry its slot.
__global__ void __launch_bounds__(kLocThreads) localize_kernel(const int32_t* __restrict__ idx,
                                                               int k, int lo, int hi,
                                                               int32_t* __restrict__ local) {
  __shared__ uint32_t s_wave[kLocThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t q = blockIdx.x;
  const int c = (k + kLocThreads - 1) / kLocThreads;
  const int i0 = min(k, tid * c), i1 = min(k, i0 + c);
  const int32_t* in = idx + q * k;
  int32_t* out = local + q * k;
  uint32_t mine = 0;
  for (int i = i0; i < i1; ++i) mine += (in[i] >= lo && in[i] < hi) ? 1u : 0u;
  uint32_t v = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wave[wv] = v;
  __syncthreads();
  uint32_t before = 0, total = 0;
  for (int w = 0; w < kLocThreads / 64; ++w) {
    if (w < wv) before += s_wave[w];
    total += s_wave[w];
  }
  uint32_t slot = before + v - mine;
  for (int i = i0; i < i1; ++i) {
    const int p = in[i];
    if (p >= lo && p < hi) out[slot++] = p - lo;
  }
  for (int i = (int)total + tid; i < k; i += kLocThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk_candidates(const float* scores, const int32_t* idx, int64_t queries, int L,
                                  int k, int pos_base, float* cand_score, int32_t* cand_idx,
                                  hipStream_t stream) {
  const int64_t n = queries * k;
  if (n == 0) return hipSuccess;
  return launch_kernel(candidates_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       scores, idx, n, L, k, pos_base, cand_score, cand_idx);
}

hipError_t launch_topk_merge(const float* cand_score, const int32_t* cand_idx, int G,
                             int64_t queries, int k_in, int k, int32_t* idx, hipStream_t stream) {
  if (queries == 0) return hipSuccess;
  return launch_kernel(topk_merge_kernel, dim3((unsigned)queries), dim3(kMergeThreads), 0, stream,
                       cand_score, cand_idx, G, queries, k_in, k, idx);
}

hipError_t launch_idx_localize(const int32_t* idx, int64_t queries, int k, int lo, int hi,
                               int32_t* local, hipStream_t stream) {
  if (queries == 0) return hipSuccess;
  return launch_kernel(localize_kernel, dim3((unsigned)queries), dim3(kLocThreads), 0, stream, idx,
                       k, lo, hi, local);
}

}  // namespace lcs
