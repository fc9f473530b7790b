// common.h -- shared device helpers and launcher declarations of the gfx950
// DSA + IndexShare kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace lcs {

// Launch through hipLaunchKernel, which returns this launch's own status (the
// per-thread sticky error of hipGetLastError may hold an unrelated earlier
// failure of the caller's HIP calls).
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = (void*)&v), ...);
  }, vals);
  return hipLaunchKernel((const void*)kernel, grid, block, ptrs, shmem, stream);
}


constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kAttHeads = 64;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kKvDim = kLatent + kRope;  // 576
constexpr int kMaxTopk = 2048;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Order-preserving map of an fp32 score onto uint32: a larger float gives a
// larger key. -0.0 is folded onto +0.0 so that equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int clamp_vis(int v, int L) { return v < 0 ? 0 : (v > L ? L : v); }

// two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const v2bf r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// s_waitcnt vmcnt(N) with the other counters left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for data exchanged through LDS only. A workgroup fence
// would also wait for every outstanding global store and global->LDS load of
// the wave (vmcnt(0)), which a pipeline keeps in flight on purpose; instead
// each wave waits for its own LDS accesses (lgkmcnt), and the empty asm
// statements keep the compiler from moving memory accesses across s_barrier.
// Global->LDS loads must be waited for (vmcnt) by the issuing wave before it
// reaches the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- launchers (host) ----

// kstride: rows (tokens) from one sequence's keys (and key scales) to the next
hipError_t launch_idx_score(const uint8_t* q8, const float* q_scale, const float* w,
                            const uint8_t* k8, const float* k_scale, int64_t kstride,
                            const int32_t* vis_len, int B, int T, int L, float* scores,
                            hipStream_t stream);

hipError_t launch_idx_score_paged(const uint8_t* q8, const float* q_scale, const float* w,
                                  const uint8_t* k8, const float* k_scale,
                                  const int32_t* block_table, int max_blocks, int lbs,
                                  int n_blocks, const int32_t* vis_len, int B, int T, int L,
                                  float* scores, hipStream_t stream);

size_t topk_workspace_bytes(int64_t rows, int L, int k);
hipError_t launch_topk(const float* scores, const int32_t* vis_len, int rows, int L, int k,
                       int32_t* idx, void* workspace, hipStream_t stream);

// Decode steps with one query per sequence can build the selection's first
// radix-digit histogram inside the indexer launch: launch_topk_clear zeroes
// the histograms in the top-k workspace (topk_hist_area), launch_idx_score_hist
// scores and accumulates them, and launch_topk_prebuilt selects without a
// histogram pass. Every chunked selection leaves the histograms zero again, so
// the clear is needed once per workspace, before the first such indexer launch.
// topk_takes_prebuilt_hist: the selection for these shapes uses the chunked
// launches (the only ones that read the histograms).
bool topk_takes_prebuilt_hist(int64_t rows, int L);
uint32_t* topk_hist_area(void* workspace, int64_t rows, int L);
hipError_t launch_topk_clear(void* workspace, int rows, int L, hipStream_t stream);
hipError_t launch_topk_prebuilt(const float* scores, const int32_t* vis_len, int rows, int L,
                                int k, int32_t* idx, void* workspace, hipStream_t stream);
hipError_t launch_idx_score_hist(const uint8_t* q8, const float* q_scale, const float* w,
                                 const uint8_t* k8, const float* k_scale, const int32_t* vis_len,
                                 int B, int L, float* scores, uint32_t* hist, hipStream_t stream);

size_t attn_workspace_bytes(int64_t queries, int k);
// the static scratch of the allocation-free attention call: its size, and its
// address on the current device (looked up once per device)
constexpr size_t kNoAllocScratchBytes = (size_t)20 << 20;
hipError_t noalloc_scratch(void** ptr);
// kv_stride: rows (tokens) from one sequence's latent rows (and row scales) to the next
hipError_t launch_sparse_mla(const uint16_t* q, const void* kv, bool kv_fp8,
                             const float* kv_scale, int64_t kv_stride, const int32_t* idx, int B,
                             int T, int L, int k, float sm_scale, uint16_t* out, float* lse,
                             void* workspace, hipStream_t stream);

// paged KV: kv/kv_scale are pools of 2^lbs-row blocks, block_table [B][max_blocks]
hipError_t launch_sparse_mla_paged(const uint16_t* q, const void* kv, bool kv_fp8,
                                   const float* kv_scale, const int32_t* block_table,
                                   int max_blocks, int lbs, int n_blocks, const int32_t* idx,
                                   int B, int T, int L, int k, float sm_scale, uint16_t* out,
                                   float* lse, void* workspace, hipStream_t stream);
// merge of `splits` query-major attention partials (the attention's own workspace)
hipError_t launch_split_combine(const uint16_t* part_o, const float* part_lse, int splits,
                                int64_t queries, uint16_t* out, float* lse, hipStream_t stream);

// D = 128 or 576
hipError_t launch_quantize_e4m3(const uint16_t* x, int64_t rows, int D, uint8_t* codes,
                                float* scales, hipStream_t stream);
// block_table == nullptr: contiguous caches [B][L]; else pools of 2^lbs-row blocks
hipError_t launch_cache_append(const uint16_t* k_new, const uint16_t* kv_new, bool kv_fp8,
                               const int32_t* pos, int B, int T, int L, uint8_t* k8,
                               float* k_scale, void* kv, float* kv_scale,
                               const int32_t* block_table, int max_blocks, int lbs, int n_blocks,
                               hipStream_t stream);

// context-parallel halves (cp.hip; the combine lives beside the split combine)
hipError_t launch_topk_candidates(const float* scores, const int32_t* idx, int64_t queries, int L,
                                  int k, int pos_base, float* cand_score, int32_t* cand_idx,
                                  hipStream_t stream);
hipError_t launch_topk_merge(const float* cand_score, const int32_t* cand_idx, int G,
                             int64_t queries, int k_in, int k, int32_t* idx, hipStream_t stream);
hipError_t launch_idx_localize(const int32_t* idx, int64_t queries, int k, int lo, int hi,
                               int32_t* local, hipStream_t stream);
hipError_t launch_lse_combine(const uint16_t* part_out, const float* part_lse, int G,
                              int64_t queries, uint16_t* out, float* lse, hipStream_t stream);

}  // namespace lcs
