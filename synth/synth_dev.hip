// synth_dev.hip -- device fill routines of the synthetic-input generator.
// Same definitions as synth_host.c (both include synth.h), so a device fill
// is bit-identical to the host fill of the same block. Used only to create
// inputs in device memory; holds none of the method's arithmetic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <tuple>

#define SYN_FN __host__ __device__ static inline
#include "synth.h"

namespace {

constexpr int kMaxPerLane = 16;  // D <= 1024

__global__ void __launch_bounds__(256) fp8_rows_kernel(
    uint64_t seed, uint32_t tensor, uint32_t layer, int64_t R, int32_t D,
    uint32_t permyriad, int32_t b0, int32_t nb, int64_t r0, int64_t nr,
    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t waves_per_block = blockDim.x >> 6;
  const int64_t total = (int64_t)nb * nr;
  for (int64_t row = (int64_t)blockIdx.x * waves_per_block + (threadIdx.x >> 6);
       row < total; row += (int64_t)gridDim.x * waves_per_block) {
    const int32_t bi = (int32_t)(row / nr);
    const int64_t ri = row - (int64_t)bi * nr;
    const uint32_t b = (uint32_t)(b0 + bi);
    const uint64_t r = (uint64_t)(r0 + ri);
    const uint64_t key = syn_rowkey(seed, tensor, layer, b, r);
    const int planted = syn_planted(seed, layer, b, r, (uint64_t)R, permyriad);
    float x[kMaxPerLane];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int d = lane + 64 * i;
      x[i] = 0.0f;
      if (d < D) {
        x[i] = syn_value(key, (uint32_t)d, planted);
        amax = fmaxf(amax, fabsf(x[i]));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float scale = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int d = lane + 64 * i;
      if (d < D) codes[row * D + d] = syn_e4m3((double)x[i] / (double)scale);
    }
    if (lane == 0) scales[row] = scale;
  }
}

__global__ void __launch_bounds__(256) bf16_rows_kernel(
    uint64_t seed, uint32_t tensor, uint32_t layer, int32_t D, int32_t b0,
    int64_t nr, int64_t r0, int64_t total, uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / D;
    const int32_t d = (int32_t)(i - row * D);
    const int32_t bi = (int32_t)(row / nr);
    const int64_t ri = row - (int64_t)bi * nr;
    const uint64_t key = syn_rowkey(seed, tensor, layer, (uint32_t)(b0 + bi), (uint64_t)(r0 + ri));
    out[i] = syn_bf16(syn_normal(key, (uint32_t)d));
  }
}

__global__ void __launch_bounds__(256) uniform_rows_kernel(
    uint64_t seed, uint32_t tensor, uint32_t layer, int32_t D, int32_t b0,
    int64_t nr, int64_t r0, int64_t total, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / D;
    const int32_t d = (int32_t)(i - row * D);
    const int32_t bi = (int32_t)(row / nr);
    const int64_t ri = row - (int64_t)bi * nr;
    const uint64_t key = syn_rowkey(seed, tensor, layer, (uint32_t)(b0 + bi), (uint64_t)(r0 + ri));
    out[i] = syn_uniform(key, (uint32_t)d);
  }
}

// hipLaunchKernel returns this launch's own status
template <typename... KArgs, typename... Args>
int launch(const char* what, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
           Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = (void*)&v), ...);
  }, vals);
  const hipError_t e = hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, stream);
  if (e == hipSuccess) return 0;
  fprintf(stderr, "synth %s: %s\n", what, hipGetErrorString(e));
  return 2;
}

int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

int synth_dev_fp8_rows(uint64_t seed, uint32_t tensor, uint32_t layer, int64_t R,
                       int32_t D, uint32_t plant_permyriad, int32_t b0, int32_t nb,
                       int64_t r0, int64_t nr, uint8_t* codes, float* scales,
                       hipStream_t stream) {
  if (D <= 0 || D > 64 * kMaxPerLane || nb < 0 || nr < 0 || !codes || !scales) return 1;
  if ((int64_t)nb * nr == 0) return 0;
  return launch("fp8 rows", fp8_rows_kernel, dim3(grid_for((int64_t)nb * nr, 4)), dim3(256),
                stream, seed, tensor, layer, R, D, plant_permyriad, b0, nb, r0, nr, codes, scales);
}

int synth_dev_bf16_rows(uint64_t seed, uint32_t tensor, uint32_t layer, int32_t D,
                        int32_t b0, int32_t nb, int64_t r0, int64_t nr, uint16_t* out,
                        hipStream_t stream) {
  if (D <= 0 || nb < 0 || nr < 0 || !out) return 1;
  const int64_t total = (int64_t)nb * nr * D;
  if (total == 0) return 0;
  return launch("bf16 rows", bf16_rows_kernel, dim3(grid_for(total, 256)), dim3(256), stream,
                seed, tensor, layer, D, b0, nr, r0, total, out);
}

int synth_dev_uniform_rows(uint64_t seed, uint32_t tensor, uint32_t layer, int32_t D,
                           int32_t b0, int32_t nb, int64_t r0, int64_t nr, float* out,
                           hipStream_t stream) {
  if (D <= 0 || nb < 0 || nr < 0 || !out) return 1;
  const int64_t total = (int64_t)nb * nr * D;
  if (total == 0) return 0;
  return launch("uniform rows", uniform_rows_kernel, dim3(grid_for(total, 256)), dim3(256), stream,
                seed, tensor, layer, D, b0, nr, r0, total, out);
}

}  // extern "C"
