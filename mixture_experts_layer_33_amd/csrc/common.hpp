// Shared device helpers for the gfx950 MoE kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kWave = 64;

// Slots per tile of the permutation's per-tile histograms.
constexpr int kRankTile = 256;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bf16 round-to-nearest-even (gfx950 converts in hardware).
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ int wave_lane() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Exclusive prefix sum over a block of `nthreads` threads, one value per
// thread; returns the exclusive prefix, writes the block total to *total.
// `scratch` needs nthreads/64 + 1 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) scratch[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      int c = scratch[w];
      scratch[w] = run;
      run += c;
    }
    scratch[nw] = run;
  }
  __syncthreads();
  int excl = scratch[wid] + incl - v;
  *total = scratch[nw];
  __syncthreads();
  return excl;
}

// Lane j's value of v (j wave-uniform), read into a scalar register: for
// broadcasts within a wavefront that works on one token.
__device__ __forceinline__ int lane_value(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ __forceinline__ float lane_value(float v, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}

// a compile-time int as a value (selects an unrolled step's buffers)
template <int V>
struct Ic {
  static constexpr int value = V;
};

}  // namespace moe
