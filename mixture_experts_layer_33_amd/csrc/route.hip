// Gate routing on gfx950: router logits, top-k selection and gate weights.
//
// A Survey on Mixture of Experts, §5 System Design (first paragraph): gate
// routing is the first step of the expert-parallel pipeline; PopFetcher
// notes §2.1.2: each token goes to its top-k experts, k usually 1 or 2.
//
// One workgroup handles kRouteTok tokens.  The router product runs in
// float32 FMA with W_gate staged through LDS; each token's logits then sit
// in one 16-lane group, which selects the top k by k rounds of a 16-lane
// (value, index) max reduction.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRouteTok = 16;      // tokens per workgroup
constexpr int kRouteK = 64;        // d rows of W_gate per LDS stage
constexpr int kRouteThreads = 256; // 16 tokens x 16 lanes

// a ranks before b: larger value, or equal value and smaller index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <typename ActT>
__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const ActT* __restrict__ x, const float* __restrict__ w_gate,
             const float* __restrict__ b_gate, const float* __restrict__ logits_in,
             float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
             float* __restrict__ topk_w, int T, int d, int E, int k) {
  __shared__ float xs[kRouteTok][kRouteK + 1];
  __shared__ float ws[kRouteK * MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int tl = tid >> 4;   // token within tile
  const int g = tid & 15;    // lane within the token's 16-lane group
  const int t = blockIdx.x * kRouteTok + tl;
  const bool tok_ok = t < T;
  constexpr int EPT = MOE_MAX_EXPERTS / 16;  // experts per lane (max)
  float acc[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) acc[j] = 0.f;

  if (logits_in != nullptr) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      int e = g + 16 * j;
      if (e < E && tok_ok) acc[j] = logits_in[(size_t)t * E + e];
    }
  } else {
    for (int k0 = 0; k0 < d; k0 += kRouteK) {
      // stage x[16 tokens][64] and W_gate[64][E]
      for (int i = tid; i < kRouteTok * kRouteK; i += kRouteThreads) {
        int r = i / kRouteK, c = i % kRouteK;
        int tt = blockIdx.x * kRouteTok + r;
        xs[r][c] = (tt < T) ? to_f32(x[(size_t)tt * d + k0 + c]) : 0.f;
      }
      for (int i = tid; i < kRouteK * E; i += kRouteThreads)
        ws[i] = w_gate[(size_t)k0 * E + i];
      __syncthreads();
      for (int kk = 0; kk < kRouteK; ++kk) {
        float xv = xs[tl][kk];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          int e = g + 16 * j;
          if (e < E) acc[j] = fmaf(xv, ws[kk * E + e], acc[j]);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      int e = g + 16 * j;
      if (e < E) acc[j] += b_gate[e];
    }
  }
  if (logits_out != nullptr && tok_ok) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      int e = g + 16 * j;
      if (e < E) logits_out[(size_t)t * E + e] = acc[j];
    }
  }

  // top-k: k rounds of a (value desc, index asc) max over the 16-lane group
  unsigned taken = 0;
  float sel_v[MOE_MAX_TOPK];
  int sel_i[MOE_MAX_TOPK];
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      int e = g + 16 * j;
      if (e < E && !((taken >> j) & 1u) && better(acc[j], e, bv, bi)) {
        bv = acc[j];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 15) == g) taken |= 1u << (bi >> 4);
    sel_v[r] = bv;
    sel_i[r] = bi;
  }
  if (g == 0 && tok_ok) {
    float p[MOE_MAX_TOPK];
    float sum = 0.f;
    for (int r = 0; r < k; ++r) {
      p[r] = expf(sel_v[r] - sel_v[0]);
      sum += p[r];
    }
    float inv = 1.0f / sum;
    for (int r = 0; r < k; ++r) {
      topk_idx[(size_t)t * k + r] = sel_i[r];
      topk_w[(size_t)t * k + r] = p[r] * inv;
    }
  }
}

hipError_t launch_route(int act, const void* x, const float* w_gate, const float* b_gate,
                        const float* logits_in, float* logits_out, int32_t* topk_idx,
                        float* topk_w, int T, int d, int E, int k, hipStream_t s) {
  dim3 grid((T + kRouteTok - 1) / kRouteTok), block(kRouteThreads);
  if (act == MOE_BF16)
    hipLaunchKernelGGL(route_kernel<bf16>, grid, block, 0, s, (const bf16*)x, w_gate, b_gate,
                       logits_in, logits_out, topk_idx, topk_w, T, d, E, k);
  else
    hipLaunchKernelGGL(route_kernel<float>, grid, block, 0, s, (const float*)x, w_gate, b_gate,
                       logits_in, logits_out, topk_idx, topk_w, T, d, E, k);
  return hipGetLastError();
}

}  // namespace moe
