// Cross-layer expert correlation and popularity prediction on gfx950.
//
// PopFetcher notes §4.1: a token that picks expert x in layer j and x' in
// layer j+1 contributes the tuple (x, x'); the conditional probability of
// x' given x shows which next-layer experts follow which.  §4.2: statistics
// over a sliding window of iterations (Eq. 1) and a correlation-based
// popularity of the next layer (Eq. 2, Eq. 3; both bodies are missing from
// the page - the reading taken: P(x'|x) = windowed tuple count / row total,
// pred(x') = sum over x of this layer's count of x times P(x'|x)).
//
// Counts are exact integers (LDS histograms per workgroup, then integer
// atomics, whose sum does not depend on their order).  The prediction runs
// in float64 with every product, quotient and sum a separate correctly
// rounded operation in index order, so it is reproducible bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kCoThreads = 256;
constexpr int kCoLdsBins = 16384;  // E_a * E_b up to this uses an LDS histogram

__global__ void __launch_bounds__(256) fill_i32_kernel(int32_t* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (long long)gridDim.x * 256)
    p[i] = 0;
}

// tuples of T tokens into `slice` [E_a][E_b] (zeroed before)
__global__ void __launch_bounds__(kCoThreads)
cooccur_kernel(const int32_t* __restrict__ idx_a, const int32_t* __restrict__ idx_b, int T,
               int k_a, int k_b, int E_a, int E_b, int32_t* __restrict__ slice) {
  __shared__ int hist[kCoLdsBins];
  const int bins = E_a * E_b;
  const bool in_lds = bins <= kCoLdsBins;
  if (in_lds)
    for (int i = threadIdx.x; i < bins; i += kCoThreads) hist[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * kCoThreads + threadIdx.x;
  if (t < T) {
    int b[MOE_MAX_TOPK];
    for (int j = 0; j < k_b; ++j) b[j] = idx_b[(size_t)t * k_b + j];
    for (int i = 0; i < k_a; ++i) {
      const int a = idx_a[(size_t)t * k_a + i];
      for (int j = 0; j < k_b; ++j) {
        if (in_lds)
          atomicAdd(&hist[a * E_b + b[j]], 1);
        else
          atomicAdd(&slice[(size_t)a * E_b + b[j]], 1);
      }
    }
  }
  if (!in_lds) return;
  __syncthreads();
  for (int i = threadIdx.x; i < bins; i += kCoThreads)
    if (hist[i] != 0) atomicAdd(&slice[i], hist[i]);
}

// window_sum = sum of the last min(iter + 1, W) slices of the ring
__global__ void __launch_bounds__(256)
co_window_kernel(const int32_t* __restrict__ ring, int window, int64_t iter, int bins,
                 int32_t* __restrict__ window_sum) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= bins) return;
  const int slot = (int)(iter % window);
  const int n = (int)((iter + 1 < (int64_t)window) ? iter + 1 : window);
  int s = 0;
  for (int b = 0; b < n; ++b) s += ring[(size_t)((slot - b + window) % window) * bins + i];
  window_sum[i] = s;
}

__global__ void __launch_bounds__(256)
predict_kernel(int E_a, int E_b, const int32_t* __restrict__ counts_a,
               const int32_t* __restrict__ cooc, double* __restrict__ pred,
               int32_t* __restrict__ order) {
  __shared__ long long s_row[MOE_MAX_EXPERTS];
  __shared__ double s_pred[MOE_MAX_EXPERTS];
  for (int i = threadIdx.x; i < E_a; i += 256) {
    long long r = 0;
    for (int h = 0; h < E_b; ++h) r += cooc[(size_t)i * E_b + h];
    s_row[i] = r;
  }
  __syncthreads();
  for (int h = threadIdx.x; h < E_b; h += 256) {
#pragma clang fp contract(off)  // a product and a sum, never fused
    double acc = 0.0;
    for (int i = 0; i < E_a; ++i) {
      if (s_row[i] == 0) continue;
      const double p = (double)cooc[(size_t)i * E_b + h] / (double)s_row[i];
      const double m = (double)counts_a[i] * p;
      acc = acc + m;
    }
    s_pred[h] = acc;
    pred[h] = acc;
  }
  __syncthreads();
  for (int h = threadIdx.x; h < E_b; h += 256) {
    const double v = s_pred[h];
    int pos = 0;
    for (int o = 0; o < E_b; ++o) pos += (s_pred[o] > v) || (s_pred[o] == v && o < h);
    order[pos] = h;
  }
}

hipError_t launch_cooccurrence(int E_a, int E_b, int k_a, int k_b, int T, int window,
                               int64_t iter, const int32_t* idx_a, const int32_t* idx_b,
                               int32_t* ring, int32_t* window_sum, hipStream_t s) {
  const int bins = E_a * E_b;
  int32_t* slice = ring + (size_t)(iter % window) * bins;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((bins + 255) / 256), dim3(256), 0, s, slice,
                     (long long)bins);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cooccur_kernel, dim3((T + kCoThreads - 1) / kCoThreads), dim3(kCoThreads),
                     0, s, idx_a, idx_b, T, k_a, k_b, E_a, E_b, slice);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(co_window_kernel, dim3((bins + 255) / 256), dim3(256), 0, s, ring, window,
                     iter, bins, window_sum);
  return hipGetLastError();
}

hipError_t launch_predict(int E_a, int E_b, const int32_t* counts_a, const int32_t* cooc,
                          double* pred, int32_t* order, hipStream_t s) {
  hipLaunchKernelGGL(predict_kernel, dim3(1), dim3(256), 0, s, E_a, E_b, counts_a, cooc, pred,
                     order);
  return hipGetLastError();
}

}  // namespace moe
