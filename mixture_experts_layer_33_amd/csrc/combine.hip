// Output decode, the elementwise backward steps of the layer, and the
// popularity window, on gfx950.
//
// A Survey on Mixture of Experts, §5 System Design (first paragraph): output
// decode restores the original token order from the gating indices and, with
// top-k gating, sums the k expert outputs weighted by the gate.  The backward
// steps here are the transposes of decode, of the gate softmax and of encode.
// PopFetcher notes §3.1 and §4.2 (Eq. 1): per-expert token counts over a
// sliding window of iterations.
//
// All row work is one wavefront per token with 16-byte accesses; sums run in
// float32 in a fixed order (slot order j = 0..k-1), never with atomics.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRowThreads = 256;  // 4 tokens per workgroup

// 16 bytes of activations as float32 values.
template <typename ActT>
struct Chunk;
template <>
struct Chunk<bf16> {
  static constexpr int N = 8;
  __device__ static void load(const bf16* p, float* v) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
  }
  __device__ static void store(bf16* p, const float* v) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = a;
  }
};
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = a[i];
  }
  __device__ static void store(float* p, const float* v) {
    f32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = v[i];
    *reinterpret_cast<f32x4*>(p) = a;
  }
};

// Load token t's k (row, weight) pairs into every lane (one token per
// wavefront).
__device__ __forceinline__ void token_slots(int t, int k, const int32_t* slot_row,
                                            const float* topk_w, int* rows, float* w) {
  const int lane = threadIdx.x & 63;
  int r = -1;
  float wv = 0.f;
  if (lane < k) {
    r = slot_row[(size_t)t * k + lane];
    wv = topk_w[(size_t)t * k + lane];
  }
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    rows[j] = lane_value(r, j);
    w[j] = lane_value(wv, j);
  }
}

// w_gate [d, E] -> w_gate_t [E, d], 32 x 32 tile `tile_id` (row-major over
// ceil(d/32) x ceil(E/32) tiles) by one 256-thread workgroup
__device__ __forceinline__ void transpose_gate_tile(const float* __restrict__ w_gate,
                                                    float* __restrict__ wt, int d, int E,
                                                    int tile_id) {
  __shared__ float tile[32][33];
  const int te = (E + 31) / 32;
  const int i0 = (tile_id / te) * 32, e0 = (tile_id % te) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, e = e0 + tx;
    tile[r][tx] = (i < d && e < E) ? w_gate[(size_t)i * E + e] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, i = i0 + tx;
    if (e < E && i < d) wt[(size_t)e * d + i] = tile[tx][r];
  }
}

// Dropped slots still carry gate gradient (through the renormalised
// weights).  The permutation lists them after the kept rows:
// row_token[S_kept + j] = slot of the j-th dropped slot, ordered by expert and
// then slot.  Block `b` (of E x ceil(d/256)) finds its expert's run by binary
// search and adds that run's contribution to dW_gate[:, e] and db[e]
// (written before by the kept-row pass), walking the run in order.
template <typename ActT>
__device__ __forceinline__ void gate_dropped_block(const ActT* __restrict__ x,
                                                   const float* __restrict__ dsel,
                                                   const int32_t* __restrict__ topk_idx,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ row_token,
                                                   float* __restrict__ dw_gate,
                                                   float* __restrict__ db_gate, int S, int d,
                                                   int E, int k, int b) {
  const int cb = (d + 255) / 256;
  const int e = b / cb;
  const int i = (b % cb) * 256 + threadIdx.x;
  const int kept = offsets[E];
  const int32_t* list = row_token + kept;
  const int n = S - kept;
  // first j with expert(list[j]) >= v
  // (an entry that is not a slot index sorts last and is skipped)
  auto expert_of = [&](int j) {
    const int s = list[j];
    return (unsigned)s < (unsigned)S ? topk_idx[s] : E;
  };
  auto lower = [&](int v) {
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (expert_of(mid) < v) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  const int j0 = lower(e), j1 = lower(e + 1);
  if (j0 == j1) return;
  float acc = 0.f, db = 0.f;
  for (int j = j0; j < j1; ++j) {
    const int s = list[j];
    if ((unsigned)s >= (unsigned)S) continue;
    const float g = dsel[s];
    db += g;
    if (i < d) acc = fmaf(g, to_f32(x[(size_t)(s / k) * d + i]), acc);
  }
  if (i < d) dw_gate[(size_t)i * E + e] += acc;
  if (b % cb == 0 && threadIdx.x == 0) db_gate[e] += db;
}

template <typename ActT>
__global__ void __launch_bounds__(kRowThreads)
combine_kernel(const ActT* __restrict__ out_perm, const float* __restrict__ topk_w,
               const int32_t* __restrict__ slot_row, ActT* __restrict__ y, int T, int d, int k,
               bool slot_order) {
  using CK = Chunk<ActT>;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[MOE_MAX_TOPK];
  float w[MOE_MAX_TOPK];
  token_slots(t, k, slot_row, topk_w, rows, w);
  if (slot_order) {  // expert outputs stored by slot (gather-fused forward)
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (rows[j] >= 0) rows[j] = t * k + j;
  }
  for (int c = lane * CK::N; c < d; c += 64 * CK::N) {
    float acc[CK::N];
#pragma unroll
    for (int i = 0; i < CK::N; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && rows[j] >= 0) {
        float v[CK::N];
        CK::load(out_perm + (size_t)rows[j] * d + c, v);
#pragma unroll
        for (int i = 0; i < CK::N; ++i) acc[i] = fmaf(w[j], v[i], acc[i]);
      }
    }
    CK::store(y + (size_t)t * d + c, acc);
  }
}

// Decode backward.  For each kept slot (t, j) with row r:
//   d_out[r] = w[t,j] * dy[t]      (stored in the activation type)
//   dg[t,j]  = <dy[t], out_perm[r]>  (0 for a dropped slot)
// then the gate softmax backward dsel[t,j] = w_j (dg_j - sum_i w_i dg_i),
// also written per packed row (dsel_perm[r]) for the gate weight gradient,
// and dlogits[t, :] (dense, optional) holding dsel at the selected experts.
// Workgroups past the tokens write W_gate^T for dx_kernel.
template <typename ActT>
__global__ void __launch_bounds__(kRowThreads)
combine_bwd_kernel(const ActT* __restrict__ dy, const ActT* __restrict__ out_perm,
                   const float* __restrict__ topk_w, const int32_t* __restrict__ topk_idx,
                   const int32_t* __restrict__ slot_row, ActT* __restrict__ d_out,
                   float* __restrict__ dsel, float* __restrict__ dsel_perm,
                   float* __restrict__ dlogits, const float* __restrict__ w_gate,
                   float* __restrict__ w_gate_t, int32_t* __restrict__ counters, int T, int d,
                   int E, int k) {
  using CK = Chunk<ActT>;
  // the weight-gradient GEMMs later on this stream take their tiles from
  // these counters: they start at zero
  if (counters != nullptr && blockIdx.x == 0 && threadIdx.x < kBwdCounters)
    counters[threadIdx.x] = 0;
  const int tok_blocks = (T + kRowThreads / 64 - 1) / (kRowThreads / 64);
  if ((int)blockIdx.x >= tok_blocks) {  // the blocks past the tokens transpose W_gate
    transpose_gate_tile(w_gate, w_gate_t, d, E, blockIdx.x - tok_blocks);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[MOE_MAX_TOPK];
  float w[MOE_MAX_TOPK];
  token_slots(t, k, slot_row, topk_w, rows, w);
  float part[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) part[j] = 0.f;
  for (int c = lane * CK::N; c < d; c += 64 * CK::N) {
    float g[CK::N];
    CK::load(dy + (size_t)t * d + c, g);
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && rows[j] >= 0) {
        float o[CK::N], s[CK::N];
        CK::load(out_perm + (size_t)rows[j] * d + c, o);
#pragma unroll
        for (int i = 0; i < CK::N; ++i) {
          part[j] = fmaf(g[i], o[i], part[j]);
          s[i] = w[j] * g[i];
        }
        CK::store(d_out + (size_t)rows[j] * d + c, s);
      }
    }
  }
  float dg[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) dg[j] = wave_sum(part[j]);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    if (j < k) s = fmaf(w[j], dg[j], s);
  float ds[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) ds[j] = w[j] * (dg[j] - s);
  if (lane < k) {
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j == lane) mine = ds[j];
    dsel[(size_t)t * k + lane] = mine;
    int my_row = -1;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j == lane) my_row = rows[j];
    if (my_row >= 0) dsel_perm[my_row] = mine;
  }
  if (dlogits != nullptr) {
    int idx[MOE_MAX_TOPK];
    const int my = (lane < k) ? topk_idx[(size_t)t * k + lane] : -1;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) idx[j] = lane_value(my, j);
    for (int e = lane; e < E; e += 64) {
      float v = 0.f;
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        if (j < k && idx[j] == e) v = ds[j];
      dlogits[(size_t)t * E + e] = v;
    }
  }
}

// Encode backward plus the router's input gradient:
//   dx[t] = sum_j dx_perm[row_j] + sum_j dsel[t,j] * w_gate[:, idx_j]
// both sums in slot order, in float32, rounded once.  With drops possible,
// workgroups past the tokens add the dropped slots' gate gradient
// (gate_dropped_block).
template <typename ActT>
__global__ void __launch_bounds__(kRowThreads)
dx_kernel(const ActT* __restrict__ dx_perm, const float* __restrict__ dsel,
          const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ slot_row,
          const float* __restrict__ wt, ActT* __restrict__ dx, int T, int d, int k,
          const ActT* __restrict__ x, const int32_t* __restrict__ offsets,
          const int32_t* __restrict__ row_token, float* __restrict__ dw_gate,
          float* __restrict__ db_gate, int E) {
  using CK = Chunk<ActT>;
  const int tok_blocks = (T + kRowThreads / 64 - 1) / (kRowThreads / 64);
  if ((int)blockIdx.x >= tok_blocks) {  // the blocks past the tokens: dropped slots
    gate_dropped_block(x, dsel, topk_idx, offsets, row_token, dw_gate, db_gate, T * k, d, E, k,
                       blockIdx.x - tok_blocks);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[MOE_MAX_TOPK], idx[MOE_MAX_TOPK];
  float ds[MOE_MAX_TOPK];
  {
    int r = -1, e = 0;
    float v = 0.f;
    if (lane < k) {
      r = slot_row[(size_t)t * k + lane];
      e = topk_idx[(size_t)t * k + lane];
      v = dsel[(size_t)t * k + lane];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      rows[j] = lane_value(r, j);
      idx[j] = lane_value(e, j);
      ds[j] = lane_value(v, j);
    }
  }
  for (int c = lane * CK::N; c < d; c += 64 * CK::N) {
    float acc[CK::N];
#pragma unroll
    for (int i = 0; i < CK::N; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && rows[j] >= 0) {
        float v[CK::N];
        CK::load(dx_perm + (size_t)rows[j] * d + c, v);
#pragma unroll
        for (int i = 0; i < CK::N; ++i) acc[i] += v[i];
      }
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && (unsigned)idx[j] < (unsigned)E) {
        const float* wr = wt + (size_t)idx[j] * d + c;
#pragma unroll
        for (int i = 0; i < CK::N; ++i) acc[i] = fmaf(ds[j], wr[i], acc[i]);
      }
    }
    CK::store(dx + (size_t)t * d + c, acc);
  }
}

// Gate weight gradient over packed rows (float32 path; the bf16 path folds
// this product into FC1's weight-gradient GEMM):
//   dW_gate[i, e] = sum over e's rows r of dsel_perm[r] * x_perm[r, i],
//   db[e] = sum over e's rows of dsel_perm[r].
// One thread per column walks the rows in order.
template <typename ActT>
__global__ void __launch_bounds__(64)
gate_rows_kernel(const ActT* __restrict__ x_perm, const float* __restrict__ dsel_perm,
                 const int32_t* __restrict__ offsets, float* __restrict__ dw_gate,
                 float* __restrict__ db_gate, int d, int E) {
  const int e = blockIdx.x;
  const int i = blockIdx.y * 64 + threadIdx.x;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  float acc = 0.f, db = 0.f;
  for (int r = r0; r < r1; ++r) {
    const float g = dsel_perm[r];
    db += g;
    if (i < d) acc = fmaf(g, to_f32(x_perm[(size_t)r * d + i]), acc);
  }
  if (i < d) dw_gate[(size_t)i * E + e] = acc;
  if (blockIdx.y == 0 && threadIdx.x == 0) db_gate[e] = db;
}

__global__ void popularity_kernel(int E, int window, int64_t iter,
                                  const int32_t* __restrict__ counts_raw,
                                  int32_t* __restrict__ ring, int32_t* __restrict__ window_sum) {
  const int slot = (int)(iter % window);
  const int n = (int)((iter + 1 < (int64_t)window) ? iter + 1 : window);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int c = counts_raw[e];
    ring[(size_t)slot * E + e] = c;
    int s = c;
    for (int b = 1; b < n; ++b) s += ring[(size_t)((slot - b + window) % window) * E + e];
    window_sum[e] = s;
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_combine(int act, const void* out_perm, const float* topk_w,
                          const int32_t* slot_row, void* y, int T, int d, int k, hipStream_t s,
                          bool slot_order) {
  dim3 grid((T + 3) / 4), block(kRowThreads);
  if (act == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, block, 0, s, (const bf16*)out_perm, topk_w,
                       slot_row, (bf16*)y, T, d, k, slot_order);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, (const float*)out_perm, topk_w,
                       slot_row, (float*)y, T, d, k, slot_order);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int act, const void* dy, const void* out_perm,
                              const float* topk_w, const int32_t* topk_idx,
                              const int32_t* slot_row, void* d_out, float* dsel,
                              float* dsel_perm, float* dlogits, const float* w_gate,
                              float* w_gate_t, int32_t* counters, int T, int d, int E, int k,
                              hipStream_t s) {
  const int tok_blocks = (T + 3) / 4;
  const int tr_blocks = ((d + 31) / 32) * ((E + 31) / 32);
  dim3 grid(tok_blocks + tr_blocks), block(kRowThreads);
  if (act == MOE_BF16)
    hipLaunchKernelGGL(combine_bwd_kernel<bf16>, grid, block, 0, s, (const bf16*)dy,
                       (const bf16*)out_perm, topk_w, topk_idx, slot_row, (bf16*)d_out, dsel,
                       dsel_perm, dlogits, w_gate, w_gate_t, counters, T, d, E, k);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, grid, block, 0, s, (const float*)dy,
                       (const float*)out_perm, topk_w, topk_idx, slot_row, (float*)d_out, dsel,
                       dsel_perm, dlogits, w_gate, w_gate_t, counters, T, d, E, k);
  return hipGetLastError();
}

hipError_t launch_dx(int act, const void* dx_perm, const float* dsel, const int32_t* topk_idx,
                     const int32_t* slot_row, const float* w_gate_t, void* dx, int T, int d,
                     int k, bool dropped, const void* x, const int32_t* offsets,
                     const int32_t* row_token, float* dw_gate, float* db_gate, int E,
                     hipStream_t s) {
  const int tok_blocks = (T + 3) / 4;
  const int drop_blocks = dropped ? E * ((d + 255) / 256) : 0;
  dim3 grid(tok_blocks + drop_blocks), block(kRowThreads);
  if (act == MOE_BF16)
    hipLaunchKernelGGL(dx_kernel<bf16>, grid, block, 0, s, (const bf16*)dx_perm, dsel, topk_idx,
                       slot_row, w_gate_t, (bf16*)dx, T, d, k, (const bf16*)x, offsets,
                       row_token, dw_gate, db_gate, E);
  else
    hipLaunchKernelGGL(dx_kernel<float>, grid, block, 0, s, (const float*)dx_perm, dsel,
                       topk_idx, slot_row, w_gate_t, (float*)dx, T, d, k, (const float*)x,
                       offsets, row_token, dw_gate, db_gate, E);
  return hipGetLastError();
}

hipError_t launch_gate_rows(int act, const void* x_perm, const float* dsel_perm,
                            const int32_t* offsets, float* dw_gate, float* db_gate, int d, int E,
                            hipStream_t s) {
  dim3 grid(E, (d + 63) / 64), block(64);
  if (act == MOE_BF16)
    hipLaunchKernelGGL(gate_rows_kernel<bf16>, grid, block, 0, s, (const bf16*)x_perm, dsel_perm,
                       offsets, dw_gate, db_gate, d, E);
  else
    hipLaunchKernelGGL(gate_rows_kernel<float>, grid, block, 0, s, (const float*)x_perm,
                       dsel_perm, offsets, dw_gate, db_gate, d, E);
  return hipGetLastError();
}

hipError_t launch_popularity(int E, int window, int64_t iter, const int32_t* counts_raw,
                             int32_t* ring, int32_t* window_sum, hipStream_t s) {
  hipLaunchKernelGGL(popularity_kernel, dim3(1), dim3(256), 0, s, E, window, iter, counts_raw,
                     ring, window_sum);
  return hipGetLastError();
}

}  // namespace moe
