// Expert-parallel dispatch plan on gfx950: which copies of which experts run
// on which rank, from the per-expert packed-row counts.
//
// Fast MoE Inference via Predictive Prefetching and Expert Replication, main
// contributions 2 and 3: experts get physical copies by token demand, and the
// number of copies is capped by GPU memory.  MoE
// training optimisation: the LLEP algorithm and dynamic load balancing, §2.1:
// work goes to the least-loaded GPU.  A Survey on Mixture of Experts, §5
// System Design (first paragraph): the packed per-expert rows are what the
// All-to-All dispatch sends, so a copy's rows are one contiguous range.
//
// One workgroup: the copy counts by a wavefront-wide argmax per extra copy,
// the row split and a rank order of the copies in parallel, then the
// least-loaded placement with one rank per lane.  Everything is integer, so
// the plan is exact and deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPlanThreads = 256;

// (c_a / r_a, expert a) ranks before (c_b / r_b, expert b): more rows per
// copy, or equal and a lower index
__device__ __forceinline__ bool more_per_copy(int ca, int ra, int ea, int cb, int rb, int eb) {
  const long long l = (long long)ca * rb, r = (long long)cb * ra;
  return l > r || (l == r && ea < eb);
}

__global__ void __launch_bounds__(kPlanThreads)
ep_plan_kernel(int E, int R, int extra, const int32_t* __restrict__ offsets,
               int32_t* __restrict__ replica_start, int32_t* __restrict__ replica_row0,
               int32_t* __restrict__ replica_rows, int32_t* __restrict__ replica_rank,
               int32_t* __restrict__ rank_rows) {
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_rep[MOE_MAX_EXPERTS];
  __shared__ int s_start[MOE_MAX_EXPERTS + 1];
  __shared__ int s_rows[MOE_PLAN_MAX_COPIES];
  __shared__ int s_order[MOE_PLAN_MAX_COPIES];
  __shared__ int s_scratch[kPlanThreads / 64 + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e <= E; e += kPlanThreads) s_off[e] = offsets[e];
  __syncthreads();

  // 1. copies per expert: one wavefront, lane owns experts lane + 64 q
  if (tid < 64) {
    constexpr int Q = MOE_MAX_EXPERTS / 64;
    int c[Q], r[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + 64 * q;
      c[q] = e < E ? s_off[e + 1] - s_off[e] : 0;
      r[q] = 1;
    }
    for (int it = 0; it < extra; ++it) {
      int bc = 0, br = 1, be = 0x7fffffff;  // ranks after every expert
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        if (e < E && more_per_copy(c[q], r[q], e, bc, br, be)) {
          bc = c[q];
          br = r[q];
          be = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int oc = __shfl_xor(bc, o, 64), orr = __shfl_xor(br, o, 64),
                  oe = __shfl_xor(be, o, 64);
        if (more_per_copy(oc, orr, oe, bc, br, be)) {
          bc = oc;
          br = orr;
          be = oe;
        }
      }
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (lane + 64 * q == be) ++r[q];
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + 64 * q;
      if (e < E) s_rep[e] = r[q];
    }
  }
  __syncthreads();

  // 2. copy index ranges: exclusive prefix of the copy counts
  {
    int total;
    const int ex = block_exclusive_scan(tid < E ? s_rep[tid] : 0, s_scratch, &total);
    if (tid < E) s_start[tid] = ex;
    if (tid == 0) s_start[E] = total;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kPlanThreads) replica_start[e] = s_start[e];

  // 3. copy i of expert e: rows offsets[e] + [floor(i c / r), floor((i+1) c / r))
  for (int e = tid; e < E; e += kPlanThreads) {
    const long long c = s_off[e + 1] - s_off[e];
    const int rr = s_rep[e];
    for (int i = 0; i < rr; ++i) {
      const int a = (int)((i * c) / rr), b = (int)(((i + 1) * c) / rr);
      const int p = s_start[e] + i;
      s_rows[p] = b - a;
      replica_row0[p] = s_off[e] + a;
      replica_rows[p] = b - a;
    }
  }
  __syncthreads();

  // 4. placement order: decreasing rows, ties by copy index
  const int P = s_start[E];
  for (int p = tid; p < P; p += kPlanThreads) {
    const int n = s_rows[p];
    int pos = 0;
    for (int q = 0; q < P; ++q) {
      const int m = s_rows[q];
      pos += (m > n) || (m == n && q < p);
    }
    s_order[pos] = p;
  }
  __syncthreads();

  // 5. least-loaded placement.  Up to 16 ranks: one lane, loads in
  // registers (a short scan per copy); more: lane = rank, wave argmin.
  if (R <= 16) {
    if (tid == 0) {
      int load[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) load[q] = 0;
      for (int j = 0; j < P; ++j) {
        const int p = s_order[j];
        int bq = 0, bl = load[0];
#pragma unroll
        for (int q = 1; q < 16; ++q)
          if (q < R && load[q] < bl) {
            bl = load[q];
            bq = q;
          }
        const int rows = s_rows[p];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (q == bq) load[q] += rows;
        replica_rank[p] = bq;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (q < R) rank_rows[q] = load[q];
    }
  } else if (tid < 64) {
    int load = lane < R ? 0 : 0x7fffffff;
    for (int j = 0; j < P; ++j) {
      const int p = s_order[j];
      int bl = load, bq = lane;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int ol = __shfl_xor(bl, o, 64), oq = __shfl_xor(bq, o, 64);
        if (ol < bl || (ol == bl && oq < bq)) {
          bl = ol;
          bq = oq;
        }
      }
      if (lane == bq) load += s_rows[p];
      if (lane == 0) replica_rank[p] = bq;
    }
    if (lane < R) rank_rows[lane] = load;
  }
}

hipError_t launch_ep_plan(int E, int R, int extra, const int32_t* offsets,
                          int32_t* replica_start, int32_t* replica_row0, int32_t* replica_rows,
                          int32_t* replica_rank, int32_t* rank_rows, hipStream_t s) {
  hipLaunchKernelGGL(ep_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, E, R, extra, offsets,
                     replica_start, replica_row0, replica_rows, replica_rank, rank_rows);
  return hipGetLastError();
}

// All-to-All split sizes of a dispatch (A Survey on Mixture of Experts, §5
// System Design, first paragraph: the packed per-expert rows are what the
// All-to-All sends).  Segment i (an expert's packed rows, or a copy's share
// of them) holds seg_rows[i] rows for rank seg_rank[i]; the send buffer holds
// rank 0's rows, then rank 1's, ..., segments of one rank in index order.
// One wavefront, lane r owning rank r: it walks the segments in order (their
// rows and ranks staged in LDS) and gives each of its own the running row
// count; a wavefront scan of the per-rank totals gives the rank offsets.  A
// segment whose rank is outside [0, R) is in no count and gets offset -1.
__global__ void __launch_bounds__(64)
dispatch_layout_kernel(int n, int R, const int32_t* __restrict__ seg_rows,
                       const int32_t* __restrict__ seg_rank, int32_t* __restrict__ send_counts,
                       int32_t* __restrict__ send_offsets, int32_t* __restrict__ seg_send_offset) {
  __shared__ int s_rows[MOE_PLAN_MAX_COPIES];
  __shared__ int s_rank[MOE_PLAN_MAX_COPIES];
  __shared__ int s_local[MOE_PLAN_MAX_COPIES];
  __shared__ int s_base[MOE_PLAN_MAX_RANKS];
  const int lane = threadIdx.x;
  for (int i = lane; i < n; i += 64) {
    s_rows[i] = seg_rows[i];
    s_rank[i] = seg_rank[i];
  }
  __syncthreads();
  int run = 0;
  for (int i = 0; i < n; ++i) {
    if (s_rank[i] == lane) {
      s_local[i] = run;
      run += s_rows[i];
    }
  }
  // exclusive scan of the per-rank totals (lanes >= R hold nothing)
  const int total_r = lane < R ? run : 0;
  int incl = total_r;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const int base = incl - total_r;
  if (lane < R) {
    send_counts[lane] = total_r;
    send_offsets[lane] = base;
    s_base[lane] = base;
  }
  if (lane == 63) send_offsets[R] = incl;
  __syncthreads();
  for (int i = lane; i < n; i += 64) {
    const int r = s_rank[i];
    seg_send_offset[i] = (r >= 0 && r < R) ? s_base[r] + s_local[i] : -1;
  }
}

hipError_t launch_dispatch_layout(int n, int R, const int32_t* seg_rows, const int32_t* seg_rank,
                                  int32_t* send_counts, int32_t* send_offsets,
                                  int32_t* seg_send_offset, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_layout_kernel, dim3(1), dim3(64), 0, s, n, R, seg_rows, seg_rank,
                     send_counts, send_offsets, seg_send_offset);
  return hipGetLastError();
}

}  // namespace moe
