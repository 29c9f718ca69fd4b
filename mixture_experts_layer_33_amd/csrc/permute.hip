// Input encode on gfx950: per-expert histogram, exclusive scan, stable
// permutation into contiguous per-expert rows, and the row gather.
//
// A Survey on Mixture of Experts, §5 System Design (first paragraph): input
// encode gathers the tokens of one expert into contiguous memory from the
// gate's token-to-expert map, so each expert's GEMM sees one dense block; the
// expert capacity limit of GShard (cited there, and in the PopFetcher notes
// §2.2) drops the slots beyond an expert's capacity.
//
// Three kernels, no host round trip:
// Slots are ranked in capacity-priority order: position q of the walk is slot
// s(q) = q (slot order) or (q % T) * k + q / T (choice-major: all first
// choices, then all second choices, ...); ranks and tiles are over q.
//
//  1. rank_hist: tiles of kRankTile positions.  Each 64-slot wavefront finds, for
//     every lane, the lower lanes routed to the same expert with ceil(log2)
//     ballots over the expert id bits (warp-level multisplit), which gives the
//     stable rank inside the wavefront; LDS counters carry the rank across
//     the tile's wavefronts and rounds.  Output: the rank of each slot inside
//     its tile and the tile histogram hist[e][tile].
//  2. scan: one workgroup per expert scans hist[e][*] over tiles, giving each
//     tile's base position within the expert, the raw count and the kept
//     count min(raw, C).
//  3. gather: offsets = exclusive scan of the kept counts; a slot's position
//     in its expert is tile base + in-tile rank; it is kept iff that
//     position is below C.  One wavefront per token reads the token's row
//     once and writes it to each of its kept rows with 16-byte accesses.
//     Dropped slots are listed after the kept rows, ordered by expert and
//     then position: row_token[S_kept + j] = slot index (the backward needs
//     them for the gate gradient).
//  3'. index (the gather-fused forward): the same indices with one thread per
//     slot and no row copy, plus row_slot[r] = the slot of kept row r; the
//     expert GEMM then reads token rows through row_token itself.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRankThreads = 256;

__global__ void __launch_bounds__(kRankThreads)
rank_hist_kernel(const int32_t* __restrict__ topk_idx, int T, int k, bool choice, int E,
                 int32_t* __restrict__ local_rank, int32_t* __restrict__ hist, int n_tiles) {
  const int S = T * k;
  __shared__ int running[MOE_MAX_EXPERTS + 1];
  __shared__ int wcnt[kRankThreads / 64][MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i <= E; i += kRankThreads) {
    running[i] = 0;
    for (int w = 0; w < kRankThreads / 64; ++w) wcnt[w][i] = 0;
  }
  __syncthreads();
  // bits needed to tell buckets 0..E apart (bucket E = slot past the end)
  const int nbits = 32 - __clz(E);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int tile = blockIdx.x;
  for (int r = 0; r < kRankTile / kRankThreads; ++r) {
    const int q = tile * kRankTile + r * kRankThreads + tid;
    const bool valid = q < S;
    const int s = choice ? (q % T) * k + q / T : q;
    // bucket E: past the end, or an expert id outside [0, E) (not counted)
    int e = valid ? topk_idx[s] : E;
    if ((unsigned)e > (unsigned)E) e = E;
    uint64_t m = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank_w = __popcll(m & lt_mask);
    if (rank_w == 0) wcnt[wid][e] = __popcll(m);
    __syncthreads();
    int rank = running[e] + rank_w;
    for (int w = 0; w < wid; ++w) rank += wcnt[w][e];
    if (valid) local_rank[q] = rank;
    __syncthreads();
    for (int i = tid; i <= E; i += kRankThreads) {
      int add = 0;
      for (int w = 0; w < kRankThreads / 64; ++w) {
        add += wcnt[w][i];
        wcnt[w][i] = 0;
      }
      running[i] += add;
    }
    __syncthreads();
  }
  for (int i = tid; i < E; i += kRankThreads) hist[(size_t)i * n_tiles + tile] = running[i];
}

constexpr int kScanThreads = 256;

__global__ void __launch_bounds__(kScanThreads)
scan_kernel(const int32_t* __restrict__ hist, int n_tiles, int E, int C,
            int32_t* __restrict__ tile_base, int32_t* __restrict__ counts_raw,
            int32_t* __restrict__ counts_kept) {
  __shared__ int scratch[kScanThreads / 64 + 1];
  const int e = blockIdx.x;
  const int32_t* h = hist + (size_t)e * n_tiles;
  int32_t* tb = tile_base + (size_t)e * n_tiles;
  int carry = 0;
  for (int b0 = 0; b0 < n_tiles; b0 += kScanThreads) {
    const int b = b0 + threadIdx.x;
    const int v = (b < n_tiles) ? h[b] : 0;
    int total;
    const int ex = block_exclusive_scan(v, scratch, &total);
    if (b < n_tiles) tb[b] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) {
    if (counts_raw) counts_raw[e] = carry;
    counts_kept[e] = carry < C ? carry : C;
  }
}

constexpr int kGatherThreads = 256;

template <typename ActT>
__global__ void __launch_bounds__(kGatherThreads)
gather_kernel(const ActT* __restrict__ x, const int32_t* __restrict__ topk_idx,
              const int32_t* __restrict__ local_rank, const int32_t* __restrict__ tile_base,
              const int32_t* __restrict__ counts_raw, const int32_t* __restrict__ counts_kept,
              int n_tiles, int T, int d, int E, int k, int C, bool choice,
              int32_t* __restrict__ offsets,
              int32_t* __restrict__ slot_row, int32_t* __restrict__ row_token,
              ActT* __restrict__ x_perm) {
  __shared__ int off[MOE_MAX_EXPERTS + 1];
  __shared__ int doff[MOE_MAX_EXPERTS + 1];
  __shared__ int scratch[kGatherThreads / 64 + 1];
  {
    const int e = threadIdx.x;
    const int kept = (e < E) ? counts_kept[e] : 0;
    const int drop = (e < E) ? counts_raw[e] - kept : 0;
    int total, dtotal;
    const int ex = block_exclusive_scan(kept, scratch, &total);
    const int dex = block_exclusive_scan(drop, scratch, &dtotal);
    if (e < E) {
      off[e] = ex;
      doff[e] = total + dex;  // dropped slots are listed after the kept rows
    }
    if (e == 0) off[E] = total;
    __syncthreads();
    if (blockIdx.x == 0) {
      if (e < E) offsets[e] = ex;
      if (e == 0) offsets[E] = total;
    }
  }
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kGatherThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_row = -1;
  if (lane < k) {
    const int s = t * k + lane;
    const int q = choice ? lane * T + t : s;  // position in the capacity walk
    const int e = topk_idx[s];
    if ((unsigned)e < (unsigned)E) {  // an id outside [0, E) stays unrouted
      const int pos = tile_base[(size_t)e * n_tiles + q / kRankTile] + local_rank[q];
      if (pos < C) {
        my_row = off[e] + pos;
        row_token[my_row] = t;
      } else {
        row_token[doff[e] + pos - C] = s;
      }
    }
    slot_row[s] = my_row;
  }
  int rows[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) rows[j] = lane_value(my_row, j);
  // 16-byte chunks of the row
  const int nchunk = d * (int)sizeof(ActT) / 16;
  const i32x4* src = reinterpret_cast<const i32x4*>(x + (size_t)t * d);
  for (int c = lane; c < nchunk; c += 64) {
    const i32x4 v = src[c];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && rows[j] >= 0)
        reinterpret_cast<i32x4*>(x_perm + (size_t)rows[j] * d)[c] = v;
    }
  }
}

hipError_t launch_rank_hist(const int32_t* topk_idx, int T, int k, bool choice, int E,
                            int32_t* local_rank, int32_t* hist, int n_tiles, hipStream_t s) {
  hipLaunchKernelGGL(rank_hist_kernel, dim3(n_tiles), dim3(kRankThreads), 0, s, topk_idx, T, k,
                     choice, E, local_rank, hist, n_tiles);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* hist, int n_tiles, int E, int C, int32_t* tile_base,
                       int32_t* counts_raw, int32_t* counts_kept, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(E), dim3(kScanThreads), 0, s, hist, n_tiles, E, C,
                     tile_base, counts_raw, counts_kept);
  return hipGetLastError();
}

// Index-only encode: offsets, slot_row, row_token (kept rows, then the
// dropped-slot list) and row_slot, one thread per slot.
__global__ void __launch_bounds__(kGatherThreads)
index_kernel(const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ local_rank,
             const int32_t* __restrict__ tile_base, const int32_t* __restrict__ counts_raw,
             const int32_t* __restrict__ counts_kept, int n_tiles, int T, int E, int k, int C,
             bool choice, int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row,
             int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot) {
  __shared__ int off[MOE_MAX_EXPERTS + 1];
  __shared__ int doff[MOE_MAX_EXPERTS + 1];
  __shared__ int scratch[kGatherThreads / 64 + 1];
  {
    const int e = threadIdx.x;
    const int kept = (e < E) ? counts_kept[e] : 0;
    const int drop = (e < E) ? counts_raw[e] - kept : 0;
    int total, dtotal;
    const int ex = block_exclusive_scan(kept, scratch, &total);
    const int dex = block_exclusive_scan(drop, scratch, &dtotal);
    if (e < E) {
      off[e] = ex;
      doff[e] = total + dex;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
      if (e < E) offsets[e] = ex;
      if (e == 0) offsets[E] = total;
    }
  }
  const long long s = (long long)blockIdx.x * kGatherThreads + threadIdx.x;
  if (s >= (long long)T * k) return;
  const int t = (int)(s / k), j = (int)(s - (long long)t * k);
  const int q = choice ? j * T + t : (int)s;
  const int e = topk_idx[s];
  int row = -1;
  if ((unsigned)e < (unsigned)E) {  // an id outside [0, E) stays unrouted
    const int pos = tile_base[(size_t)e * n_tiles + q / kRankTile] + local_rank[q];
    if (pos < C) {
      row = off[e] + pos;
      row_token[row] = t;
      row_slot[row] = (int)s;
    } else {
      row_token[doff[e] + pos - C] = (int)s;
    }
  }
  slot_row[s] = row;
}

hipError_t launch_index(const int32_t* topk_idx, const int32_t* local_rank,
                        const int32_t* tile_base, const int32_t* counts_raw,
                        const int32_t* counts_kept, int n_tiles, int T, int E, int k, int C,
                        bool choice, int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                        int32_t* row_slot, hipStream_t s) {
  const long long S = (long long)T * k;
  dim3 grid((unsigned)((S + kGatherThreads - 1) / kGatherThreads)), block(kGatherThreads);
  hipLaunchKernelGGL(index_kernel, grid, block, 0, s, topk_idx, local_rank, tile_base,
                     counts_raw, counts_kept, n_tiles, T, E, k, C, choice, offsets, slot_row,
                     row_token, row_slot);
  return hipGetLastError();
}

hipError_t launch_gather(int act, const void* x, const int32_t* topk_idx,
                         const int32_t* local_rank, const int32_t* tile_base,
                         const int32_t* counts_raw, const int32_t* counts_kept, int n_tiles,
                         int T, int d, int E, int k, int C, bool choice, int32_t* offsets,
                         int32_t* slot_row, int32_t* row_token, void* x_perm, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(kGatherThreads);
  if (act == MOE_BF16)
    hipLaunchKernelGGL(gather_kernel<bf16>, grid, block, 0, s, (const bf16*)x, topk_idx,
                       local_rank, tile_base, counts_raw, counts_kept, n_tiles, T, d, E, k, C,
                       choice, offsets, slot_row, row_token, (bf16*)x_perm);
  else
    hipLaunchKernelGGL(gather_kernel<float>, grid, block, 0, s, (const float*)x, topk_idx,
                       local_rank, tile_base, counts_raw, counts_kept, n_tiles, T, d, E, k, C,
                       choice, offsets, slot_row, row_token, (float*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
