// Expert FFN as grouped GEMMs on gfx950 MFMA (bf16 in, float32 accumulate).
//
// PopFetcher notes §2.1.1 and §5.1: each expert is FC -> ReLU -> FC with an
// H x aH and an aH x H matrix; §5.2.1: one GEMM pass forward and two backward
// (input gradient and weight gradient) per FC.  A Survey on Mixture of
// Experts, §5.1 (Computation): the layer waits for the most loaded expert, so
// skewed token counts must not leave the matrix cores idle.
//
// Weights are [E, out, in].  Five products share one kernel template:
//   forward   h  = ReLU(x_perm_e W1[e]^T)      A [rows][d]  B [F][d]   (NT)
//             O  = h_e W2[e]^T                 A [rows][F]  B [d][F]   (NT)
//   dgrad     dz = (dO_e W2[e]) * [h_e > 0]    A [rows][d]  B [d][F]   (NN)
//             dx = dz_e W1[e]                  A [rows][F]  B [F][d]   (NN)
//   wgrad     dW2[e] = dO_e^T h_e              A [rows][d]  B [rows][F] (TN)
//             dW1[e] = dz_e^T x_perm_e         A [rows][F]  B [rows][d] (TN)
// Both operands always reach LDS as [row][64 k] bf16 tiles (16-byte chunks
// XOR-swizzled by row) so every MFMA fragment is one 16-byte LDS read;
// operands that are contiguous along M or N in memory are transposed in
// registers on their way to LDS (8 consecutive k of one row per chunk).
//
// Scheduling: forward and dgrad tiles cover each expert's packed rows; the
// tile list is built inside the kernel from the device offsets (no host
// sync), grouped along M for operand reuse and laid out so each XCD (one L2)
// gets a contiguous range.  wgrad tiles are ordered hottest expert first so
// the long K loops of popular experts start early (longest-processing-time
// first); experts with no rows store zeros.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kBK = 64;          // k per LDS stage
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round robin

enum Epi { EPI_RELU = 0, EPI_STORE = 1, EPI_MASK = 2, EPI_F32 = 3 };

// 16-byte chunk kc of LDS row `row` (rows of 64 bf16 = 8 chunks).  The XOR
// uses row bits 0-2, 3-5 and 6-8 so that both 8 consecutive rows (MFMA
// fragment reads) and rows 8 apart (transposed stores) spread over banks.
__device__ __forceinline__ int swz(int row, int kc) {
  return (row * 8 + (kc ^ ((row ^ (row >> 3) ^ (row >> 6)) & 7))) * 8;
}

// ---------------------------------------------------------------------------
// Operand tiles, copied global -> LDS directly (global_load_lds_dwordx4: the
// 16 bytes of lane L land at the wave's LDS base + 16 L; one wave instruction
// fills 1 KiB).  Each lane fetches whichever global chunk the LDS swizzle
// puts at its position.
//
// K-contiguous operand (element (r, k) at base[r * ld + k]): LDS [ROWS][64],
// 16-byte chunk kc of row r at position kc ^ f(r); read back as one 16-byte
// fragment per lane.  Rows >= nrows re-read row nrows-1 (never stored).
template <int ROWS>
struct TileK {
  static constexpr int N = ROWS / 32;  // wave instructions per thread per stage
  uint32_t off[N];                     // byte offsets from the stage base
  __device__ void init(int ld, int nrows) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int row = (i * 4 + wid) * 8 + (lane >> 3), p = lane & 7;
      const int kc = p ^ ((row ^ (row >> 3) ^ (row >> 6)) & 7);
      off[i] = (uint32_t)(((size_t)min(row, nrows - 1) * ld + kc * 8) * sizeof(bf16));
    }
  }
  // stage with k in [k0, k0 + 64)
  __device__ void issue(const bf16* base, int ld, int k0, int, bf16* lds) const {
    const int wid = threadIdx.x >> 6;
    const char* b = reinterpret_cast<const char*>(base + k0);
#pragma unroll
    for (int i = 0; i < N; ++i)
      __builtin_amdgcn_global_load_lds(
          b + off[i], (__attribute__((address_space(3))) void*)(lds + (i * 4 + wid) * 8 * kBK),
          16, 0, 0);
  }
  // 32 x 16 MFMA operand block at rows r0..r0+31, k = kk*16 ..: lane l holds
  // row r0 + l%32, the 8 consecutive k from kk*16 + 8*(l/32)
  __device__ static bf16x8 frag(const bf16* lds, int r0, int kk) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x8*>(lds + swz(r0 + (lane & 31), kk * 2 + (lane >> 5)));
  }
};

// MN-contiguous operand (element (r, k) at base[k * ld + r]): LDS [64][ROWS]
// as in memory, 16-byte chunk c of k-row k at position c ^ sw(k), read back
// transposed by ds_read_b64_tr_b16.  Within each 16-lane group that
// instruction hands lane i the elements M[4j + i/4][i%4] (j = 0..3) of the
// 4-element pieces M[r] addressed by the group's lanes r; addressing k-row
// kb + r/4, columns c0 + 4 (r%4) gives lane i four consecutive k of column
// c0 + i.  Two reads give the 8 k of a fragment, in the same k order as the
// K-contiguous fragments.  k rows >= kmax re-read row kmax-1 (zeroed in the
// fragment where it matters); columns >= ncols re-read valid columns.
template <int ROWS>
struct TileMN {
  static constexpr int R = ROWS * 2;          // bytes per k-row
  static constexpr int CPR = R / 16;          // chunks per k-row
  static constexpr int RPI = 1024 / R;        // k-rows per wave instruction
  static constexpr int N = 64 / RPI / 4;      // wave instructions per thread per stage
  __device__ static int sw(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }
  int kl[N];       // k-row of this lane's chunk, within the stage
  uint32_t col[N]; // byte offset of its column chunk
  __device__ void init(int ld, int ncols) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = (i * 4 + wid) * RPI + lane / CPR, p = lane % CPR;
      const int c = min(p ^ sw(k), ncols / 8 - 1);
      kl[i] = k;
      col[i] = (uint32_t)(c * 8 * sizeof(bf16));
    }
  }
  __device__ void issue(const bf16* base, int ld, int k0, int kmax, bf16* lds) const {
    const int wid = threadIdx.x >> 6;
    const char* b = reinterpret_cast<const char*>(base + (size_t)k0 * ld);
    const int kend = kmax - k0;  // rows of this stage that exist
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = min(kl[i], kend - 1);
      __builtin_amdgcn_global_load_lds(
          b + (uint32_t)(k * ld * (int)sizeof(bf16)) + col[i],
          (__attribute__((address_space(3))) void*)(lds + (i * 4 + wid) * RPI * ROWS), 16, 0, 0);
    }
  }
  // Same operand block from the transposed layout: 16-lane group G = l/16
  // covers columns r0 + 16*(G&1) .. +15 and k from kk*16 + 8*(G>>1); two
  // transposed reads of 4 k each.
  __device__ static bf16x8 frag(const bf16* lds, int r0, int kk) {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    typedef __attribute__((ext_vector_type(2))) int i32x2;
    const int lane = threadIdx.x & 63, G = lane >> 4, r = lane & 15;
    const int n = r0 + 16 * (G & 1) + 4 * (r & 3);
    i32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = kk * 16 + 8 * (G >> 1) + h * 4 + (r >> 2);
      const int byte = k * R + (((n >> 3) ^ sw(k)) << 4) + (((n >> 2) & 1) << 3);
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((const char*)lds + byte));
      // reinterpret all 8 bytes at once (element-wise casts of this result
      // have been seen to be lowered wrongly)
      const i32x2 w = __builtin_bit_cast(i32x2, v);
      out[2 * h] = w[0];
      out[2 * h + 1] = w[1];
    }
    return __builtin_bit_cast(bf16x8, out);
  }
  // zero fragment entries whose k (stage-relative) is >= kend
  __device__ static void mask_k(bf16x8& f, int kk, int kend) {
    const int k0 = kk * 16 + ((threadIdx.x & 63) >> 5) * 8;
    i32x4 w = __builtin_bit_cast(i32x4, f);  // element 2q = low half of dword q
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned keep = (k0 + 2 * q < kend ? 0x0000ffffu : 0u) |
                            (k0 + 2 * q + 1 < kend ? 0xffff0000u : 0u);
      w[q] = (int)((unsigned)w[q] & keep);
    }
    f = __builtin_bit_cast(bf16x8, w);
  }
  // 16 bytes (8 columns) of k-row k at column chunk c, for the gate product
  __device__ static bf16x8 chunk(const bf16* lds, int k, int c) {
    return *reinterpret_cast<const bf16x8*>((const char*)lds + k * R + ((c ^ sw(k)) << 4));
  }
};

template <bool KMAJOR, int ROWS>
struct Tile;
template <int ROWS>
struct Tile<true, ROWS> : TileK<ROWS> {};
template <int ROWS>
struct Tile<false, ROWS> : TileMN<ROWS> {};

// ---------------------------------------------------------------------------
// One output tile: C[BM x BN] = sum_k A(m, k) B(n, k), k in [0, K), on 4
// wavefronts in a 2 x 2 grid, each owning a (BM/2) x (BN/2) block of 32 x 32
// MFMA blocks (v_mfma_f32_32x32x16_bf16: twice the work per issue of the
// 16 x 16 x 32 form, which measured at about 60% of its rate here).  The
// MFMA takes the B tile as its first operand and the A tile as its second,
// so each result block is C^T: lane l holds C[m][n..n+3] with m = l % 32 and
// n = 4 * (l / 32) + 8p, four consecutive columns of one row, which the
// epilogue writes as one 8- or 16-byte store.
//
// Pipeline: three LDS stages, one barrier per 64-deep k step; stage kt+2 is
// in flight while stage kt is computed, and before the barrier each wave
// waits only for its loads of stage kt+1 (vmcnt = one stage's count).
//
// With GATE (B MN-contiguous) and a non-null `gsel`, the tile also forms
// g[n] = sum_k gsel[k] B(n, k) for its columns from the LDS stages (gacc: per
// thread, 8 columns over its share of the rows) and sum_k gsel[k] (gdb);
// see gate_reduce().
template <int BM, int BN, bool A_K, bool B_K, bool GATE = false>
struct TileGemm {
  static constexpr int WM = BM / 2, WN = BN / 2;  // 2 x 2 waves
  static constexpr int FM = WM / 32, FN = WN / 32;  // 32 x 32 MFMA blocks per wave
  static constexpr size_t kStageBytes = (size_t)(BM + BN) * kBK * sizeof(bf16);
  // three stages when they fit in LDS (next to ~2 KiB of scheduler state),
  // else two
  static constexpr int kStages = 3 * kStageBytes <= 152 * 1024 ? 3 : 2;
  static constexpr int kStageOps = Tile<A_K, BM>::N + Tile<B_K, BN>::N;
  static constexpr size_t kLdsPipe = (size_t)kStages * kStageBytes;
  f32x16 acc[FN][FM];  // acc[i][j]: n-block i, m-block j
  float gacc[8];
  float gdb;

  __device__ void run(const bf16* A, int lda, int a_rows, const bf16* B, int ldb, int b_rows,
                      int K, bf16* lds, const float* gsel = nullptr) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};
    if constexpr (GATE) {
#pragma unroll
      for (int m = 0; m < 8; ++m) gacc[m] = 0.f;
      gdb = 0.f;
    }
    const int nk = (K + kBK - 1) / kBK;
    if (nk == 0) return;
    bf16* const a_lds = lds;                          // [3][BM * 64]
    bf16* const b_lds = lds + kStages * BM * kBK;     // [3][BN * 64]
    Tile<A_K, BM> ta;
    Tile<B_K, BN> tb;
    ta.init(lda, a_rows);
    tb.init(ldb, b_rows);
    auto issue = [&](int kt) {
      const int s = kt % kStages;
      ta.issue(A, lda, kt * kBK, K, a_lds + s * (BM * kBK));
      tb.issue(B, ldb, kt * kBK, K, b_lds + s * (BN * kBK));
    };
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    constexpr int kGateRows = GATE ? kBK * (BN / 8) / kGemmThreads : 1;
    float gv[kGateRows];
    auto compute = [&](int kt) {
      const int s = kt % kStages;
      const bf16* as = a_lds + s * (BM * kBK);
      const bf16* bs = b_lds + s * (BN * kBK);
      const int kend = K - kt * kBK;  // < 64 only on a ragged last step
      // all A and B fragments of one 16-deep k slice
      auto load = [&](int kk, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int r0 = wm * WM + j * 32;
          if constexpr (A_K) {
            a[j] = TileK<BM>::frag(as, r0, kk);
          } else {
            a[j] = TileMN<BM>::frag(as, r0, kk);
            if (kend < kBK) TileMN<BM>::mask_k(a[j], kk, kend);
          }
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int r0 = wn * WN + i * 32;
          if constexpr (B_K)
            b[i] = TileK<BN>::frag(bs, r0, kk);
          else
            b[i] = TileMN<BN>::frag(bs, r0, kk);
        }
      };
      auto mma = [&](const bf16x8 (&a)[FM], const bf16x8 (&b)[FN]) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[i], a[j], acc[i][j], 0, 0, 0);
      };
      // software pipeline: slice kk+1's fragments load while slice kk's
      // MFMAs run (two register sets, alternating)
      // (scheduling barriers keep the compiler from sinking each load next
      // to its first use, which exposes the LDS latency every 4 MFMAs)
      bf16x8 a0[FM], b0[FN], a1[FM], b1[FN];
      load(0, a0, b0);
      load(1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mma(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      load(2, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      load(3, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mma(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma(a1, b1);
      if constexpr (GATE) {
        if (gsel != nullptr) {
          // thread: 8 columns (chunk c) of rows kg*kGateRows .. of this stage
          const int c = threadIdx.x % (BN / 8), kg = threadIdx.x / (BN / 8);
#pragma unroll
          for (int q = 0; q < kGateRows; ++q) {
            const int k = kg * kGateRows + q;
            const float g = gv[q];
            const bf16x8 v = TileMN<BN>::chunk(bs, k, c);
            gdb += g;
#pragma unroll
            for (int m = 0; m < 8; ++m) gacc[m] = fmaf(g, (float)v[m], gacc[m]);
          }
        }
      }
    };
    // gate weights of stage kt's rows for this thread (loaded before the
    // stage kt+2 copies are issued, so waiting for them never waits for those)
    auto load_gate = [&](int kt) {
      if constexpr (GATE) {
        if (gsel != nullptr) {
          const int kg = threadIdx.x / (BN / 8);
#pragma unroll
          for (int q = 0; q < kGateRows; ++q) {
            const int k = kt * kBK + kg * kGateRows + q;
            gv[q] = (k < K) ? gsel[k] : 0.f;
          }
        }
      }
    };
    // stages 0 .. kStages-2 in flight before the loop; step kt issues stage
    // kt + kStages - 1 and, before its barrier, waits for stage kt+1 (with
    // three stages the one issued this step may stay in flight)
    issue(0);
    if (kStages == 3 && nk > 1) {
      issue(1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStageOps) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool ahead = kt + kStages - 1 < nk;
      load_gate(kt);
      if (ahead) issue(kt + kStages - 1);
      compute(kt);
      if (kStages == 3 && ahead)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStageOps) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

  // Sum the per-thread gate partials over the row groups (fixed order) and
  // write out[n * out_stride] = g[n] for n < cols, and *db_out (if non-null).
  // Uses the first LDS bytes; call after run() (which ends with a barrier).
  __device__ void gate_reduce(float* red, int cols, float* out, int out_stride,
                              float* db_out) const {
    constexpr int RB = BN / 8, G = kGemmThreads / RB;
    const int rb = threadIdx.x % RB, kb = threadIdx.x / RB;
#pragma unroll
    for (int m = 0; m < 8; ++m) red[kb * BN + rb * 8 + m] = gacc[m];
    if (rb == 0) red[G * BN + kb] = gdb;
    __syncthreads();
    for (int n = threadIdx.x; n < cols; n += kGemmThreads) {
      float sum = 0.f;
      for (int g = 0; g < G; ++g) sum += red[g * BN + n];
      out[(size_t)n * out_stride] = sum;
    }
    if (db_out != nullptr && threadIdx.x == 0) {
      float sum = 0.f;
      for (int g = 0; g < G; ++g) sum += red[G * BN + g];
      *db_out = sum;
    }
  }
};
// Epilogue: in each 32 x 32 block lane l holds C[m][n..n+3] for m = l%32 and
// n = 4*(l/32) + 8p (p = 0..3) (see TileGemm).  rows/cols bound the valid
// part of the tile (cols is a multiple of 4).
template <int EPI, class TG>
__device__ __forceinline__ void store_tile(const TG& tg, void* C, int ldc, int rows, int cols,
                                           const bf16* aux, int ld_aux) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
#pragma unroll
  for (int j = 0; j < TG::FM; ++j) {
    const int m = wm * TG::WM + j * 32 + (lane & 31);
    if (m >= rows) continue;
#pragma unroll
    for (int i = 0; i < TG::FN; ++i) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int n = wn * TG::WN + i * 32 + 4 * (lane >> 5) + 8 * p;
        if (n >= cols) continue;
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = tg.acc[i][j][4 * p + q];
        if constexpr (EPI == EPI_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(C) + (size_t)m * ldc + n) = v;
        } else {
          if constexpr (EPI == EPI_RELU) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = fmaxf(v[q], 0.f);
          }
          if constexpr (EPI == EPI_MASK) {
            const bf16x4 hv = *reinterpret_cast<const bf16x4*>(aux + (size_t)m * ld_aux + n);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (!((float)hv[q] > 0.f)) v[q] = 0.f;
          }
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = (bf16)v[q];
          *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(C) + (size_t)m * ldc + n) = o;
        }
      }
      // keep the scheduler from hoisting every accumulator read to the top
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// Row-grouped GEMM (forward and dgrad): for every expert e, rows
// offsets[e]..offsets[e+1] of A times expert e's weight matrix.
struct RowsArgs {
  const bf16* A;        // [rows][K]
  const bf16* B;        // per expert: [N][K] (B_K) or [K][N]; expert stride b_stride
  bf16* C;              // [rows][N]
  const bf16* aux;      // mask source for EPI_MASK, [rows][N]
  const int32_t* offsets;
  long long b_stride;
  int K, N, E;
};

template <int BM, int BN, bool B_K, int EPI>
__global__ void __launch_bounds__(kGemmThreads)
rows_gemm_kernel(RowsArgs p) {
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_tstart[MOE_MAX_EXPERTS + 1];
  __shared__ int s_scratch[kGemmThreads / 64 + 1];
  __shared__ int s_expert;
  const int tid = threadIdx.x;
  // m-tiles per expert and their prefix sum
  {
    int mt = 0;
    if (tid < p.E) {
      const int a = p.offsets[tid], b = p.offsets[tid + 1];
      s_off[tid] = a;
      if (tid == p.E - 1) s_off[p.E] = b;
      mt = (b - a + BM - 1) / BM;
    }
    int total;
    const int ex = block_exclusive_scan(mt, s_scratch, &total);
    if (tid < p.E) s_tstart[tid] = ex;
    if (tid == 0) s_tstart[p.E] = total;
    __syncthreads();
  }
  const int MT = s_tstart[p.E];
  const int NT = (p.N + BN - 1) / BN;
  const int total = MT * NT;
  const int bid = blockIdx.x;
  if (bid >= total) return;
  // XCD-contiguous ranges: workgroup bid runs on XCD bid % 8.
  const int x = bid % kXcds, i = bid / kXcds;
  const int q = total / kXcds, rmd = total % kXcds;
  const int logical = x * q + min(x, rmd) + i;
  // group 8 m-tiles; walk n inside the group column by column
  constexpr int G = 8;
  const int grp = logical / (G * NT);
  const int gm0 = grp * G;
  const int gsz = min(G, MT - gm0);
  const int in = logical - grp * G * NT;
  const int mt = gm0 + in % gsz;
  const int nt = in / gsz;
  if (tid < p.E && s_tstart[tid] <= mt && mt < s_tstart[tid + 1]) s_expert = tid;
  __syncthreads();
  const int e = s_expert;
  const int row0 = s_off[e] + (mt - s_tstart[e]) * BM;
  const int rows = min(BM, s_off[e + 1] - row0);
  const int n0 = nt * BN;
  const int cols = min(BN, p.N - n0);

  TileGemm<BM, BN, true, B_K> tg;
  const bf16* A = p.A + (size_t)row0 * p.K;
  const bf16* Bm = p.B + (size_t)e * p.b_stride;
  if (B_K) {
    tg.run(A, p.K, rows, Bm + (size_t)n0 * p.K, p.K, cols, p.K, lds);
  } else {
    tg.run(A, p.K, rows, Bm + n0, p.N, cols, p.K, lds);
  }
  store_tile<EPI>(tg, p.C + (size_t)row0 * p.N + n0, p.N, rows, cols,
                  p.aux ? p.aux + (size_t)row0 * p.N + n0 : nullptr, p.N);
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM: dW[e] [N1][N2] = X1_e^T X2_e over expert e's rows.
struct WgradArgs {
  const bf16* X1;  // [rows][N1]
  const bf16* X2;  // [rows][N2]
  float* C;        // [E][N1][N2]
  const int32_t* offsets;
  // gate gradient (GATE only): gsel[r] per packed row; dW_gate [N2][E], db [E]
  const float* gsel;
  float* dw_gate;
  float* db_gate;
  int N1, N2, E;
};

// With GATE, the workgroups of the first N1 tile also produce the gate's
// weight gradient over the same rows, dW_gate[:, e] = X2_e^T gsel_e and
// db[e] = sum(gsel_e), from the X2 tiles they already stream (for FC1's
// weight gradient X2 is x_perm and gsel the gate-softmax gradient per row).
template <int BM, int BN, bool GATE>
__global__ void __launch_bounds__(kGemmThreads)
wgrad_kernel(WgradArgs p) {
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];
  __shared__ int s_perm[MOE_MAX_EXPERTS];
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  if (tid < p.E) s_cnt[tid] = p.offsets[tid + 1] - p.offsets[tid];
  __syncthreads();
  if (tid < p.E) {  // rank experts by row count, most rows first, ties by index
    const int c = s_cnt[tid];
    int r = 0;
    for (int o = 0; o < p.E; ++o) {
      const int co = s_cnt[o];
      r += (co > c) || (co == c && o < tid);
    }
    s_perm[r] = tid;
  }
  __syncthreads();
  const int T1 = (p.N1 + BM - 1) / BM, T2 = (p.N2 + BN - 1) / BN;
  const int per = T1 * T2;
  const int bid = blockIdx.x;
  const int rank = bid / per, in = bid % per;
  const int e = s_perm[rank];
  const int t1 = in / T2, t2 = in % T2;
  const int n1 = t1 * BM, n2 = t2 * BN;
  const int r0 = p.offsets[e], K = s_cnt[e];
  const int rows = min(BM, p.N1 - n1), cols = min(BN, p.N2 - n2);
  TileGemm<BM, BN, false, false, GATE> tg;
  const bool gate_here = GATE && t1 == 0;
  tg.run(p.X1 + (size_t)r0 * p.N1 + n1, p.N1, rows, p.X2 + (size_t)r0 * p.N2 + n2, p.N2, cols, K,
         lds, gate_here ? p.gsel + r0 : nullptr);
  store_tile<EPI_F32>(tg, p.C + (size_t)e * p.N1 * p.N2 + (size_t)n1 * p.N2 + n2, p.N2, rows,
                      cols, nullptr, 0);
  if constexpr (GATE) {
    if (gate_here) {
      __syncthreads();
      tg.gate_reduce(reinterpret_cast<float*>(lds), cols, p.dw_gate + (size_t)n2 * p.E + e, p.E,
                     t2 == 0 ? p.db_gate + e : nullptr);
    }
  }
}

// ---------------------------------------------------------------------------
// float32 path (act = MOE_F32): plain FMA kernels, no reduced precision.
constexpr int kF32Rows = 16;

// C[r][n] = epi(sum_k A[r][k] B_e(n, k)); B_e(n,k) = B[e][n][k] (B_K) or B[e][k][n].
template <bool B_K, int EPI>
__global__ void __launch_bounds__(256)
f32_rows_kernel(const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C,
                const float* __restrict__ aux, const int32_t* __restrict__ offsets, int K, int N,
                int E, int S_max) {
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  for (int i = threadIdx.x; i <= E; i += 256) s_off[i] = offsets[i];
  __syncthreads();
  const int r = blockIdx.x * kF32Rows + (threadIdx.x >> 4);
  const int g = threadIdx.x & 15;
  if (r >= s_off[E] || r >= S_max) return;
  int e = 0;
  while (!(s_off[e] <= r && r < s_off[e + 1])) ++e;
  const float* a = A + (size_t)r * K;
  const float* b = B + (size_t)e * N * K;
  for (int n = blockIdx.y * 64 + g; n < min(N, blockIdx.y * 64 + 64); n += 16) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(a[k], B_K ? b[(size_t)n * K + k] : b[(size_t)k * N + n], acc);
    if (EPI == EPI_RELU) acc = fmaxf(acc, 0.f);
    if (EPI == EPI_MASK && !(aux[(size_t)r * N + n] > 0.f)) acc = 0.f;
    C[(size_t)r * N + n] = acc;
  }
}

// dW[e][n1][n2] = sum over e's rows m of X1[m][n1] X2[m][n2]
__global__ void __launch_bounds__(256)
f32_wgrad_kernel(const float* __restrict__ X1, const float* __restrict__ X2, float* __restrict__ C,
                 const int32_t* __restrict__ offsets, int N1, int N2) {
  const int e = blockIdx.x;
  const int n1 = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int g = threadIdx.x & 15;
  if (n1 >= N1) return;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  for (int n2 = blockIdx.z * 64 + g; n2 < min(N2, blockIdx.z * 64 + 64); n2 += 16) {
    float acc = 0.f;
    for (int m = r0; m < r1; ++m) acc = fmaf(X1[(size_t)m * N1 + n1], X2[(size_t)m * N2 + n2], acc);
    C[((size_t)e * N1 + n1) * N2 + n2] = acc;
  }
}

// Every kernel variant the launchers can pick, instantiated explicitly (so
// each is emitted whatever order the launchers reference them in).
#define MOE_ROWS_VARIANTS(BM, BN)                                        \
  template __global__ void rows_gemm_kernel<BM, BN, true, EPI_RELU>(RowsArgs);   \
  template __global__ void rows_gemm_kernel<BM, BN, true, EPI_STORE>(RowsArgs);  \
  template __global__ void rows_gemm_kernel<BM, BN, false, EPI_MASK>(RowsArgs);  \
  template __global__ void rows_gemm_kernel<BM, BN, false, EPI_STORE>(RowsArgs); \
  template __global__ void wgrad_kernel<BM, BN, false>(WgradArgs);               \
  template __global__ void wgrad_kernel<BM, BN, true>(WgradArgs);
MOE_ROWS_VARIANTS(256, 256)
MOE_ROWS_VARIANTS(256, 128)
MOE_ROWS_VARIANTS(128, 256)
MOE_ROWS_VARIANTS(128, 128)
#undef MOE_ROWS_VARIANTS

// ---------------------------------------------------------------------------
// launchers

// Tile shape per product: the largest tiles (fewest LDS bytes per flop) that
// still give every CU work.  `mt(bm)` = number of row tiles for tile height bm.
struct Shape2 {
  int bm, bn;
};
template <class MT>
static Shape2 pick_tile(MT mt, int N) {
  const long long want = 2 * 256;  // two tiles per CU
  const Shape2 cand[] = {{256, 256}, {256, 128}, {128, 256}, {128, 128}};
  for (const Shape2& c : cand) {
    const long long tiles = mt(c.bm) * (long long)((N + c.bn - 1) / c.bn);
    if (tiles >= want) return c;
  }
  return {128, 128};
}

template <int BM, int BN, bool B_K, int EPI>
static hipError_t launch_rows_t(const RowsArgs& p, int S_max, hipStream_t s) {
  // worst case: sum over experts of ceil(rows_e / BM) <= S_max / BM + E
  const long long mt_max = (S_max + BM - 1) / BM + p.E;
  const long long nt = (p.N + BN - 1) / BN;
  const long long grid = mt_max * nt;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  constexpr size_t shm = TileGemm<BM, BN, true, B_K>::kLdsPipe;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&rows_gemm_kernel<BM, BN, B_K, EPI>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((rows_gemm_kernel<BM, BN, B_K, EPI>), dim3((unsigned)grid),
                     dim3(kGemmThreads), shm, s, p);
  return hipGetLastError();
}

template <bool B_K, int EPI>
static hipError_t launch_rows(const bf16* A, const bf16* B, bf16* C, const bf16* aux,
                              const int32_t* offsets, long long b_stride, int K, int N, int E,
                              int S_max, hipStream_t s) {
  RowsArgs p{A, B, C, aux, offsets, b_stride, K, N, E};
  // row tiles for an even spread of S_max rows over E experts
  auto mt = [&](int bm) {
    const long long per = ((long long)S_max / E + bm - 1) / bm;
    return per * E;
  };
  const Shape2 t = pick_tile(mt, N);
  if (t.bm == 256 && t.bn == 256) return launch_rows_t<256, 256, B_K, EPI>(p, S_max, s);
  if (t.bm == 256 && t.bn == 128) return launch_rows_t<256, 128, B_K, EPI>(p, S_max, s);
  if (t.bm == 128 && t.bn == 256) return launch_rows_t<128, 256, B_K, EPI>(p, S_max, s);
  return launch_rows_t<128, 128, B_K, EPI>(p, S_max, s);
}

template <int BM, int BN, bool GATE>
static hipError_t launch_wgrad_t(const WgradArgs& p, hipStream_t s) {
  const long long grid = (long long)p.E * ((p.N1 + BM - 1) / BM) * ((p.N2 + BN - 1) / BN);
  constexpr size_t shm = TileGemm<BM, BN, false, false, GATE>::kLdsPipe;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&wgrad_kernel<BM, BN, GATE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((wgrad_kernel<BM, BN, GATE>), dim3((unsigned)grid), dim3(kGemmThreads), shm,
                     s, p);
  return hipGetLastError();
}

template <bool GATE>
static hipError_t launch_wgrad(const bf16* X1, const bf16* X2, float* C, const int32_t* offsets,
                               const float* gsel, float* dw_gate, float* db_gate, int N1, int N2,
                               int E, hipStream_t s) {
  WgradArgs p{X1, X2, C, offsets, gsel, dw_gate, db_gate, N1, N2, E};
  auto mt = [&](int bm) { return (long long)E * ((N1 + bm - 1) / bm); };
  const Shape2 t = pick_tile(mt, N2);
  if (t.bm == 256 && t.bn == 256) return launch_wgrad_t<256, 256, GATE>(p, s);
  if (t.bm == 256 && t.bn == 128) return launch_wgrad_t<256, 128, GATE>(p, s);
  if (t.bm == 128 && t.bn == 256) return launch_wgrad_t<128, 256, GATE>(p, s);
  return launch_wgrad_t<128, 128, GATE>(p, s);
}

#define MOE_TRY(expr)                         \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return _e;          \
  } while (0)

hipError_t launch_expert_fwd(int act, const void* x_perm, const int32_t* offsets, const void* w1,
                             const void* w2, void* h, void* out_perm, int S_max, int d, int F,
                             int E, hipStream_t s) {
  if (act == MOE_BF16) {
    MOE_TRY((launch_rows<true, EPI_RELU>((const bf16*)x_perm, (const bf16*)w1, (bf16*)h, nullptr,
                                         offsets, (long long)F * d, d, F, E, S_max, s)));
    MOE_TRY((launch_rows<true, EPI_STORE>((const bf16*)h, (const bf16*)w2, (bf16*)out_perm,
                                          nullptr, offsets, (long long)d * F, F, d, E, S_max,
                                          s)));
    return hipSuccess;
  }
  dim3 b(256);
  dim3 g1((S_max + kF32Rows - 1) / kF32Rows, (F + 63) / 64),
      g2((S_max + kF32Rows - 1) / kF32Rows, (d + 63) / 64);
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_RELU>), g1, b, 0, s, (const float*)x_perm,
                     (const float*)w1, (float*)h, nullptr, offsets, d, F, E, S_max);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_STORE>), g2, b, 0, s, (const float*)h,
                     (const float*)w2, (float*)out_perm, nullptr, offsets, F, d, E, S_max);
  return hipGetLastError();
}

hipError_t launch_expert_bwd(int act, const void* d_out, const void* x_perm, const void* h,
                             const int32_t* offsets, const void* w1, const void* w2, void* dz,
                             void* dx_perm, float* dw1, float* dw2, const float* dsel_perm,
                             float* dw_gate, float* db_gate, int S_max, int d, int F, int E,
                             hipStream_t s) {
  if (act == MOE_BF16) {
    // dz = (dO W2[e]) * [h > 0]: A = dO [rows][d], B = W2[e] as [K=d][N=F]
    MOE_TRY((launch_rows<false, EPI_MASK>((const bf16*)d_out, (const bf16*)w2, (bf16*)dz,
                                          (const bf16*)h, offsets, (long long)d * F, d, F, E,
                                          S_max, s)));
    // dW2[e] = dO^T h  ([d][F])
    MOE_TRY((launch_wgrad<false>((const bf16*)d_out, (const bf16*)h, dw2, offsets, nullptr,
                                 nullptr, nullptr, d, F, E, s)));
    // dx_perm = dz W1[e]: A = dz [rows][F], B = W1[e] as [K=F][N=d]  (may reuse dO's memory)
    MOE_TRY((launch_rows<false, EPI_STORE>((const bf16*)dz, (const bf16*)w1, (bf16*)dx_perm,
                                           nullptr, offsets, (long long)F * d, F, d, E, S_max,
                                           s)));
    // dW1[e] = dz^T x_perm  ([F][d]), with the gate's dW_gate / db over the kept rows
    MOE_TRY((launch_wgrad<true>((const bf16*)dz, (const bf16*)x_perm, dw1, offsets, dsel_perm,
                                dw_gate, db_gate, F, d, E, s)));
    return hipSuccess;
  }
  dim3 b(256);
  const int rt = (S_max + kF32Rows - 1) / kF32Rows;
  hipLaunchKernelGGL((f32_rows_kernel<false, EPI_MASK>), dim3(rt, (F + 63) / 64), b, 0, s,
                     (const float*)d_out, (const float*)w2, (float*)dz, (const float*)h, offsets, d,
                     F, E, S_max);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL(f32_wgrad_kernel, dim3(E, (d + 15) / 16, (F + 63) / 64), b, 0, s,
                     (const float*)d_out, (const float*)h, dw2, offsets, d, F);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL((f32_rows_kernel<false, EPI_STORE>), dim3(rt, (d + 63) / 64), b, 0, s,
                     (const float*)dz, (const float*)w1, (float*)dx_perm, nullptr, offsets, F, d,
                     E, S_max);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL(f32_wgrad_kernel, dim3(E, (F + 15) / 16, (d + 63) / 64), b, 0, s,
                     (const float*)dz, (const float*)x_perm, dw1, offsets, F, d);
  return hipGetLastError();
}

}  // namespace moe
