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

__device__ __forceinline__ int swz(int row, int kc) { return (row * 8 + (kc ^ (row & 7))) * 8; }

// ---------------------------------------------------------------------------
// Operand tile loaders: global -> registers -> LDS [ROWS][64] (bf16).
// K-contiguous operand: element (r, k) at base[r * ld + k].
template <int ROWS>
struct LoadK {
  static constexpr int N = ROWS * 8 / kGemmThreads;  // 16-byte chunks per thread
  i32x4 v[N];
  // rows >= nrows are clamped to row nrows-1 (their results are never stored)
  __device__ void load(const bf16* base, int ld, int nrows, int k0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * kGemmThreads;
      const int r = min(c >> 3, nrows - 1), kc = c & 7;
      v[i] = *reinterpret_cast<const i32x4*>(base + (size_t)r * ld + k0 + kc * 8);
    }
  }
  __device__ void store(bf16* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * kGemmThreads;
      const int r = c >> 3, kc = c & 7;
      *reinterpret_cast<i32x4*>(lds + swz(r, kc)) = v[i];
    }
  }
};

// MN-contiguous operand: element (r, k) at base[k * ld + r].  Each thread
// loads KB consecutive k of 8 consecutive r and writes them transposed.
// k >= kmax reads as zero; r >= nrows is clamped (never stored).
template <int ROWS>
struct LoadMN {
  static constexpr int RB = ROWS / 8;                 // 8-row blocks
  static constexpr int KB = kBK * RB / kGemmThreads;  // k per thread (4 or 8)
  i32x4 v[KB];  // v[i] = 8 bf16 of k-row i, two per dword
  __device__ void load(const bf16* base, int ld, int nrows, int k0, int kmax) {
    const int rb = threadIdx.x % RB, kb = threadIdx.x / RB;
    const int r = min(rb * 8, nrows - 8);
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int k = k0 + kb * KB + i;
      if (k < kmax)
        v[i] = *reinterpret_cast<const i32x4*>(base + (size_t)k * ld + r);
      else
        v[i] = i32x4{0, 0, 0, 0};
    }
  }
  // (v[i] element m, v[i+1] element m) as one dword: low halves for even m,
  // high halves for odd m.
  __device__ static int pair(int lo_src, int hi_src, int odd) {
    return (int)__builtin_amdgcn_perm((unsigned)hi_src, (unsigned)lo_src,
                                      odd ? 0x07060302u : 0x05040100u);
  }
  __device__ void store(bf16* lds) const {
    const int rb = threadIdx.x % RB, kb = threadIdx.x / RB;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int row = rb * 8 + m, p = m >> 1, odd = m & 1;
      if constexpr (KB == 8) {
        i32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pair(v[2 * q][p], v[2 * q + 1][p], odd);
        *reinterpret_cast<i32x4*>(lds + swz(row, kb)) = o;
      } else {
        typedef __attribute__((ext_vector_type(2))) int i32x2;
        i32x2 o;
#pragma unroll
        for (int q = 0; q < 2; ++q) o[q] = pair(v[2 * q][p], v[2 * q + 1][p], odd);
        *reinterpret_cast<i32x2*>(lds + swz(row, kb >> 1) + (kb & 1) * 4) = o;
      }
    }
  }
};

template <bool KMAJOR, int ROWS>
struct Loader;
template <int ROWS>
struct Loader<true, ROWS> {
  LoadK<ROWS> l;
  __device__ void load(const bf16* base, int ld, int nrows, int k0, int) {
    l.load(base, ld, nrows, k0);
  }
  __device__ void store(bf16* lds) const { l.store(lds); }
};
template <int ROWS>
struct Loader<false, ROWS> {
  LoadMN<ROWS> l;
  __device__ void load(const bf16* base, int ld, int nrows, int k0, int kmax) {
    l.load(base, ld, nrows, k0, kmax);
  }
  __device__ void store(bf16* lds) const { l.store(lds); }
};

// ---------------------------------------------------------------------------
// One output tile: C[BM x BN] = sum_k A(r, k) B(n, k), k in [0, K).
// A/B pointers address element (0, 0) of the tile; kmax bounds k for
// MN-contiguous operands (wgrad's ragged expert rows).
template <int BM, int BN, bool A_K, bool B_K>
struct TileGemm {
  static constexpr int WM = BM / 2, WN = BN / 2;  // 2 x 2 waves
  static constexpr int FM = WM / 16, FN = WN / 16;
  f32x4 acc[FM][FN];

  __device__ void run(const bf16* A, int lda, int a_rows, const bf16* B, int ldb, int b_rows,
                      int K, bf16* lds) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nk = (K + kBK - 1) / kBK;
    if (nk == 0) return;
    Loader<A_K, BM> la;
    Loader<B_K, BN> lb;
    la.load(A_K ? A : A, lda, a_rows, 0, K);
    lb.load(B, ldb, b_rows, 0, K);
    la.store(lds);
    lb.store(lds + 2 * BM * kBK);
    __syncthreads();
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        if (A_K)
          la.load(A, lda, a_rows, (kt + 1) * kBK, K);
        else
          la.load(A + (size_t)(kt + 1) * kBK * lda, lda, a_rows, 0, K - (kt + 1) * kBK);
        if (B_K)
          lb.load(B, ldb, b_rows, (kt + 1) * kBK, K);
        else
          lb.load(B + (size_t)(kt + 1) * kBK * ldb, ldb, b_rows, 0, K - (kt + 1) * kBK);
      }
      const bf16* as = lds + cur * (BM * kBK);
      const bf16* bs = lds + 2 * BM * kBK + cur * (BN * kBK);
#pragma unroll
      for (int ks = 0; ks < kBK / 32; ++ks) {
        bf16x8 a[FM], b[FN];
        const int kc = ks * 4 + (lane >> 4);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WM + i * 16 + (lane & 15);
          a[i] = *reinterpret_cast<const bf16x8*>(as + swz(r, kc));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * WN + j * 16 + (lane & 15);
          b[j] = *reinterpret_cast<const bf16x8*>(bs + swz(r, kc));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (more) {
        la.store(lds + (cur ^ 1) * (BM * kBK));
        lb.store(lds + 2 * BM * kBK + (cur ^ 1) * (BN * kBK));
      }
      __syncthreads();
    }
  }
};

// Epilogue: element (r, n) of the tile is acc[i][j][q] with
// r = wm*WM + i*16 + (lane/16)*4 + q and n = wn*WN + j*16 + lane%16.
template <int BM, int BN, bool A_K, bool B_K, int EPI>
__device__ __forceinline__ void store_tile(const TileGemm<BM, BN, A_K, B_K>& tg, void* C, int ldc,
                                           int rows, int cols, const bf16* aux, int ld_aux) {
  using TG = TileGemm<BM, BN, A_K, B_K>;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
#pragma unroll
  for (int i = 0; i < TG::FM; ++i)
#pragma unroll
    for (int j = 0; j < TG::FN; ++j) {
      const int n = wn * TG::WN + j * 16 + (lane & 15);
      if (n >= cols) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm * TG::WM + i * 16 + (lane >> 4) * 4 + q;
        if (r >= rows) continue;
        float v = tg.acc[i][j][q];
        if constexpr (EPI == EPI_F32) {
          reinterpret_cast<float*>(C)[(size_t)r * ldc + n] = v;
        } else {
          if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.f);
          if constexpr (EPI == EPI_MASK) {
            if (!((float)aux[(size_t)r * ld_aux + n] > 0.f)) v = 0.f;
          }
          reinterpret_cast<bf16*>(C)[(size_t)r * ldc + n] = (bf16)v;
        }
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
  store_tile<BM, BN, true, B_K, EPI>(tg, p.C + (size_t)row0 * p.N + n0, p.N, rows, cols,
                                     p.aux ? p.aux + (size_t)row0 * p.N + n0 : nullptr, p.N);
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM: dW[e] [N1][N2] = X1_e^T X2_e over expert e's rows.
struct WgradArgs {
  const bf16* X1;  // [rows][N1]
  const bf16* X2;  // [rows][N2]
  float* C;        // [E][N1][N2]
  const int32_t* offsets;
  int N1, N2, E;
};

template <int BM, int BN>
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
  TileGemm<BM, BN, false, false> tg;
  tg.run(p.X1 + (size_t)r0 * p.N1 + n1, p.N1, rows, p.X2 + (size_t)r0 * p.N2 + n2, p.N2, cols, K,
         lds);
  store_tile<BM, BN, false, false, EPI_F32>(tg, p.C + (size_t)e * p.N1 * p.N2 + (size_t)n1 * p.N2 + n2,
                                            p.N2, rows, cols, nullptr, 0);
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

// ---------------------------------------------------------------------------
// launchers
constexpr int kFwdBM = 128, kFwdBN = 128;
constexpr int kWgBM = 128, kWgBN = 128;

template <int BM, int BN>
constexpr size_t gemm_lds_bytes() {
  return (size_t)2 * (BM + BN) * kBK * sizeof(bf16);
}

template <int BM, int BN, bool B_K, int EPI>
static hipError_t launch_rows(const bf16* A, const bf16* B, bf16* C, const bf16* aux,
                              const int32_t* offsets, long long b_stride, int K, int N, int E,
                              int S_max, hipStream_t s) {
  RowsArgs p{A, B, C, aux, offsets, b_stride, K, N, E};
  // worst case: sum over experts of ceil(rows_e / BM) <= S_max / BM + E
  const long long mt_max = (S_max + BM - 1) / BM + E;
  const long long nt = (N + BN - 1) / BN;
  const long long grid = mt_max * nt;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  constexpr size_t shm = gemm_lds_bytes<BM, BN>();
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&rows_gemm_kernel<BM, BN, B_K, EPI>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((rows_gemm_kernel<BM, BN, B_K, EPI>), dim3((unsigned)grid), dim3(kGemmThreads),
                     shm, s, p);
  return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_wgrad(const bf16* X1, const bf16* X2, float* C, const int32_t* offsets,
                               int N1, int N2, int E, hipStream_t s) {
  WgradArgs p{X1, X2, C, offsets, N1, N2, E};
  const long long grid = (long long)E * ((N1 + BM - 1) / BM) * ((N2 + BN - 1) / BN);
  constexpr size_t shm = gemm_lds_bytes<BM, BN>();
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&wgrad_kernel<BM, BN>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((wgrad_kernel<BM, BN>), dim3((unsigned)grid), dim3(kGemmThreads), shm, s, p);
  return hipGetLastError();
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
    MOE_TRY((launch_rows<kFwdBM, kFwdBN, true, EPI_RELU>(
        (const bf16*)x_perm, (const bf16*)w1, (bf16*)h, nullptr, offsets, (long long)F * d, d, F,
        E, S_max, s)));
    MOE_TRY((launch_rows<kFwdBM, kFwdBN, true, EPI_STORE>(
        (const bf16*)h, (const bf16*)w2, (bf16*)out_perm, nullptr, offsets, (long long)d * F, F,
        d, E, S_max, s)));
    return hipSuccess;
  }
  dim3 b(256);
  dim3 g1((S_max + kF32Rows - 1) / kF32Rows, (F + 63) / 64), g2((S_max + kF32Rows - 1) / kF32Rows, (d + 63) / 64);
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_RELU>), g1, b, 0, s, (const float*)x_perm,
                     (const float*)w1, (float*)h, nullptr, offsets, d, F, E, S_max);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_STORE>), g2, b, 0, s, (const float*)h,
                     (const float*)w2, (float*)out_perm, nullptr, offsets, F, d, E, S_max);
  return hipGetLastError();
}

hipError_t launch_expert_bwd(int act, const void* d_out, const void* x_perm, const void* h,
                             const int32_t* offsets, const void* w1, const void* w2, void* dz,
                             void* dx_perm, float* dw1, float* dw2, int S_max, int d, int F,
                             int E, hipStream_t s) {
  if (act == MOE_BF16) {
    // dz = (dO W2[e]) * [h > 0]: A = dO [rows][d], B = W2[e] as [K=d][N=F]
    MOE_TRY((launch_rows<kFwdBM, kFwdBN, false, EPI_MASK>(
        (const bf16*)d_out, (const bf16*)w2, (bf16*)dz, (const bf16*)h, offsets, (long long)d * F,
        d, F, E, S_max, s)));
    // dW2[e] = dO^T h  ([d][F])
    MOE_TRY((launch_wgrad<kWgBM, kWgBN>((const bf16*)d_out, (const bf16*)h, dw2, offsets, d, F, E, s)));
    // dx_perm = dz W1[e]: A = dz [rows][F], B = W1[e] as [K=F][N=d]  (may reuse dO's memory)
    MOE_TRY((launch_rows<kFwdBM, kFwdBN, false, EPI_STORE>(
        (const bf16*)dz, (const bf16*)w1, (bf16*)dx_perm, nullptr, offsets, (long long)F * d, F,
        d, E, S_max, s)));
    // dW1[e] = dz^T x_perm  ([F][d])
    MOE_TRY((launch_wgrad<kWgBM, kWgBN>((const bf16*)dz, (const bf16*)x_perm, dw1, offsets, F, d, E, s)));
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
