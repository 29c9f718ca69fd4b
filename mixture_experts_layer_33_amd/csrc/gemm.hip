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
// Operands are copied global -> LDS by the buffer unit directly
// (buffer_load_dwordx4 ... lds, no staging registers) and read back as MFMA
// fragments: K-contiguous operands as 16-byte rows, M/N-contiguous operands
// transposed by ds_read_b64_tr_b16.  Buffer range checks turn rows past the
// end of an operand into zeros, so ragged tiles need no clamping or masking.
//
// Scheduling: forward and dgrad tiles cover each expert's packed rows; the
// tile list is built inside the kernel from the device offsets (no host
// sync), grouped along M for operand reuse and laid out so each XCD (one L2)
// gets a contiguous range.  wgrad tiles are ordered hottest expert first so
// the long K loops of popular experts start early (longest-processing-time
// first); experts with no rows store zeros.
#include "buffer.hpp"
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace moe {

constexpr int kBK = 64;          // k per LDS stage
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round robin

enum Epi { EPI_RELU = 0, EPI_STORE = 1, EPI_MASK = 2, EPI_F32 = 3 };

// ---------------------------------------------------------------------------
// Operand tiles.  Each stage holds 64 k of the tile; one wave instruction
// copies 1 KiB.  issue<Q, NQ> issues the instructions i with i % NQ == Q, so
// a stage's copies can be spread over NQ scheduling regions.
//
// K-contiguous operand (element (r, k) at base[r * ld + k]), valid rows
// [0, nrows): LDS [ROWS][64] bf16, 16-byte chunk kc of row r at position
// kc ^ ((r >> 1) & 7), so a fragment read (16-byte chunks of 16 consecutive
// rows per 256 bytes of banks) is free of bank conflicts.  K is a multiple of
// 64 for these operands.
template <int ROWS>
struct TileK {
  static constexpr int N = ROWS / 32;          // wave instructions per thread per stage
  static constexpr int kBytes = ROWS * kBK * 2;
  static constexpr int NLO = 4;                // lane offsets (one per 16-deep slice)
  const bf16* base;
  uint32_t bytes;
  uint32_t off[N];
  __device__ void init(const bf16* b, int ld, int nrows, int /*kmax*/, int wid) {
    const int lane = threadIdx.x & 63;
    base = b;
    bytes = (uint32_t)nrows * (uint32_t)ld * 2u;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int row = (i * 4 + wid) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ ((row >> 1) & 7);
      off[i] = (uint32_t)(row * ld + kc * 8) * 2u;
    }
  }
  // Gathered rows: tile row r is row idx[r] of b ([src_rows][ld]); rows past
  // nrows point past the resource's range and land as zeros.
  __device__ void init_gather(const bf16* b, int ld, int nrows, int src_rows,
                              const int32_t* idx, int wid) {
    const int lane = threadIdx.x & 63;
    base = b;
    bytes = (uint32_t)src_rows * (uint32_t)ld * 2u;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int row = (i * 4 + wid) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ ((row >> 1) & 7);
      off[i] = row < nrows ? (uint32_t)(idx[row] * ld + kc * 8) * 2u : kPadOffset;
    }
  }
  // resource and stage offset for the stage starting at k0 (dead: zeros)
  __device__ Rsrc rsrc(bool live) const { return make_rsrc(base, live ? bytes : 0u); }
  __device__ static uint32_t soff(int k0) { return (uint32_t)k0 * 2u; }
  template <int Q, int NQ, int AUX = 0>
  __device__ void issue(Rsrc r, uint32_t so, char* stage, int wid) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i % NQ == Q) copy16<AUX>(r, stage + (i * 4 + wid) * 1024, off[i], so);
  }
  static constexpr int issued(int Q, int NQ) {
    int n = 0;
    for (int i = 0; i < N; ++i) n += (i % NQ == Q);
    return n;
  }
  // lane byte offsets: slice kk, lane l holds row l%32 of the block, k from
  // kk*16 + 8*(l/32)
  __device__ static void lane_offsets(uint32_t (&lo)[NLO]) {
    const int lane = threadIdx.x & 63, r = lane & 31;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      lo[kk] = (uint32_t)(r * 8 + ((kk * 2 + (lane >> 5)) ^ ((r >> 1) & 7))) * 16u;
  }
  static constexpr int kReads = 1;  // LDS reads per fragment
  // 32 x 16 MFMA operand block at rows r0..r0+31, slice kk
  __device__ static bf16x8 frag(const char* stage, int r0, int kk, const uint32_t (&lo)[NLO]) {
    return *reinterpret_cast<const bf16x8*>(stage + r0 * (kBK * 2) + lo[kk]);
  }
};

// M/N-contiguous operand (element (r, k) at base[k * ld + r]), valid columns
// [0, ncols) and k rows [0, kmax): LDS [64][ROWS] as in memory, with a pitch
// of ROWS*2 + 64 bytes (four unused 16-byte slots after each k-row) so that
// four consecutive k-rows start in four different 64-byte groups of banks.
// Read back transposed by ds_read_b64_tr_b16: within each 16-lane group that
// instruction hands lane i the elements M[4j + i/4][i%4] (j = 0..3) of the
// 4-element pieces M[r] addressed by the group's lanes r; addressing k-row
// kb + r/4, columns c0 + 4 (r%4) gives lane i four consecutive k of column
// c0 + i.  Two reads give the 8 k of a fragment, in the same k order as the
// K-contiguous fragments.  k rows >= kmax read as zeros (buffer range);
// columns >= ncols re-read a valid column chunk; pad slots read nothing.
template <int ROWS>
struct TileMN {
  static constexpr int R = ROWS * 2;            // bytes of a k-row
  static constexpr int P = R + 64;              // LDS pitch
  static constexpr int SPR = P / 16;            // 16-byte slots per k-row
  static constexpr int N = kBK * SPR / 256;     // wave instructions per thread per stage
  static constexpr int kBytes = kBK * P;
  static constexpr int NLO = 1;
  static_assert(kBK * SPR % 256 == 0, "stage must be whole wave instructions");
  const bf16* base;
  uint32_t bytes, ld2;
  uint32_t off[N];
  __device__ void init(const bf16* b, int ld, int ncols, int kmax, int wid) {
    const int lane = threadIdx.x & 63;
    base = b;
    ld2 = (uint32_t)ld * 2u;
    bytes = (uint32_t)kmax * ld2;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int slot = (i * 4 + wid) * 64 + lane;
      const int k = slot / SPR, s = slot % SPR;
      off[i] = s < R / 16 ? (uint32_t)k * ld2 + (uint32_t)min(s, ncols / 8 - 1) * 16u
                          : kPadOffset;
    }
  }
  __device__ Rsrc rsrc(bool live) const { return make_rsrc(base, live ? bytes : 0u); }
  __device__ uint32_t soff(int k0) const { return (uint32_t)k0 * ld2; }
  template <int Q, int NQ, int AUX = 0>
  __device__ void issue(Rsrc r, uint32_t so, char* stage, int wid) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i % NQ == Q) copy16<AUX>(r, stage + (i * 4 + wid) * 1024, off[i], so);
  }
  static constexpr int issued(int Q, int NQ) {
    int n = 0;
    for (int i = 0; i < N; ++i) n += (i % NQ == Q);
    return n;
  }
  // 16-lane group G = l/16 covers columns r0 + 16*(G&1) .. +15 and k from
  // kk*16 + 8*(G>>1): lane r of the group addresses k-row + r/4, column
  // + 4*(r%4)
  __device__ static void lane_offsets(uint32_t (&lo)[NLO]) {
    const int lane = threadIdx.x & 63, G = lane >> 4, r = lane & 15;
    lo[0] = (uint32_t)((8 * (G >> 1) + (r >> 2)) * P + (16 * (G & 1) + 4 * (r & 3)) * 2);
  }
  static constexpr int kReads = 2;
  __device__ static bf16x8 frag(const char* stage, int r0, int kk, const uint32_t (&lo)[NLO]) {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    typedef __attribute__((ext_vector_type(2))) int i32x2;
    i32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(stage + r0 * 2 + (kk * 16 + h * 4) * P +
                                                     lo[0]));
      // reinterpret all 8 bytes at once (element-wise casts of this result
      // have been seen to be lowered wrongly)
      const i32x2 w = __builtin_bit_cast(i32x2, v);
      out[2 * h] = w[0];
      out[2 * h + 1] = w[1];
    }
    return __builtin_bit_cast(bf16x8, out);
  }
  // 16 bytes (8 columns) of k-row k at column chunk c, for the gate product
  __device__ static bf16x8 chunk(const char* stage, int k, int c) {
    return *reinterpret_cast<const bf16x8*>(stage + k * P + c * 16);
  }
};

template <bool KMAJOR, int ROWS>
struct Tile;
template <int ROWS>
struct Tile<true, ROWS> : TileK<ROWS> {};
template <int ROWS>
struct Tile<false, ROWS> : TileMN<ROWS> {};

// Spread a region's LDS reads and copies between its MFMAs (one MFMA runs 32
// cycles; the wave issues other instructions meanwhile).
template <int NM, int ND, int NV>
__device__ __forceinline__ void interleave() {
  constexpr int a = NM < ND ? NM : ND;
  constexpr int m2 = NM - a;
  constexpr int b = m2 < NV ? m2 : NV;
#pragma unroll
  for (int t = 0; t < a; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
#pragma unroll
  for (int t = 0; t < b; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
  }
  if constexpr (ND > a) __builtin_amdgcn_sched_group_barrier(0x100, ND - a, 0);
  if constexpr (NV > b) __builtin_amdgcn_sched_group_barrier(0x010, NV - b, 0);
  if constexpr (m2 > b) __builtin_amdgcn_sched_group_barrier(0x008, m2 - b, 0);
}

// The LDS stage buffers of a tile, each its own LDS object: the compiler can
// then tell that the buffer being read is not the one the copies are filling
// (with one shared array it waits for every copy before each transposed
// read).  Unused third stages are 16 bytes.
struct StageBufs {
  char* a[3];
  char* b[3];
};
template <class TG>
__device__ __forceinline__ StageBufs tile_lds() {
  constexpr int A3 = TG::kStages == 3 ? TG::TA::kBytes : 16;
  constexpr int B3 = TG::kStages == 3 ? TG::TB::kBytes : 16;
  __shared__ __attribute__((aligned(16))) char a0[TG::TA::kBytes];
  __shared__ __attribute__((aligned(16))) char a1[TG::TA::kBytes];
  __shared__ __attribute__((aligned(16))) char a2[A3];
  __shared__ __attribute__((aligned(16))) char b0[TG::TB::kBytes];
  __shared__ __attribute__((aligned(16))) char b1[TG::TB::kBytes];
  __shared__ __attribute__((aligned(16))) char b2[B3];
  return StageBufs{{a0, a1, a2}, {b0, b1, b2}};
}

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
// Pipeline: 3 LDS stages (2 where 3 do not fit), one barrier per 64-deep k
// step.  Step kt reads stage kt in four 16-deep slices, software-pipelined
// over two register sets, and copies stage kt + stages - 1 into the buffer
// stage kt - 1 used; the copies (all at the step's start with two stages)
// and the reads of the next slice are spread between the MFMAs.  The last
// slice's MFMAs run after the barrier, covering
// the latency of the first reads of the next stage.  Every step issues a full
// stage of copies (past the end of K they are out of range and read nothing),
// so a wave's outstanding-copy count is the same at every barrier.
//
// With GATE (B MN-contiguous) and a non-null `gsel`, the tile also forms
// g[n] = sum_k gsel[k] B(n, k) for its columns from the LDS stages (gacc: per
// thread, 8 columns over its share of the rows) and sum_k gsel[k] (gdb);
// see gate_reduce().
template <int BM, int BN, bool A_K, bool B_K, bool GATE = false, int STAGES = 0,
          int B_AUX = 0>
struct TileGemm {
  using TA = Tile<A_K, BM>;
  using TB = Tile<B_K, BN>;
  static constexpr int WM = BM / 2, WN = BN / 2;  // 2 x 2 waves
  static constexpr int FM = WM / 32, FN = WN / 32;  // 32 x 32 MFMA blocks per wave
  static constexpr size_t kStageBytes = (size_t)TA::kBytes + TB::kBytes;
  // three stages when they fit in LDS next to the kernels' own few KiB
  static constexpr int kStages =
      STAGES != 0 ? STAGES : (3 * kStageBytes + 4096 <= 160 * 1024 ? 3 : 2);
  static constexpr int kStageOps = TA::N + TB::N;
  static constexpr int kBAux = B_AUX;  // cache policy of B's copies
  static constexpr int kReads = FM * TA::kReads + FN * TB::kReads;  // LDS reads per slice
  f32x16 acc[FN][FM];  // acc[i][j]: n-block i, m-block j
  float gacc[8];
  float gdb;

  // A: rows [0, a_rows) (K-contiguous) or columns [0, a_rows) over k rows
  // [0, K) (MN-contiguous); likewise B.  With a_idx (K-contiguous A only),
  // tile row r is row a_idx[r] of A ([a_src_rows][lda]).
  __device__ void run(const bf16* A, int lda, int a_rows, const bf16* B, int ldb, int b_rows,
                      int K, const StageBufs& L, const float* gsel = nullptr,
                      const int32_t* a_idx = nullptr, int a_src_rows = 0) {
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
    const int wid = (int)uniform(threadIdx.x >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    TA ta;
    TB tb;
    if constexpr (A_K) {
      if (a_idx != nullptr)
        ta.init_gather(A, lda, a_rows, a_src_rows, a_idx, wid);
      else
        ta.init(A, lda, a_rows, K, wid);
    } else {
      ta.init(A, lda, a_rows, K, wid);
    }
    tb.init(B, ldb, b_rows, K, wid);
    uint32_t alo[TA::NLO], blo[TB::NLO];
    TA::lane_offsets(alo);
    TB::lane_offsets(blo);

    auto load = [&](const char* as, const char* bs, int kk, bf16x8(&a)[FM], bf16x8(&b)[FN]) {
#pragma unroll
      for (int j = 0; j < FM; ++j) a[j] = TA::frag(as, wm * WM + j * 32, kk, alo);
#pragma unroll
      for (int i = 0; i < FN; ++i) b[i] = TB::frag(bs, wn * WN + i * 32, kk, blo);
    };
    auto mma = [&](const bf16x8(&a)[FM], const bf16x8(&b)[FN]) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[i], a[j], acc[i][j], 0, 0, 0);
    };
    // a full stage of copies (prologue)
    auto issue_all = [&](int kt, char* ad, char* bd) {
      const bool live = kt < nk;
      const Rsrc ra = ta.rsrc(live), rb = tb.rsrc(live);
      const uint32_t sa = ta.soff(kt * kBK), sb = tb.soff(kt * kBK);
      ta.template issue<0, 1>(ra, sa, ad, wid);
      tb.template issue<0, 1, kBAux>(rb, sb, bd, wid);
    };
    constexpr int kGateRows = GATE ? kBK * (BN / 8) / kGemmThreads : 1;
    float gv[kGateRows];
    // gate weights of stage kt's rows for this thread
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
    auto gate_stage = [&](const char* bs) {
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
    // Wait for this wave's copies of the next stage (with three stages those
    // of the stage after it stay in flight) and its own LDS reads, then meet
    // the other waves.  Written out because __syncthreads() adds a release
    // fence, which waits for every outstanding copy.
    auto sync = [&]() {
      if constexpr (kStages == 3)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kStageOps) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    bf16x8 a0[FM], b0[FN], a1[FM], b1[FN];
    // step kt on stage S = kt % stages; FIRST: no previous slice to finish
    auto step = [&](auto S_, auto FIRST_, int kt) {
      constexpr int S = decltype(S_)::value;
      constexpr bool FIRST = decltype(FIRST_)::value != 0;
      constexpr int SD = (S + kStages - 1) % kStages;  // buffer of stage kt-1
      const char* as = L.a[S];
      const char* bs = L.b[S];
      char* const ad = L.a[SD];
      char* const bd = L.b[SD];
      const int kd = kt + kStages - 1;
      const bool live = kd < nk;
      const Rsrc ra = ta.rsrc(live), rb = tb.rsrc(live);
      const uint32_t sa = ta.soff(kd * kBK), sb = tb.soff(kd * kBK);
      constexpr int NM = FM * FN;
      load_gate(kt);
      __builtin_amdgcn_sched_barrier(0);
      // region 0: slice 0 -> set 0; finish slice 3 of step kt-1 (set 1).
      // With two stages the next stage must land within this step, so all of
      // its copies go out here; with three they are spread over the regions.
      constexpr int NQ = kStages == 2 ? 1 : 4;
      load(as, bs, 0, a0, b0);
      ta.template issue<0, NQ>(ra, sa, ad, wid);
      tb.template issue<0, NQ, kBAux>(rb, sb, bd, wid);
      if constexpr (!FIRST) mma(a1, b1);
      interleave<FIRST ? 0 : NM, kReads, TA::issued(0, NQ) + TB::issued(0, NQ)>();
      __builtin_amdgcn_sched_barrier(0);
      // region 1: slice 1 -> set 1; slice 0
      load(as, bs, 1, a1, b1);
      ta.template issue<1, NQ>(ra, sa, ad, wid);
      tb.template issue<1, NQ, kBAux>(rb, sb, bd, wid);
      mma(a0, b0);
      interleave<NM, kReads, TA::issued(1, NQ) + TB::issued(1, NQ)>();
      __builtin_amdgcn_sched_barrier(0);
      // region 2: slice 2 -> set 0; slice 1
      load(as, bs, 2, a0, b0);
      ta.template issue<2, NQ>(ra, sa, ad, wid);
      tb.template issue<2, NQ, kBAux>(rb, sb, bd, wid);
      mma(a1, b1);
      interleave<NM, kReads, TA::issued(2, NQ) + TB::issued(2, NQ)>();
      __builtin_amdgcn_sched_barrier(0);
      // region 3: slice 3 -> set 1; slice 2
      load(as, bs, 3, a1, b1);
      ta.template issue<3, NQ>(ra, sa, ad, wid);
      tb.template issue<3, NQ, kBAux>(rb, sb, bd, wid);
      mma(a0, b0);
      interleave<NM, kReads, TA::issued(3, NQ) + TB::issued(3, NQ)>();
      __builtin_amdgcn_sched_barrier(0);
      gate_stage(bs);
      sync();
    };

    // prologue: stages 0 .. stages-2 in flight, wait for stage 0
    issue_all(0, L.a[0], L.b[0]);
    if constexpr (kStages == 3) issue_all(1, L.a[1], L.b[1]);
    sync();
    step(Ic<0>{}, Ic<1>{}, 0);
    // whole rounds of `stages` steps, then the rest (one loop exit)
    int kt = 1;
    for (; kt + kStages <= nk; kt += kStages) {
      step(Ic<1 % kStages>{}, Ic<0>{}, kt);
      if constexpr (kStages == 3) {
        step(Ic<2>{}, Ic<0>{}, kt + 1);
        step(Ic<0>{}, Ic<0>{}, kt + 2);
      } else {
        step(Ic<0>{}, Ic<0>{}, kt + 1);
      }
    }
    if (kt < nk) {
      step(Ic<1 % kStages>{}, Ic<0>{}, kt);
      if constexpr (kStages == 3) {
        if (kt + 1 < nk) step(Ic<2>{}, Ic<0>{}, kt + 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1);
    // copies past the end are still in flight: let them land before the
    // caller reuses LDS
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // Sum the per-thread gate partials over the row groups (fixed order) and
  // write out[n * out_stride] = g[n] for n < cols, and *db_out (if non-null).
  // `red` is LDS (a stage buffer); call after run() (which ends with a barrier).
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
// Epilogue, staged through LDS so that global stores are whole row segments
// (the MFMA layout puts 32 different rows in one wave's store).  In each
// 32 x 32 block lane l holds C[m][n..n+3] for m = l%32 and n = 4*(l/32) + 8p
// (p = 0..3) (see TileGemm).  Each wave writes one 32-row strip of its block
// at a time to its own LDS region (rows padded by 16 bytes, so the 32 rows of
// a write fall in different banks), then reads it back as 16-byte pieces of
// whole rows, applies the mask and stores.  ReLU and the bf16 rounding happen
// on the way in.  EPI_MASK: `aux` is a bit mask, bit (n % 32) of word
// aux[m * ld_aux + n / 32] keeps element (m, n); a lane's words for the whole
// tile are loaded first, in one round trip.  rows/cols bound the valid part
// of the tile (cols is a multiple of 8).  Call after run(); uses the stage
// buffers.
// With crow, tile row m is stored at row crow[m] of C (C then points at the
// tile's first column of row 0).
template <int EPI, class TG>
__device__ __forceinline__ void store_tile(const TG& tg, const StageBufs& L, void* C, int ldc,
                                           int rows, int cols, const uint32_t* aux, int ld_aux,
                                           uint8_t* bits_out = nullptr,
                                           const int32_t* crow = nullptr) {
  using OutT = typename std::conditional<EPI == EPI_F32, float, bf16>::type;
  constexpr int ES = sizeof(OutT);
  constexpr int WN = TG::WN, WM = TG::WM;
  constexpr int PITCH = WN * ES + 16;    // bytes per staged row
  constexpr int CPR = WN * ES / 16;      // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;          // rows per wave instruction
  static_assert(32 * PITCH <= TG::TA::kBytes && 32 * PITCH <= TG::TB::kBytes,
                "a wave's strip must fit in one stage buffer");
  const int lane = threadIdx.x & 63, wid = (int)uniform(threadIdx.x >> 6);
  const int wm = wid >> 1, wn = wid & 1;
  // wave w stages in a[0], a[1], b[0], b[1]
  char* const strip = wid == 0 ? L.a[0] : wid == 1 ? L.a[1] : wid == 2 ? L.b[0] : L.b[1];
  const int n0 = wn * WN;
  constexpr int IT = 32 / RPI;  // row-phase iterations per strip
  uint32_t mw[EPI == EPI_MASK ? TG::FM * IT : 1];
  int cr[TG::FM * IT];  // destination row of each staged row this lane stores
#pragma unroll
  for (int j = 0; j < TG::FM; ++j)
#pragma unroll
    for (int t = 0; t < IT; ++t) {
      const int m = wm * WM + j * 32 + t * RPI + lane / CPR;
      cr[j * IT + t] = crow == nullptr ? m : (m < rows ? crow[m] : 0);
    }
  if constexpr (EPI == EPI_MASK) {
#pragma unroll
    for (int j = 0; j < TG::FM; ++j)
#pragma unroll
      for (int t = 0; t < IT; ++t) {
        const int m = wm * WM + j * 32 + t * RPI + lane / CPR;
        const int n = n0 + (lane % CPR) * 8;
        mw[j * IT + t] = m < rows ? aux[(size_t)m * ld_aux + n / 32] : 0u;
      }
  }
#pragma unroll
  for (int j = 0; j < TG::FM; ++j) {
    const int m0 = wm * WM + j * 32;
    // registers -> LDS
#pragma unroll
    for (int i = 0; i < TG::FN; ++i) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int c = i * 32 + 4 * (lane >> 5) + 8 * p;
        char* dst = strip + (lane & 31) * PITCH + c * ES;
        if constexpr (EPI == EPI_F32) {
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = tg.acc[i][j][4 * p + q];
          *reinterpret_cast<f32x4*>(dst) = v;
        } else {
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v = tg.acc[i][j][4 * p + q];
            if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.f);
            o[q] = (bf16)v;
          }
          *reinterpret_cast<bf16x4*>(dst) = o;
        }
      }
    }
    // LDS -> global, whole row pieces (LDS accesses of one wave stay in order)
#pragma unroll
    for (int t = 0; t < IT; ++t) {
      const int r = t * RPI + lane / CPR, c = (lane % CPR) * (16 / ES);
      const i32x4 v = *reinterpret_cast<const i32x4*>(strip + r * PITCH + c * ES);
      const int m = m0 + r, n = n0 + c;
      const bool ok = m < rows && n < cols;
      if (ok) {
        const size_t at = (size_t)cr[j * IT + t] * ldc + n;
        if constexpr (EPI == EPI_MASK) {
          const uint32_t keep = mw[j * IT + t] >> (n & 31);
          i32x4 o = v;
#pragma unroll
          for (int q = 0; q < 4; ++q)  // dword q holds elements 2q (low) and 2q+1
            o[q] &= (int)(((keep >> (2 * q)) & 1u ? 0x0000ffffu : 0u) |
                          ((keep >> (2 * q + 1)) & 1u ? 0xffff0000u : 0u));
          *reinterpret_cast<i32x4*>(reinterpret_cast<bf16*>(C) + at) = o;
        } else if constexpr (EPI == EPI_F32) {
          // weight gradients are written once and not read back here:
          // streaming stores keep them from evicting the operands
          __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(reinterpret_cast<OutT*>(C) + at));
        } else {
          *reinterpret_cast<i32x4*>(reinterpret_cast<OutT*>(C) + at) = v;
        }
      }
      if constexpr (EPI == EPI_RELU) {
        if (bits_out != nullptr) {
          // byte n/8 of row m: bit q <=> element n + q > 0.  Four consecutive
          // lanes hold 32 consecutive columns of one row (CPR is a multiple
          // of 4); the first of them stores the four bytes as one word.
          static_assert(CPR % 4 == 0, "a lane quad stays in one row");
          const bf16x8 hv = __builtin_bit_cast(bf16x8, v);
          uint32_t b = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q) b |= ((float)hv[q] > 0.f ? 1u : 0u) << q;
          const uint32_t b1 = __shfl_down(b, 1, 64), b2 = __shfl_down(b, 2, 64),
                         b3 = __shfl_down(b, 3, 64);
          if (ok && (lane & 3) == 0)
            *reinterpret_cast<uint32_t*>(bits_out + (size_t)m * (ldc / 8) + n / 8) =
                b | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
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
  const uint32_t* aux;  // EPI_MASK: keep bits, [rows][N / 32] words
  uint8_t* bits_out;    // EPI_RELU (optional): keep bits [C > 0], [rows][N / 8] bytes
  const int32_t* offsets;
  // MAP_GATHER_A: packed row r of A is row a_map[r] of A ([a_src_rows][K]);
  // MAP_SCATTER_C: packed row r is stored at row c_map[r] of C
  const int32_t* a_map;
  const int32_t* c_map;
  // split tail (null: off): float32 partial tiles, kMaxSplitUnits x BM x BN
  float* partial;
  long long b_stride;
  int K, N, E, a_src_rows;
  int cus;  // compute units: workgroups of one full round of tiles
};
enum RowMap { MAP_NONE = 0, MAP_GATHER_A = 1, MAP_SCATTER_C = 2 };

// Split tail.  With one workgroup per CU, a launch of `total` tiles runs
// total / cus full rounds and a last round that leaves most CUs idle when
// only a few tiles remain.  The first n_dp tiles run whole; each of the
// `tail` remaining tiles runs as s segments of its K range on separate
// workgroups (so the last round fills the chip), which store float32
// partial tiles; rows_fixup_kernel then sums each tile's segments in
// segment order and applies the epilogue.  Deterministic: the plan depends
// only on the tile count, K and the CU count.
constexpr int kMaxSplitUnits = 256;  // partial tiles the workspace holds
constexpr int kMaxRowTileArea = 256 * 128;  // largest row tile (256 x 128, 128 x 256)
constexpr int kMaxSplit = 16;
// A split pays only when it cuts the last round to a quarter or less: the
// fixup reads s partial tiles per tail tile (measured: 2-way splits of
// 16-step tiles cost more in the fixup than they save).
constexpr int kMinSplit = 4;
constexpr int kMinSplitSteps = 4;    // k steps (of kBK) per segment, at least
// Products with a shorter K are never split, so they launch no fixup (a
// launch costs ~5 us even when it finds nothing to do; a tile of K < 2048 is
// too short for a split to win that back).
constexpr int kMinSplitK = 2048;
struct SplitPlan {
  int n_dp, tail, s;
};
__host__ __device__ inline SplitPlan split_plan(int total, int nk, int cus, bool enabled) {
  SplitPlan p{total, 0, 1};
  if (!enabled || cus <= 0) return p;
  const int tail = total % cus;
  if (tail == 0) return p;
  const int fill = (cus < kMaxSplitUnits ? cus : kMaxSplitUnits) / tail;
  const int deep = nk / kMinSplitSteps;
  int s = fill < deep ? fill : deep;
  s = s < kMaxSplit ? s : kMaxSplit;
  if (s < kMinSplit) return p;
  p.n_dp = total - tail;
  p.tail = tail;
  p.s = s;
  return p;
}

// Per-expert m-tile counts and their prefix sum (shared arrays, whole block).
template <int BM>
__device__ __forceinline__ void rows_scan(const RowsArgs& p, int* s_off, int* s_tstart,
                                          int* s_scratch) {
  const int tid = threadIdx.x;
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

struct RowTile {
  int e, row0, rows, n0, cols;
};
// Row tiles of one expert run in groups of this many m-tiles, each group
// sweeping the n-tiles, so concurrent tiles share the expert's weight tiles.
constexpr int kGroupM = 8;

// Tile `logical` (whole block, uniform): expert by expert (tiles of expert e
// are logical [s_tstart[e] * NT, s_tstart[e+1] * NT)); inside an expert,
// groups of up to kGroupM m-tiles, n walked column by column inside a group.
// A group never mixes experts, so the workgroups running together on one XCD
// share one expert's weights.
template <int BM, int BN>
__device__ __forceinline__ RowTile find_tile(int logical, int NT, int N, int E, const int* s_off,
                                             const int* s_tstart, int* s_expert) {
  const int tid = threadIdx.x;
  if (tid < E && s_tstart[tid] * NT <= logical && logical < s_tstart[tid + 1] * NT)
    *s_expert = tid;
  __syncthreads();
  RowTile t;
  t.e = *s_expert;
  constexpr int G = kGroupM;
  const int mte = s_tstart[t.e + 1] - s_tstart[t.e];
  const int j = logical - s_tstart[t.e] * NT;
  const int grp = j / (G * NT);
  const int gm0 = grp * G;
  const int gsz = min(G, mte - gm0);
  const int in = j - grp * G * NT;
  const int mt = gm0 + in % gsz;  // m-tile within the expert
  const int nt = in / gsz;
  t.row0 = s_off[t.e] + mt * BM;
  t.rows = min(BM, s_off[t.e + 1] - t.row0);
  t.n0 = nt * BN;
  t.cols = min(BN, N - t.n0);
  return t;
}

// A partial tile in the accumulators' own layout: wave w, block (i, j),
// lane l holds 16 floats at ((w * FN + i) * FM + j) * 1024 + 16 l, element
// 4p + q being C[m][n] with m = 32 j + l % 32 and n = 32 i + 4 (l / 32) +
// 8p + q within the wave's WM x WN part (see TileGemm).
template <class TG>
__device__ __forceinline__ void store_partial(const TG& tg, float* dst) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < TG::FN; ++i)
#pragma unroll
    for (int j = 0; j < TG::FM; ++j) {
      f32x4* o = reinterpret_cast<f32x4*>(
          dst + ((size_t)(wid * TG::FN + i) * TG::FM + j) * 1024 + lane * 16);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = tg.acc[i][j][4 * p + q];
        o[p] = v;
      }
    }
}

// PERSIST (no split tail, p.partial null): one workgroup per CU walks its
// XCD's tiles; otherwise one workgroup per tile or split unit.  STREAM_B:
// the expert weights (B) are copied with the non-temporal hint.
template <int BM, int BN, bool B_K, int EPI, int MAP, bool PERSIST, bool STREAM_B>
__global__ void __launch_bounds__(kGemmThreads)
rows_gemm_kernel(RowsArgs p) {
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_tstart[MOE_MAX_EXPERTS + 1];
  __shared__ int s_scratch[kGemmThreads / 64 + 1];
  __shared__ int s_expert;
  rows_scan<BM>(p, s_off, s_tstart, s_scratch);
  const int MT = s_tstart[p.E];
  const int NT = (p.N + BN - 1) / BN;
  const int total = MT * NT;
  const int nk = p.K / kBK;
  using TG = TileGemm<BM, BN, true, B_K, false, 0, STREAM_B ? kNonTemporal : 0>;
  const StageBufs L = tile_lds<TG>();
  // one tile; seg >= 0: that K segment of a split tail tile, stored as a
  // partial tile (unit u)
  auto do_tile = [&](int logical, int seg, int s_parts, int u) {
    const RowTile t = find_tile<BM, BN>(logical, NT, p.N, p.E, s_off, s_tstart, &s_expert);
    const int k0 = seg < 0 ? 0 : (seg * nk / s_parts) * kBK;
    const int k1 = seg < 0 ? p.K : ((seg + 1) * nk / s_parts) * kBK;
    TG tg;
    const bf16* Bm = p.B + (size_t)t.e * p.b_stride;
    if constexpr (MAP == MAP_GATHER_A) {
      static_assert(B_K, "gathered rows are a forward (NT) product");
      tg.run(p.A + k0, p.K, t.rows, Bm + (size_t)t.n0 * p.K + k0, p.K, t.cols, k1 - k0, L,
             nullptr, p.a_map + t.row0, p.a_src_rows);
    } else {
      const bf16* A = p.A + (size_t)t.row0 * p.K + k0;
      if (B_K) {
        tg.run(A, p.K, t.rows, Bm + (size_t)t.n0 * p.K + k0, p.K, t.cols, k1 - k0, L);
      } else {
        tg.run(A, p.K, t.rows, Bm + (size_t)k0 * p.N + t.n0, p.N, t.cols, k1 - k0, L);
      }
    }
    if (seg >= 0) {
      store_partial(tg, p.partial + (size_t)u * (BM * BN));
      return;
    }
    if constexpr (MAP == MAP_SCATTER_C) {
      store_tile<EPI>(tg, L, p.C + t.n0, p.N, t.rows, t.cols, nullptr, 0, nullptr,
                      p.c_map + t.row0);
    } else {
      store_tile<EPI>(tg, L, p.C + (size_t)t.row0 * p.N + t.n0, p.N, t.rows, t.cols,
                      p.aux ? p.aux + (size_t)t.row0 * (p.N / 32) + t.n0 / 32 : nullptr, p.N / 32,
                      p.bits_out ? p.bits_out + (size_t)t.row0 * (p.N / 8) + t.n0 / 8 : nullptr);
    }
  };
  if constexpr (PERSIST) {
    // Persistent: workgroup b (on XCD b % 8) runs every (workgroups on its
    // XCD)-th tile of that XCD's contiguous range, so consecutive tiles of
    // one CU need no new workgroup and one XCD's L2 serves one expert group.
    const int G = gridDim.x, x = blockIdx.x % kXcds, w = blockIdx.x / kXcds;
    const int per_x = G / kXcds + (x < G % kXcds ? 1 : 0);
    const int q = total / kXcds, rmd = total % kXcds;
    const int lo = x * q + min(x, rmd), hi = lo + q + (x < rmd ? 1 : 0);
    for (int logical = lo + w; logical < hi; logical += per_x) {
      do_tile(logical, -1, 1, 0);
      // every wave has read its epilogue strip before the next tile's copies
      // reuse the stage buffers (LDS only: the stores may stay in flight)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  } else {
    const SplitPlan sp = split_plan(total, nk, p.cus, p.partial != nullptr);
    const int bid = blockIdx.x;
    if (bid < sp.n_dp) {
      // XCD-contiguous ranges: workgroup bid runs on XCD bid % 8.
      const int x = bid % kXcds, i = bid / kXcds;
      const int q = sp.n_dp / kXcds, rmd = sp.n_dp % kXcds;
      do_tile(x * q + min(x, rmd) + i, -1, 1, 0);
    } else {
      const int u = bid - sp.n_dp;  // split unit: tile n_dp + u / s, segment u % s
      if (u >= sp.tail * sp.s) return;
      do_tile(sp.n_dp + u / sp.s, u % sp.s, sp.s, u);
    }
  }
}

// Sum of the split tail's partial tiles (segment order) and the epilogue of
// rows_gemm_kernel on it: ReLU + keep bits, plain store, or the ReLU mask,
// bf16 rounding to nearest even, to the same destination rows.  Tail tile b
// is cut into fixup_parts(BM, BN) items of kGemmThreads / (BN / 8) rows each,
// dealt to the workgroups in turn; a thread takes 8 consecutive columns of
// one row and issues the loads of four segments ahead of their (in-order)
// sums.  One workgroup per CU: the launch follows every split-capable GEMM
// launch and must cost little when the device-side plan has no split.
constexpr int kFixupBlocks = 256;
constexpr int fixup_parts(int BM, int BN) { return BM / (kGemmThreads / (BN / 8)); }
template <int BM, int BN, int EPI, int MAP>
__global__ void __launch_bounds__(kGemmThreads)
rows_fixup_kernel(RowsArgs p) {
  constexpr int kFixupRows = kGemmThreads / (BN / 8);
  constexpr int kParts = fixup_parts(BM, BN);
  static_assert(kParts * kFixupRows == BM, "whole rows per item");
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_tstart[MOE_MAX_EXPERTS + 1];
  __shared__ int s_scratch[kGemmThreads / 64 + 1];
  __shared__ int s_expert;
  rows_scan<BM>(p, s_off, s_tstart, s_scratch);
  const int NT = (p.N + BN - 1) / BN;
  const SplitPlan sp = split_plan(s_tstart[p.E] * NT, p.K / kBK, p.cus, true);
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  for (int item = blockIdx.x; item < sp.tail * kParts; item += gridDim.x) {
    const int tb = item / kParts, part_rows = (item % kParts) * kFixupRows;
    const RowTile t = find_tile<BM, BN>(sp.n_dp + tb, NT, p.N, p.E, s_off, s_tstart, &s_expert);
    __syncthreads();  // every thread has read s_expert before the next item rewrites it
    const float* part = p.partial + (size_t)tb * sp.s * (BM * BN);
    const int g = threadIdx.x;
    const int m = part_rows + g / (BN / 8), n = (g % (BN / 8)) * 8;
    if (m >= t.rows || n >= t.cols) continue;
    const int wm = m / WM, j = (m % WM) / 32, ml = m % 32;
    const int wn = n / WN, i = (n % WN) / 32, pq = (n % 32) / 8;
    const size_t blk = ((size_t)((wm * 2 + wn) * FN + i) * FM + j) * 1024;
    const size_t o0 = blk + ml * 16 + 4 * pq, o1 = blk + (ml + 32) * 16 + 4 * pq;
    float v[8];  // -0 is the identity of +, so v becomes exactly segment 0 first
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = -0.f;
    for (int s0 = 0; s0 < sp.s; s0 += 4) {
      f32x4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (s0 + u < sp.s) {
          const float* ps = part + (size_t)(s0 + u) * (BM * BN);
          a[u] = *reinterpret_cast<const f32x4*>(ps + o0);
          b[u] = *reinterpret_cast<const f32x4*>(ps + o1);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (s0 + u < sp.s) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] += a[u][q];
            v[4 + q] += b[u][q];
          }
        }
      }
    }
    const int row = t.row0 + m, col = t.n0 + n;
    const size_t orow = MAP == MAP_SCATTER_C ? (size_t)p.c_map[row] : (size_t)row;
    bf16x8 o;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = (bf16)(EPI == EPI_RELU ? fmaxf(v[q], 0.f) : v[q]);
    if constexpr (EPI == EPI_MASK) {
      const uint32_t keep = p.aux[(size_t)row * (p.N / 32) + col / 32] >> (col % 32);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (!((keep >> q) & 1u)) o[q] = __builtin_bit_cast(bf16, (uint16_t)0);
    }
    *reinterpret_cast<bf16x8*>(p.C + orow * p.N + col) = o;
    if constexpr (EPI == EPI_RELU) {
      if (p.bits_out != nullptr) {
        uint32_t b = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) b |= ((float)o[q] > 0.f ? 1u : 0u) << q;
        p.bits_out[(size_t)row * (p.N / 8) + col / 8] = (uint8_t)b;
      }
    }
  }
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
  int32_t* next_tile;  // tile queue: zero at launch
  // Replicas (null rep_start: none).  Copy p = rep_start[e] + c of expert e
  // takes the packed rows [rep_row0[p], rep_row0[p] + rep_rows[p]).  An
  // expert split over its copies gets one float32 partial dW per copy
  // (part [slot][N1][N2], gate partials gpart [slot][N2], dbpart [slot]),
  // summed in copy order by wgrad_reduce_kernel.
  const int32_t* rep_start;
  const int32_t* rep_row0;
  const int32_t* rep_rows;
  float* part;
  float* gpart;
  float* dbpart;
  int n_copies, max_slots;  // sizes of rep_row0 / rep_rows and of part
  int tiles_per_copy, grid;  // output tiles of one expert; workgroups launched
  int N1, N2, E;
};

// Per-expert copy counts in the schedule and the partial slots of the
// experts split over their copies (LDS, whole block): s_nc[e] copies (1 when
// not split), s_slot[e] first slot or -1.
//
// An expert with several copies is split over them only where that can
// shorten the schedule: when one of its unsplit tiles (a K loop over all its
// rows) would take longer than a workgroup's mean share of the whole launch,
// rows_e * grid > tiles_per_copy * rows of all experts.  Otherwise its tiles
// run over all its rows, exactly as without copies, and the tile queue
// balances the load by itself.  The rule reads only the offsets and the
// launch shape, so both kernels of a launch (and every call with the same
// inputs) take the same decision.
__device__ __forceinline__ void wgrad_copies(const WgradArgs& p, int* s_nc, int* s_slot,
                                             int* s_scratch) {
  const int tid = threadIdx.x;
  int nc = 1;
  if (tid < p.E && p.rep_start != nullptr) {
    nc = p.rep_start[tid + 1] - p.rep_start[tid];
    const long long rows = p.offsets[tid + 1] - p.offsets[tid];
    const long long all_rows = p.offsets[p.E];
    if (nc > 1 && rows * p.grid <= (long long)p.tiles_per_copy * all_rows) nc = 1;
  }
  const int multi = (tid < p.E && nc > 1) ? nc : 0;
  int total;
  const int ex = block_exclusive_scan(multi, s_scratch, &total);
  if (tid < p.E) {
    s_nc[tid] = nc;
    s_slot[tid] = multi > 0 ? ex : -1;
  }
}

// Persistent: one workgroup per CU takes tiles from a queue (an atomic
// counter) in longest-processing-time order - the experts by decreasing row
// count (ties by index), a split expert's copies in order, each copy's tiles
// row by row - so the long K loops of popular experts start first and the
// short ones fill in behind them.  A tile's float32 dW leaves through non-temporal
// stores that stay in flight while the next tile's k loop runs (only LDS is
// fenced between tiles).  Which workgroup takes which tile varies; each tile
// is computed the same way, so the results are bitwise reproducible.
// Experts with no rows store zeros.  An expert that is not split (always,
// without replicas) computes exactly the unreplicated tiles.
//
// With GATE, the tiles of the first N1 tile row also produce the gate's
// weight gradient over the same rows, dW_gate[:, e] = X2_e^T gsel_e and
// db[e] = sum(gsel_e), from the X2 tiles they already stream (for FC1's
// weight gradient X2 is x_perm and gsel the gate-softmax gradient per row).
template <int BM, int BN, bool GATE>
__global__ void __launch_bounds__(kGemmThreads)
wgrad_kernel(WgradArgs p) {
  __shared__ int s_perm[MOE_MAX_EXPERTS];
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  __shared__ int s_nc[MOE_MAX_EXPERTS];
  __shared__ int s_slot[MOE_MAX_EXPERTS];
  __shared__ int s_tpre[MOE_MAX_EXPERTS + 1];  // first tile of each expert rank
  __shared__ int s_scratch[kGemmThreads / 64 + 1];
  __shared__ int s_tile;
  const int tid = threadIdx.x;
  if (tid < p.E) s_cnt[tid] = p.offsets[tid + 1] - p.offsets[tid];
  wgrad_copies(p, s_nc, s_slot, s_scratch);  // (ends with a barrier)
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
  {
    const int nt = tid < p.E ? s_nc[s_perm[tid]] * per : 0;
    int total;
    const int ex = block_exclusive_scan(nt, s_scratch, &total);
    if (tid < p.E) s_tpre[tid] = ex;
    if (tid == 0) s_tpre[p.E] = total;
  }
  using TG = TileGemm<BM, BN, false, false, GATE>;
  const StageBufs L = tile_lds<TG>();
  for (;;) {
    if (tid == 0) s_tile = atomicAdd(p.next_tile, 1);
    __syncthreads();  // s_tpre written; s_tile visible
    const int tile = s_tile;
    if (tile >= s_tpre[p.E]) break;
    int lo = 0, hi = p.E - 1;  // expert rank holding this tile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tpre[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int e = s_perm[lo], j = tile - s_tpre[lo];
    const int c = j / per, in = j % per;
    const int t1 = in / T2, t2 = in % T2;
    const int n1 = t1 * BM, n2 = t2 * BN;
    int r0 = p.offsets[e], K = s_cnt[e];
    if (p.rep_start != nullptr && s_nc[e] > 1) {
      // a copy's rows, kept inside the expert's own rows whatever the plan
      // holds (copies that do not tile the rows give unspecified results,
      // never an access outside the operands)
      const int cp = p.rep_start[e] + c;
      const bool ok = cp >= 0 && cp < p.n_copies;
      const int a = ok ? p.rep_row0[cp] : r0;
      const int n = ok ? p.rep_rows[cp] : 0;
      const int lo_r = r0, hi_r = r0 + K;
      r0 = min(max(a, lo_r), hi_r);
      K = max(0, min(n, hi_r - r0));
    }
    const int slot = s_slot[e] < 0 ? -1 : s_slot[e] + c;
    if (slot >= p.max_slots) {  // more copies than the plan's size: skipped
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      continue;
    }
    const int rows = min(BM, p.N1 - n1), cols = min(BN, p.N2 - n2);
    TG tg;
    const bool gate_here = GATE && t1 == 0;
    tg.run(p.X1 + (size_t)r0 * p.N1 + n1, p.N1, rows, p.X2 + (size_t)r0 * p.N2 + n2, p.N2, cols,
           K, L, gate_here ? p.gsel + r0 : nullptr);
    float* dst = slot < 0 ? p.C + (size_t)e * p.N1 * p.N2 : p.part + (size_t)slot * p.N1 * p.N2;
    store_tile<EPI_F32>(tg, L, dst + (size_t)n1 * p.N2 + n2, p.N2, rows, cols, nullptr, 0);
    if constexpr (GATE) {
      if (gate_here) {
        __syncthreads();
        if (slot < 0)
          tg.gate_reduce(reinterpret_cast<float*>(L.a[0]), cols,
                         p.dw_gate + (size_t)n2 * p.E + e, p.E,
                         t2 == 0 ? p.db_gate + e : nullptr);
        else
          tg.gate_reduce(reinterpret_cast<float*>(L.a[0]), cols,
                         p.gpart + (size_t)slot * p.N2 + n2, 1,
                         t2 == 0 ? p.dbpart + slot : nullptr);
      }
    }
    // every wave has read its epilogue strip (and the gate sums) before the
    // next tile's copies reuse the stage buffers, and thread 0 has read
    // s_tile before the next take rewrites it; the dW stores stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// Weight gradients of the experts split over their copies: the sum of the
// copies' partial dW in copy order (the fixed-order reduction a replicated
// expert's gradient needs), plus, with gate partials, dW_gate[:, e] and db[e].
// Every workgroup walks the split experts in index order (none: it exits at
// once), its threads striding over each one's N1 x N2 elements, 4 per thread.
__global__ void __launch_bounds__(256)
wgrad_reduce_kernel(WgradArgs p) {
  __shared__ int s_nc[MOE_MAX_EXPERTS];
  __shared__ int s_slot[MOE_MAX_EXPERTS];
  __shared__ int s_scratch[256 / 64 + 1];
  wgrad_copies(p, s_nc, s_slot, s_scratch);
  __syncthreads();
  const size_t n = (size_t)p.N1 * p.N2;  // a multiple of 4 (N2 is)
  for (int e = 0; e < p.E; ++e) {
    const int nc = s_nc[e], slot0 = s_slot[e];
    if (nc <= 1 || slot0 + nc > p.max_slots) continue;  // not split / beyond the plan's size
    float* dst = p.C + (size_t)e * n;
    for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n;
         i += (size_t)gridDim.x * 256 * 4) {
      f32x4 acc = *reinterpret_cast<const f32x4*>(p.part + (size_t)slot0 * n + i);
      for (int c = 1; c < nc; ++c) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p.part + (size_t)(slot0 + c) * n + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += v[q];
      }
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(dst + i));
    }
    if (p.gpart != nullptr && (int)blockIdx.x == e % (int)gridDim.x) {
      for (int i = threadIdx.x; i < p.N2; i += 256) {
        float acc = p.gpart[(size_t)slot0 * p.N2 + i];
        for (int c = 1; c < nc; ++c) acc += p.gpart[(size_t)(slot0 + c) * p.N2 + i];
        p.dw_gate[(size_t)i * p.E + e] = acc;
      }
      if (threadIdx.x == 0) {
        float acc = p.dbpart[slot0];
        for (int c = 1; c < nc; ++c) acc += p.dbpart[slot0 + c];
        p.db_gate[e] = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Keep bits of the ReLU for the FC1 input gradient: bit q of word w is
// h[32 w + q] > 0 over the packed rows [0, offsets[E]) of h [rows][F] (F is a
// multiple of 32, so a word never spans two rows).  The dgrad epilogue then
// reads one bit per element instead of h.
__global__ void __launch_bounds__(256)
relu_bits_kernel(const bf16* __restrict__ h, const int32_t* __restrict__ offsets, int E, int F,
                 uint32_t* __restrict__ bits) {
  const long long total = (long long)offsets[E] * (F / 32);
  for (long long w = (long long)blockIdx.x * 256 + threadIdx.x; w < total;
       w += (long long)gridDim.x * 256) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(h + w * 32);
    uint32_t b = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 v = src[q];
#pragma unroll
      for (int t = 0; t < 8; ++t) b |= ((float)v[t] > 0.f ? 1u : 0u) << (q * 8 + t);
    }
    bits[w] = b;
  }
}

// ---------------------------------------------------------------------------
// float32 path (act = MOE_F32): FMA kernels, no reduced precision.  Operands
// are staged through LDS in k chunks; every output still accumulates its k
// terms in increasing k order, one fmaf each, as a plain loop would.
constexpr int kF32Rows = 16;
constexpr int kF32Chunk = 32;  // k (rows of the expert for dW) per LDS chunk

// C[r][n] = epi(sum_k A[r][k] B_e(n, k)); B_e(n,k) = B[e][n][k] (B_K) or B[e][k][n].
// A workgroup takes 16 consecutive packed rows and 64 columns; its rows lie
// in a contiguous range of experts (rows are packed by expert), and each
// expert of that range gets its own pass over B_e.  Thread (row r, lane g)
// computes columns g, g + 16, g + 32, g + 48.
// Optional maps as in RowsArgs: A row a_map[r], C row c_map[r] (null: r).
template <bool B_K, int EPI>
__global__ void __launch_bounds__(256)
f32_rows_kernel(const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C,
                const float* __restrict__ aux, const int32_t* __restrict__ offsets, int K, int N,
                int E, int S_max, const int32_t* __restrict__ a_map,
                const int32_t* __restrict__ c_map) {
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ float sa[kF32Rows][kF32Chunk + 1];
  __shared__ float sb[64][kF32Chunk + 1];
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += 256) s_off[i] = offsets[i];
  __syncthreads();
  const int rows = min(s_off[E], S_max);
  const int rb = blockIdx.x * kF32Rows;
  if (rb >= rows) return;  // (the whole workgroup)
  const int rl = min(rb + kF32Rows, rows) - 1;  // last live row of the workgroup
  auto expert_of = [&](int row) {
    int e = 0;
    while (!(s_off[e] <= row && row < s_off[e + 1])) ++e;
    return e;
  };
  const int lr = tid >> 4, g = tid & 15;
  const int r = rb + lr;
  const bool live = r <= rl;
  const int e = live ? expert_of(r) : -1;
  const int e_first = expert_of(rb), e_last = expert_of(rl);
  const int n0 = blockIdx.y * 64;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int ee = e_first; ee <= e_last; ++ee) {
    if (s_off[ee] == s_off[ee + 1]) continue;  // no rows (same for the whole workgroup)
    const float* b = B + (size_t)ee * N * K;
    for (int k0 = 0; k0 < K; k0 += kF32Chunk) {
      __syncthreads();  // the previous chunk has been used
      for (int i = tid; i < kF32Rows * kF32Chunk; i += 256) {
        const int rr = i / kF32Chunk, kk = i % kF32Chunk, row = rb + rr, k = k0 + kk;
        sa[rr][kk] = (row <= rl && k < K) ? A[(size_t)(a_map ? a_map[row] : row) * K + k] : 0.f;
      }
      for (int i = tid; i < 64 * kF32Chunk; i += 256) {
        // B_K: consecutive threads along k, else along n (both read memory in order)
        const int nn = B_K ? i / kF32Chunk : i % 64, kk = B_K ? i % kF32Chunk : i / 64;
        const int n = n0 + nn, k = k0 + kk;
        sb[nn][kk] = (n < N && k < K) ? (B_K ? b[(size_t)n * K + k] : b[(size_t)k * N + n]) : 0.f;
      }
      __syncthreads();
      if (e == ee) {
        const int kn = min(kF32Chunk, K - k0);
        for (int kk = 0; kk < kn; ++kk) {
          const float av = sa[lr][kk];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = fmaf(av, sb[g + 16 * q][kk], acc[q]);
        }
      }
    }
  }
  if (!live) return;
  const size_t cr = (size_t)(c_map ? c_map[r] : r);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n0 + g + 16 * q;
    if (n >= N) continue;
    float v = acc[q];
    if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
    if (EPI == EPI_MASK && !(aux[(size_t)r * N + n] > 0.f)) v = 0.f;
    C[cr * N + n] = v;
  }
}

// dW[e][n1][n2] = sum over e's rows m of X1[m][n1] X2[m][n2]: a workgroup
// takes 16 n1 x 64 n2 of one expert and stages chunks of its rows; thread
// (n1, lane g) computes n2 = g, g + 16, g + 32, g + 48.
__global__ void __launch_bounds__(256)
f32_wgrad_kernel(const float* __restrict__ X1, const float* __restrict__ X2, float* __restrict__ C,
                 const int32_t* __restrict__ offsets, int N1, int N2) {
  __shared__ float s1[kF32Chunk][16 + 1];
  __shared__ float s2[kF32Chunk][64 + 1];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int n1b = blockIdx.y * 16, n2b = blockIdx.z * 64;
  const int l1 = tid >> 4, g = tid & 15;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int m0 = r0; m0 < r1; m0 += kF32Chunk) {
    __syncthreads();  // the previous chunk has been used
    for (int i = tid; i < kF32Chunk * 16; i += 256) {
      const int mm = i / 16, c = i % 16, m = m0 + mm;
      s1[mm][c] = (m < r1 && n1b + c < N1) ? X1[(size_t)m * N1 + n1b + c] : 0.f;
    }
    for (int i = tid; i < kF32Chunk * 64; i += 256) {
      const int mm = i / 64, c = i % 64, m = m0 + mm;
      s2[mm][c] = (m < r1 && n2b + c < N2) ? X2[(size_t)m * N2 + n2b + c] : 0.f;
    }
    __syncthreads();
    const int mn = min(kF32Chunk, r1 - m0);
    for (int mm = 0; mm < mn; ++mm) {
      const float x1 = s1[mm][l1];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(x1, s2[mm][g + 16 * q], acc[q]);
    }
  }
  const int n1 = n1b + l1;
  if (n1 >= N1) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n2 = n2b + g + 16 * q;
    if (n2 < N2) C[((size_t)e * N1 + n1) * N2 + n2] = acc[q];
  }
}

// Every kernel variant the launchers can pick, instantiated explicitly (so
// each is emitted whatever order the launchers reference them in).
#define MOE_ROWS_PERSIST(BM, BN, P, W)                                                           \
  template __global__ void rows_gemm_kernel<BM, BN, true, EPI_RELU, MAP_NONE, P, W>(RowsArgs);     \
  template __global__ void rows_gemm_kernel<BM, BN, true, EPI_STORE, MAP_NONE, P, W>(RowsArgs);    \
  template __global__ void rows_gemm_kernel<BM, BN, false, EPI_MASK, MAP_NONE, P, W>(RowsArgs);    \
  template __global__ void rows_gemm_kernel<BM, BN, false, EPI_STORE, MAP_NONE, P, W>(RowsArgs);   \
  template __global__ void rows_gemm_kernel<BM, BN, true, EPI_RELU, MAP_GATHER_A, P, W>(RowsArgs); \
  template __global__ void rows_gemm_kernel<BM, BN, true, EPI_STORE, MAP_SCATTER_C, P, W>(RowsArgs);
#define MOE_ROWS_VARIANTS(BM, BN)                                                      \
  MOE_ROWS_PERSIST(BM, BN, true, false)                                                        \
  MOE_ROWS_PERSIST(BM, BN, false, false)                                                       \
  MOE_ROWS_PERSIST(BM, BN, true, true)                                                         \
  MOE_ROWS_PERSIST(BM, BN, false, true)                                                        \
  template __global__ void rows_fixup_kernel<BM, BN, EPI_RELU, MAP_NONE>(RowsArgs);            \
  template __global__ void rows_fixup_kernel<BM, BN, EPI_STORE, MAP_NONE>(RowsArgs);           \
  template __global__ void rows_fixup_kernel<BM, BN, EPI_MASK, MAP_NONE>(RowsArgs);            \
  template __global__ void rows_fixup_kernel<BM, BN, EPI_RELU, MAP_GATHER_A>(RowsArgs);        \
  template __global__ void rows_fixup_kernel<BM, BN, EPI_STORE, MAP_SCATTER_C>(RowsArgs);
#define MOE_WGRAD_VARIANTS(BM, BN)                                   \
  template __global__ void wgrad_kernel<BM, BN, false>(WgradArgs);   \
  template __global__ void wgrad_kernel<BM, BN, true>(WgradArgs);
// (a 256 x 256 row tile holds 256 accumulators per lane and would spill)
MOE_ROWS_VARIANTS(256, 128)
MOE_ROWS_VARIANTS(128, 256)
MOE_ROWS_VARIANTS(128, 128)
MOE_WGRAD_VARIANTS(256, 256)
MOE_WGRAD_VARIANTS(256, 128)
MOE_WGRAD_VARIANTS(128, 256)
MOE_WGRAD_VARIANTS(128, 128)
#undef MOE_ROWS_VARIANTS
#undef MOE_ROWS_PERSIST
#undef MOE_WGRAD_VARIANTS

// ---------------------------------------------------------------------------
// launchers

#define MOE_TRY(expr)                         \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return _e;          \
  } while (0)

// Compute units of the current device (tiles per full round), cached per
// device.
static int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

// Tile shape per product.  Row-grouped products: a small cost model, time ~
// (rounds of one tile per CU) x (tile area) / (relative speed of the shape on
// random bf16 data: 128x256 and 256x128 tiles do the most work per cycle,
// 128x128 the least; 256x256 is left out, its accumulators leave too few
// registers), with the row tiles estimated as an even spread of
// S_max rows plus half a ragged tile per expert, and a split last round
// costing 1/s of a round plus the fixup.  Weight gradients: the largest
// tiles that still give every CU two.
struct Shape2 {
  int bm, bn;
};
static Shape2 pick_rows_tile(int S_max, int E, int K, int N, int cus, bool split) {
  struct C {
    int bm, bn;
    double speed;
  };
  const C cand[] = {{128, 256, 1.15}, {256, 128, 1.12}, {128, 128, 0.95}};
  Shape2 best{128, 128};
  double best_t = 1e300;
  for (const C& c : cand) {
    const int tiles = ((S_max + c.bm - 1) / c.bm + E / 2) * ((N + c.bn - 1) / c.bn);
    const SplitPlan sp = split_plan(tiles, K / kBK, cus, split);
    const double rounds = sp.s > 1 ? sp.n_dp / cus + 1.0 / sp.s + 0.1
                                   : std::ceil((double)tiles / cus);
    const double t = rounds * c.bm * c.bn / c.speed;
    if (t < best_t) {
      best_t = t;
      best = {c.bm, c.bn};
    }
  }
  return best;
}
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

template <int BM, int BN, bool B_K, int EPI, int MAP, bool STREAM_B>
static hipError_t launch_rows_t(const RowsArgs& p, int S_max, hipStream_t s) {
  static_assert(BM * BN <= kMaxRowTileArea, "partial tiles must fit the workspace");
  // worst case: sum over experts of ceil(rows_e / BM) <= S_max / BM + E
  // tiles, plus up to kMaxSplitUnits segments replacing the split tail
  const long long mt_max = (S_max + BM - 1) / BM + p.E;
  const long long nt = (p.N + BN - 1) / BN;
  // without a split tail the kernel is persistent: one workgroup per CU
  const long long grid = p.partial != nullptr ? mt_max * nt + kMaxSplitUnits
                                              : std::min<long long>(mt_max * nt, p.cus);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.partial != nullptr)
    hipLaunchKernelGGL((rows_gemm_kernel<BM, BN, B_K, EPI, MAP, false, STREAM_B>),
                       dim3((unsigned)grid), dim3(kGemmThreads), 0, s, p);
  else
    hipLaunchKernelGGL((rows_gemm_kernel<BM, BN, B_K, EPI, MAP, true, STREAM_B>),
                       dim3((unsigned)grid), dim3(kGemmThreads), 0, s, p);
  if (p.partial != nullptr) {
    MOE_TRY(hipGetLastError());
    hipLaunchKernelGGL((rows_fixup_kernel<BM, BN, EPI, MAP>),
                       dim3(kFixupBlocks), dim3(kGemmThreads), 0, s, p);
  }
  return hipGetLastError();
}

// max_rows: the most rows one expert can hold (its capacity).  When no
// expert can need more than one group of m-tiles, the tiles that share a
// weight tile all run together, so the weights are read once per launch and
// are copied with the streaming hint (they then leave the caches to the
// activations that later launches re-read).  With more m-tiles per expert
// the later groups re-read the weight tiles, which must stay cached.
template <bool B_K, int EPI, int MAP, int BM, int BN>
static hipError_t launch_rows_s(const RowsArgs& p, int S_max, int max_rows, hipStream_t s) {
  if ((max_rows + BM - 1) / BM <= kGroupM)
    return launch_rows_t<BM, BN, B_K, EPI, MAP, true>(p, S_max, s);
  return launch_rows_t<BM, BN, B_K, EPI, MAP, false>(p, S_max, s);
}
template <bool B_K, int EPI, int MAP = MAP_NONE>
static hipError_t launch_rows(const bf16* A, const bf16* B, bf16* C, const uint32_t* aux,
                              const int32_t* offsets, long long b_stride, int K, int N, int E,
                              int S_max, int max_rows, float* partial, hipStream_t s,
                              uint32_t* bits_out = nullptr, const int32_t* a_map = nullptr,
                              const int32_t* c_map = nullptr, int a_src_rows = 0) {
  const int cus = device_cus();
  if (K < kMinSplitK) partial = nullptr;
  RowsArgs p{A, B, C, aux, reinterpret_cast<uint8_t*>(bits_out), offsets, a_map, c_map,
             partial, b_stride, K, N, E, a_src_rows, cus};
  const Shape2 t = pick_rows_tile(S_max, E, K, N, cus, partial != nullptr);
  if (t.bm == 256 && t.bn == 128)
    return launch_rows_s<B_K, EPI, MAP, 256, 128>(p, S_max, max_rows, s);
  if (t.bm == 128 && t.bn == 256)
    return launch_rows_s<B_K, EPI, MAP, 128, 256>(p, S_max, max_rows, s);
  return launch_rows_s<B_K, EPI, MAP, 128, 128>(p, S_max, max_rows, s);
}

template <int BM, int BN, bool GATE>
static hipError_t launch_wgrad_t(WgradArgs p, int n_copies, hipStream_t s) {
  p.tiles_per_copy = ((p.N1 + BM - 1) / BM) * ((p.N2 + BN - 1) / BN);
  const long long tiles = (long long)n_copies * p.tiles_per_copy;
  // one workgroup per CU (at most as many as the tiles of a schedule that
  // splits every expert over all its copies)
  p.grid = (int)std::min<long long>(tiles, device_cus());
  hipLaunchKernelGGL((wgrad_kernel<BM, BN, GATE>), dim3((unsigned)p.grid), dim3(kGemmThreads),
                     0, s, p);
  MOE_TRY(hipGetLastError());
  if (p.rep_start != nullptr && n_copies > p.E) {
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(2 * device_cus()), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

// Replicas of the weight-gradient GEMMs (see WgradArgs); null = none.
struct WgradReplicas {
  const int32_t* start;
  const int32_t* row0;
  const int32_t* rows;
  int n_copies;
  float* part;
  float* gpart;
  float* dbpart;
};

template <bool GATE>
static hipError_t launch_wgrad(const bf16* X1, const bf16* X2, float* C, const int32_t* offsets,
                               const float* gsel, float* dw_gate, float* db_gate,
                               int32_t* next_tile, int N1, int N2, int E,
                               const WgradReplicas* rep, hipStream_t s) {
  const int max_slots = rep && rep->n_copies > E ? 2 * (rep->n_copies - E) : 0;
  WgradArgs p{X1, X2, C, offsets, gsel, dw_gate, db_gate, next_tile,
              rep ? rep->start : nullptr, rep ? rep->row0 : nullptr, rep ? rep->rows : nullptr,
              rep ? rep->part : nullptr, rep && GATE ? rep->gpart : nullptr,
              rep && GATE ? rep->dbpart : nullptr, rep ? rep->n_copies : 0, max_slots,
              0, 0, N1, N2, E};
  const int n_copies = rep ? rep->n_copies : E;
  auto mt = [&](int bm) { return (long long)E * ((N1 + bm - 1) / bm); };
  const Shape2 t = pick_tile(mt, N2);
  if (t.bm == 256 && t.bn == 256) return launch_wgrad_t<256, 256, GATE>(p, n_copies, s);
  if (t.bm == 256 && t.bn == 128) return launch_wgrad_t<256, 128, GATE>(p, n_copies, s);
  if (t.bm == 128 && t.bn == 256) return launch_wgrad_t<128, 256, GATE>(p, n_copies, s);
  return launch_wgrad_t<128, 128, GATE>(p, n_copies, s);
}

// Bytes of float32 partial tiles a row-grouped launch may use: the split
// tail never holds more than kMaxSplitUnits tiles of the largest row tile.
size_t wgrad_replica_bytes(int n_copies, int E, int d, int F) {
  const size_t slots = n_copies > E ? 2 * (size_t)(n_copies - E) : 0;
  return slots * ((size_t)d * F + d + 1) * sizeof(float);
}

size_t rows_partial_bytes(int act) {
  return act == MOE_BF16 ? (size_t)kMaxSplitUnits * kMaxRowTileArea * sizeof(float) : 0;
}

hipError_t launch_expert_fwd(int act, const void* x_perm, const int32_t* offsets, const void* w1,
                             const void* w2, void* h, void* out_perm, uint32_t* relu_bits,
                             float* partial, int S_max, int max_rows, int d, int F, int E,
                             hipStream_t s) {
  if (act == MOE_BF16) {
    MOE_TRY((launch_rows<true, EPI_RELU>((const bf16*)x_perm, (const bf16*)w1, (bf16*)h, nullptr,
                                         offsets, (long long)F * d, d, F, E, S_max, max_rows,
                                         partial, s, relu_bits)));
    MOE_TRY((launch_rows<true, EPI_STORE>((const bf16*)h, (const bf16*)w2, (bf16*)out_perm,
                                          nullptr, offsets, (long long)d * F, F, d, E, S_max,
                                          max_rows, partial, s)));
    return hipSuccess;
  }
  dim3 b(256);
  dim3 g1((S_max + kF32Rows - 1) / kF32Rows, (F + 63) / 64),
      g2((S_max + kF32Rows - 1) / kF32Rows, (d + 63) / 64);
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_RELU>), g1, b, 0, s, (const float*)x_perm,
                     (const float*)w1, (float*)h, nullptr, offsets, d, F, E, S_max, nullptr,
                     nullptr);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_STORE>), g2, b, 0, s, (const float*)h,
                     (const float*)w2, (float*)out_perm, nullptr, offsets, F, d, E, S_max,
                     nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_expert_fwd_fused(int act, const void* x, const int32_t* row_token, int T,
                                   const int32_t* offsets, const int32_t* row_slot,
                                   const void* w1, const void* w2, void* h, void* out_slot,
                                   uint32_t* relu_bits, float* partial, int S_max, int max_rows,
                                   int d, int F, int E, hipStream_t s) {
  if (act == MOE_BF16) {
    // FC1 reads token rows x[row_token[r]]; FC2 stores row r at slot row_slot[r]
    MOE_TRY((launch_rows<true, EPI_RELU, MAP_GATHER_A>(
        (const bf16*)x, (const bf16*)w1, (bf16*)h, nullptr, offsets, (long long)F * d, d, F, E,
        S_max, max_rows, partial, s, relu_bits, row_token, nullptr, T)));
    MOE_TRY((launch_rows<true, EPI_STORE, MAP_SCATTER_C>(
        (const bf16*)h, (const bf16*)w2, (bf16*)out_slot, nullptr, offsets, (long long)d * F, F,
        d, E, S_max, max_rows, partial, s, nullptr, nullptr, row_slot, 0)));
    return hipSuccess;
  }
  dim3 b(256);
  dim3 g1((S_max + kF32Rows - 1) / kF32Rows, (F + 63) / 64),
      g2((S_max + kF32Rows - 1) / kF32Rows, (d + 63) / 64);
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_RELU>), g1, b, 0, s, (const float*)x,
                     (const float*)w1, (float*)h, nullptr, offsets, d, F, E, S_max, row_token,
                     nullptr);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL((f32_rows_kernel<true, EPI_STORE>), g2, b, 0, s, (const float*)h,
                     (const float*)w2, (float*)out_slot, nullptr, offsets, F, d, E, S_max,
                     nullptr, row_slot);
  return hipGetLastError();
}

hipError_t launch_expert_bwd(int act, const void* d_out, const void* x_perm, const void* h,
                             const int32_t* offsets, const void* w1, const void* w2, void* dz,
                             void* dx_perm, float* dw1, float* dw2, const float* dsel_perm,
                             float* dw_gate, float* db_gate, const uint32_t* relu_bits_in,
                             uint32_t* relu_bits_ws, float* partial, int32_t* counters,
                             int S_max, int max_rows, int d, int F, int E, hipStream_t s,
                             const int32_t* rep_start, const int32_t* rep_row0,
                             const int32_t* rep_rows, int n_copies, float* rep_part) {
  const size_t rep_slots = n_copies > E ? 2 * (size_t)(n_copies - E) : 0;
  const WgradReplicas rep{rep_start, rep_row0, rep_rows, n_copies, rep_part,
                          rep_part + rep_slots * (size_t)d * F,
                          rep_part + rep_slots * (size_t)d * F + rep_slots * (size_t)d};
  const WgradReplicas* repp = rep_start != nullptr ? &rep : nullptr;
  if (act == MOE_BF16) {
    // keep bits of the ReLU (unless the forward kept them), then
    // dz = (dO W2[e]) * [h > 0]: A = dO [rows][d], B = W2[e] as [K=d][N=F]
    const uint32_t* relu_bits = relu_bits_in;
    if (relu_bits == nullptr) {
      const long long words = (long long)S_max * (F / 32);
      const int blocks = (int)std::min<long long>((words + 255) / 256, 4096);
      hipLaunchKernelGGL(relu_bits_kernel, dim3(std::max(blocks, 1)), dim3(256), 0, s,
                         (const bf16*)h, offsets, E, F, relu_bits_ws);
      MOE_TRY(hipGetLastError());
      relu_bits = relu_bits_ws;
    }
    MOE_TRY((launch_rows<false, EPI_MASK>((const bf16*)d_out, (const bf16*)w2, (bf16*)dz,
                                          relu_bits, offsets, (long long)d * F, d, F, E, S_max,
                                          max_rows, partial, s)));
    // dW2[e] = dO^T h  ([d][F])
    MOE_TRY((launch_wgrad<false>((const bf16*)d_out, (const bf16*)h, dw2, offsets, nullptr,
                                 nullptr, nullptr, counters, d, F, E, repp, s)));
    // dW1[e] = dz^T x_perm  ([F][d]), with the gate's dW_gate / db over the kept rows
    MOE_TRY((launch_wgrad<true>((const bf16*)dz, (const bf16*)x_perm, dw1, offsets, dsel_perm,
                                dw_gate, db_gate, counters + 1, F, d, E, repp, s)));
    // dx_perm = dz W1[e]: A = dz [rows][F], B = W1[e] as [K=F][N=d]  (may reuse dO's
    // memory: it runs after the last reader of dO).  Last of the four, so the
    // decode of dX that follows reads dx_perm while it is still cached.
    MOE_TRY((launch_rows<false, EPI_STORE>((const bf16*)dz, (const bf16*)w1, (bf16*)dx_perm,
                                           nullptr, offsets, (long long)F * d, F, d, E, S_max,
                                           max_rows, partial, s)));
    return hipSuccess;
  }
  if (rep_start != nullptr) return hipErrorInvalidValue;  // replicas: bf16 only
  dim3 b(256);
  const int rt = (S_max + kF32Rows - 1) / kF32Rows;
  hipLaunchKernelGGL((f32_rows_kernel<false, EPI_MASK>), dim3(rt, (F + 63) / 64), b, 0, s,
                     (const float*)d_out, (const float*)w2, (float*)dz, (const float*)h, offsets, d,
                     F, E, S_max, nullptr, nullptr);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL(f32_wgrad_kernel, dim3(E, (d + 15) / 16, (F + 63) / 64), b, 0, s,
                     (const float*)d_out, (const float*)h, dw2, offsets, d, F);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL((f32_rows_kernel<false, EPI_STORE>), dim3(rt, (d + 63) / 64), b, 0, s,
                     (const float*)dz, (const float*)w1, (float*)dx_perm, nullptr, offsets, F, d,
                     E, S_max, nullptr, nullptr);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL(f32_wgrad_kernel, dim3(E, (F + 15) / 16, (d + 63) / 64), b, 0, s,
                     (const float*)dz, (const float*)x_perm, dw1, offsets, F, d);
  return hipGetLastError();
}

}  // namespace moe
