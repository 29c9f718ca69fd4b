// Gate routing on gfx950: router logits, top-k selection and gate weights.
//
// A Survey on Mixture of Experts, §5 System Design (first paragraph): gate
// routing is the first step of the expert-parallel pipeline; PopFetcher
// notes §2.1.2: each token goes to its top-k experts, k usually 1 or 2.
//
// Two router kernels: for bf16 activations an MFMA kernel (three exact bf16
// parts of W_gate, below), which selects the top k by merging sorted lists;
// for float32 activations, or when the caller passes the logits, a float32
// FMA kernel with W_gate staged through LDS, where each token's logits sit
// in one 16-lane group that selects the top k by k rounds of a (value,
// index) max reduction.
#include <type_traits>

#include "buffer.hpp"
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

  // Selection keys: a NaN logit ranks as -inf, so every round finds a winner
  // among the experts not yet taken and the indices stay in [0, E) whatever
  // the logits hold (finite logits are the contract; this keeps a violation
  // from producing indices that later kernels would use as addresses).
#pragma unroll
  for (int j = 0; j < EPT; ++j) acc[j] = acc[j] != acc[j] ? -INFINITY : acc[j];
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

// ---------------------------------------------------------------------------
// bf16 activations: router logits as a tiled product on the matrix cores.
//
// Each float32 W_gate value is split exactly into three bf16 parts,
// W = hi + mid + lo: hi keeps the top 8 significant bits (the float's upper
// half), mid the top 8 of the remainder, lo what is left, at most 8 bits
// (exact while |W| >= 2^-103; below, lo's bits under float32's normal range
// are dropped).  Both subtractions are exact.  A bf16 x times a bf16 part is
// exact in float32, so summing x*hi + x*mid + x*lo with float32 accumulation
// gives float32 accuracy at matrix-core rate.  The split happens in
// registers, on the fragment a wavefront is about to use, so every W_gate
// value is split once per workgroup and W_gate is staged in its own float32
// layout.  Two values at a time: each part of the pair is the upper halves
// of the two floats, packed by one byte permute (11 operations per pair).
__device__ __forceinline__ void split3_pair(float w0, float w1, uint32_t& hi, uint32_t& mid,
                                            uint32_t& lo) {
  constexpr uint32_t kUpper = 0xffff0000u;  // upper half of a float: its bf16 truncation
  constexpr uint32_t kPackUpper = 0x07060302u;  // perm: upper half of S1, then of S0
  const uint32_t b0 = __builtin_bit_cast(uint32_t, w0), b1 = __builtin_bit_cast(uint32_t, w1);
  const float r0 = w0 - __builtin_bit_cast(float, b0 & kUpper);
  const float r1 = w1 - __builtin_bit_cast(float, b1 & kUpper);
  const uint32_t c0 = __builtin_bit_cast(uint32_t, r0), c1 = __builtin_bit_cast(uint32_t, r1);
  const float q0 = r0 - __builtin_bit_cast(float, c0 & kUpper);
  const float q1 = r1 - __builtin_bit_cast(float, c1 & kUpper);
  hi = __builtin_amdgcn_perm(b1, b0, kPackUpper);
  mid = __builtin_amdgcn_perm(c1, c0, kPackUpper);
  lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, q1), __builtin_bit_cast(uint32_t, q0),
                             kPackUpper);
}
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// s_waitcnt vmcnt(VM) lgkmcnt(LGKM) (expcnt not waited), then s_barrier.  As
// builtins rather than inline assembly, so that the compiler's own wait
// counting sees them and adds no waits for loads already known complete;
// s_barrier alone, without __syncthreads()' fence, which would wait for
// every copy in flight.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_barrier() {
  static_assert(VM >= 0 && VM <= 63 && LGKM >= 0 && LGKM <= 15, "wait counts");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (LGKM << 8) | ((VM >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

// f(Ic<P>{}) for P = P0 .. N - 1, unrolled at compile time
template <int P0, int N, class F>
__device__ __forceinline__ void unroll_stages(F&& f) {
  if constexpr (P0 < N) {
    f(Ic<P0>{});
    unroll_stages<P0 + 1, N>(f);
  }
}

// Router tile: one workgroup per BM tokens computes their logits against all
// experts (v_mfma_f32_16x16x32_bf16, blocks of 16 tokens x 16 experts; EP =
// E rounded up to a power of two >= 16), then selects each token's top k.
//
// The four or eight wavefronts split the work WM x WN x WK ways: token
// blocks, expert blocks, and the 32-deep k slices of each stage (their
// partial logits are summed in a fixed order at the end).  Eight wavefronts
// (two per SIMD) let one wavefront's split run beside another's MFMAs.
// Splitting k keeps the LDS reads per MFMA lowest and has every W_gate value
// split by one wavefront only, so it is preferred while the accumulators fit
// in registers.  A stage holds the x tile [BM][KD] (bf16) and the KD rows of
// W_gate [KD][E] (float32, one contiguous run of memory), copied global ->
// LDS by the buffer unit (16 bytes a lane, no registers; rows past the last
// token land as zeros; d is a multiple of KD).  STAGES stages rotate, up to
// STAGES - 1 of them in flight, each its own LDS object so that the compiler
// keeps the copies in flight past the reads of other stages; the epilogue
// reuses them (partial logits in the first, the summed logits in the
// others).
// With few experts the kernel streams x from HBM; the stage count sets how
// many bytes each CU keeps in flight.
//
// x rows in LDS are KD * 2 bytes.  Rows shorter than 256 bytes: chunk kc of
// row r sits at kc ^ ((r / rows per 256 bytes) % chunks per row); longer
// rows: at kc ^ (r % 16).  Either way the 16 rows of a fragment read (one
// 16-byte chunk each) fall in 16 different 16-byte bank groups.
// Padding after each 1 KiB of staged W_gate (WP, only when E = EW, a power
// of two from 32 to 128): the four k groups of a fragment read (rows 8 apart)
// then start 16 banks apart instead of on the same banks.
constexpr int route_wpad(int EW) { return EW == 32 ? 64 : EW == 64 ? 32 : EW == 128 ? 16 : 0; }

template <int BM, int EP, int EW, int WM, int WN, int WK, int KD, int STAGES, bool WP>
struct RouteCfg {
  static constexpr int NWV = WM * WN * WK;          // wavefronts per workgroup
  static constexpr int FM = BM / 16 / WM;           // token blocks per wavefront
  static constexpr int FN = EP / 16 / WN;           // expert blocks per wavefront
  static constexpr int ROWB = KD * 2;               // bytes of an x row in LDS
  static constexpr int CPR = KD / 8;                // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;           // rows per wave copy instruction
  static constexpr int XB = BM * ROWB;              // x tile bytes
  static constexpr int WCH = WP ? 1024 + route_wpad(EW) : 1024;  // LDS pitch of 1 KiB of W
  static constexpr int WB = (KD * EW * 4 + 1023) / 1024 * WCH;  // W_gate rows (E <= EW)
  static constexpr int STAGE = XB + WB;
  static constexpr int NX = XB / 1024, NW = WB / WCH;  // copy instructions per stage (most)
  static constexpr int NXW = (NX + NWV - 1) / NWV, NWW = (NW + NWV - 1) / NWV;  // per wavefront
  static constexpr int NPW = NXW + NWW;             // copies per wavefront per stage
  static constexpr int SL = KD / 32 / WK;           // MFMA k slices per wavefront per stage
  static_assert(NWV == 4 || NWV == 8, "four or eight wavefronts");
  static_assert(FM >= 1 && FN >= 1 && FM * 16 * WM == BM && FN * 16 * WN == EP, "blocks");
  static_assert(EW == EP || (EW == 8 && EP == 16), "staged experts");
  static_assert(SL >= 1 && SL * 32 * WK == KD, "whole slices per wavefront");
  static_assert(XB % 1024 == 0 && ROWB <= 1024, "whole copy instructions");
  // Software-pipelined main loop (split of the next stage under this one's
  // MFMAs) where a wavefront has 8 or more token blocks: enough MFMAs per
  // W_gate fragment to hide its split.  Its prologue waits with one more
  // stage in flight.
  static constexpr bool PIPE = FM >= 8 && STAGES >= 3;
  static_assert(NPW * (STAGES - (PIPE ? 1 : 2)) <= 63, "s_waitcnt vmcnt counts at most 63");
  static_assert(STAGES >= 2, "double buffering at least");
  static_assert(!WP || (route_wpad(EW) > 0 && EW == EP), "padded W_gate rows");
};

// Top-k by sorted lists (route_tile_kernel's epilogue).  A list holds the
// best KL (value, expert) pairs seen so far, best first in the order of
// better(); empty slots are (-inf, INT_MAX), which every real pair beats.
template <int KL>
struct TopList {
  float v[KL];
  int i[KL];
};

// Merge with the list of the partner lane that DPP control CTRL names (an
// involution within 16-lane rows): the better of each slot and the partner's
// slot KL - 1 - j keeps the best KL of the two lists (they form a bitonic
// sequence), then half-cleaners sort them.  Both partners end with the same
// list: better() is a total order on distinct experts.
template <int CTRL, int KL>
__device__ __forceinline__ void merge_partner(TopList<KL>& L) {
  float ov[KL];
  int oi[KL];
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    const int vb = __builtin_bit_cast(int, L.v[j]);
    ov[j] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(vb, vb, CTRL, 0xF, 0xF, false));
    oi[j] = __builtin_amdgcn_update_dpp(L.i[j], L.i[j], CTRL, 0xF, 0xF, false);
  }
  float mv[KL];
  int mi[KL];
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    const bool t = better(ov[KL - 1 - j], oi[KL - 1 - j], L.v[j], L.i[j]);
    mv[j] = t ? ov[KL - 1 - j] : L.v[j];
    mi[j] = t ? oi[KL - 1 - j] : L.i[j];
  }
#pragma unroll
  for (int h = KL / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int j = 0; j < KL; ++j)
      if ((j & h) == 0) {
        const bool sw = better(mv[j + h], mi[j + h], mv[j], mi[j]);
        const float a = mv[j], b = mv[j + h];
        const int ia = mi[j], ib = mi[j + h];
        mv[j] = sw ? b : a;
        mv[j + h] = sw ? a : b;
        mi[j] = sw ? ib : ia;
        mi[j + h] = sw ? ia : ib;
      }
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    L.v[j] = mv[j];
    L.i[j] = mi[j];
  }
}

// One token's top k from its row of logits in LDS, by TPT consecutive lanes
// (s = this lane's place): lane s takes experts s, s + TPT, ...  Inserting
// in increasing index order, a new pair beats a filled slot only with a
// strictly larger value (ties go to the smaller index already there), and
// the first j pairs fill slots 0..j-1.  A NaN logit ranks as -inf, so the
// selection is total and every index written is in [0, E).  Lane s writes
// choices s, s + TPT, ... < k: the expert, and its gate weight
// exp(v_r - v_0) / sum_{r' < k} exp(v_r' - v_0).
template <int KL, int TPT, int EPT>
__device__ __forceinline__ void route_select(const float* row, int s, int E, int k, int t, int T,
                                             int32_t* __restrict__ topk_idx,
                                             float* __restrict__ topk_w) {
  TopList<KL> L;
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    L.v[j] = -INFINITY;
    L.i[j] = 0x7fffffff;
  }
#pragma unroll
  for (int jj = 0; jj < EPT; ++jj) {
    const int e = s + TPT * jj;
    float x = row[e];
    x = x != x ? -INFINITY : x;
    const bool valid = e < E;
    bool c[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) c[j] = valid && (j >= jj || x > L.v[j]);
#pragma unroll
    for (int j = KL - 1; j >= 1; --j) {
      L.v[j] = c[j - 1] ? L.v[j - 1] : (c[j] ? x : L.v[j]);
      L.i[j] = c[j - 1] ? L.i[j - 1] : (c[j] ? e : L.i[j]);
    }
    L.v[0] = c[0] ? x : L.v[0];
    L.i[0] = c[0] ? e : L.i[0];
  }
  // partners: lane ^ 1, lane ^ 2 (quads now agree), then lane i of each 8
  // with 7 - i (one in each quad), then i of each 16 with 15 - i
  if constexpr (TPT >= 2) merge_partner<0xB1>(L);   // quad_perm [1, 0, 3, 2]
  if constexpr (TPT >= 4) merge_partner<0x4E>(L);   // quad_perm [2, 3, 0, 1]
  if constexpr (TPT >= 8) merge_partner<0x141>(L);  // row_half_mirror
  if constexpr (TPT >= 16) merge_partner<0x140>(L); // row_mirror
  if (t >= T) return;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < KL; ++r)
    if (r < k) sum += expf(L.v[r] - L.v[0]);
#pragma unroll
  for (int r = 0; r < KL; ++r)
    if (r < k && r % TPT == s) {
      topk_idx[(size_t)t * k + r] = L.i[r];
      topk_w[(size_t)t * k + r] = expf(L.v[r] - L.v[0]) * (1.0f / sum);
    }
}

constexpr int pow2_floor(int v) { return v >= 2 ? 2 * pow2_floor(v / 2) : 1; }
// threads per token when nt threads select for `tokens` tokens: a power of two,
// 1 to 16 (a DPP row)
constexpr int route_tpt(int nt, int tokens) {
  return nt / tokens >= 16 ? 16 : (nt / tokens >= 1 ? pow2_floor(nt / tokens) : 1);
}

template <int KD>
__device__ __forceinline__ int route_swz(int row) {
  if constexpr (KD * 2 >= 256) return row & 15;
  else return (row / (256 / (KD * 2))) & (KD / 8 - 1);
}

template <int BM, int EP, int EW, int WM, int WN, int WK, int KD, int STAGES, bool WP>
__global__ void __launch_bounds__(64 * WM * WN * WK)
route_tile_kernel(const bf16* __restrict__ x, const float* __restrict__ w_gate,
                  const float* __restrict__ b_gate, float* __restrict__ logits_out,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int T, int d, int E,
                  int k) {
  using Cf = RouteCfg<BM, EP, EW, WM, WN, WK, KD, STAGES, WP>;
  constexpr int FM = Cf::FM, FN = Cf::FN, NWV = Cf::NWV;
  constexpr bool PIPE = Cf::PIPE;
  constexpr int S1 = STAGES > 1 ? Cf::STAGE : 16, S2 = STAGES > 2 ? Cf::STAGE : 16;
  constexpr int S3 = STAGES > 3 ? Cf::STAGE : 16, S4 = STAGES > 4 ? Cf::STAGE : 16;
  constexpr int S5 = STAGES > 5 ? Cf::STAGE : 16, S6 = STAGES > 6 ? Cf::STAGE : 16;
  constexpr int S7 = STAGES > 7 ? Cf::STAGE : 16;
  static_assert(STAGES <= 8, "at most eight stages");
  __shared__ __attribute__((aligned(16))) char st0[Cf::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[S1];
  __shared__ __attribute__((aligned(16))) char st2[S2];
  __shared__ __attribute__((aligned(16))) char st3[S3];
  __shared__ __attribute__((aligned(16))) char st4[S4];
  __shared__ __attribute__((aligned(16))) char st5[S5];
  __shared__ __attribute__((aligned(16))) char st6[S6];
  __shared__ __attribute__((aligned(16))) char st7[S7];
  __shared__ __attribute__((aligned(16))) char dummy[1024];  // target of padding copies
  // one token block's logits, after the main loop: in stage 0's memory
  typedef float RedRow[16][EP + 1];
  static_assert(sizeof(RedRow) * WK <= Cf::STAGE, "the epilogue fits in a stage buffer");
  RedRow* const red = reinterpret_cast<RedRow*>(st0);
  char* const stage[8] = {st0, st1, st2, st3, st4, st5, st6, st7};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = (int)uniform((uint32_t)tid >> 6);
  const int kw = wid % WK, wn = (wid / WK) % WN, wm = wid / (WK * WN);
  const int t0 = blockIdx.x * BM;
  const int rows_valid = min(BM, T - t0);
  const int nst = d / KD;
  // this stage's W_gate rows: KD * E floats, copied as whole 1 KiB pieces
  const int nw = (KD * E * 4 + 1023) / 1024;

  // Copy slots of this wavefront: NXW of x (instruction wid + NWV i of the
  // stage's NX) then NWW of W_gate (wid + NWV i of nw).  A slot past its count
  // is padding: no bytes, written to `dummy`.  Only the lane offsets are
  // kept; the stage's k offset goes into the scalar offset.
  uint32_t voff[Cf::NPW];
  int ldst[Cf::NPW];  // LDS offset in the stage, or -1 (padding)
  unroll_stages<0, Cf::NPW>([&](auto J_) __attribute__((always_inline)) {
    constexpr int j = decltype(J_)::value;
    constexpr bool isx = j < Cf::NXW;
    const int q = wid + NWV * (isx ? j : j - Cf::NXW);
    const bool pad = q >= (isx ? Cf::NX : nw);
    if constexpr (isx) {
      const int row = q * Cf::RPI + lane / Cf::CPR;
      const int kc = (lane % Cf::CPR) ^ route_swz<KD>(row);
      voff[j] = pad ? kPadOffset : (uint32_t)(row * d + kc * 8) * 2u;
    } else {
      voff[j] = pad ? kPadOffset : (uint32_t)(q * 1024 + lane * 16);
    }
    ldst[j] = pad ? -1 : (isx ? q * 1024 : Cf::XB + q * Cf::WCH);
  });
  const bf16* xbase = x + (size_t)t0 * d;
  const uint32_t xbytes = (uint32_t)rows_valid * (uint32_t)d * 2u;
  const uint32_t wbytes = (uint32_t)d * (uint32_t)E * 4u;

  auto issue = [&](int kt, char* dst) __attribute__((always_inline)) {
    const bool live = kt < nst;
    const Rsrc rx = make_rsrc(xbase, live ? xbytes : 0u);
    const Rsrc rw = make_rsrc(w_gate, live ? wbytes : 0u);
    unroll_stages<0, Cf::NPW>([&](auto J_) __attribute__((always_inline)) {
      constexpr int j = decltype(J_)::value;
      char* to = ldst[j] < 0 ? dummy : dst + ldst[j];
      if constexpr (j < Cf::NXW)
        copy16(rx, to, voff[j], (uint32_t)(kt * KD) * 2u);
      else
        copy16(rw, to, voff[j], (uint32_t)(kt * KD) * (uint32_t)E * 4u);
    });
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int m = 0; m < FM; ++m)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r16 = lane & 15, kq = lane >> 4;
  // this lane's expert in each of the wavefront's expert blocks (experts past
  // E read a real expert's weights; their logit columns are never used)
  int ecol[FN];
#pragma unroll
  for (int n = 0; n < FN; ++n) ecol[n] = min((wn * FN + n) * 16 + r16, E - 1);
  // One stage's operands in registers: this wavefront's x fragments and, per
  // expert block, the 8 W_gate values of each lane, for each of its slices.
  struct Frag {
    bf16x8 a[Cf::SL][FM];
    float w[Cf::SL][FN][8];
  };
  auto load_x = [&](const char* st, Frag& f, int s, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < FM; ++m) {
      const int row = (wm * FM + m) * 16 + r16;
      f.a[s][m] = *reinterpret_cast<const bf16x8*>(st + row * Cf::ROWB +
                                                   ((kc ^ route_swz<KD>(row)) * 16));
    }
  };
  auto load_w = [&](const char* st, Frag& f, int s, int kc) __attribute__((always_inline)) {
    const float* ws = reinterpret_cast<const float*>(st + Cf::XB);
#pragma unroll
    for (int n = 0; n < FN; ++n) {
      // WP: row kc * 8 starts kc * EW / 32 padded KiB in; row kc * 8 + i
      // at a compile-time offset from it
      const char* wrow = reinterpret_cast<const char*>(ws) + kc * (EW / 32) * Cf::WCH +
                         ecol[n] * 4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (WP)
          f.w[s][n][i] = *reinterpret_cast<const float*>(
              wrow + ((i * EW * 4) >> 10) * Cf::WCH + ((i * EW * 4) & 1023));
        else
          f.w[s][n][i] = ws[(kc * 8 + i) * E + ecol[n]];
      }
    }
  };
  // (pipelined: W_gate's values first, which the split waits for)
  auto load = [&](const char* st, Frag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < Cf::SL; ++s) {
      const int kc = (kw * Cf::SL + s) * 4 + kq;  // this lane's 8-deep k chunk
      if constexpr (PIPE) {
        load_w(st, f, s, kc);
        load_x(st, f, s, kc);
      } else {
        load_x(st, f, s, kc);
        load_w(st, f, s, kc);
      }
    }
  };
  auto split_mma = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < Cf::SL; ++s)
#pragma unroll
      for (int n = 0; n < FN; ++n) {
        // 8 consecutive k of this lane's expert, split into the 3 parts
        u32x4 ph, pm, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t h, md, l;
          split3_pair(f.w[s][n][2 * i], f.w[s][n][2 * i + 1], h, md, l);
          ph[i] = h;
          pm[i] = md;
          pl[i] = l;
        }
        const bf16x8 pw[3] = {__builtin_bit_cast(bf16x8, ph), __builtin_bit_cast(bf16x8, pm),
                              __builtin_bit_cast(bf16x8, pl)};
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int m = 0; m < FM; ++m)
            acc[m][n] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[s][m], pw[p], acc[m][n], 0, 0, 0);
      }
  };
  // The three bf16 parts of a stage's W_gate fragments.
  struct Parts {
    bf16x8 p[Cf::SL][FN][3];
  };
  auto split = [&](const Frag& f, Parts& q) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < Cf::SL; ++s)
#pragma unroll
      for (int n = 0; n < FN; ++n) {
        // 8 consecutive k of this lane's expert, split into the 3 parts
        u32x4 ph, pm, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t h, md, l;
          split3_pair(f.w[s][n][2 * i], f.w[s][n][2 * i + 1], h, md, l);
          ph[i] = h;
          pm[i] = md;
          pl[i] = l;
        }
        q.p[s][n][0] = __builtin_bit_cast(bf16x8, ph);
        q.p[s][n][1] = __builtin_bit_cast(bf16x8, pm);
        q.p[s][n][2] = __builtin_bit_cast(bf16x8, pl);
      }
  };
  auto mma = [&](const Frag& f, const Parts& q) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < Cf::SL; ++s)
#pragma unroll
      for (int n = 0; n < FN; ++n)
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int m = 0; m < FM; ++m)
            acc[m][n] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[s][m], q.p[s][n][p], acc[m][n], 0, 0, 0);
  };
  if constexpr (!PIPE) {
    unroll_stages<0, STAGES - 1>([&](auto P_) __attribute__((always_inline)) {
      issue(decltype(P_)::value, stage[decltype(P_)::value]);
    });
    // Step kt on stage buffer P = kt % STAGES: wait until this wavefront's
    // copies of stage kt have landed (the later STAGES - 2 stay in flight) and
    // its LDS reads are done, meet the other wavefronts, refill the buffer
    // stage kt - 1 used with stage kt + STAGES - 1, then read and compute stage
    // kt, each fragment's split just before its MFMAs.
    for (int kt = 0; kt < nst; kt += STAGES)
      unroll_stages<0, STAGES>([&](auto P_) __attribute__((always_inline)) {
        constexpr int P = decltype(P_)::value;
        if (kt + P < nst) {
          wait_barrier<Cf::NPW * (STAGES - 2), 0>();
          issue(kt + P + STAGES - 1, stage[(P + STAGES - 1) % STAGES]);
          Frag f;
          load(stage[P], f);
          split_mma(f);
        }
      });
  } else {
    // Three or more stages, software-pipelined: while the MFMAs of stage kt
    // run on operands already in registers, the wavefront reads stage kt + 1
    // from LDS and splits its W_gate fragments.  Step kt waits until its
    // copies of stage kt + 1 have landed (the later STAGES - 2 stay in flight)
    // and its reads of stage kt are done, meets the other wavefronts (so
    // every read of stage kt is done), and refills that buffer with stage
    // kt + STAGES.  Register sets alternate, so the loop is unrolled over a
    // multiple of 2 and of STAGES.
    unroll_stages<0, STAGES>([&](auto P_) __attribute__((always_inline)) {
      issue(decltype(P_)::value, stage[decltype(P_)::value]);
    });
    Frag f[2];
    Parts q[2];
    wait_barrier<Cf::NPW * (STAGES - 1), 15>();
    load(stage[0], f[0]);
    split(f[0], q[0]);
    constexpr int L = STAGES % 2 == 0 ? STAGES : 2 * STAGES;
    for (int kt = 0; kt < nst; kt += L)
      unroll_stages<0, L>([&](auto P_) __attribute__((always_inline)) {
        constexpr int P = decltype(P_)::value;
        const int kk = kt + P;
        if (kk < nst) {
          wait_barrier<Cf::NPW * (STAGES - 2), 0>();
          issue(kk + STAGES, stage[P % STAGES]);
          // (after the last stage this reads the zeros of a copy past the
          // end: in bounds, and unused)
          load(stage[(P + 1) % STAGES], f[(P + 1) % 2]);
          split(f[(P + 1) % 2], q[(P + 1) % 2]);
          mma(f[P % 2], q[P % 2]);
          // the LDS reads first, then the split's VALU work spread over the
          // MFMAs (without this the compiler runs the split as one block)
          constexpr int NMF = Cf::SL * FN * 3 * FM, NDS = Cf::SL * (FM + 4 * FN);
          constexpr int NV = (Cf::SL * FN * 48 + NMF - 1) / NMF;
          __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);  // LDS reads
          unroll_stages<0, NMF>([&](auto) __attribute__((always_inline)) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // NV VALU
          });
        }
      });
  }

  // padding copies past the last stage are still in flight
  wait_barrier<0, 15>();

  // Epilogue.  Per block of 16 tokens, the wavefronts holding its logits
  // write their partial sums (one per k group) to `red`; after a barrier
  // every thread sums some of them in k order, adds the bias, and stores the
  // logit in the token-major table `fl` in the other stage buffers.  Once a
  // chunk of blocks is in `fl`, TPT threads per token select its top k:
  // each inserts its experts, in increasing index order, into a sorted list
  // of the best KL (KL = k rounded up to 2, 4 or 8), then partner lanes merge
  // their lists by register moves until all TPT hold the token's best KL.
  constexpr int NT = 64 * NWV;
  constexpr int RBUF = (2 * WK * (int)sizeof(RedRow) <= Cf::STAGE) ? 2 : 1;  // red copies
  // fl: 16-token blocks of rows of RS floats; RS = EP + (threads per token
  // when the tile is one chunk) keeps the threads of the tokens a wavefront
  // reads on distinct banks
  constexpr int RS = EP + route_tpt(NT, BM);
  constexpr int FLB = 16 * RS * 4;                 // bytes of one block in fl
  constexpr int BPB = Cf::STAGE / FLB;             // blocks per stage buffer
  static_assert(STAGES >= 2 && BPB >= 1, "the logits table fits in the stage buffers");
  constexpr int NB = BM / 16;
  constexpr int CHB = (STAGES - 1) * BPB < NB ? (STAGES - 1) * BPB : NB;  // blocks per chunk
  constexpr int CT = CHB * 16;                     // tokens per chunk
  constexpr int TPT = route_tpt(NT, CT);           // threads per token
  constexpr int EPT = EP / TPT;                    // experts per thread
  constexpr int TPP = NT / TPT;                    // tokens per pass
  static_assert(NT % EP == 0, "a thread sums one expert column of each block");
  auto fl_row = [&](int tc) __attribute__((always_inline)) -> float* {
    const int b = tc >> 4, sb = b / BPB;  // block within the chunk, its buffer
    char* const base = sb == 0   ? st1
                       : sb == 1 ? st2
                       : sb == 2 ? st3
                       : sb == 3 ? st4
                       : sb == 4 ? st5
                       : sb == 5 ? st6
                                 : st7;
    return reinterpret_cast<float*>(base) + (b % BPB) * 16 * RS + (tc & 15) * RS;
  };
  const int ecl = tid % EP;  // this thread's expert column when summing
  const float bias_e = ecl < E ? b_gate[ecl] : 0.f;
  for (int cb = 0; cb < NB; cb += CHB) {
    for (int mb = cb; mb < cb + CHB && mb < NB; ++mb) {
      RedRow* const rb = red + (mb % RBUF) * WK;
      // (m compile-time: the accumulators stay in registers)
#pragma unroll
      for (int m = 0; m < FM; ++m) {
        if (mb != wm * FM + m) continue;
#pragma unroll
        for (int n = 0; n < FN; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            rb[kw][kq * 4 + i][(wn * FN + n) * 16 + r16] = acc[m][n][i];
      }
      __syncthreads();
#pragma unroll
      for (int qq = 0; qq < (16 * EP + NT - 1) / NT; ++qq) {
        const int q = tid / EP + qq * (NT / EP);  // token of the block
        if (q >= 16) break;
        float sum = rb[0][q][ecl];
#pragma unroll
        for (int w = 1; w < WK; ++w) sum += rb[w][q][ecl];
        const float v = sum + bias_e;
        fl_row((mb - cb) * 16 + q)[ecl] = v;
        const int t = t0 + mb * 16 + q;
        if (logits_out != nullptr && ecl < E && t < T) logits_out[(size_t)t * E + ecl] = v;
      }
      // the next block's partial sums go to the other copy of red, or wait
      if constexpr (RBUF == 1) __syncthreads();
    }
    if constexpr (RBUF == 2) __syncthreads();
    const int nct = min(CT, BM - cb * 16);
    for (int tc0 = 0; tc0 < nct; tc0 += TPP) {
      const int tc = tc0 + tid / TPT;  // whole TPT-lane groups share a token
      if (tc < nct) {
        const float* row = fl_row(tc);
        const int t = t0 + cb * 16 + tc, s = tid % TPT;
        if (k <= 2)
          route_select<2, TPT, EPT>(row, s, E, k, t, T, topk_idx, topk_w);
        else if (k <= 4)
          route_select<4, TPT, EPT>(row, s, E, k, t, T, topk_idx, topk_w);
        else
          route_select<8, TPT, EPT>(row, s, E, k, t, T, topk_idx, topk_w);
      }
    }
    __syncthreads();  // fl (and red) are rewritten by the next chunk
  }
}

// Launch shapes, from timings on the four workloads' sizes (cold and warm).
// Tokens per workgroup BM: enough workgroups for every CU (BM = T / 256
// rounded down to a power of two, 16..128; 64 at most with 256 experts).
// Wavefronts split k as far as the accumulators allow, then experts, then
// tokens; eight wavefronts (two per SIMD) where the split's VALU work is
// large against the MFMAs and the accumulators fit in half the registers:
// with 16 padded experts (k eight ways, 256-deep stages, BM <= 64, d a
// multiple of 256), 32 (experts two ways, k four ways) and 128 at BM = 128
// (experts four ways, k two ways).  Stage depth KD: 128 where four
// wavefronts split it (d a multiple of 128), else 64 (32 with 256 experts).
// Stages: as many as fit in LDS, at most eight.
struct RouteShape {
  int bm, wm, wn, wk, kd;
};
static RouteShape route_shape(int T, int d, int EP) {
  int bm = 16;
  while (bm < 128 && T / (2 * bm) >= 256) bm *= 2;
  if (EP == 256) return {bm > 64 ? 64 : bm, 1, 4, 1, 32};
  if (EP == 128) return bm == 128 ? RouteShape{128, 1, 4, 2, 64} : RouteShape{bm, 1, 2, 2, 64};
  if (EP == 64) return bm == 128 ? RouteShape{128, 1, 4, 1, 64} : RouteShape{bm, 1, 2, 2, 64};
  const bool k128 = d % 128 == 0;
  if (EP == 32) {
    if (bm == 128) return {128, 1, 2, 2, k128 ? 128 : 64};
    return k128 ? RouteShape{bm, 1, 2, 4, 128} : RouteShape{bm, 1, 2, 2, 64};
  }
  // EP == 16
  if (d % 256 == 0 && bm <= 64) return {bm, 1, 1, 8, 256};
  if (k128) return {bm, 1, 1, 4, 128};
  return {bm < 32 ? 32 : bm, 2, 1, 2, 64};
}

template <int BM, int EP, int EW, int WM, int WN, int WK, int KD, bool WP>
static void launch_route_tile(hipStream_t s, const bf16* x, const float* w_gate, const float* b,
                              float* lo, int32_t* idx, float* w, int T, int d, int E, int k) {
  using C2 = RouteCfg<BM, EP, EW, WM, WN, WK, KD, 2, WP>;
  // LDS: the stages (the epilogue reuses the first) and the padding target
  constexpr int FIT = (160 * 1024 - 1024 - 512) / C2::STAGE;
  constexpr int VM = 63 / C2::NPW + (C2::FM >= 8 ? 1 : 2);  // vmcnt limit (see PIPE)
  constexpr int MAXS = FIT < VM ? FIT : VM;
  constexpr int STAGES = MAXS < 2 ? 2 : (MAXS > 8 ? 8 : MAXS);
  hipLaunchKernelGGL((route_tile_kernel<BM, EP, EW, WM, WN, WK, KD, STAGES, WP>),
                     dim3((T + BM - 1) / BM), dim3(64 * C2::NWV), 0, s, x, w_gate, b, lo, idx, w,
                     T, d, E, k);
}

int route_padded_experts(int E) {
  int ep = 16;
  while (ep < E) ep *= 2;
  return ep;
}

hipError_t launch_route(int act, const void* x, const float* w_gate, const float* b_gate,
                        const float* logits_in, float* logits_out, int32_t* topk_idx,
                        float* topk_w, int T, int d, int E, int k, hipStream_t s) {
  if (act == MOE_BF16 && logits_in == nullptr) {
    const int EP = route_padded_experts(E), EW = E <= 8 ? 8 : EP;
    const RouteShape r = route_shape(T, d, EP);
    const bf16* xs = static_cast<const bf16*>(x);
    const long long key =
        (((((long long)EW * 1000 + r.bm) * 10 + r.wm) * 10 + r.wn) * 10 + r.wk) * 10 + r.kd / 32;
    const bool wp = E == EW && route_wpad(EW) > 0;
#define MOE_RT(BM, EPV, EWV, WM, WN, WK, KD)                                                    \
  case ((((EWV * 1000LL + BM) * 10 + WM) * 10 + WN) * 10 + WK) * 10 + KD / 32:                  \
    if (wp)                                                                                     \
      launch_route_tile<BM, EPV, EWV, WM, WN, WK, KD, (route_wpad(EWV) > 0)>(                   \
          s, xs, w_gate, b_gate, logits_out, topk_idx, topk_w, T, d, E, k);                     \
    else                                                                                        \
      launch_route_tile<BM, EPV, EWV, WM, WN, WK, KD, false>(s, xs, w_gate, b_gate, logits_out, \
                                                             topk_idx, topk_w, T, d, E, k);     \
    break;
#define MOE_RT16(EWV)                       \
  MOE_RT(16, 16, EWV, 1, 1, 8, 256)         \
  MOE_RT(32, 16, EWV, 1, 1, 8, 256)         \
  MOE_RT(64, 16, EWV, 1, 1, 8, 256)         \
  MOE_RT(16, 16, EWV, 1, 1, 4, 128)         \
  MOE_RT(32, 16, EWV, 1, 1, 4, 128)         \
  MOE_RT(64, 16, EWV, 1, 1, 4, 128)         \
  MOE_RT(128, 16, EWV, 1, 1, 4, 128)        \
  MOE_RT(32, 16, EWV, 2, 1, 2, 64)          \
  MOE_RT(64, 16, EWV, 2, 1, 2, 64)          \
  MOE_RT(128, 16, EWV, 2, 1, 2, 64)
#define MOE_RT_BM(EPV, WM, WN, WK, KD) \
  MOE_RT(16, EPV, EPV, WM, WN, WK, KD)  \
  MOE_RT(32, EPV, EPV, WM, WN, WK, KD)  \
  MOE_RT(64, EPV, EPV, WM, WN, WK, KD)
    switch (key) {
      MOE_RT16(8)
      MOE_RT16(16)
      MOE_RT_BM(32, 1, 2, 4, 128)
      MOE_RT_BM(32, 1, 2, 2, 64)
      MOE_RT(128, 32, 32, 1, 2, 2, 128)
      MOE_RT(128, 32, 32, 1, 2, 2, 64)
      MOE_RT_BM(64, 1, 2, 2, 64)
      MOE_RT(128, 64, 64, 1, 4, 1, 64)
      MOE_RT_BM(128, 1, 2, 2, 64)
      MOE_RT(128, 128, 128, 1, 4, 2, 64)
      MOE_RT_BM(256, 1, 4, 1, 32)
      default:
        return hipErrorInvalidValue;
    }
#undef MOE_RT_BM
#undef MOE_RT16
#undef MOE_RT
    return hipGetLastError();
  }
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
