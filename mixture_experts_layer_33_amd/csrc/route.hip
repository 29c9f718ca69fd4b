// Gate routing on gfx950: router logits, top-k selection and gate weights.
//
// A Survey on Mixture of Experts, §5 System Design (first paragraph): gate
// routing is the first step of the expert-parallel pipeline; PopFetcher
// notes §2.1.2: each token goes to its top-k experts, k usually 1 or 2.
//
// Two router kernels: for bf16 activations an MFMA kernel (three exact bf16
// parts of W_gate, below); for float32 activations, or when the caller
// passes the logits, a float32 FMA kernel with W_gate staged through LDS.  In
// both, each token's logits sit in one 16-lane group, which selects the top k
// by k rounds of a 16-lane (value, index) max reduction.
#include <type_traits>

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

// Keep the better of (bv, bi) and the pair that DPP control CTRL brings from
// another lane of the same 16-lane row.
template <int CTRL>
__device__ __forceinline__ void dpp_better(float& bv, int& bi) {
  const int vb = __builtin_bit_cast(int, bv);
  const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(vb, vb, CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

// The best (value, index) pair of each row of 16 lanes, left in every lane of
// the row, by register moves between lanes (no LDS): after the mirror
// (lane i with 15 - i) and the half-row mirror (i with 7 - i in each half) the
// four lanes of every quad hold four disjoint quarters of the row, which the
// two quad swaps combine.  The order is total, so any pairing gives the same
// winner.
__device__ __forceinline__ void row16_best(float& bv, int& bi) {
  dpp_better<0x140>(bv, bi);  // row_mirror
  dpp_better<0x141>(bv, bi);  // row_half_mirror
  dpp_better<0x4E>(bv, bi);   // quad_perm [2, 3, 0, 1]
  dpp_better<0xB1>(bv, bi);   // quad_perm [1, 0, 3, 2]
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
// bf16 activations: the router product on MFMA.  W_gate (float32) is split
// exactly into three bf16 parts, W = hi + mid + lo (each part takes the next
// 8 bits of the 24-bit significand); bf16 x times each bf16 part is exact in
// float32, so logits = sum over the three parts of x W_p with float32
// accumulation: float32 accuracy at matrix-core rate.  The split happens
// while W_gate is staged into LDS, as [3][EP][SW] (EP = E rounded up to 16,
// extra rows zero), so there is no separate pass over W_gate.
__device__ __forceinline__ void split3(float v, bf16& hi, bf16& mid, bf16& lo) {
  hi = (bf16)v;
  const float r1 = v - (float)hi;
  mid = (bf16)r1;
  lo = (bf16)(r1 - (float)mid);
}

// f(Ic<P>{}) for P = P0 .. N - 1, unrolled at compile time
template <int P0, int N, class F>
__device__ __forceinline__ void unroll_stages(F&& f) {
  if constexpr (P0 < N) {
    f(Ic<P0>{});
    unroll_stages<P0 + 1, N>(f);
  }
}

// LDS row of SW bf16 (SW/8 16-byte chunks), chunks XOR-swizzled by the low
// row bits so that the 16 rows of an MFMA operand read fall in different
// banks.
template <int SW>
__device__ __forceinline__ int rswz(int row, int kc) {
  constexpr int XM = (SW / 8 < 16 ? SW / 8 : 16) - 1;
  return row * SW + ((kc ^ (row & XM)) * 8);
}

// Router logits on MFMA (v_mfma_f32_16x16x32_bf16, 16 tokens x 16 experts per
// block).  Four wavefronts; KS of them share TG groups of 16 tokens and split
// the k range of every LDS stage between them, their partial logits summed
// in LDS in a fixed order, so a workgroup covers 64 TG / KS tokens (KS > 1
// gives small batches enough workgroups; TG > 1 reuses each staged W_gate
// slice for more tokens when experts are many).  Loads run D stages ahead, in
// D register sets: W_gate through registers into LDS (split on the way, two
// LDS buffers), x fragments straight into registers.  With few experts each
// stage holds little work, so the kernel is bound by how many bytes each CU
// keeps in flight: D sets the depth of that queue.
template <int EP, int KS, int TG, int D, int UW>
__global__ void __launch_bounds__(256)
route_mfma_kernel(const bf16* __restrict__ x, const float* __restrict__ w_gate,
                  const float* __restrict__ b_gate, float* __restrict__ logits_out,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int T, int d, int E,
                  int k) {
  constexpr int BK = EP > 128 ? 32 : 64;          // k per wavefront per stage
  constexpr int SW = KS * BK;                     // k per stage
  constexpr int FN = EP / 16;
  constexpr int ROWS = 3 * EP;                    // LDS rows per stage
  constexpr int CPR = SW / 8;                     // 8-k chunks per row
  constexpr int EU = EP / UW;                     // expert groups of a copy unit
  constexpr int NU = EU * CPR;                    // (group, chunk) copy units per stage
  constexpr int NCH = (NU + 255) / 256;           // copy units per thread
  constexpr int TPW = 64 / KS * TG;               // tokens per workgroup
  constexpr int NS = BK / 32;                     // MFMA k slices per wavefront per stage
  __shared__ __attribute__((aligned(16))) bf16 lds[2][ROWS * SW];
  __shared__ f32x4 red[KS > 1 ? 4 : 1][KS > 1 ? 64 * FN * TG : 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int grp = wid / KS, ks = wid % KS;
  const int t0 = blockIdx.x * TPW + grp * 16 * TG;
  const bf16* xrow[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    const int ta = min(t0 + g * 16 + (lane & 15), T - 1);  // A-fragment row (clamped)
    xrow[g] = x + (size_t)ta * d + ks * BK + (lane >> 4) * 8;
  }
  f32x4 acc[TG][FN];
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the epilogue's gate bias (expert 16 j + lane % 16), loaded before the k
  // loop so that its latency is hidden
  float bias[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int e = j * 16 + (lane & 15);
    bias[j] = (e < E) ? b_gate[e] : 0.f;
  }

  // A copy unit is 8 consecutive k rows of W_gate (one LDS chunk) for UW
  // consecutive experts: eight 16-byte loads when UW = 4 (E a multiple of 4,
  // so with W_gate 16-byte aligned every row is), eight 4-byte ones when
  // UW = 1.  Wide units pay
  // off only when there are enough of them to occupy every thread.  Experts
  // from E up to EP read a real expert's weights instead (clamped address,
  // no branch): their logit columns are never read, and each output column
  // of the product depends only on its own W_gate column.
  static_assert(UW == 1 || UW == 4, "copy units are 1 or 4 experts wide");
  static_assert(D >= 2 && D % 2 == 0, "register sets alternate over the two LDS buffers");
  using WV = std::conditional_t<UW == 4, f32x4, float>;
  WV wr[D][NCH][8];         // W_gate of the stages ahead (D register sets)
  bf16x8 xr[D][TG][NS];     // x fragments of the stages ahead
  int woff[NCH];            // element offset of each unit's first W_gate entry
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int q = tid + c * 256, eu = q % EU, kc = q / EU;
    woff[c] = kc * 8 * E + min(UW * eu, E - UW);
  }
  auto load_w = [&](int kt, WV(&dst)[NCH][8]) {
    const float* wk = w_gate + (size_t)kt * SW * E;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (NU % 256 != 0 && tid + c * 256 >= NU) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dst[c][i] = *reinterpret_cast<const WV*>(wk + (size_t)i * E + woff[c]);
    }
  };
  auto store_w = [&](int buf, const WV(&src)[NCH][8]) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int q = tid + c * 256, eu = q % EU, kc = q / EU;
      if (NU % 256 != 0 && q >= NU) continue;
#pragma unroll
      for (int u = 0; u < UW; ++u) {
        bf16x8 hi, mid, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float v;
          if constexpr (UW == 4) v = src[c][i][u];
          else v = src[c][i];
          bf16 h, m, l;
          split3(v, h, m, l);
          hi[i] = h;
          mid[i] = m;
          lo[i] = l;
        }
        const int e = UW * eu + u;
        *reinterpret_cast<bf16x8*>(&lds[buf][rswz<SW>(e, kc)]) = hi;
        *reinterpret_cast<bf16x8*>(&lds[buf][rswz<SW>(EP + e, kc)]) = mid;
        *reinterpret_cast<bf16x8*>(&lds[buf][rswz<SW>(2 * EP + e, kc)]) = lo;
      }
    }
  };
  auto load_x = [&](int kt, bf16x8(&dst)[TG][NS]) {
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        dst[g][s] = *reinterpret_cast<const bf16x8*>(xrow[g] + (size_t)kt * SW + s * 32);
  };
  const int nk = d / SW;
  // step kt: register set P = kt % D, LDS buffer kt % 2.  Stage kt's W_gate
  // is already in LDS, so wr[P] takes the loads of stage kt + D; after the
  // MFMAs, stage kt + 1 (loaded D - 1 steps earlier) goes into the other LDS
  // buffer, and xr[P] takes the x fragments of stage kt + D
  auto step = [&](auto P_, int kt) {
    constexpr int P = decltype(P_)::value;
    constexpr int L = P % 2;
    if (kt + D < nk) load_w(kt + D, wr[P]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int kc = ks * (BK / 8) + s * 4 + (lane >> 4);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = p * EP + j * 16 + (lane & 15);
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(&lds[L][rswz<SW>(row, kc)]);
#pragma unroll
          for (int g = 0; g < TG; ++g)
            acc[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xr[P][g][s], b, acc[g][j], 0, 0,
                                                                0);
        }
    }
    if (kt + 1 < nk) store_w(L ^ 1, wr[(P + 1) % D]);
    if (kt + D < nk) load_x(kt + D, xr[P]);
    __syncthreads();
  };
  unroll_stages<0, D>([&](auto P_) {
    constexpr int P = decltype(P_)::value;
    if (P < nk) {
      load_w(P, wr[P]);
      load_x(P, xr[P]);
    }
  });
  store_w(0, wr[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += D)
    unroll_stages<0, D>([&](auto P_) {
      if (kt + decltype(P_)::value < nk) step(P_, kt + decltype(P_)::value);
    });
  if constexpr (KS > 1) {
#pragma unroll
    for (int j = 0; j < FN; ++j) red[wid][lane * FN + j] = acc[0][j];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      f32x4 sum = red[wid][lane * FN + j];
#pragma unroll
      for (int q = 1; q < KS; ++q) {
        const f32x4 o = red[wid + q][lane * FN + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += o[i];
      }
      acc[0][j] = sum;
    }
  }

  // lane holds tokens t0 + 16 g + (lane/16)*4 + i (i < 4), experts j*16 + lane%16
  const int gl = lane & 15;
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + g * 16 + (lane >> 4) * 4 + i;
      float v[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) v[j] = acc[g][j][i] + bias[j];
      if (logits_out != nullptr && t < T) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int e = j * 16 + gl;
          if (e < E) logits_out[(size_t)t * E + e] = v[j];
        }
      }
      // a NaN logit ranks as -inf (selection stays total, indices in [0, E))
#pragma unroll
      for (int j = 0; j < FN; ++j) v[j] = v[j] != v[j] ? -INFINITY : v[j];
      unsigned taken = 0;
      float sv[MOE_MAX_TOPK];
      int si[MOE_MAX_TOPK];
      for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int e = j * 16 + gl;
          if (e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) {
            bv = v[j];
            bi = e;
          }
        }
        row16_best(bv, bi);
        if ((bi & 15) == gl) taken |= 1u << (bi >> 4);
        sv[r] = bv;
        si[r] = bi;
      }
      if (gl == 0 && t < T) {
        float pr[MOE_MAX_TOPK];
        float sum = 0.f;
        for (int r = 0; r < k; ++r) {
          pr[r] = expf(sv[r] - sv[0]);
          sum += pr[r];
        }
        const float inv = 1.0f / sum;
        for (int r = 0; r < k; ++r) {
          topk_idx[(size_t)t * k + r] = si[r];
          topk_w[(size_t)t * k + r] = pr[r] * inv;
        }
      }
    }
}

// Stages of loads in flight: deeper only where one wavefront covers a whole
// stage's k range (the per-stage work is least there).
constexpr int route_depth(int EP, int KS, int TG) { return KS == 1 && EP * TG < 128 ? 4 : 2; }

// Experts per W_gate copy unit: 4 once that still leaves 256 units per stage.
constexpr int route_unit(int EP, int KS) { return EP * KS * (EP > 128 ? 32 : 64) >= 8192 ? 4 : 1; }

int route_padded_experts(int E) {
  int ep = 16;
  while (ep < E) ep *= 2;
  return ep;
}

hipError_t launch_route(int act, const void* x, const float* w_gate, const float* b_gate,
                        const float* logits_in, float* logits_out, int32_t* topk_idx,
                        float* topk_w, int T, int d, int E, int k, hipStream_t s) {
  if (act == MOE_BF16 && logits_in == nullptr) {
    const int EP = route_padded_experts(E);
    // Token groups per wavefront (TG): as many as keep one workgroup per CU
    // (and the registers unspilled); then, for batches too
    // small for that, split each stage's k range over KS wavefronts (LDS
    // and d permitting).
    const int bk = EP > 128 ? 32 : 64;
    const int max_tg = EP <= 64 ? 4 : EP == 128 ? 2 : 1;  // more would spill
    const int max_ks = EP <= 32 ? 4 : EP == 64 ? 2 : 1;
    int tg = 1, ks = 1;
    while (tg < max_tg && (T + 64 * 2 * tg - 1) / (64 * 2 * tg) >= 256) tg *= 2;
    if (tg == 1)
      while (ks < max_ks && (T + 64 / ks - 1) / (64 / ks) < 256 && d % (2 * ks * bk) == 0)
        ks *= 2;
    const int tpw = 64 / ks * tg;
    dim3 grid((T + tpw - 1) / tpw), block(256);
    const bf16* xs = (const bf16*)x;
#define MOE_ROUTE_U(EPV, KSV, TGV, UWV)                                                      \
  hipLaunchKernelGGL((route_mfma_kernel<EPV, KSV, TGV, route_depth(EPV, KSV, TGV), UWV>), grid, \
                     block, 0, s, xs, w_gate, b_gate, logits_out, topk_idx, topk_w, T, d, E, k)
#define MOE_ROUTE(EPV, KSV, TGV) MOE_ROUTE_U(EPV, KSV, TGV, route_unit(EPV, KSV))
    if (route_unit(EP, ks) == 4 && E % 4 != 0) {
      // rows of W_gate not 16-byte aligned: copied one expert at a time, one
      // token group per wavefront
      grid = dim3((T + 63) / 64);
      switch (EP) {  // four-expert units never run at EP = 16
        case 32: MOE_ROUTE_U(32, 1, 1, 1); break;
        case 64: MOE_ROUTE_U(64, 1, 1, 1); break;
        case 128: MOE_ROUTE_U(128, 1, 1, 1); break;
        default: MOE_ROUTE_U(256, 1, 1, 1); break;
      }
      return hipGetLastError();
    }
    switch ((EP * 8 + ks) * 8 + tg) {
      case (16 * 8 + 4) * 8 + 1: MOE_ROUTE(16, 4, 1); break;
      case (16 * 8 + 2) * 8 + 1: MOE_ROUTE(16, 2, 1); break;
      case (16 * 8 + 1) * 8 + 1: MOE_ROUTE(16, 1, 1); break;
      case (16 * 8 + 1) * 8 + 2: MOE_ROUTE(16, 1, 2); break;
      case (16 * 8 + 1) * 8 + 4: MOE_ROUTE(16, 1, 4); break;
      case (32 * 8 + 4) * 8 + 1: MOE_ROUTE(32, 4, 1); break;
      case (32 * 8 + 2) * 8 + 1: MOE_ROUTE(32, 2, 1); break;
      case (32 * 8 + 1) * 8 + 1: MOE_ROUTE(32, 1, 1); break;
      case (32 * 8 + 1) * 8 + 2: MOE_ROUTE(32, 1, 2); break;
      case (32 * 8 + 1) * 8 + 4: MOE_ROUTE(32, 1, 4); break;
      case (64 * 8 + 2) * 8 + 1: MOE_ROUTE(64, 2, 1); break;
      case (64 * 8 + 1) * 8 + 1: MOE_ROUTE(64, 1, 1); break;
      case (64 * 8 + 1) * 8 + 2: MOE_ROUTE(64, 1, 2); break;
      case (64 * 8 + 1) * 8 + 4: MOE_ROUTE(64, 1, 4); break;
      case (128 * 8 + 1) * 8 + 1: MOE_ROUTE(128, 1, 1); break;
      case (128 * 8 + 1) * 8 + 2: MOE_ROUTE(128, 1, 2); break;
      default: MOE_ROUTE(256, 1, 1); break;
    }
#undef MOE_ROUTE_U
#undef MOE_ROUTE
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
