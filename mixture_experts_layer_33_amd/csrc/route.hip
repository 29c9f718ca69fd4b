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

// ---------------------------------------------------------------------------
// bf16 activations: the router product on MFMA.  W_gate (float32) is split
// exactly into three bf16 parts, W = hi + mid + lo (each part takes the next
// 8 bits of the 24-bit significand), stored transposed as [3][EP][d] with
// EP = E rounded up to 16 (extra rows zero).  bf16 x times each bf16 part is
// exact in float32, so logits = sum over the three parts of x W_p with
// float32 accumulation: float32 accuracy at matrix-core rate.
__global__ void split_gate_kernel(const float* __restrict__ w_gate, bf16* __restrict__ wsplit,
                                  int d, int E, int EP) {
  __shared__ float tile[32][33];
  const int i0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, e = e0 + tx;
    tile[r][tx] = (i < d && e < E) ? w_gate[(size_t)i * E + e] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, i = i0 + tx;
    if (e < EP && i < d) {
      const float v = tile[tx][r];
      const bf16 hi = (bf16)v;
      const float r1 = v - (float)hi;
      const bf16 mid = (bf16)r1;
      const bf16 lo = (bf16)(r1 - (float)mid);
      const size_t plane = (size_t)EP * d;
      wsplit[(size_t)e * d + i] = hi;
      wsplit[plane + (size_t)e * d + i] = mid;
      wsplit[2 * plane + (size_t)e * d + i] = lo;
    }
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
// block).  Four wavefronts; KS of them share one group of 16 tokens and split
// the k range of every LDS stage between them, their partial logits summed
// in LDS in a fixed order, so a workgroup covers 64 / KS tokens (KS > 1 gives
// small batches enough workgroups).  The three bf16 parts of W_gate go
// through LDS; x fragments are read straight from memory one stage ahead.
template <int EP, int KS>
__global__ void __launch_bounds__(256)
route_mfma_kernel(const bf16* __restrict__ x, const bf16* __restrict__ wsplit,
                  const float* __restrict__ b_gate, float* __restrict__ logits_out,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int T, int d, int E,
                  int k) {
  constexpr int BK = EP > 128 ? 32 : 64;          // k per wavefront per stage
  constexpr int SW = KS * BK;                     // k per stage
  constexpr int FN = EP / 16;
  constexpr int ROWS = 3 * EP;                    // LDS rows per stage
  constexpr int CPR = SW / 8;                     // chunks per row
  constexpr int NQ = ROWS * CPR;                  // chunks per stage
  constexpr int NCH = (NQ + 255) / 256;           // chunks per thread
  constexpr int TPW = 64 / KS;                    // tokens per workgroup
  constexpr int NS = BK / 32;                     // MFMA k slices per wavefront per stage
  __shared__ __attribute__((aligned(16))) bf16 lds[2][ROWS * SW];
  __shared__ f32x4 red[KS > 1 ? 4 : 1][KS > 1 ? 64 * FN : 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int grp = wid / KS, ks = wid % KS;
  const int t0 = blockIdx.x * TPW + grp * 16;
  const int ta = min(t0 + (lane & 15), T - 1);  // A-fragment row (clamped)
  const bf16* xrow = x + (size_t)ta * d + ks * BK + (lane >> 4) * 8;
  f32x4 acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x4 stage[NCH];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int q = tid + c * 256, row = q / CPR, kc = q % CPR;
      if (NQ % 256 == 0 || q < NQ)
        stage[c] = *reinterpret_cast<const i32x4*>(wsplit + (size_t)row * d + k0 + kc * 8);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int q = tid + c * 256, row = q / CPR, kc = q % CPR;
      if (NQ % 256 == 0 || q < NQ)
        *reinterpret_cast<i32x4*>(&lds[buf][rswz<SW>(row, kc)]) = stage[c];
    }
  };
  bf16x8 xc[NS], xn[NS];
  auto load_x = [&](int kt, bf16x8(&dst)[NS]) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      dst[s] = *reinterpret_cast<const bf16x8*>(xrow + (size_t)kt * SW + s * 32);
  };
  const int nk = d / SW;
  load_stage(0);
  load_x(0, xc);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_stage((kt + 1) * SW);
      load_x(kt + 1, xn);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int kc = ks * (BK / 8) + s * 4 + (lane >> 4);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = p * EP + j * 16 + (lane & 15);
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(&lds[cur][rswz<SW>(row, kc)]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xc[s], b, acc[j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) xc[s] = xn[s];
  }
  if constexpr (KS > 1) {
#pragma unroll
    for (int j = 0; j < FN; ++j) red[wid][lane * FN + j] = acc[j];
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
      acc[j] = sum;
    }
  }

  // lane holds tokens t0 + (lane/16)*4 + i (i < 4), experts j*16 + lane%16
  const int g = lane & 15;
  float bias[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int e = j * 16 + g;
    bias[j] = (e < E) ? b_gate[e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + (lane >> 4) * 4 + i;
    float v[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) v[j] = acc[j][i] + bias[j];
    if (logits_out != nullptr && t < T) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int e = j * 16 + g;
        if (e < E) logits_out[(size_t)t * E + e] = v[j];
      }
    }
    unsigned taken = 0;
    float sv[MOE_MAX_TOPK];
    int si[MOE_MAX_TOPK];
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int e = j * 16 + g;
        if (e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) {
          bv = v[j];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 15) == g) taken |= 1u << (bi >> 4);
      sv[r] = bv;
      si[r] = bi;
    }
    if (g == 0 && t < T) {
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

int route_padded_experts(int E) {
  int ep = 16;
  while (ep < E) ep *= 2;
  return ep;
}

size_t route_split_bytes(int d, int E) {
  return (size_t)3 * route_padded_experts(E) * d * sizeof(bf16);
}

hipError_t launch_route(int act, const void* x, const float* w_gate, const float* b_gate,
                        const float* logits_in, float* logits_out, int32_t* topk_idx,
                        float* topk_w, int T, int d, int E, int k, void* wsplit, hipStream_t s) {
  if (act == MOE_BF16 && logits_in == nullptr) {
    const int EP = route_padded_experts(E);
    hipLaunchKernelGGL(split_gate_kernel, dim3((d + 31) / 32, (EP + 31) / 32), dim3(256), 0, s,
                       w_gate, (bf16*)wsplit, d, E, EP);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // split each stage's k range over KS wavefronts when the batch is too
    // small to give every CU two workgroups of 64 tokens (LDS and d permitting)
    int ks = 1;
    const int bk = EP > 128 ? 32 : 64;
    const int max_ks = EP <= 32 ? 4 : EP == 64 ? 2 : 1;
    while (ks < max_ks && (T + 64 / ks - 1) / (64 / ks) < 512 && d % (2 * ks * bk) == 0) ks *= 2;
    dim3 grid((T + 64 / ks - 1) / (64 / ks)), block(256);
    const bf16* xs = (const bf16*)x;
    const bf16* wsp = (const bf16*)wsplit;
#define MOE_ROUTE(EPV, KSV)                                                                 \
  hipLaunchKernelGGL((route_mfma_kernel<EPV, KSV>), grid, block, 0, s, xs, wsp, b_gate,      \
                     logits_out, topk_idx, topk_w, T, d, E, k)
    switch (EP * 8 + ks) {
      case 16 * 8 + 4: MOE_ROUTE(16, 4); break;
      case 16 * 8 + 2: MOE_ROUTE(16, 2); break;
      case 16 * 8 + 1: MOE_ROUTE(16, 1); break;
      case 32 * 8 + 4: MOE_ROUTE(32, 4); break;
      case 32 * 8 + 2: MOE_ROUTE(32, 2); break;
      case 32 * 8 + 1: MOE_ROUTE(32, 1); break;
      case 64 * 8 + 2: MOE_ROUTE(64, 2); break;
      case 64 * 8 + 1: MOE_ROUTE(64, 1); break;
      case 128 * 8 + 1: MOE_ROUTE(128, 1); break;
      default: MOE_ROUTE(256, 1); break;
    }
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
