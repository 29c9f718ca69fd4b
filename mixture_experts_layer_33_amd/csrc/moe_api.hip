// C ABI of libmoe: argument checks, workspace carving and the launch order of
// each step.  The entry points and their semantics are documented in
// include/moe.h.  Nothing here reads device memory or synchronises; every
// call only enqueues kernels on the caller's stream.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_bytes(const moe_shape* s) { return s->act_dtype == MOE_BF16 ? 2 : 4; }

int64_t slots(const moe_shape* s) { return (int64_t)s->T * s->k; }

int rank_tiles(const moe_shape* s) { return (int)((slots(s) + kRankTile - 1) / kRankTile); }

moe_status check_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->T <= 0 || s->d_model <= 0 || s->d_ff <= 0 || s->E <= 0 || s->k <= 0)
    return MOE_ERR_INVALID_ARG;
  if (s->k > s->E) return MOE_ERR_INVALID_ARG;
  if (s->d_model % 64 != 0 || s->d_ff % 64 != 0) return MOE_ERR_INVALID_ARG;
  if (isnan(s->capacity_factor) || isinf(s->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (s->act_dtype != MOE_F32 && s->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->capacity_priority != MOE_PRIORITY_SLOT && s->capacity_priority != MOE_PRIORITY_CHOICE)
    return MOE_ERR_INVALID_ARG;
  if (s->E > MOE_MAX_EXPERTS || s->k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  // row indices, slot indices and per-row element offsets stay in int32
  const int64_t S = slots(s);
  if (S > (int64_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  // the GEMM's buffer resources address an operand tile in 31-bit offsets
  const int64_t wide = s->d_model > s->d_ff ? s->d_model : s->d_ff;
  const int64_t limit = 0x7ffffff0;  // bytes addressable from one resource
  if (S * wide * 2 >= limit || (int64_t)s->d_model * s->d_ff * 2 >= limit ||
      (int64_t)s->d_model * s->E * 4 >= limit)  // the router's float32 W_gate
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int capacity_of(const moe_shape* s) {
  const double cf = (double)s->capacity_factor;
  if (cf <= 0.0) return s->T;
  const double c = ceil(cf * (double)s->T * (double)s->k / (double)s->E);
  if (c < 1.0) return 1;
  if (c > (double)s->T) return s->T;
  return (int)c;
}

// Workspace carving: the routing/permutation buffers, then backward buffers.
struct PermWs {
  int32_t* local_rank;  // [S]
  int32_t* hist;        // [E][n_tiles]
  int32_t* tile_base;   // [E][n_tiles]
  int32_t* raw_tmp;     // [E] raw counts when the caller passes none
  int32_t* kept_tmp;    // [E] kept counts when the caller passes none
};

size_t perm_ws_bytes(const moe_shape* s) {
  const size_t S = (size_t)slots(s);
  const size_t nt = (size_t)rank_tiles(s) * (size_t)s->E;
  size_t b = align_up(S * 4) + 2 * align_up(nt * 4) + 2 * align_up((size_t)s->E * 4);
  return b;
}

PermWs carve_perm(const moe_shape* s, void* ws) {
  char* p = static_cast<char*>(ws);
  PermWs w;
  const size_t S = (size_t)slots(s);
  const size_t nt = (size_t)rank_tiles(s) * (size_t)s->E;
  w.local_rank = reinterpret_cast<int32_t*>(p);
  p += align_up(S * 4);
  w.hist = reinterpret_cast<int32_t*>(p);
  p += align_up(nt * 4);
  w.tile_base = reinterpret_cast<int32_t*>(p);
  p += align_up(nt * 4);
  w.raw_tmp = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)s->E * 4);
  w.kept_tmp = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)s->E * 4);
  return w;
}

struct BwdWs {
  void* d_out;      // [S][d] act (later dx_perm)
  void* dz;         // [S][F] act
  float* dsel;      // [T][k]  gate-softmax gradient per slot
  float* dsel_perm; // [S]     the same per packed row
  float* w_gate_t;  // [E][d]
  uint32_t* relu_bits;  // [S][F/32] keep bits of the ReLU (bf16 path)
  int32_t* counters;    // tile queues of the two weight-gradient GEMMs
  float* partial;       // split-tail partial tiles of the row-grouped GEMMs
};

size_t bwd_ws_bytes(const moe_shape* s) {
  const size_t S = (size_t)slots(s), a = act_bytes(s);
  return align_up(S * s->d_model * a) + align_up(S * s->d_ff * a) + 2 * align_up(S * 4) +
         align_up((size_t)s->E * s->d_model * 4) + align_up(S * (size_t)s->d_ff / 8) +
         align_up(kBwdCounters * 4) + rows_partial_bytes(s->act_dtype);
}

BwdWs carve_bwd(const moe_shape* s, void* ws) {
  char* p = static_cast<char*>(ws);
  const size_t S = (size_t)slots(s), a = act_bytes(s);
  BwdWs w;
  w.d_out = p;
  p += align_up(S * s->d_model * a);
  w.dz = p;
  p += align_up(S * s->d_ff * a);
  w.dsel = reinterpret_cast<float*>(p);
  p += align_up(S * 4);
  w.dsel_perm = reinterpret_cast<float*>(p);
  p += align_up(S * 4);
  w.w_gate_t = reinterpret_cast<float*>(p);
  p += align_up((size_t)s->E * s->d_model * 4);
  w.relu_bits = reinterpret_cast<uint32_t*>(p);
  p += align_up(S * (size_t)s->d_ff / 8);
  w.counters = reinterpret_cast<int32_t*>(p);
  p += align_up(kBwdCounters * 4);
  w.partial = rows_partial_bytes(s->act_dtype) ? reinterpret_cast<float*>(p) : nullptr;
  return w;
}

// Forward workspaces: the routing/permutation part, [row_slot [S] for the
// fused forward], then the GEMMs' split-tail partial tiles.
size_t fwd_ws_bytes(const moe_shape* s, bool fused) {
  return perm_ws_bytes(s) + (fused ? align_up((size_t)slots(s) * 4) : 0) +
         rows_partial_bytes(s->act_dtype);
}
float* fwd_partial(const moe_shape* s, void* ws, bool fused) {
  if (rows_partial_bytes(s->act_dtype) == 0) return nullptr;
  return reinterpret_cast<float*>(static_cast<char*>(ws) + perm_ws_bytes(s) +
                                  (fused ? align_up((size_t)slots(s) * 4) : 0));
}

moe_status check_ws(const moe_shape* s, int op, const void* ws, size_t bytes) {
  const size_t need = moe_workspace_bytes(s, op);
  if (need == 0) return MOE_OK;
  if (ws == nullptr || bytes < need) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// all pointers non-null and 16-byte aligned
template <typename... P>
bool ptrs_ok(P... p) {
  const void* arr[] = {static_cast<const void*>(p)...};
  for (const void* q : arr)
    if (q == nullptr || !aligned16(q)) return false;
  return true;
}

bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }

#define MOE_HIP(expr)                                \
  do {                                               \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;    \
  } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// route kernel + per-tile ranks + scan (counts)
moe_status do_route(const moe_shape* s, const void* x, const float* w_gate, const float* b_gate,
                    const float* logits_in, float* logits_out, int32_t* idx, float* w,
                    int32_t* counts_raw, int32_t* counts_kept, const PermWs& pw, hipStream_t st) {
  MOE_HIP(launch_route(s->act_dtype, x, w_gate, b_gate, logits_in, logits_out, idx, w, s->T,
                       s->d_model, s->E, s->k, st));
  const int nt = rank_tiles(s);
  MOE_HIP(launch_rank_hist(idx, s->T, s->k, s->capacity_priority == MOE_PRIORITY_CHOICE, s->E,
                           pw.local_rank, pw.hist, nt, st));
  MOE_HIP(launch_scan(pw.hist, nt, s->E, capacity_of(s), pw.tile_base, counts_raw, counts_kept,
                      st));
  return MOE_OK;
}

}  // namespace

// Workspace of moe_forward_noalloc: a library-owned device array, one copy
// per GPU (the loader places it with the code object on each device the
// library runs on; it lives until the process ends).  Its size covers
// moe_forward's workspace for every shape with T*k <= MOE_NOALLOC_MAX_SLOTS:
// the per-slot ranks (4 bytes a slot), two per-(expert, 256-slot tile)
// tables, two per-expert count vectors, and the expert GEMMs' split-tail
// partial tiles (32 MiB).  In host code `scratch` names a host-side stand-in,
// not the device memory: only the address hipGetSymbolAddress returns for the
// current device is ever passed to kernels.
constexpr size_t kNoallocScratchBytes = 36u << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];
static_assert(((size_t)MOE_NOALLOC_MAX_SLOTS * 4 +
               2 * (size_t)MOE_MAX_EXPERTS * (MOE_NOALLOC_MAX_SLOTS / kRankTile) * 4 +
               2 * (size_t)MOE_MAX_EXPERTS * 4 + 5 * 256 + ((size_t)32 << 20)) <=
                  kNoallocScratchBytes,
              "the static workspace must hold the largest forward workspace");

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's `scratch`, looked up once per
// device (with that device current) and kept.
hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & (kAlign - 1)) != 0)
      return hipErrorInvalidValue;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_check_shape(const moe_shape* shape) { return check_shape(shape); }

size_t moe_workspace_bytes(const moe_shape* s, int32_t op) {
  if (check_shape(s) != MOE_OK) return 0;
  switch (op) {
    case MOE_OP_ROUTE:
    case MOE_OP_PERMUTE:
      return perm_ws_bytes(s);
    case MOE_OP_FORWARD:
      return fwd_ws_bytes(s, false);
    case MOE_OP_FORWARD_FUSED:
      return fwd_ws_bytes(s, true);
    case MOE_OP_EXPERT_FFN:
      return rows_partial_bytes(s->act_dtype);
    case MOE_OP_COMBINE:
      return 0;
    case MOE_OP_BACKWARD:
      return bwd_ws_bytes(s);
    default:
      return 0;
  }
}

int32_t moe_capacity(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return -1;
  return capacity_of(s);
}

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK:
      return "ok";
    case MOE_ERR_INVALID_ARG:
      return "invalid argument (null or misaligned pointer, bad size, k > E, d or F not a multiple of 64)";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported dtype or shape (E > 256, k > 8, T*k too large)";
    case MOE_ERR_WORKSPACE:
      return "workspace missing, misaligned or smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP:
      return "HIP kernel launch failed";
    default:
      return "unknown status";
  }
}

moe_status moe_route(const moe_shape* s, const void* x, const float* w_gate, const float* b_gate,
                     const float* logits_in, float* logits_out, int32_t* topk_idx, float* topk_w,
                     int32_t* counts_raw, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ptrs_ok(topk_idx, topk_w) || !opt_ok(counts_raw) || !opt_ok(logits_out) ||
      !opt_ok(logits_in))
    return MOE_ERR_INVALID_ARG;
  if (logits_in == nullptr && !ptrs_ok(x, w_gate, b_gate)) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_ROUTE, ws, ws_bytes)) != MOE_OK) return st;
  PermWs pw = carve_perm(s, ws);
  if (counts_raw == nullptr) {  // routing only; moe_permute counts
    MOE_HIP(launch_route(s->act_dtype, x, w_gate, b_gate, logits_in, logits_out, topk_idx,
                         topk_w, s->T, s->d_model, s->E, s->k, as_stream(stream)));
    return MOE_OK;
  }
  return do_route(s, x, w_gate, b_gate, logits_in, logits_out, topk_idx, topk_w, counts_raw,
                  pw.kept_tmp, pw, as_stream(stream));
}

moe_status moe_permute(const moe_shape* s, const void* x, const int32_t* topk_idx,
                       int32_t* counts_raw, int32_t* counts_kept, int32_t* offsets,
                       int32_t* slot_row, int32_t* row_token, void* x_perm, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ptrs_ok(x, topk_idx, counts_kept, offsets, slot_row, row_token, x_perm) ||
      !opt_ok(counts_raw))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_PERMUTE, ws, ws_bytes)) != MOE_OK) return st;
  PermWs pw = carve_perm(s, ws);
  hipStream_t stream_ = as_stream(stream);
  const int nt = rank_tiles(s);
  const int C = capacity_of(s);
  int32_t* raw = counts_raw ? counts_raw : pw.raw_tmp;
  MOE_HIP(launch_rank_hist(topk_idx, s->T, s->k, s->capacity_priority == MOE_PRIORITY_CHOICE,
                           s->E, pw.local_rank, pw.hist, nt, stream_));
  MOE_HIP(launch_scan(pw.hist, nt, s->E, C, pw.tile_base, raw, counts_kept, stream_));
  MOE_HIP(launch_gather(s->act_dtype, x, topk_idx, pw.local_rank, pw.tile_base, raw, counts_kept,
                        nt, s->T, s->d_model, s->E, s->k, C,
                        s->capacity_priority == MOE_PRIORITY_CHOICE, offsets, slot_row, row_token,
                        x_perm, stream_));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_shape* s, const void* x_perm, const int32_t* offsets,
                          const void* w1, const void* w2, void* h, void* out_perm,
                          uint32_t* relu_bits, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ptrs_ok(x_perm, offsets, w1, w2, h, out_perm) || !opt_ok(relu_bits))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_EXPERT_FFN, ws, ws_bytes)) != MOE_OK) return st;
  float* partial = rows_partial_bytes(s->act_dtype) ? static_cast<float*>(ws) : nullptr;
  MOE_HIP(launch_expert_fwd(s->act_dtype, x_perm, offsets, w1, w2, h, out_perm, relu_bits,
                            partial, (int)slots(s), capacity_of(s), s->d_model, s->d_ff, s->E,
                            as_stream(stream)));
  return MOE_OK;
}

moe_status moe_combine(const moe_shape* s, const void* out_perm, const float* topk_w,
                       const int32_t* slot_row, void* y, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ptrs_ok(out_perm, topk_w, slot_row, y)) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_combine(s->act_dtype, out_perm, topk_w, slot_row, y, s->T, s->d_model, s->k,
                         as_stream(stream)));
  return MOE_OK;
}

moe_status moe_forward(const moe_shape* s, const void* x, const float* w_gate,
                       const float* b_gate, const void* w1, const void* w2, void* y,
                       float* logits_out, int32_t* topk_idx, float* topk_w, int32_t* counts_raw,
                       int32_t* counts_kept, int32_t* offsets, int32_t* slot_row,
                       int32_t* row_token, void* x_perm, void* h, void* out_perm,
                       uint32_t* relu_bits, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ptrs_ok(x, w_gate, b_gate, w1, w2, y, topk_idx, topk_w, counts_kept, offsets, slot_row,
               row_token, x_perm, h, out_perm) ||
      !opt_ok(logits_out) || !opt_ok(counts_raw) || !opt_ok(relu_bits))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_FORWARD, ws, ws_bytes)) != MOE_OK) return st;
  PermWs pw = carve_perm(s, ws);
  hipStream_t stream_ = as_stream(stream);
  int32_t* raw = counts_raw ? counts_raw : pw.raw_tmp;
  st = do_route(s, x, w_gate, b_gate, nullptr, logits_out, topk_idx, topk_w, raw, counts_kept, pw,
                stream_);
  if (st != MOE_OK) return st;
  const int nt = rank_tiles(s);
  MOE_HIP(launch_gather(s->act_dtype, x, topk_idx, pw.local_rank, pw.tile_base, raw, counts_kept,
                        nt, s->T, s->d_model, s->E, s->k, capacity_of(s),
                        s->capacity_priority == MOE_PRIORITY_CHOICE, offsets, slot_row, row_token,
                        x_perm, stream_));
  MOE_HIP(launch_expert_fwd(s->act_dtype, x_perm, offsets, w1, w2, h, out_perm, relu_bits,
                            fwd_partial(s, ws, false), (int)slots(s), capacity_of(s), s->d_model,
                            s->d_ff, s->E, stream_));
  MOE_HIP(launch_combine(s->act_dtype, out_perm, topk_w, slot_row, y, s->T, s->d_model, s->k,
                         stream_));
  return MOE_OK;
}

moe_status moe_forward_fused(const moe_shape* s, const void* x, const float* w_gate,
                             const float* b_gate, const void* w1, const void* w2, void* y,
                             float* logits_out, int32_t* topk_idx, float* topk_w,
                             int32_t* counts_raw, int32_t* counts_kept, int32_t* offsets,
                             int32_t* slot_row, int32_t* row_token, void* h, void* out_slot,
                             uint32_t* relu_bits, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ptrs_ok(x, w_gate, b_gate, w1, w2, y, topk_idx, topk_w, counts_kept, offsets, slot_row,
               row_token, h, out_slot) ||
      !opt_ok(logits_out) || !opt_ok(counts_raw) || !opt_ok(relu_bits))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_FORWARD_FUSED, ws, ws_bytes)) != MOE_OK) return st;
  PermWs pw = carve_perm(s, ws);
  int32_t* row_slot = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + perm_ws_bytes(s));
  hipStream_t stream_ = as_stream(stream);
  int32_t* raw = counts_raw ? counts_raw : pw.raw_tmp;
  st = do_route(s, x, w_gate, b_gate, nullptr, logits_out, topk_idx, topk_w, raw, counts_kept, pw,
                stream_);
  if (st != MOE_OK) return st;
  MOE_HIP(launch_index(topk_idx, pw.local_rank, pw.tile_base, raw, counts_kept, rank_tiles(s),
                       s->T, s->E, s->k, capacity_of(s),
                       s->capacity_priority == MOE_PRIORITY_CHOICE, offsets, slot_row, row_token,
                       row_slot, stream_));
  MOE_HIP(launch_expert_fwd_fused(s->act_dtype, x, row_token, s->T, offsets, row_slot, w1, w2, h,
                                  out_slot, relu_bits, fwd_partial(s, ws, true), (int)slots(s),
                                  capacity_of(s), s->d_model, s->d_ff, s->E, stream_));
  MOE_HIP(launch_combine(s->act_dtype, out_slot, topk_w, slot_row, y, s->T, s->d_model, s->k,
                         stream_, true));
  return MOE_OK;
}

}  // extern "C"

namespace {

// moe_backward, with the weight gradients optionally split over replicas
moe_status backward_impl(const moe_shape* s, const void* dy, const void* x, const float* w_gate,
                         const void* w1, const void* w2, const int32_t* topk_idx,
                         const float* topk_w, const int32_t* slot_row, const int32_t* row_token,
                         const int32_t* offsets, const void* x_perm, const void* h,
                         const void* out_perm, const uint32_t* relu_bits, void* dx, float* dw1,
                         float* dw2, float* dw_gate, float* db_gate, float* dlogits, void* ws,
                         const int32_t* rep_start, const int32_t* rep_row0,
                         const int32_t* rep_rows, int n_copies, hipStream_t stream_) {
  BwdWs bw = carve_bwd(s, ws);
  float* rep_part = rep_start != nullptr
                        ? reinterpret_cast<float*>(static_cast<char*>(ws) + bwd_ws_bytes(s))
                        : nullptr;
  const int act = s->act_dtype;
  MOE_HIP(launch_combine_bwd(act, dy, out_perm, topk_w, topk_idx, slot_row, bw.d_out, bw.dsel,
                             bw.dsel_perm, dlogits, w_gate, bw.w_gate_t, bw.counters, s->T,
                             s->d_model, s->E, s->k, stream_));
  // dx_perm reuses d_out's memory: the FC1 dgrad runs after the FC2 wgrad,
  // the last reader of d_out.  For bf16 the FC1 wgrad also writes dW_gate and
  // db over the kept rows.
  MOE_HIP(launch_expert_bwd(act, bw.d_out, x_perm, h, offsets, w1, w2, bw.dz, bw.d_out, dw1, dw2,
                            bw.dsel_perm, dw_gate, db_gate, relu_bits, bw.relu_bits, bw.partial,
                            bw.counters, (int)slots(s), capacity_of(s), s->d_model, s->d_ff, s->E,
                            stream_, rep_start, rep_row0, rep_rows, n_copies, rep_part));
  if (act != MOE_BF16)
    MOE_HIP(launch_gate_rows(act, x_perm, bw.dsel_perm, offsets, dw_gate, db_gate, s->d_model,
                             s->E, stream_));
  // with a capacity below T slots can be dropped: dx also adds their gate gradient
  MOE_HIP(launch_dx(act, bw.d_out, bw.dsel, topk_idx, slot_row, bw.w_gate_t, dx, s->T,
                    s->d_model, s->k, capacity_of(s) < s->T, x, offsets, row_token, dw_gate,
                    db_gate, s->E, stream_));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_backward(const moe_shape* s, const void* dy, const void* x, const float* w_gate,
                        const void* w1, const void* w2, const int32_t* topk_idx,
                        const float* topk_w, const int32_t* slot_row, const int32_t* row_token,
                        const int32_t* offsets, const void* x_perm, const void* h,
                        const void* out_perm, const uint32_t* relu_bits, void* dx, float* dw1,
                        float* dw2, float* dw_gate, float* db_gate, float* dlogits, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ptrs_ok(dy, x, w_gate, w1, w2, topk_idx, topk_w, slot_row, row_token, offsets, x_perm, h,
               out_perm, dx, dw1, dw2, dw_gate, db_gate) ||
      !opt_ok(dlogits) || !opt_ok(relu_bits))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_BACKWARD, ws, ws_bytes)) != MOE_OK) return st;
  return backward_impl(s, dy, x, w_gate, w1, w2, topk_idx, topk_w, slot_row, row_token, offsets,
                       x_perm, h, out_perm, relu_bits, dx, dw1, dw2, dw_gate, db_gate, dlogits,
                       ws, nullptr, nullptr, nullptr, 0, as_stream(stream));
}

size_t moe_backward_replicated_workspace_bytes(const moe_shape* s, int32_t n_copies) {
  if (check_shape(s) != MOE_OK || s->act_dtype != MOE_BF16 || n_copies < s->E ||
      n_copies > MOE_PLAN_MAX_COPIES)
    return 0;
  return bwd_ws_bytes(s) + align_up(wgrad_replica_bytes(n_copies, s->E, s->d_model, s->d_ff));
}

moe_status moe_backward_replicated(const moe_shape* s, const void* dy, const void* x,
                                   const float* w_gate, const void* w1, const void* w2,
                                   const int32_t* topk_idx, const float* topk_w,
                                   const int32_t* slot_row, const int32_t* row_token,
                                   const int32_t* offsets, const void* x_perm, const void* h,
                                   const void* out_perm, const uint32_t* relu_bits,
                                   int32_t n_copies, const int32_t* replica_start,
                                   const int32_t* replica_row0, const int32_t* replica_rows,
                                   void* dx, float* dw1, float* dw2, float* dw_gate,
                                   float* db_gate, float* dlogits, void* ws, size_t ws_bytes,
                                   void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (n_copies < s->E || n_copies > MOE_PLAN_MAX_COPIES) return MOE_ERR_INVALID_ARG;
  if (!ptrs_ok(dy, x, w_gate, w1, w2, topk_idx, topk_w, slot_row, row_token, offsets, x_perm, h,
               out_perm, dx, dw1, dw2, dw_gate, db_gate, replica_start, replica_row0,
               replica_rows) ||
      !opt_ok(dlogits) || !opt_ok(relu_bits))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe_backward_replicated_workspace_bytes(s, n_copies);
  if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return MOE_ERR_WORKSPACE;
  return backward_impl(s, dy, x, w_gate, w1, w2, topk_idx, topk_w, slot_row, row_token, offsets,
                       x_perm, h, out_perm, relu_bits, dx, dw1, dw2, dw_gate, db_gate, dlogits,
                       ws, replica_start, replica_row0, replica_rows, n_copies,
                       as_stream(stream));
}

moe_status moe_popularity_update(int32_t E, int32_t window, int64_t iter,
                                 const int32_t* counts_raw, int32_t* ring, int32_t* window_sum,
                                 void* stream) {
  if (E <= 0 || window <= 0 || window > 64 || iter < 0) return MOE_ERR_INVALID_ARG;
  if (!ptrs_ok(counts_raw, ring, window_sum)) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_popularity(E, window, iter, counts_raw, ring, window_sum, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_ep_plan(int32_t E, int32_t R, int32_t extra, const int32_t* offsets,
                       int32_t* replica_start, int32_t* replica_row0, int32_t* replica_rows,
                       int32_t* replica_rank, int32_t* rank_rows, void* stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || R < 1 || R > MOE_PLAN_MAX_RANKS || extra < 0 ||
      extra > MOE_PLAN_MAX_COPIES - E)  // (no int overflow: E <= MOE_MAX_EXPERTS here)
    return MOE_ERR_INVALID_ARG;
  if (!ptrs_ok(offsets, replica_start, replica_row0, replica_rows, replica_rank, rank_rows))
    return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_ep_plan(E, R, extra, offsets, replica_start, replica_row0, replica_rows,
                         replica_rank, rank_rows, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_dispatch_layout(int32_t n, int32_t R, const int32_t* seg_rows,
                               const int32_t* seg_rank, int32_t* send_counts,
                               int32_t* send_offsets, int32_t* seg_send_offset, void* stream) {
  if (n < 1 || n > MOE_PLAN_MAX_COPIES || R < 1 || R > MOE_PLAN_MAX_RANKS)
    return MOE_ERR_INVALID_ARG;
  if (!ptrs_ok(seg_rows, seg_rank, send_counts, send_offsets, seg_send_offset))
    return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_dispatch_layout(n, R, seg_rows, seg_rank, send_counts, send_offsets,
                                 seg_send_offset, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_cooccurrence_update(int32_t E_a, int32_t E_b, int32_t k_a, int32_t k_b,
                                   int32_t T, int32_t window, int64_t iter,
                                   const int32_t* idx_a, const int32_t* idx_b, int32_t* ring,
                                   int32_t* window_sum, void* stream) {
  if (E_a < 1 || E_b < 1 || E_a > MOE_MAX_EXPERTS || E_b > MOE_MAX_EXPERTS || k_a < 1 ||
      k_b < 1 || k_a > MOE_MAX_TOPK || k_b > MOE_MAX_TOPK || k_a > E_a || k_b > E_b || T < 1 ||
      window < 1 || window > 64 || iter < 0)
    return MOE_ERR_INVALID_ARG;
  if (!ptrs_ok(idx_a, idx_b, ring, window_sum)) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_cooccurrence(E_a, E_b, k_a, k_b, T, window, iter, idx_a, idx_b, ring,
                              window_sum, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_predict_popularity(int32_t E_a, int32_t E_b, const int32_t* counts_a,
                                  const int32_t* cooc, double* pred, int32_t* order,
                                  void* stream) {
  if (E_a < 1 || E_b < 1 || E_a > MOE_MAX_EXPERTS || E_b > MOE_MAX_EXPERTS)
    return MOE_ERR_INVALID_ARG;
  if (!ptrs_ok(counts_a, cooc, pred, order)) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_predict(E_a, E_b, counts_a, cooc, pred, order, as_stream(stream)));
  return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_shape* s, const void* x, const float* w_gate,
                               const float* b_gate, const void* w1, const void* w2, void* y,
                               float* logits_out, int32_t* topk_idx, float* topk_w,
                               int32_t* counts_raw, int32_t* counts_kept, int32_t* offsets,
                               int32_t* slot_row, int32_t* row_token, void* x_perm, void* h,
                               void* out_perm, uint32_t* relu_bits, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (slots(s) > MOE_NOALLOC_MAX_SLOTS) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_workspace_bytes(s, MOE_OP_FORWARD);
  if (need > kNoallocScratchBytes) return MOE_ERR_UNSUPPORTED;
  if (!ptrs_ok(x, w_gate, b_gate, w1, w2, y, topk_idx, topk_w, counts_kept, offsets, slot_row,
               row_token, x_perm, h, out_perm) ||
      !opt_ok(logits_out) || !opt_ok(counts_raw) || !opt_ok(relu_bits))
    return MOE_ERR_INVALID_ARG;
  void* ws = nullptr;
  MOE_HIP(noalloc_scratch(&ws));
  // The forward workspace holds nothing that must start at zero: every
  // kernel writes its part before any kernel reads it.
  return moe_forward(s, x, w_gate, b_gate, w1, w2, y, logits_out, topk_idx, topk_w, counts_raw,
                     counts_kept, offsets, slot_row, row_token, x_perm, h, out_perm, relu_bits,
                     ws, kNoallocScratchBytes, stream);
}

}  // extern "C"
