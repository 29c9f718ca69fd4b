/*
 * moe.h - C ABI of libmoe, one GPU's mixture-of-experts layer on MI355X (gfx950).
 *
 * The layer follows the expert-parallel pipeline the survey "A Survey on
 * Mixture of Experts" lays out in §5 (System Design), first paragraph:
 * gate routing -> input encode -> expert computation -> output decode, here
 * on one GPU (no All-to-All: the packed per-expert buffers are exactly what
 * a dispatch would send).  Experts are FC -> ReLU -> FC with two weight
 * matrices and no biases (PopFetcher notes, §2.1.1 and §5.1); the gate is a
 * linear router with top-k selection (PopFetcher notes, §2.1.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers: every tensor argument is a DEVICE pointer to memory the caller
 *   owns.  The library never allocates or frees device memory; scratch space
 *   is a caller-provided workspace of moe_workspace_bytes(shape, op) bytes
 *   (256-byte aligned).  The shape struct is a HOST pointer.
 * - Layout: row-major and contiguous; tensors start 16-byte aligned.
 *     x, y, dy, dx      [T, d]        activation type
 *     w_gate            [d, E]        float32, b_gate [E] float32
 *     logits            [T, E]        float32
 *     topk_idx          [T, k]        int32, topk_w [T, k] float32
 *     w1                [E, F, d]     activation type (output x input)
 *     w2                [E, d, F]     activation type (output x input)
 *     x_perm, out_perm  [T*k, d]      activation type (first S_kept rows used)
 *     h                 [T*k, F]      activation type
 *     slot_row          [T*k]         int32; slot s = t*k + j; -1 = dropped
 *     row_token         [T*k]         int32; first S_kept entries valid
 *     counts_*          [E] int32;  offsets [E+1] int32 (offsets[E] = S_kept)
 *     dw1, dw2          same shapes as w1, w2, float32
 *     dw_gate [d, E], db_gate [E], dlogits [T, E]: float32
 *   Activation type: MOE_F32 (everything float32) or MOE_BF16 (bf16 storage,
 *   float32 accumulation, round-to-nearest-even stores).
 * - Asynchrony: every call only enqueues work on `stream` (a hipStream_t;
 *   NULL = the default stream) and returns; it never synchronises and never
 *   reads device data on the host.  Device faults show at the caller's next
 *   synchronisation.
 * - Errors: argument checks happen on the host before anything is enqueued;
 *   a failing call enqueues nothing and returns a negative moe_status.
 *   MOE_ERR_HIP means a launch was rejected after earlier launches of the
 *   same call may already be enqueued.
 * - Determinism: results are bitwise identical run to run (no float atomics;
 *   integer results never depend on thread order).
 * - Thread safety: the entry points with a workspace argument touch no
 *   memory but their arguments; concurrent calls need distinct outputs and
 *   workspaces.  The library keeps one host-side cache: the compute-unit
 *   count of each device (read once), which sizes the expert GEMMs' last
 *   round of tiles.  The float32 summation order of those tiles, and so the
 *   exact bits of h, out_perm and the input gradients, depends on that count
 *   (identical run to run on one device model).
 * - Finite inputs: router logits must be finite (NaN/Inf are a precondition
 *   violation).  The outputs of such a token are then unspecified, but every
 *   index the router writes stays in [0, E): a NaN logit ranks below every
 *   other logit.  moe_permute leaves a topk_idx entry outside [0, E)
 *   unrouted (slot_row -1, in no count and not in the dropped-slot list);
 *   such a permutation must not be passed to moe_backward.
 * - Routing semantics (the pages leave these open; this is the reading
 *   taken): selection on the float32 logits, ties to the lowest expert index
 *   (+0.0 == -0.0); gate weights are a softmax over the k selected logits;
 *   capacity C = ceil(cf*T*k/E) clamped to [1, T], or T when cf <= 0
 *   (dropless); slots claim capacity in the shape's capacity_priority order
 *   (slot order t*k + j by default); kept weights are not renormalised
 *   after drops; a token with every slot dropped outputs 0.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null required pointer, bad size, k > E ... */
#define MOE_ERR_UNSUPPORTED (-2) /* dtype or shape outside the compiled kernels */
#define MOE_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define MOE_ERR_HIP (-4)         /* a HIP launch failed */

#define MOE_F32 0
#define MOE_BF16 1

/* Capacity priority: the order in which slots claim expert capacity (and the
 * order of an expert's packed rows).  SLOT: s = t*k + j increasing, so each
 * expert keeps its earliest tokens.  CHOICE: every token's first choice in
 * token order, then every second choice, ... (the GShard gating that the
 * PopFetcher notes name beside plain top-k, §2.2 and §8.2). */
#define MOE_PRIORITY_SLOT 0
#define MOE_PRIORITY_CHOICE 1

/* Limits of the compiled kernels (MOE_ERR_UNSUPPORTED beyond them).  Besides
 * these, every operand a kernel addresses through one buffer resource stays
 * under 2 GiB: T*k*max(d, F)*2, d*F*2 and d*E*4 bytes (an unsupported shape
 * returns the error; it is never run with wrapped offsets). */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
#define MOE_PLAN_MAX_RANKS 64
#define MOE_PLAN_MAX_COPIES 1024 /* E + extra copies in moe_ep_plan */

typedef struct moe_shape {
  int32_t T;               /* tokens, >= 1 (an empty batch is MOE_ERR_INVALID_ARG) */
  int32_t d_model;         /* d: multiple of 64 */
  int32_t d_ff;            /* F: multiple of 64 */
  int32_t E;               /* experts, 1..MOE_MAX_EXPERTS */
  int32_t k;               /* experts per token, 1..min(E, MOE_MAX_TOPK) */
  float capacity_factor;   /* <= 0: dropless */
  int32_t act_dtype;       /* MOE_F32 or MOE_BF16 */
  int32_t capacity_priority; /* MOE_PRIORITY_SLOT or MOE_PRIORITY_CHOICE */
} moe_shape;

/* Operations, for moe_workspace_bytes. */
#define MOE_OP_ROUTE 0
#define MOE_OP_PERMUTE 1
#define MOE_OP_EXPERT_FFN 2
#define MOE_OP_COMBINE 3
#define MOE_OP_FORWARD 4
#define MOE_OP_BACKWARD 5
#define MOE_OP_FORWARD_FUSED 6

/* Workspace bytes `op` needs for `shape` (0 if none).  Returns 0 and sets
 * nothing on an invalid shape; validate with moe_check_shape first. */
size_t moe_workspace_bytes(const moe_shape* shape, int32_t op);

/* MOE_OK if the shape is valid and supported, else the error code. */
moe_status moe_check_shape(const moe_shape* shape);

/* Expert capacity C (see the routing semantics above); -1 on a bad shape. */
int32_t moe_capacity(const moe_shape* shape);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Gate routing (A Survey on Mixture of Experts, §5 System Design, first
 * paragraph: gate routing; PopFetcher notes §2.1.2: top-k selection).
 * logits[t,e] = b_gate[e] + sum_i x[t,i] * w_gate[i,e] in float32, unless
 * logits_in is given (then x/w_gate/b_gate may be NULL and those logits are
 * used as they are).  Writes logits_out if non-NULL, the top-k experts in
 * descending logit order, their renormalised weights, and counts_raw[e] =
 * number of slots routed to e (before capacity).  counts_raw may be NULL:
 * then only the routing kernel runs (moe_permute counts the slots again and
 * can write counts_raw; moe_route followed by moe_permute with counts_raw
 * given there launches exactly the kernels of moe_forward's first half).
 * Workspace: MOE_OP_ROUTE. */
moe_status moe_route(const moe_shape* shape, const void* x, const float* w_gate,
                     const float* b_gate, const float* logits_in, float* logits_out,
                     int32_t* topk_idx, float* topk_w, int32_t* counts_raw,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Input encode (survey §5, first paragraph: gathering each expert's tokens
 * into contiguous memory; capacity limit as in GShard, cited there).  From
 * topk_idx: counts_kept[e] = min(raw count, C); offsets = exclusive prefix
 * sum of counts_kept; slot_row[s] = offsets[e] + position of slot s among
 * e's slots in capacity-priority order, or -1 if that position is >= C;
 * row_token[r] = token of packed row r; x_perm[r] = x[row_token[r]] (exact
 * copy).  Dropped slots are listed after the kept rows: row_token[S_kept + j],
 * for j < T*k - S_kept, is the slot index t*k+j' of the j-th dropped slot,
 * ordered by expert and then by position (moe_backward reads this list).
 * counts_raw may be NULL.  Workspace: MOE_OP_PERMUTE. */
moe_status moe_permute(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                       int32_t* counts_raw, int32_t* counts_kept, int32_t* offsets,
                       int32_t* slot_row, int32_t* row_token, void* x_perm,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Expert computation (PopFetcher notes §2.1.1 FC-ReLU-FC and §5.1 weight
 * shapes; survey §5 "expert computation" on the packed buffers).  For each
 * expert e over packed rows offsets[e]..offsets[e+1]:
 *   h = ReLU(x_perm_e * w1[e]^T), out_perm = h * w2[e]^T
 * with float32 accumulation; h and out_perm stored in the activation type
 * (h is kept for the backward).  Rows past offsets[E] are not touched.
 * relu_bits (optional, bf16 only; NULL = not written): [T*k][d_ff/32]
 * words, bit (f % 32) of word [r][f / 32] set iff h[r][f] > 0, over rows
 * [0, offsets[E]); moe_backward can take it instead of deriving the ReLU
 * mask from h.  Ignored for MOE_F32.
 * Workspace: MOE_OP_EXPERT_FFN: bf16 needs 32 MiB of scratch for float32
 * partial tiles (when the last round of GEMM tiles would leave compute
 * units idle, its tiles are split along the reduction dimension and summed
 * in a fixed order, so results are deterministic); MOE_F32 needs none (the
 * argument may then be NULL). */
moe_status moe_expert_ffn(const moe_shape* shape, const void* x_perm, const int32_t* offsets,
                          const void* w1, const void* w2, void* h, void* out_perm,
                          uint32_t* relu_bits, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Output decode (survey §5, first paragraph: the inverse of input encode,
 * restoring token order from the gating indices).  y[t] = sum over kept
 * slots j, in order j = 0..k-1, of topk_w[t,j] * out_perm[slot_row[t*k+j]],
 * accumulated in float32 and rounded once; 0 if all of t's slots dropped. */
moe_status moe_combine(const moe_shape* shape, const void* out_perm, const float* topk_w,
                       const int32_t* slot_row, void* y, void* stream);

/* The whole forward: moe_route, moe_permute, moe_expert_ffn, moe_combine on
 * one stream.  logits_out, counts_raw and relu_bits may be NULL.  Every
 * other output (and relu_bits if given) is kept for moe_backward.
 * Workspace: MOE_OP_FORWARD. */
moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_gate,
                       const float* b_gate, const void* w1, const void* w2, void* y,
                       float* logits_out, int32_t* topk_idx, float* topk_w,
                       int32_t* counts_raw, int32_t* counts_kept, int32_t* offsets,
                       int32_t* slot_row, int32_t* row_token, void* x_perm, void* h,
                       void* out_perm, uint32_t* relu_bits, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Gather/scatter-fused forward (A Survey on Mixture of Experts, §5.1
 * Computation: ScatterMoE's grouped product on scattered rows avoids
 * copying tokens into per-expert groups).  Same routing and the same y,
 * bit for bit, as moe_forward, without the packed copy x_perm: the first
 * expert GEMM reads row row_token[r] of x for packed row r, the second
 * stores each kept slot's expert output at that slot, out_slot[t*k+j]
 * ([T*k][d_model], activation type; rows of dropped slots are not
 * written), and the decode reads slot rows directly.  topk_idx, topk_w,
 * counts, offsets, slot_row, row_token, h and relu_bits are as moe_forward
 * writes them; out_slot[s] = out_perm[slot_row[s]] for every kept slot s.
 * For inference or any forward not followed by moe_backward, which takes
 * moe_forward's packed tensors.  logits_out, counts_raw and relu_bits may
 * be NULL.  Workspace: MOE_OP_FORWARD_FUSED. */
moe_status moe_forward_fused(const moe_shape* shape, const void* x, const float* w_gate,
                             const float* b_gate, const void* w1, const void* w2, void* y,
                             float* logits_out, int32_t* topk_idx, float* topk_w,
                             int32_t* counts_raw, int32_t* counts_kept, int32_t* offsets,
                             int32_t* slot_row, int32_t* row_token, void* h, void* out_slot,
                             uint32_t* relu_bits, void* workspace, size_t workspace_bytes,
                             void* stream);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus the workspace),
 * same kernels and the same results, bit for bit, as moe_forward.  The
 * workspace is a library-owned static device array of 36 MiB, one per GPU,
 * held until the process ends; no call allocates or frees anything.
 * Limit: T*k <= MOE_NOALLOC_MAX_SLOTS (else MOE_ERR_UNSUPPORTED, nothing
 * enqueued).  Every call on one GPU uses that GPU's one array, so calls that
 * overlap on a GPU (other streams, other threads, a graph replay beside an
 * eager call) race and corrupt each other; serialize them.  The array keeps
 * the last call's contents; no call depends on them.  The first call on each
 * device looks up the array's device address (host side, once). */
#define MOE_NOALLOC_MAX_SLOTS 262144
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_gate,
                               const float* b_gate, const void* w1, const void* w2, void* y,
                               float* logits_out, int32_t* topk_idx, float* topk_w,
                               int32_t* counts_raw, int32_t* counts_kept, int32_t* offsets,
                               int32_t* slot_row, int32_t* row_token, void* x_perm, void* h,
                               void* out_perm, uint32_t* relu_bits, void* stream);

/* Backward of moe_forward for output gradient dy (PopFetcher notes §5.2.1:
 * one GEMM pass forward, two backward - gradients of the inputs and of the
 * expert parameters).  Reads the saved forward tensors and writes
 *   dx [T,d]     full input gradient, expert path plus router path
 *   dw1, dw2     float32; experts with no rows get zeros
 *   dw_gate, db_gate  float32 gate gradients
 *   dlogits      float32 [T,E] if non-NULL
 * Gate: w = softmax of the selected logits, so dlogits[t, idx_j] =
 * w_j (dg_j - sum_i w_i dg_i) with dg_j = <dy[t], out_perm[row_j]> (0 for a
 * dropped slot); other logits get 0.  ReLU'(0) = 0, mask [h > 0]: from
 * relu_bits when given (as written by moe_forward / moe_expert_ffn for
 * these h), else derived from h.  Workspace: MOE_OP_BACKWARD. */
moe_status moe_backward(const moe_shape* shape, const void* dy, const void* x,
                        const float* w_gate, const void* w1, const void* w2,
                        const int32_t* topk_idx, const float* topk_w,
                        const int32_t* slot_row, const int32_t* row_token,
                        const int32_t* offsets, const void* x_perm, const void* h,
                        const void* out_perm, const uint32_t* relu_bits, void* dx,
                        float* dw1, float* dw2, float* dw_gate, float* db_gate,
                        float* dlogits, void* workspace, size_t workspace_bytes,
                        void* stream);

/* moe_backward with each expert's weight gradients split over its replicas
 * (Fast MoE Inference via Predictive Prefetching and Expert Replication,
 * main contributions 2 and 3: hot experts get physical copies, each serving
 * a share of their tokens; A Survey on Mixture of Experts, §5.1
 * Computation: the layer waits for the most loaded expert).  Copy p =
 * replica_start[e] + c of expert e takes the packed rows
 * [replica_row0[p], replica_row0[p] + replica_rows[p]) - moe_ep_plan's
 * outputs, n_copies = replica_start[E] = E + extra.  The weight-gradient
 * tile scheduler splits an expert with several copies over them when one of
 * its unsplit output tiles would outlast a workgroup's mean share of the
 * launch (rows_e * workgroups > output tiles per expert * all rows; the
 * workgroups are min(the device's CUs, n_copies * output tiles per expert)):
 * each copy is then a K range of its own (what that copy's rank would
 * compute), and dW1[e], dW2[e], dW_gate[:, e] and db[e] are the sum of its
 * copies' float32 partial gradients in copy order (the fixed-order reduction
 * of the copies' gradients).  Every other expert, whatever its copies, gets
 * exactly moe_backward's values, as do dx and dlogits.  bf16 only (MOE_ERR_UNSUPPORTED otherwise); E <=
 * n_copies <= MOE_PLAN_MAX_COPIES.  Copies that do not tile their expert's
 * rows give unspecified weight gradients (never an access outside the
 * operands).  Workspace: moe_backward_replicated_workspace_bytes(shape,
 * n_copies) (moe_backward's plus 2 (n_copies - E) partial gradients). */
size_t moe_backward_replicated_workspace_bytes(const moe_shape* shape, int32_t n_copies);
moe_status moe_backward_replicated(const moe_shape* shape, const void* dy, const void* x,
                                   const float* w_gate, const void* w1, const void* w2,
                                   const int32_t* topk_idx, const float* topk_w,
                                   const int32_t* slot_row, const int32_t* row_token,
                                   const int32_t* offsets, const void* x_perm, const void* h,
                                   const void* out_perm, const uint32_t* relu_bits,
                                   int32_t n_copies, const int32_t* replica_start,
                                   const int32_t* replica_row0, const int32_t* replica_rows,
                                   void* dx, float* dw1, float* dw2, float* dw_gate,
                                   float* db_gate, float* dlogits, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Per-expert popularity over a sliding window of iterations (PopFetcher
 * notes §3.1, routing-information collector; §4.2, Eq. 1: token
 * distribution over the last s iterations).  Writes counts_raw into row
 * iter % window of ring [window, E], then window_sum[e] = sum of the rows of
 * the last min(iter + 1, window) iterations.  Rows of iterations not yet
 * recorded are never read.  Integers, exact.  iter >= 0, 1 <= window <= 64. */
moe_status moe_popularity_update(int32_t E, int32_t window, int64_t iter,
                                 const int32_t* counts_raw, int32_t* ring,
                                 int32_t* window_sum, void* stream);

/* Expert-parallel dispatch plan from one GPU's packed rows (offsets [E+1]
 * from moe_permute; counts c_e = offsets[e+1] - offsets[e]).
 * - Copies (Fast MoE Inference via Predictive Prefetching and Expert
 *   Replication: replication by token demand, capped by GPU memory): every
 *   expert has one copy and the `extra` copies the memory budget allows go
 *   one at a time to the expert with the most rows per copy (c_e / r_e,
 *   compared exactly; ties to the lowest index).  Copies of expert e are
 *   p = replica_start[e] .. replica_start[e+1]-1; copy i takes the packed
 *   rows offsets[e] + [floor(i c/r), floor((i+1) c/r)) (replica_row0,
 *   replica_rows) - one contiguous range, as the All-to-All sends them.
 * - Placement (LLEP notes §2.1: work goes to the least-loaded GPU): copies in
 *   order of decreasing rows (ties by copy index) each go to the rank with
 *   the fewest rows so far (ties to the lowest rank): replica_rank[p];
 *   rank_rows[r] = rows rank r computes (the All-to-All split sizes).
 * All arrays are int32 device memory: replica_start [E+1], replica_row0,
 * replica_rows, replica_rank [E+extra], rank_rows [R].  Limits: 1 <= E <=
 * MOE_MAX_EXPERTS, 1 <= R <= MOE_PLAN_MAX_RANKS, 0 <= extra,
 * E + extra <= MOE_PLAN_MAX_COPIES (else MOE_ERR_INVALID_ARG).  One
 * workgroup; enqueues only. */
moe_status moe_ep_plan(int32_t E, int32_t R, int32_t extra, const int32_t* offsets,
                       int32_t* replica_start, int32_t* replica_row0, int32_t* replica_rows,
                       int32_t* replica_rank, int32_t* rank_rows, void* stream);

/* All-to-All split sizes and send-buffer layout of an expert-parallel
 * dispatch (A Survey on Mixture of Experts, §5 System Design, first
 * paragraph: the per-expert packed rows are what the All-to-All sends).
 * Segment i holds seg_rows[i] packed rows bound for rank seg_rank[i]: with an
 * expert -> rank map, the segments are the experts (seg_rows = counts_kept,
 * seg_rank = the map); with moe_ep_plan's copies, the copies (replica_rows,
 * replica_rank).  The send buffer holds rank 0's rows, then rank 1's, ...,
 * the segments of one rank in index order:
 *   send_counts[r]      rows for rank r (the split sizes)        [R]
 *   send_offsets[r]     exclusive prefix sum, send_offsets[R] = total  [R+1]
 *   seg_send_offset[i]  first send-buffer row of segment i        [n]
 * A segment whose rank is outside [0, R) is in no count and gets -1.  All
 * int32 device memory; 1 <= n <= MOE_PLAN_MAX_COPIES, 1 <= R <=
 * MOE_PLAN_MAX_RANKS, else MOE_ERR_INVALID_ARG.  One wavefront; enqueues
 * only. */
moe_status moe_dispatch_layout(int32_t n, int32_t R, const int32_t* seg_rows,
                               const int32_t* seg_rank, int32_t* send_counts,
                               int32_t* send_offsets, int32_t* seg_send_offset, void* stream);

/* Cross-layer expert correlation (PopFetcher notes §4.1: a token choosing
 * expert x in layer j and x' in layer j+1 gives the tuple (x, x')).  Counts
 * this iteration's tuples of T tokens, idx_a [T, k_a] (layer j, experts
 * < E_a) against idx_b [T, k_b] (layer j+1, experts < E_b), into
 * ring[iter % window] ([window][E_a][E_b] int32) and writes window_sum
 * [E_a][E_b] = sum of the last min(iter + 1, window) slices (the sliding
 * window of §4.2).  Exact integers.  Limits: 1 <= E_a, E_b <=
 * MOE_MAX_EXPERTS, 1 <= k <= MOE_MAX_TOPK (k_a <= E_a, k_b <= E_b),
 * 1 <= window <= 64, iter >= 0, T >= 1, else MOE_ERR_INVALID_ARG; expert
 * ids outside the ranges are a precondition violation.  Device pointers;
 * enqueues only. */
moe_status moe_cooccurrence_update(int32_t E_a, int32_t E_b, int32_t k_a, int32_t k_b,
                                   int32_t T, int32_t window, int64_t iter,
                                   const int32_t* idx_a, const int32_t* idx_b, int32_t* ring,
                                   int32_t* window_sum, void* stream);

/* Next-layer popularity from this layer's selections (PopFetcher notes
 * §4.2, Eq. 2 and Eq. 3, bodies missing from the page; reading taken):
 * P(x'|x) = cooc[x][x'] / sum_x'' cooc[x][x''] and
 * pred[x'] = sum over x = 0..E_a-1 (rows with zero total skipped) of
 * counts_a[x] * P(x'|x), each quotient, product and sum one correctly rounded
 * float64 operation in that order.  order [E_b] lists the experts by
 * decreasing pred, ties to the lower index.  counts_a [E_a], cooc
 * [E_a][E_b] int32 (e.g. moe_cooccurrence_update's window_sum), pred [E_b]
 * float64, order [E_b] int32; device pointers; enqueues only. */
moe_status moe_predict_popularity(int32_t E_a, int32_t E_b, const int32_t* counts_a,
                                  const int32_t* cooc, double* pred, int32_t* order,
                                  void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
