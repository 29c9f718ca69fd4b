// Host-side launchers of the gfx950 MoE kernels (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- gate routing (route.hip)
// logits = x * w_gate + b (float32); top-k with lowest-index ties; weights =
// softmax over the selected logits.
// bf16 without logits_in runs the router on MFMA (W_gate split into three
// exact bf16 parts in registers as its fragments are used).
hipError_t launch_route(int act, const void* x, const float* w_gate, const float* b_gate,
                        const float* logits_in, float* logits_out, int32_t* topk_idx,
                        float* topk_w, int T, int d, int E, int k, hipStream_t s);
int route_padded_experts(int E);

// ---- input encode (permute.hip)
// Per tile of kRankTile slots: stable rank of each slot among the tile's
// slots of the same expert, and the tile histogram hist[e][tile].
hipError_t launch_rank_hist(const int32_t* topk_idx, int T, int k, bool choice, int E,
                            int32_t* local_rank, int32_t* hist, int n_tiles, hipStream_t s);
// Exclusive scan of hist over tiles per expert (tile_base, in place of hist
// is not allowed), counts_raw and counts_kept = min(raw, C).
hipError_t launch_scan(const int32_t* hist, int n_tiles, int E, int C, int32_t* tile_base,
                       int32_t* counts_raw, int32_t* counts_kept, hipStream_t s);
// slot_row, row_token, offsets and the row copy x -> x_perm.
// Dropped slots are listed after the kept rows: row_token[S_kept + j].
hipError_t launch_gather(int act, const void* x, const int32_t* topk_idx,
                         const int32_t* local_rank, const int32_t* tile_base,
                         const int32_t* counts_raw, const int32_t* counts_kept, int n_tiles,
                         int T, int d, int E, int k,
                         int C, bool choice, int32_t* offsets, int32_t* slot_row,
                         int32_t* row_token, void* x_perm, hipStream_t s);
// The same indices without the row copy, plus row_slot[r] = slot of kept row r.
hipError_t launch_index(const int32_t* topk_idx, const int32_t* local_rank,
                        const int32_t* tile_base, const int32_t* counts_raw,
                        const int32_t* counts_kept, int n_tiles, int T, int E, int k, int C,
                        bool choice, int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                        int32_t* row_slot, hipStream_t s);

// ---- output decode and the elementwise backward steps (combine.hip)
// slot_order: expert output of kept slot s is row s of out_perm (else row
// slot_row[s]).
hipError_t launch_combine(int act, const void* out_perm, const float* topk_w,
                          const int32_t* slot_row, void* y, int T, int d, int k, hipStream_t s,
                          bool slot_order = false);
// Decode backward; its extra workgroups also write w_gate_t = W_gate^T, and
// it zeroes the kBwdCounters tile counters of the weight-gradient GEMMs that
// follow on the stream (counters may be null).
constexpr int kBwdCounters = 2;
hipError_t launch_combine_bwd(int act, const void* dy, const void* out_perm,
                              const float* topk_w, const int32_t* topk_idx,
                              const int32_t* slot_row, void* d_out, float* dsel,
                              float* dsel_perm, float* dlogits, const float* w_gate,
                              float* w_gate_t, int32_t* counters, int T, int d, int E, int k,
                              hipStream_t s);
// dW_gate / db over each expert's packed rows (float32 path; bf16 folds it
// into the FC1 weight gradient) ...
hipError_t launch_gate_rows(int act, const void* x_perm, const float* dsel_perm,
                            const int32_t* offsets, float* dw_gate, float* db_gate, int d, int E,
                            hipStream_t s);
// dX; with `dropped`, its extra workgroups add the gate gradient of the
// dropped slots listed after the kept rows in row_token to dW_gate / db.
hipError_t launch_dx(int act, const void* dx_perm, const float* dsel, const int32_t* topk_idx,
                     const int32_t* slot_row, const float* w_gate_t, void* dx, int T, int d,
                     int k, bool dropped, const void* x, const int32_t* offsets,
                     const int32_t* row_token, float* dw_gate, float* db_gate, int E,
                     hipStream_t s);
hipError_t launch_popularity(int E, int window, int64_t iter, const int32_t* counts_raw,
                             int32_t* ring, int32_t* window_sum, hipStream_t s);

// ---- expert GEMMs (gemm.hip)
// Forward: h = ReLU(x_perm W1[e]^T), out = h W2[e]^T over each expert's rows.
// relu_bits (bf16, optional): keep bits [h > 0] written by FC1's epilogue.
// partial (bf16; rows_partial_bytes, or null): scratch for splitting the
// last round of tiles along K.  max_rows: the most rows one expert can hold
// (the capacity; T when dropless), which picks the weights' cache policy.
size_t rows_partial_bytes(int act);
hipError_t launch_expert_fwd(int act, const void* x_perm, const int32_t* offsets,
                             const void* w1, const void* w2, void* h, void* out_perm,
                             uint32_t* relu_bits, float* partial, int S_max, int max_rows, int d,
                             int F, int E, hipStream_t s);
// Gather/scatter-fused forward: FC1 reads token rows x[row_token[r]] ([T][d]);
// FC2 stores packed row r at row row_slot[r] of out_slot ([T*k][d]).
hipError_t launch_expert_fwd_fused(int act, const void* x, const int32_t* row_token, int T,
                                   const int32_t* offsets, const int32_t* row_slot,
                                   const void* w1, const void* w2, void* h, void* out_slot,
                                   uint32_t* relu_bits, float* partial, int S_max, int max_rows,
                                   int d, int F, int E, hipStream_t s);
// Backward GEMMs: dz = (dO W2[e]) * [h > 0]; dW2[e] = dO^T h;
// dx_perm = dz W1[e]; dW1[e] = dz^T x_perm.
// bf16 also folds dW_gate / db over the kept rows into the FC1 wgrad and
// takes the ReLU mask from relu_bits_in if non-null, else derives it from h
// into relu_bits_ws ([S_max][F/32] words of scratch).  The two bf16 weight
// gradients take their tiles from counters[0] and counters[1], which must be
// zero at launch (launch_combine_bwd zeroes them).  With replicas (bf16
// only; rep_start [E+1], rep_row0 / rep_rows [n_copies] as moe_ep_plan writes
// them), each copy of an expert is a K range of its own and an expert with
// several copies gets the sum of the copies' partial weight gradients in copy
// order (rep_part: wgrad_replica_bytes of scratch).
hipError_t launch_expert_bwd(int act, const void* d_out, const void* x_perm, const void* h,
                             const int32_t* offsets, const void* w1, const void* w2,
                             void* dz, void* dx_perm, float* dw1, float* dw2,
                             const float* dsel_perm, float* dw_gate, float* db_gate,
                             const uint32_t* relu_bits_in, uint32_t* relu_bits_ws,
                             float* partial, int32_t* counters, int S_max, int max_rows,
                             int d, int F, int E, hipStream_t s,
                             const int32_t* rep_start = nullptr,
                             const int32_t* rep_row0 = nullptr,
                             const int32_t* rep_rows = nullptr, int n_copies = 0,
                             float* rep_part = nullptr);
// Scratch of the replicated weight gradients (bf16): per partial slot a dW,
// a gate column and a db value; at most 2 (n_copies - E) slots.
size_t wgrad_replica_bytes(int n_copies, int E, int d, int F);

// ---- expert-parallel dispatch plan (plan.hip)
hipError_t launch_ep_plan(int E, int R, int extra, const int32_t* offsets,
                          int32_t* replica_start, int32_t* replica_row0, int32_t* replica_rows,
                          int32_t* replica_rank, int32_t* rank_rows, hipStream_t s);
hipError_t launch_dispatch_layout(int n, int R, const int32_t* seg_rows, const int32_t* seg_rank,
                                  int32_t* send_counts, int32_t* send_offsets,
                                  int32_t* seg_send_offset, hipStream_t s);

// ---- cross-layer correlation and popularity prediction (correl.hip)
hipError_t launch_cooccurrence(int E_a, int E_b, int k_a, int k_b, int T, int window,
                               int64_t iter, const int32_t* idx_a, const int32_t* idx_b,
                               int32_t* ring, int32_t* window_sum, hipStream_t s);
hipError_t launch_predict(int E_a, int E_b, const int32_t* counts_a, const int32_t* cooc,
                          double* pred, int32_t* order, hipStream_t s);

}  // namespace moe
