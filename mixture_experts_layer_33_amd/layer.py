"""Device buffers for one MoE layer shape, allocated through torch.

``MoeLayer`` owns every output, saved tensor and workspace that the C entry
points write, so a caller only brings the inputs.  It computes nothing: each
method is one call of the binding.
"""
from __future__ import annotations

import torch

from . import (MOE_BF16, MOE_F32, MoeShape, moe_backward, moe_capacity, moe_check_shape,
               moe_combine, moe_expert_ffn, moe_forward, moe_forward_fused, moe_permute,
               moe_popularity_update, moe_route, moe_status_string, moe_workspace_bytes)


def act_torch_dtype(act: int):
    return torch.bfloat16 if act == MOE_BF16 else torch.float32


class MoeLayer:
    def __init__(self, T, d, F, E, k, capacity_factor=0.0, act=MOE_BF16, device="cuda",
                 window=4, backward=True, priority="slot"):
        self.shape = MoeShape.make(T, d, F, E, k, capacity_factor, act, priority)
        st = moe_check_shape(self.shape)
        if st != 0:
            raise ValueError(f"bad shape: {moe_status_string(st)}")
        self.T, self.d, self.F, self.E, self.k = T, d, F, E, k
        self.act = act
        self.dtype = act_torch_dtype(act)
        self.device = device
        S = T * k
        i32, f32 = torch.int32, torch.float32
        z = lambda *s, dt: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
        self.C = moe_capacity(self.shape)
        self.y = z(T, d, dt=self.dtype)
        self.logits = z(T, E, dt=f32)
        self.topk_idx = z(T, k, dt=i32)
        self.topk_w = z(T, k, dt=f32)
        self.counts_raw = z(E, dt=i32)
        self.counts_kept = z(E, dt=i32)
        self.offsets = z(E + 1, dt=i32)
        self.slot_row = z(S, dt=i32)
        self.row_token = z(S, dt=i32)
        self.x_perm = z(S, d, dt=self.dtype)
        self.h = z(S, F, dt=self.dtype)
        self.out_perm = z(S, d, dt=self.dtype)
        # keep bits of the ReLU, written by the forward and read by the
        # backward (bf16 only); relu_bits_used = False makes the backward
        # derive the mask from h instead
        self.relu_bits = z(S, F // 32, dt=i32) if act == MOE_BF16 else None
        self.relu_bits_used = True
        self.ws_fwd = z(max(moe_workspace_bytes(self.shape, "forward"), 256), dt=torch.uint8)
        self.window = window
        self.ring = torch.zeros(window, E, dtype=i32, device=device)
        self.window_sum = torch.zeros(E, dtype=i32, device=device)
        if backward:
            self.dx = z(T, d, dt=self.dtype)
            self.dw1 = z(E, F, d, dt=f32)
            self.dw2 = z(E, d, F, dt=f32)
            self.dw_gate = z(d, E, dt=f32)
            self.db_gate = z(E, dt=f32)
            self.dlogits = z(T, E, dt=f32)
            self.ws_bwd = z(max(moe_workspace_bytes(self.shape, "backward"), 256), dt=torch.uint8)

    # one call each -------------------------------------------------------
    def forward(self, x, w_gate, b_gate, w1, w2, logits_out=True, stream=None):
        moe_forward(self.shape, x, w_gate, b_gate, w1, w2, self.y,
                    self.logits if logits_out else None, self.topk_idx, self.topk_w,
                    self.counts_raw, self.counts_kept, self.offsets, self.slot_row,
                    self.row_token, self.x_perm, self.h, self.out_perm, self.relu_bits,
                    self.ws_fwd, stream)
        return self.y

    def forward_fused(self, x, w_gate, b_gate, w1, w2, logits_out=True, stream=None):
        """The gather/scatter-fused forward: same y and indices as forward(),
        expert outputs by slot in ``out_slot`` and no x_perm; not for the
        backward."""
        if getattr(self, "out_slot", None) is None:
            self.out_slot = torch.empty(self.T * self.k, self.d, dtype=self.dtype,
                                        device=self.device)
            nb = max(moe_workspace_bytes(self.shape, "forward_fused"), 256)
            self.ws_fused = torch.empty(nb, dtype=torch.uint8, device=self.device)
        moe_forward_fused(self.shape, x, w_gate, b_gate, w1, w2, self.y,
                          self.logits if logits_out else None, self.topk_idx, self.topk_w,
                          self.counts_raw, self.counts_kept, self.offsets, self.slot_row,
                          self.row_token, self.h, self.out_slot, self.relu_bits, self.ws_fused,
                          stream)
        return self.y

    def backward(self, dy, x, w_gate, w1, w2, dlogits=True, stream=None):
        moe_backward(self.shape, dy, x, w_gate, w1, w2, self.topk_idx, self.topk_w,
                     self.slot_row, self.row_token, self.offsets, self.x_perm, self.h,
                     self.out_perm, self.relu_bits if self.relu_bits_used else None, self.dx,
                     self.dw1, self.dw2, self.dw_gate, self.db_gate,
                     self.dlogits if dlogits else None, self.ws_bwd, stream)
        return self.dx

    def route(self, x, w_gate, b_gate, logits_in=None, logits_out=True, counts=True,
              stream=None):
        moe_route(self.shape, x, w_gate, b_gate, logits_in,
                  self.logits if logits_in is None and logits_out else None, self.topk_idx,
                  self.topk_w, self.counts_raw if counts else None, self.ws_fwd, stream)

    def permute(self, x, topk_idx=None, counts=True, stream=None):
        moe_permute(self.shape, x, self.topk_idx if topk_idx is None else topk_idx,
                    self.counts_raw if counts else None, self.counts_kept, self.offsets,
                    self.slot_row, self.row_token, self.x_perm, self.ws_fwd, stream)

    def expert_ffn(self, w1, w2, x_perm=None, offsets=None, stream=None):
        if getattr(self, "ws_ffn", None) is None:
            nb = max(moe_workspace_bytes(self.shape, "expert_ffn"), 256)
            self.ws_ffn = torch.empty(nb, dtype=torch.uint8, device=self.device)
        moe_expert_ffn(self.shape, self.x_perm if x_perm is None else x_perm,
                       self.offsets if offsets is None else offsets, w1, w2, self.h,
                       self.out_perm, self.relu_bits, self.ws_ffn, stream)

    def combine(self, out_perm=None, topk_w=None, slot_row=None, stream=None):
        moe_combine(self.shape, self.out_perm if out_perm is None else out_perm,
                    self.topk_w if topk_w is None else topk_w,
                    self.slot_row if slot_row is None else slot_row, self.y, stream)

    def popularity(self, it, counts_raw=None, stream=None):
        moe_popularity_update(self.E, self.window, it,
                              self.counts_raw if counts_raw is None else counts_raw,
                              self.ring, self.window_sum, stream)


__all__ = ["MoeLayer", "act_torch_dtype", "MOE_BF16", "MOE_F32"]
