"""Seeded synthetic workloads for the single-GPU MoE layer.

This module only draws random inputs and states their shapes.  It holds none
of the layer's arithmetic (no routing, no permutation, no expert math), so both
the CPU reference under ``oracle/`` and the GPU path can take their inputs from
it without sharing any computation.

Workload shapes and value distributions follow the pages' description of the
workloads MoE systems see: skewed expert popularity that stabilises and then
drifts slowly between iterations (PopFetcher notes, §2.2 Motivation, Fig. 3 and
§4.1), batches of 4K-32K tokens with hidden sizes 1K-4K (LLEP blog, §3.1
performance table), and up to 128 experts per layer.

Random streams: ``np.random.default_rng([SEED, tag, iteration])`` with one tag
per tensor, so every tensor can be regenerated on its own.  Normal draws are
taken in float32 and, for bf16 workloads, rounded to bf16 with
round-to-nearest-even; the float32 arrays returned then hold bf16 values
exactly, and ``bf16_bits`` gives the 16-bit patterns to upload.
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Dict, Optional

import numpy as np

SEED = 0
TAGS = {"x": 1, "w_gate": 2, "order": 3, "w1": 4, "w2": 5, "dy": 6, "drift": 7,
        "successor": 8, "next_layer": 9}

_HERE = os.path.dirname(os.path.abspath(__file__))


def rng(tag: str, it: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED, TAGS[tag], it])


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bf16-representable")
    return (u >> 16).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    F: int
    E: int
    k: int
    capacity_factor: float  # <= 0: dropless
    dtype: str  # "f32" or "bf16"
    x_std: float
    zipf_s: Optional[float]  # None: zero gate bias
    backward: bool = False
    iters: int = 1
    window: int = 4
    drift_swaps: int = 0
    description: str = ""
    priority: str = "slot"  # capacity priority: "slot" or "choice" (choice-major)

    def tokens(self) -> int:
        return self.T


def _calibrated_exponent() -> float:
    with open(os.path.join(_HERE, "calibration.json")) as f:
        return float(json.load(f)["mixtral_shaped_zipf_s"])


def workloads() -> Dict[str, Workload]:
    return {
        "tiny_fp32": Workload(
            "tiny_fp32", T=256, d=64, F=128, E=8, k=2, capacity_factor=0.0,
            dtype="f32", x_std=0.02, zipf_s=None,
            description="T=256 d=64 F=128 E=8 top-2 dropless fp32"),
        "uniform_cf125": Workload(
            "uniform_cf125", T=4096, d=1024, F=4096, E=16, k=2, capacity_factor=1.25,
            dtype="bf16", x_std=1.0, zipf_s=None,
            description="T=4096 d=1024 F=4096 E=16 top-2 capacity 1.25 bf16"),
        "skewed_zipf12": Workload(
            "skewed_zipf12", T=8192, d=2048, F=8192, E=32, k=2, capacity_factor=0.0,
            dtype="bf16", x_std=1.0, zipf_s=1.2,
            description="T=8192 d=2048 F=8192 E=32 top-2 dropless Zipf(1.2) bias bf16"),
        "mixtral_shaped": Workload(
            "mixtral_shaped", T=16384, d=4096, F=14336, E=8, k=2, capacity_factor=0.0,
            dtype="bf16", x_std=1.0, zipf_s=_calibrated_exponent(), backward=True,
            description="T=16384 d=4096 F=14336 E=8 top-2 dropless, top expert ~35% of slots, fwd+bwd bf16"),
        "fine_grained": Workload(
            "fine_grained", T=32768, d=4096, F=1024, E=128, k=4, capacity_factor=0.0,
            dtype="bf16", x_std=1.0, zipf_s=1.0, backward=True, iters=8, window=4,
            drift_swaps=4,
            description="T=32768 d=4096 F=1024 E=128 top-4 dropless Zipf(1.0) drifting over 8 iterations, window 4, fwd+bwd bf16"),
    }


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (for small parity cases).
    The description then lists the changed fields after the original's."""
    if changes and "description" not in changes:
        diff = " ".join(f"{k}={v}" for k, v in changes.items())
        changes["description"] = f"{w.name} scaled to {diff}"
    return dataclasses.replace(w, **changes)


def _normal(tag: str, shape, std: float, dtype: str, it: int = 0) -> np.ndarray:
    a = rng(tag, it).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return round_to_bf16(a) if dtype == "bf16" else a


def expert_order(w: Workload, it: int = 0) -> np.ndarray:
    """Experts listed from most to least favoured at iteration ``it``.

    Iteration 0 is a seeded random permutation; each later iteration applies
    ``drift_swaps`` seeded adjacent transpositions to the previous order.
    """
    order = rng("order").permutation(w.E)
    for i in range(1, it + 1):
        pos = rng("drift", i).integers(0, max(w.E - 1, 1), size=w.drift_swaps)
        for p in pos:
            order[p], order[p + 1] = order[p + 1], order[p]
    return order


def gate_bias(w: Workload, it: int = 0, zipf_s: Optional[float] = None) -> np.ndarray:
    """b[e] = -s * ln(rank(e)), rank 1 for the most favoured expert (log-Zipf)."""
    s = w.zipf_s if zipf_s is None else zipf_s
    if s is None:
        return np.zeros(w.E, dtype=np.float32)
    order = expert_order(w, it)
    rank = np.empty(w.E, dtype=np.float64)
    rank[order] = np.arange(1, w.E + 1, dtype=np.float64)
    return (-s * np.log(rank)).astype(np.float32)


def make_x(w: Workload, it: int = 0) -> np.ndarray:
    return _normal("x", (w.T, w.d), w.x_std, w.dtype, it)


def make_dy(w: Workload, it: int = 0) -> np.ndarray:
    return _normal("dy", (w.T, w.d), 1.0, w.dtype, it)


def make_w_gate(w: Workload) -> np.ndarray:
    return _normal("w_gate", (w.d, w.E), 0.02, "f32")


def make_w1(w: Workload) -> np.ndarray:
    """Expert FC1 weights, [E, F, d] (output x input)."""
    return _normal("w1", (w.E, w.F, w.d), 0.02, w.dtype)


def make_w2(w: Workload) -> np.ndarray:
    """Expert FC2 weights, [E, d, F] (output x input)."""
    return _normal("w2", (w.E, w.d, w.F), 0.02, w.dtype)


def make_inputs(w: Workload, it: int = 0, with_weights: bool = True,
                with_dy: bool = False) -> Dict[str, np.ndarray]:
    out = {"x": make_x(w, it), "w_gate": make_w_gate(w), "b_gate": gate_bias(w, it)}
    if with_weights:
        out["w1"] = make_w1(w)
        out["w2"] = make_w2(w)
    if with_dy:
        out["dy"] = make_dy(w, it)
    return out


def identity_experts(d: int, E: int, dtype: str = "f32"):
    """Experts whose FC-ReLU-FC is exactly the identity: F = 2d,
    W1 = [I; -I] and W2 = [I, -I], so ReLU(x) - ReLU(-x) = x."""
    eye = np.eye(d, dtype=np.float32)
    w1 = np.concatenate([eye, -eye], axis=0)  # [2d, d]
    w2 = np.concatenate([eye, -eye], axis=1)  # [d, 2d]
    return (np.broadcast_to(w1, (E, 2 * d, d)).copy(),
            np.broadcast_to(w2, (E, d, 2 * d)).copy())


def capacity_free_bound(w: Workload) -> int:
    """Largest number of rows the permuted buffers can hold: T*k."""
    return w.T * w.k


def quantize_half_steps(a: np.ndarray) -> np.ndarray:
    """Round values to multiples of 0.5 (a tie-heavy routing input)."""
    return (np.round(np.asarray(a, dtype=np.float64) * 2.0) / 2.0).astype(np.float32)



def next_layer_choices(idx_a: np.ndarray, E_b: int, k_b: int, it: int = 0,
                       follow: float = 0.7) -> np.ndarray:
    """Synthetic top-k choices of the following layer, correlated with this
    layer's: a seeded successor map sends expert x to x' = succ[x]; each of a
    token's k_b choices is, with probability ``follow``, the successor of its
    next unused layer-j choice, else a uniformly drawn expert; choices are
    made distinct by skipping repeats.  The successor map is fixed across
    iterations; the coin flips and draws change with ``it``.  (Input
    generation only: the pages' cross-layer tuples, not a learned router.)"""
    T, k_a = idx_a.shape
    succ = rng("successor", 0).permutation(E_b)
    g = rng("next_layer", it)
    flips = g.random((T, 4 * k_b))
    draws = g.integers(0, E_b, (T, 4 * k_b))
    out = np.empty((T, k_b), dtype=np.int32)
    for t in range(T):
        chosen = []
        a = 0
        c = 0
        while len(chosen) < k_b:
            if c < 4 * k_b and flips[t, c] < follow and a < k_a:
                cand = int(succ[int(idx_a[t, a]) % E_b])
                a += 1
            elif c < 4 * k_b:
                cand = int(draws[t, c])
            else:
                cand = (chosen[-1] + 1) % E_b if chosen else 0
            c += 1
            if cand not in chosen:
                chosen.append(cand)
        out[t] = chosen
    return out
