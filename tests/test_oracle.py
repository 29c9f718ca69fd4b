"""Pins for the CPU reference (runs without a GPU).

Each test ties a part of ``oracle.moe_oracle`` to something other than
itself: a hand-worked example, a library routine, a closed form, an
invariant, brute force on tiny inputs, torch autograd or finite differences.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# ---------------------------------------------------------------- routing
def test_hand_worked_routing():
    g = load("hand_routing.json")
    L = np.array(g["logits"], dtype=np.float32)
    L[3, 1] = -0.0
    idx, w = orc.topk_gate(L, g["k"])
    assert idx.tolist() == g["idx"]
    e = math.e
    want = [[e / (1 + e), 1 / (1 + e)], [0.5, 0.5], [0.5, 0.5],
            [e ** 4 / (1 + e ** 4), 1 / (1 + e ** 4)]]
    np.testing.assert_allclose(w, np.array(want), rtol=1e-7)
    assert idx.reshape(-1).tolist() == g["expert_of_slot"]
    for case in ("capacity_case", "dropless_case"):
        c = g[case]
        C = orc.capacity(g["T"], g["k"], g["E"], c["capacity_factor"])
        assert C == c["C"]
        s = orc.assign_slots(idx, g["E"], C)
        for key in ("counts_raw", "counts_kept", "offsets", "slot_row", "row_token"):
            assert s[key].tolist() == c[key], (case, key)
        assert s["drops"] == c["drops"]


def test_hand_worked_capacity_priorities():
    """Slot order and GShard's choice-major order on the hand-worked fixture
    (C = 1 tells them apart: token 3's first choice beats token 0's second)."""
    g = load("hand_routing.json")
    L = np.array(g["logits"], dtype=np.float32)
    L[3, 1] = -0.0
    idx, _ = orc.topk_gate(L, g["k"])
    cases = [("slot", g["slot_order_C1_case"])] + [("choice", c) for c in g["choice_major_cases"]]
    for prio, c in cases:
        C = orc.capacity(g["T"], g["k"], g["E"], c["capacity_factor"])
        assert C == c["C"]
        s = orc.assign_slots(idx, g["E"], C, prio)
        for key in ("counts_raw", "counts_kept", "offsets", "slot_row", "row_token", "dropped"):
            assert s[key].tolist() == c[key], (prio, c["C"], key)
        assert s["drops"] == c["drops"]


@pytest.mark.parametrize("cf", [0.5, 0.8, 1.0])
def test_choice_major_capacity_bruteforce(cf):
    """Position of a slot = number of slots of the same expert that come
    earlier in (choice, token) order, counted directly."""
    rng = np.random.default_rng(11)
    T, E, k = 37, 5, 3
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:, 1] += 1.2
    idx, _ = orc.topk_gate(L, k)
    C = orc.capacity(T, k, E, cf)
    s = orc.assign_slots(idx, E, C, "choice")
    n_kept = [0] * E
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            pos = sum(1 for jj in range(k) for tt in range(T)
                      if idx[tt, jj] == e and (jj, tt) < (j, t))
            if pos < C:
                n_kept[e] += 1
                row = int(s["offsets"][e]) + pos
                assert s["slot_row"][t * k + j] == row
                assert s["row_token"][row] == t
            else:
                assert s["slot_row"][t * k + j] == -1
    assert s["counts_kept"].tolist() == n_kept
    assert s["drops"] == T * k - sum(n_kept) > 0
    # dropped list: by expert, then position
    exp = [int(idx.reshape(-1)[q]) for q in s["dropped"]]
    assert exp == sorted(exp)


def test_hand_worked_popularity():
    p = load("hand_routing.json")["popularity_case"]
    W = p["window"]
    ring = np.zeros((W, 3), np.int32)
    for it, (cnt, want) in enumerate(zip(p["counts_per_iteration"], p["window_sum_per_iteration"])):
        ring, ws = orc.popularity_update(ring, it, np.array(cnt))
        assert ws.tolist() == want


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_lexsort_bruteforce(seed):
    rng = np.random.default_rng(seed)
    T, E = 64, 7
    L = rng.standard_normal((T, E)).astype(np.float32)
    if seed % 2:  # many exact ties
        L = workloads.quantize_half_steps(L)
    if seed == 5:  # signed zeros must tie
        L[:, :3] = np.array([0.0, -0.0, 0.0], np.float32)
        L[:, 3:] = -1.0
    for k in (1, 2, 3, E):
        idx, w = orc.topk_gate(L, k)
        for t in range(T):
            # lexsort: last key is primary -> primary -L, secondary index
            order = np.lexsort((np.arange(E), -L[t].astype(np.float64) + 0.0))
            assert idx[t].tolist() == order[:k].tolist()
        assert np.all(np.diff(w, axis=1) <= 0)
        np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=4 * 2 ** -23)


def test_topk_all_equal_and_full_softmax():
    T, E = 5, 6
    L = np.full((T, E), 0.25, np.float32)
    idx, w = orc.topk_gate(L, 3)
    assert (idx == np.arange(3)).all()
    np.testing.assert_array_equal(w, np.float32(1 / 3))
    L = rand((T, E), 3)
    idx, w = orc.topk_gate(L, E)
    full = torch.softmax(torch.from_numpy(L.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(full, idx, 1), rtol=1e-6)


def test_topk_rejects_nonfinite():
    L = np.zeros((2, 3), np.float32)
    L[1, 2] = np.nan
    with pytest.raises(ValueError):
        orc.topk_gate(L, 2)


def test_router_logits_special_cases():
    T, d, E = 9, 12, 5
    x = rand((T, d), 1)
    b = rand((E,), 2)
    eye = np.zeros((d, E), np.float32)
    eye[np.arange(E), np.arange(E)] = 1.0
    np.testing.assert_array_equal(orc.router_logits(x, eye, b), x[:, :E] + b)
    # against torch's float64 linear layer
    wg = rand((d, E), 3)
    lin = torch.nn.Linear(d, E, dtype=torch.float64)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(wg.T.astype(np.float64)))
        lin.bias.copy_(torch.from_numpy(b.astype(np.float64)))
        ref = lin(torch.from_numpy(x.astype(np.float64))).float().numpy()
    np.testing.assert_array_equal(orc.router_logits(x, wg, b), ref)


# ---------------------------------------------------------------- capacity / permutation
def test_capacity_values():
    assert orc.capacity(4096, 2, 16, 1.25) == 640
    assert orc.capacity(4096, 2, 16, 1.0) == 512
    assert orc.capacity(4096, 2, 16, 0.0) == 4096
    assert orc.capacity(10, 1, 100, 0.01) == 1          # clamp below
    assert orc.capacity(10, 4, 2, 5.0) == 10            # clamp above


@pytest.mark.parametrize("seed", range(4))
def test_assign_slots_dropless_is_stable_sort(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 300, 9, 3
    L = rng.standard_normal((T, E)).astype(np.float32) + np.log(np.arange(1, E + 1))[::-1].astype(np.float32)
    idx, _ = orc.topk_gate(L, k)
    s = orc.assign_slots(idx, E, orc.capacity(T, k, E, 0.0))
    flat = idx.reshape(-1)
    assert s["counts_raw"].tolist() == np.bincount(flat, minlength=E).tolist()
    assert s["offsets"].tolist() == [0] + np.cumsum(s["counts_kept"]).tolist()
    order = np.argsort(flat, kind="stable")          # library stable sort
    assert s["row_token"].tolist() == (order // k).tolist()
    assert sorted(s["slot_row"].tolist()) == list(range(T * k))  # bijection
    assert (s["slot_row"][order] == np.arange(T * k)).all()


@pytest.mark.parametrize("cf", [0.5, 0.8, 1.0])
def test_assign_slots_capacity_bruteforce(cf):
    rng = np.random.default_rng(7)
    T, E, k = 40, 5, 2
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:, 0] += 1.5  # make expert 0 overflow
    idx, _ = orc.topk_gate(L, k)
    C = orc.capacity(T, k, E, cf)
    s = orc.assign_slots(idx, E, C)
    flat = idx.reshape(-1)
    S = T * k
    kept_rows = []
    for sl in range(S):
        e = flat[sl]
        pos = sum(1 for p in range(sl) if flat[p] == e)   # O(S^2) brute force
        if pos < C:
            row = sum(min(C, int((flat == ee).sum())) for ee in range(e)) + pos
            assert s["slot_row"][sl] == row
            assert s["row_token"][row] == sl // k
            kept_rows.append(row)
        else:
            assert s["slot_row"][sl] == -1
    assert sorted(kept_rows) == list(range(len(kept_rows)))
    assert s["drops"] == S - len(kept_rows) == S - int(s["counts_kept"].sum())
    assert (s["counts_kept"] <= C).all()
    assert s["drops"] > 0


# ---------------------------------------------------------------- experts
def test_expert_ffn_is_torch_mlp_for_one_expert():
    T, d, F = 17, 8, 24
    x = rand((T, d), 4)
    w1 = rand((1, F, d), 5, 0.3)
    w2 = rand((1, d, F), 6, 0.3)
    mlp = torch.nn.Sequential(torch.nn.Linear(d, F, bias=False, dtype=torch.float64),
                              torch.nn.ReLU(),
                              torch.nn.Linear(F, d, bias=False, dtype=torch.float64))
    with torch.no_grad():
        mlp[0].weight.copy_(torch.from_numpy(w1[0].astype(np.float64)))
        mlp[2].weight.copy_(torch.from_numpy(w2[0].astype(np.float64)))
        ref = mlp(torch.from_numpy(x.astype(np.float64))).numpy()
    out = orc.forward(x, np.zeros((d, 1), np.float32), np.zeros(1, np.float32), w1, w2,
                      k=1, capacity_factor=0.0, act="f64")
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)
    assert out["idx"].tolist() == [[0]] * T
    np.testing.assert_array_equal(out["w"], 1.0)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_identity_experts_give_weighted_input(act):
    T, d, E, k = 50, 16, 4, 2
    x = workloads.round_to_bf16(rand((T, d), 8)) if act == "bf16" else rand((T, d), 8)
    w1, w2 = workloads.identity_experts(d, E)
    out = orc.forward(x, rand((d, E), 9), rand((E,), 10), w1, w2, k, 0.0, act)
    np.testing.assert_array_equal(out["o"], out["x_perm"].astype(np.float64))
    wsum = out["w"].astype(np.float64).sum(1, keepdims=True)
    ref = orc.round_act(wsum * x.astype(np.float64), act)
    np.testing.assert_array_equal(out["y"], ref)
    np.testing.assert_allclose(out["y"], x, rtol=2 ** -7 if act == "bf16" else 1e-6)


def test_all_dropped_token_outputs_zero():
    T, d, E, k = 8, 4, 2, 1
    x = rand((T, d), 11)
    b = np.array([5.0, -5.0], np.float32)   # everyone picks expert 0
    w1, w2 = workloads.identity_experts(d, E)
    out = orc.forward(x, np.zeros((d, E), np.float32), b, w1, w2, k, 0.5, "f32")
    C = out["C"]
    assert C == 2
    assert (out["slot_row"][:C] >= 0).all() and (out["slot_row"][C:] == -1).all()
    np.testing.assert_array_equal(out["y"][C:], 0.0)
    np.testing.assert_allclose(out["y"][:C], x[:C], rtol=1e-7)


@pytest.mark.parametrize("cf", [0.0, 0.6])
def test_forward_equals_dense_per_token(cf):
    T, d, F, E, k = 64, 12, 20, 6, 3
    x = rand((T, d), 12)
    wg = rand((d, E), 13)
    b = rand((E,), 14)
    w1 = rand((E, F, d), 15, 0.4)
    w2 = rand((E, d, F), 16, 0.4)
    out = orc.forward(x, wg, b, w1, w2, k, cf, "f64")
    if cf:
        assert out["drops"] > 0
    for t in range(T):
        ref = orc.token_output(t, x, out["w"], out["idx"], out["slot_row"], w1, w2, "f64")
        np.testing.assert_allclose(out["y"][t], ref, rtol=1e-12, atol=1e-13)
    # and against a torch dense evaluation that never permutes
    xt = torch.from_numpy(x.astype(np.float64))
    logits = torch.from_numpy(out["logits"].astype(np.float64))
    top = torch.topk(logits, k, dim=1)
    assert (top.indices.numpy() == out["idx"]).all()
    wt = torch.softmax(top.values, dim=1)
    y = torch.zeros_like(xt)
    for t in range(T):
        for j in range(k):
            if out["slot_row"][t * k + j] < 0:
                continue
            e = int(top.indices[t, j])
            hh = torch.relu(torch.nn.functional.linear(xt[t], torch.from_numpy(w1[e].astype(np.float64))))
            y[t] += wt[t, j] * torch.nn.functional.linear(hh, torch.from_numpy(w2[e].astype(np.float64)))
    # the oracle's weights are stored in float32, torch's stay float64
    ref = y.numpy()
    np.testing.assert_allclose(out["y"], ref, rtol=0, atol=2e-7 * np.abs(ref).max())


def test_capacity_ceiling_hand_worked():
    """Non-integer quotients where ceil, floor and nearest all differ
    (golden/capacity_ceiling.json, worked by hand), plus a routing case in
    which the ceiling decides which slot is dropped."""
    g = load("capacity_ceiling.json")
    for c in g["cases"]:
        got = orc.capacity(c["T"], c["k"], c["E"], c["cf"])
        assert got == c["C"], c
        assert got != c["floor"] or c["floor"] < 1
    d = g["drop_case"]
    idx, _ = orc.topk_gate(np.array(d["logits"], np.float32), d["k"])
    C = orc.capacity(d["T"], d["k"], d["E"], d["capacity_factor"])
    assert C == d["C"]
    s = orc.assign_slots(idx, d["E"], C)
    for key in ("counts_raw", "counts_kept", "offsets", "slot_row", "row_token", "dropped"):
        assert s[key].tolist() == d[key], key
    assert s["drops"] == d["drops"]


def test_capacity_is_the_least_sufficient_integer():
    """Invariant of a ceiling: C - 1 < cf*T*k/E <= C (before the clamp), on
    random shapes; exact rational arithmetic on the float32 capacity factor."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    for _ in range(500):
        T, k = int(rng.integers(1, 5000)), int(rng.integers(1, 9))
        E = int(rng.integers(k, 300))
        cf = float(np.float32(rng.uniform(0.01, 3.0)))
        q = Fraction(cf) * T * k / E
        C = orc.capacity(T, k, E, cf)
        if 1 < C < T:
            assert C - 1 < q <= C, (T, k, E, cf, C, float(q))


def test_bf16_single_rounding():
    """float64 -> bf16 in one rounding: a value just above a bf16 half-way
    point goes up (rounding through float32 first would land exactly on the
    half-way point and then tie to even, down)."""
    v = np.array([1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8 + 2 ** -30), 1 + 2 ** -8 - 2 ** -30])
    np.testing.assert_array_equal(orc.round_act(v, "bf16"),
                                  [1 + 2 ** -7, -(1 + 2 ** -7), 1.0])


def test_bf16_rounding_special_ranges():
    """bf16 subnormals (quantum 2**-133, ties to even), the largest finite
    value, overflow at the half-way point above it, signed zero, inf, NaN."""
    v = np.array([1.5 * 2 ** -133, 2 ** -134, 3 * 2 ** -135, 2.5 * 2 ** -133,
                  (2 - 2 ** -7) * 2 ** 127, (2 - 2 ** -8) * 2 ** 127, -0.0, -np.inf])
    got = orc.round_act(v, "bf16")
    np.testing.assert_array_equal(got[:6], [2 ** -132, 0.0, 2 ** -133, 2 ** -132,
                                            (2 - 2 ** -7) * 2 ** 127, np.inf])
    assert got[6] == 0.0 and np.signbit(got[6])
    assert got[7] == -np.inf
    assert np.isnan(orc.round_act(np.array([np.nan]), "bf16")[0])


def test_bf16_rounding_against_brute_force():
    """Every result is the nearest of all 65536 bf16 bit patterns (ties to
    the pattern with an even last bit), by exhaustive search."""
    pats = np.arange(1 << 16, dtype=np.uint32)
    ok = (pats & 0x7F80) != 0x7F80                     # finite patterns only
    pats = pats[ok]
    vals = (pats << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 39, 3000),
                        vals[rng.integers(0, vals.size, 500)] * (1 + 2.0 ** -8)])
    got = orc.round_act(v, "bf16")
    for x, g in zip(v, got):
        dist = np.abs(vals - x)
        best = dist.min()
        cand = pats[dist == best]
        if cand.size > 1:
            cand = cand[(cand & 1) == 0]
        want = np.array([int(cand[0]) << 16], np.uint32).view(np.float32)[0]
        if abs(x) >= (2 - 2 ** -8) * 2.0 ** 127:           # past the last half-way point
            want = np.copysign(np.inf, x)
        assert g == want, (x, g, want)


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8)], np.float64)
    np.testing.assert_array_equal(orc.round_act(vals, "bf16"),
                                  [1.0, 1.0 + 2 ** -6, 1.0, -1.0])
    t = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(orc.round_act(vals, "bf16"), t)


# ---------------------------------------------------------------- popularity
def test_popularity_against_history():
    rng = np.random.default_rng(3)
    E, W = 7, 4
    ring = np.zeros((W, E), np.int32)
    hist = []
    for it in range(11):
        c = rng.integers(0, 1000, E)
        hist.append(c)
        ring, ws = orc.popularity_update(ring, it, c)
        assert ws.tolist() == np.sum(hist[-W:], axis=0).tolist()


# ---------------------------------------------------------------- backward
def _dense_torch_loss(x, wg, b, w1, w2, k, slot_row, dy):
    """Dense per-token forward in torch float64 with autograd; routing
    structure (which experts, which slots survive) held fixed."""
    T, d = x.shape
    logits = x @ wg + b
    top = torch.topk(logits.detach(), k, dim=1).indices
    sel = torch.gather(logits, 1, top)
    wt = torch.softmax(sel, dim=1)
    y = []
    for t in range(T):
        acc = torch.zeros(d, dtype=torch.float64)
        for j in range(k):
            if slot_row[t * k + j] < 0:
                continue
            e = int(top[t, j])
            hh = torch.relu(w1[e] @ x[t])
            acc = acc + wt[t, j] * (w2[e] @ hh)
        y.append(acc)
    return (torch.stack(y) * dy).sum()


@pytest.mark.parametrize("cf", [0.0, 0.5])
def test_backward_matches_torch_autograd(cf):
    T, d, F, E, k = 24, 8, 16, 4, 2
    x = rand((T, d), 20)
    wg = rand((d, E), 21)
    b = rand((E,), 22)
    w1 = rand((E, F, d), 23, 0.5)
    w2 = rand((E, d, F), 24, 0.5)
    dy = rand((T, d), 25)
    fwd = orc.forward(x, wg, b, w1, w2, k, cf, "f64")
    if cf:
        assert fwd["drops"] > 0
    g = orc.backward(dy, fwd, x, wg, w1, w2, "f64")
    tx, twg, tb, tw1, tw2 = (torch.tensor(a.astype(np.float64), requires_grad=True)
                            for a in (x, wg, b, w1, w2))
    loss = _dense_torch_loss(tx, twg, tb, tw1, tw2, k, fwd["slot_row"],
                             torch.from_numpy(dy.astype(np.float64)))
    loss.backward()
    # the oracle stores logits and gate weights in float32, torch keeps
    # float64 throughout, so agreement is to float32 level, scaled by the
    # tensor's largest entry (a missing term or a wrong sign is O(1))
    for mine, ref in ((g["dx_f64"], tx.grad), (g["dw1_f64"], tw1.grad), (g["dw2_f64"], tw2.grad),
                      (g["dw_gate"], twg.grad), (g["db_gate"], tb.grad)):
        ref = ref.numpy()
        np.testing.assert_allclose(mine, ref, rtol=0, atol=2e-6 * np.abs(ref).max())


def _loss_f64(x, wg, b, w1, w2, k, cf, dy):
    out = orc.forward(x, wg, b, w1, w2, k, cf, "f64",
                      logits=None)
    return float((out["y"] * dy).sum()), out


@pytest.mark.parametrize("cf", [0.0, 0.5])
def test_backward_finite_differences(cf):
    """Central differences (step 1e-6) of sum(y * dy), in float64 end to end.
    The router logits are computed in float64 here (no float32 rounding) so
    the derivative is smooth; perturbations that change routing or cross a
    ReLU kink are skipped."""
    T, d, F, E, k = 8, 8, 16, 4, 2
    x = rand((T, d), 30).astype(np.float64)
    wg = rand((d, E), 31).astype(np.float64)
    b = rand((E,), 32).astype(np.float64)
    w1 = rand((E, F, d), 33, 0.5).astype(np.float64)
    w2 = rand((E, d, F), 34, 0.5).astype(np.float64)
    dy = rand((T, d), 35).astype(np.float64)

    def run(x, wg, b, w1, w2):
        logits = x @ wg + b  # float64 logits
        T_, E_ = logits.shape
        idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
        sel = np.take_along_axis(logits, idx, 1)
        p = np.exp(sel - sel[:, :1])
        w = p / p.sum(1, keepdims=True)
        C = orc.capacity(T_, k, E_, cf)
        s = orc.assign_slots(idx, E_, C)
        xp = orc.encode(x, s["row_token"])
        h, o = orc.expert_ffn(xp, s["offsets"], w1, w2, "f64")
        y = orc.decode(o, w, s["slot_row"], "f64")
        fwd = {"idx": idx, "w": w, "h": h, "o": o, "x_perm": xp}
        fwd.update(s)
        z_margin = np.inf
        for e in range(E_):
            a, bb = s["offsets"][e], s["offsets"][e + 1]
            if bb > a:
                z_margin = min(z_margin, np.abs(xp[a:bb] @ w1[e].T).min())
        return float((y * dy).sum()), fwd, idx, z_margin

    base, fwd, idx0, margin = run(x, wg, b, w1, w2)
    assert margin > 1e-3
    if cf:
        assert fwd["drops"] > 0
    g = orc.backward(dy, fwd, x, wg, w1, w2, "f64")
    grads = {"x": g["dx_f64"], "wg": g["dw_gate"], "b": g["db_gate"], "w1": g["dw1_f64"], "w2": g["dw2_f64"]}
    params = {"x": x, "wg": wg, "b": b, "w1": w1, "w2": w2}
    rng = np.random.default_rng(0)
    h = 1e-6
    checked = 0
    for name, arr in params.items():
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(flat.size, 40), replace=False):
            old = flat[i]
            flat[i] = old + h
            lp, _, ip, mp = run(**params)
            flat[i] = old - h
            lm, _, im, mm = run(**params)
            flat[i] = old
            if not ((ip == idx0).all() and (im == idx0).all()) or min(mp, mm) < 1e-4:
                continue
            fd = (lp - lm) / (2 * h)
            an = float(grads[name].reshape(-1)[i])
            tol = 1e-6 * max(1.0, abs(fd)) if name in ("x", "w1", "w2") else 2e-6 * max(1.0, abs(fd))
            assert abs(fd - an) <= tol, (name, i, fd, an)
            checked += 1
    assert checked >= 150


@pytest.mark.parametrize("act", ["f32", "f64"])
def test_backward_identity_experts_closed_form(act):
    """Identity experts, dropless: y = (sum_j w_j) x = x, so dX = dy and the
    gate gets no gradient (sum of weights is constant)."""
    T, d, E, k = 32, 8, 4, 2
    x = rand((T, d), 40)
    w1, w2 = workloads.identity_experts(d, E)
    wg, b = rand((d, E), 41), rand((E,), 42)
    dy = rand((T, d), 43)
    fwd = orc.forward(x, wg, b, w1, w2, k, 0.0, act)
    g = orc.backward(dy, fwd, x, wg, w1, w2, act)
    np.testing.assert_allclose(g["dx"], dy, rtol=1e-6, atol=1e-7)
    assert np.abs(g["dlogits"]).max() < 1e-6
    assert np.abs(g["dw_gate"]).max() < 1e-5 and np.abs(g["db_gate"]).max() < 1e-5


# ---------------------------------------------------------------- page sizes
def test_page_expert_sizes():
    g = load("popfetcher_sizes.json")
    H, a = g["H"], g["alpha"]
    w = workloads.Workload("p", T=1, d=H, F=a * H, E=1, k=1, capacity_factor=0.0,
                           dtype="f32", x_std=1.0, zipf_s=None)
    n = w.E * w.F * w.d * 2
    assert n == g["expert_params"] and 4 * n == g["expert_bytes_fp32"]
    assert n // (2 * H) == g["push_pull_crossover_tokens"]
    assert 4 * w.d * w.F == g["fwd_ops_per_token"]


# ---------------------------------------------------------------- workloads
def test_workload_recipes():
    ws = workloads.workloads()
    assert [w.name for w in ws.values()] == ["tiny_fp32", "uniform_cf125", "skewed_zipf12",
                                            "mixtral_shaped", "fine_grained"]
    w = ws["fine_grained"]
    o0, o1 = workloads.expert_order(w, 0), workloads.expert_order(w, 1)
    assert sorted(o0) == list(range(w.E)) and sorted(o1) == list(range(w.E))
    assert 0 < (o0 != o1).sum() <= 2 * w.drift_swaps
    b = workloads.gate_bias(w, 0)
    assert b.max() == 0.0 and np.isclose(b.min(), -np.log(w.E))
    x = workloads.make_x(workloads.scaled(ws["skewed_zipf12"], T=8))
    assert (workloads.round_to_bf16(x) == x).all()


@pytest.mark.parametrize("cf", [0.0, 0.6])
def test_token_backward_matches_full_backward(cf):
    T, d, F, E, k = 40, 16, 24, 5, 2
    x = rand((T, d), 50)
    wg, b = rand((d, E), 51), rand((E,), 52)
    w1, w2 = rand((E, F, d), 53, 0.4), rand((E, d, F), 54, 0.4)
    dy = rand((T, d), 55)
    fwd = orc.forward(x, wg, b, w1, w2, k, cf, "f64")
    g = orc.backward(dy, fwd, x, wg, w1, w2, "f64")
    for t in range(T):
        dx_t, dl_t = orc.token_backward(t, dy[t], x, wg, w1, w2, fwd["idx"], fwd["w"],
                                        fwd["slot_row"], "f64")
        np.testing.assert_allclose(dx_t, g["dx_f64"][t], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dl_t, g["dlogits"][t], rtol=1e-6, atol=1e-7)


def test_weight_grad_entries_match_full_backward():
    T, d, F, E, k = 60, 16, 24, 4, 2
    x = rand((T, d), 60)
    wg, b = rand((d, E), 61), rand((E,), 62)
    w1, w2 = rand((E, F, d), 63, 0.4), rand((E, d, F), 64, 0.4)
    dy = rand((T, d), 65)
    fwd = orc.forward(x, wg, b, w1, w2, k, 0.0, "f64")
    g = orc.backward(dy, fwd, x, wg, w1, w2, "f64")
    fs, is_ = [0, 5, 23], [1, 7, 15]
    for e in range(E):
        a, bb = fwd["offsets"][e], fwd["offsets"][e + 1]
        toks = fwd["row_token"][a:bb]
        # gate weight of each row: the slot of token t that points at row r
        wr = np.array([fwd["w"][t][list(fwd["slot_row"][t * k:(t + 1) * k]).index(r)]
                       for t, r in zip(toks, range(a, bb))])
        dw1, dw2 = orc.expert_weight_grad_entries(e, fs, is_, fwd["x_perm"][a:bb], dy[toks], wr,
                                                  w1[e], w2[e], "f64")
        np.testing.assert_allclose(dw1, g["dw1_f64"][e][np.ix_(fs, is_)], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dw2, g["dw2_f64"][e][np.ix_(is_, fs)], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- dispatch plan
def test_hand_worked_ep_plan():
    g = load("ep_plan.json")
    out = orc.ep_plan(g["offsets"], g["extra"], g["R"])
    for key in ("replica_start", "replica_row0", "replica_rows", "replica_rank", "rank_rows"):
        assert out[key].tolist() == g[key], key


@pytest.mark.parametrize("seed,extra", [(0, 0), (1, 5), (2, 40), (3, 200)])
def test_replica_counts_are_the_largest_quotients(seed, extra):
    """Greedy one-at-a-time replication equals taking the `extra` largest
    quotients c_e / j (j = 1, 2, ...) in (value desc, expert asc, j asc)
    order - a different formulation, evaluated with exact fractions."""
    from fractions import Fraction
    rng = np.random.default_rng(seed)
    E = 37
    counts = rng.integers(0, 500, E)
    counts[3] = 0
    counts[7] = counts[9]  # ties
    cand = [(Fraction(int(counts[e]), j), e, j) for e in range(E) for j in range(1, extra + 2)]
    cand.sort(key=lambda c: (-c[0], c[1], c[2]))
    want = [1] * E
    for _, e, _ in cand[:extra]:
        want[e] += 1
    assert orc.replica_counts(counts, extra) == want


@pytest.mark.parametrize("seed,extra,R", [(0, 0, 8), (1, 16, 8), (2, 64, 16), (3, 3, 1), (4, 9, 64)])
def test_ep_plan_invariants(seed, extra, R):
    rng = np.random.default_rng(seed)
    E = 50
    counts = (rng.zipf(1.3, E) * 7) % 3000
    counts[::11] = 0
    off = np.concatenate([[0], np.cumsum(counts)])
    out = orc.ep_plan(off, extra, R)
    start, row0, rows, rank = (out[k] for k in ("replica_start", "replica_row0", "replica_rows",
                                                "replica_rank"))
    assert start[-1] == E + extra
    for e in range(E):
        seg = slice(start[e], start[e + 1])
        # copies tile the expert's rows in order, sizes differ by at most one
        assert row0[seg][0] == off[e] and (row0[seg] + rows[seg])[-1] == off[e + 1]
        assert (row0[seg][1:] == (row0[seg] + rows[seg])[:-1]).all()
        assert rows[seg].max() - rows[seg].min() <= 1
    load = np.bincount(rank, weights=rows, minlength=R).astype(np.int64)
    assert load.tolist() == out["rank_rows"].tolist()
    assert load.sum() == counts.sum()
    # list scheduling bound (Graham): the fullest rank exceeds the mean by at
    # most one copy
    assert load.max() <= load.sum() / R + rows.max() + 1e-9


# ---------------------------------------------------------------- cross-layer correlation
def test_hand_worked_cooccurrence_and_prediction():
    g = load("cooccurrence.json")
    ring = np.zeros((g["window"], g["E_a"], g["E_b"]), np.int64)
    for it, step in enumerate(g["iterations"]):
        c = orc.cooccurrence(np.array(step["idx_a"]), np.array(step["idx_b"]), g["E_a"], g["E_b"])
        assert c.tolist() == step["cooc"]
        ring, ws = orc.window_update(ring, it, c)
        assert ws.tolist() == step["window_sum"]
    p = g["predict_case"]
    pred = orc.predict_popularity(np.array(p["counts_a"]), np.array(p["cooc"]))
    assert pred.tolist() == p["pred"]
    assert orc.rank_experts(pred).tolist() == p["order"]


def test_cooccurrence_is_a_product_of_one_hot_matrices():
    rng = np.random.default_rng(3)
    T, Ea, Eb, ka, kb = 300, 9, 7, 3, 2
    ia = np.stack([rng.choice(Ea, ka, replace=False) for _ in range(T)])
    ib = np.stack([rng.choice(Eb, kb, replace=False) for _ in range(T)])
    A = np.zeros((T, Ea), np.int64)
    B = np.zeros((T, Eb), np.int64)
    np.add.at(A, (np.repeat(np.arange(T), ka), ia.reshape(-1)), 1)
    np.add.at(B, (np.repeat(np.arange(T), kb), ib.reshape(-1)), 1)
    c = orc.cooccurrence(ia, ib, Ea, Eb)
    np.testing.assert_array_equal(c, A.T @ B)
    # each layer-j selection pairs with k_b layer-(j+1) selections
    np.testing.assert_array_equal(c.sum(1), kb * np.bincount(ia.reshape(-1), minlength=Ea))


def test_window_update_matches_popularity_window():
    rng = np.random.default_rng(4)
    ring2 = np.zeros((3, 5, 1), np.int64)
    ring1 = np.zeros((3, 5), np.int32)
    for it in range(7):
        c = rng.integers(0, 100, 5)
        ring2, ws2 = orc.window_update(ring2, it, c[:, None])
        ring1, ws1 = orc.popularity_update(ring1, it, c)
        np.testing.assert_array_equal(ws2[:, 0], ws1)


def test_prediction_special_cases():
    # deterministic successor: every token's next-layer expert is f(x)
    rng = np.random.default_rng(5)
    E, T = 11, 500
    f = rng.permutation(E)
    ia = rng.integers(0, E, (T, 1))
    ib = f[ia]
    c = orc.cooccurrence(ia, ib, E, E)
    counts = rng.integers(0, 1000, E)
    pred = orc.predict_popularity(counts, c)
    want = np.zeros(E)
    seen = np.bincount(ia[:, 0], minlength=E) > 0
    for x in range(E):
        if seen[x]:
            want[f[x]] += counts[x]
    np.testing.assert_array_equal(pred, want)
    # independent layers: P(x'|x) = q(x') for every x, so pred = (sum of the
    # counts of seen x) * q
    q = np.array([3, 0, 5, 2], np.int64)
    u = np.array([4, 1, 0, 7, 2], np.int64)
    cnt = np.array([10, 20, 30, 40, 50])
    pred = orc.predict_popularity(cnt, np.outer(u, q))
    np.testing.assert_allclose(pred, (10 + 20 + 40 + 50) * q / q.sum(), rtol=1e-15)
    assert orc.top_hit_rate(pred, q, n=2) == 1.0
    assert orc.top_hit_rate(pred, q[::-1], n=2) == 0.0


# ---------------------------------------------------------------- dispatch layout
def test_hand_worked_dispatch_layout():
    g = load("dispatch_layout.json")
    for c in g["cases"]:
        out = orc.dispatch_layout(c["seg_rows"], c["seg_rank"], c["R"])
        for key in ("send_counts", "send_offsets", "seg_send_offset"):
            assert out[key].tolist() == c[key], (c["what"], key)


@pytest.mark.parametrize("seed", range(6))
def test_dispatch_layout_invariants(seed):
    """Split sizes are the per-rank row sums (np.bincount); the send buffer
    is the segments in a stable sort by rank (np.argsort kind="stable"), so
    each segment starts at the running sum of the rows before it in that
    order; the non-empty segments tile [0, total) exactly once; with ranks
    non-decreasing in segment order the layout is the plain prefix sum."""
    rng = np.random.default_rng(seed)
    n, R = int(rng.integers(1, 300)), int(rng.integers(1, 65))
    rows = rng.integers(0, 50, n) * (rng.random(n) > 0.2)
    rank = rng.integers(0, R, n)
    out = orc.dispatch_layout(rows, rank, R)
    np.testing.assert_array_equal(out["send_counts"], np.bincount(rank, weights=rows, minlength=R))
    order = np.argsort(rank, kind="stable")
    start = np.zeros(n, np.int64)
    start[order] = np.concatenate([[0], np.cumsum(rows[order])[:-1]])
    np.testing.assert_array_equal(out["seg_send_offset"], start)
    np.testing.assert_array_equal(out["send_offsets"],
                                  np.concatenate([[0], np.cumsum(out["send_counts"])]))
    cover = np.zeros(int(rows.sum()), np.int32)
    for i in range(n):
        cover[start[i]:start[i] + rows[i]] += 1
    assert (cover == 1).all()
    srt = np.sort(rank)
    mono = orc.dispatch_layout(rows, srt, R)
    np.testing.assert_array_equal(mono["seg_send_offset"],
                                  np.concatenate([[0], np.cumsum(rows)[:-1]]))


# ---------------------------------------------------------------- replicated weight gradients
def _small_layer(seed=0, T=40, d=8, F=16, E=4, k=2, cf=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((d, E)) * 0.3
    b = np.array([0.8, 0.2, 0.0, -0.5][:E])
    w1 = rng.standard_normal((E, F, d)) * 0.3
    w2 = rng.standard_normal((E, d, F)) * 0.3
    dy = rng.standard_normal((T, d))
    fwd = orc.forward(x, wg, b, w1, w2, k, cf, "f64")
    return x, wg, w1, w2, dy, fwd


@pytest.mark.parametrize("extra,R", [(0, 2), (3, 2), (6, 3)])
def test_replicated_weight_gradients(extra, R):
    """Splitting an expert's rows over copies changes nothing but the order
    of the row sum: one copy per expert gives the unsplit gradients bit for
    bit; the dispatch plan's copies give them within float64 rounding; every
    other gradient is untouched."""
    x, wg, w1, w2, dy, fwd = _small_layer(seed=extra)
    plain = orc.backward(dy, fwd, x, wg, w1, w2, "f64")
    copies = orc.ep_plan(fwd["offsets"], extra, R)
    if extra:
        assert (np.diff(copies["replica_start"]) > 1).any()
    rep = orc.backward(dy, fwd, x, wg, w1, w2, "f64", copies=copies)
    for key in ("dw1_f64", "dw2_f64"):
        np.testing.assert_allclose(rep[key], plain[key], rtol=0,
                                   atol=1e-12 * np.abs(plain[key]).max())
        if extra == 0:
            np.testing.assert_array_equal(rep[key], plain[key])
    for key in ("dx", "dw_gate", "db_gate", "dlogits"):
        np.testing.assert_array_equal(rep[key], plain[key])


def test_replicated_weight_gradients_hand_worked():
    """One expert, three rows split 2 + 1: dW2 = dO[0:2]^T h[0:2] + dO[2:3]^T
    h[2:3], the copy partials worked by hand on integer-valued operands."""
    fwd = {"idx": np.zeros((3, 1), np.int32), "w": np.ones((3, 1), np.float32),
           "slot_row": np.array([0, 1, 2], np.int32), "offsets": np.array([0, 3], np.int32),
           "h": np.array([[1.0, 2.0], [0.0, 1.0], [3.0, 0.0]]),
           "o": np.zeros((3, 1)), "x_perm": np.array([[1.0], [2.0], [-1.0]])}
    dy = np.array([[1.0], [2.0], [-1.0]])
    w1 = np.ones((1, 2, 1))
    w2 = np.array([[[1.0, 1.0]]])
    copies = {"replica_start": [0, 2], "replica_row0": [0, 2], "replica_rows": [2, 1]}
    rep = orc.backward(dy, fwd, np.zeros((3, 1)), np.zeros((1, 1)), w1, w2, "f64", copies=copies)
    # dO = w * dy = dy; copy 0: [1*1 + 2*0, 1*2 + 2*1] = [1, 4]; copy 1: [-3, 0]
    np.testing.assert_array_equal(rep["dw2_f64"][0], [[-2.0, 4.0]])
    # dz = (dO @ W2) * [h > 0]: rows [1,1], [0,2], [-1,0]; dW1 = dz^T x_perm:
    # copy 0: [1*1 + 0*2, 1*1 + 2*2] = [1, 5]; copy 1: [(-1)(-1), 0] = [1, 0]
    np.testing.assert_array_equal(rep["dw1_f64"][0], [[2.0], [5.0]])


def test_replicated_copies_must_tile_the_rows():
    x, wg, w1, w2, dy, fwd = _small_layer()
    good = orc.ep_plan(fwd["offsets"], 2, 2)
    bad = {k: np.array(v, copy=True) for k, v in good.items()}
    p = int(np.argmax(bad["replica_rows"]))
    bad["replica_rows"][p] -= 1
    with pytest.raises(ValueError):
        orc.backward(dy, fwd, x, wg, w1, w2, "f64", copies=bad)
