"""Plain, slow CPU reference of one GPU's mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and
it shares no code with the GPU path: it imports nothing but NumPy.

What it computes (all in float64 from the stored-precision inputs, rounding
only where the layer stores a tensor):

* gate routing - a linear router with a bias, top-k selection with the lowest
  expert index winning ties, gate weights renormalised over the chosen k
  (PopFetcher notes, §2.1.2 "MoE architecture": each token goes to one or more
  experts by top-k selection; A Survey on Mixture of Experts, §5 System
  Design, first paragraph: gate routing is the first step of expert
  parallelism);
* an optional per-expert capacity limit (GShard-style capacity, cited in the
  survey's §5 first paragraph and in the PopFetcher notes §2.2); slots beyond
  an expert's capacity are dropped;
* input encode - gathering each expert's tokens into one contiguous block in a
  stable order (survey §5, first paragraph);
* the expert network FC -> ReLU -> FC with two weight matrices and no biases
  (PopFetcher notes §2.1.1, and §5.1: matrices H x aH and aH x H, 4H^2
  parameters);
* output decode - restoring token order and summing the k expert outputs
  weighted by the gate (survey §5, first paragraph);
* per-expert popularity counts over a sliding window of iterations
  (PopFetcher notes §3.1 routing-information collector and §4.2, Eq. 1,
  whose body is missing from the page: the window sum of per-expert counts
  is the reading taken here);
* the backward pass of all of the above (the notes' §5.2.1 counts one GEMM
  forward and two backward per expert layer: gradient w.r.t. input and
  w.r.t. parameters);
* an expert-parallel dispatch plan: demand-based replication of hot experts
  under a cap on extra copies (Fast MoE Inference via Predictive Prefetching
  and Expert Replication, main contributions 2 and 3: physical copies of
  experts by token demand, their number limited by GPU memory) and
  least-loaded placement of the copies on ranks (LLEP notes, §2.1: work goes
  to the least-loaded GPU); the All-to-All split sizes and send-buffer
  offsets of an expert -> rank map or of such a plan;
* cross-layer expert correlation and popularity prediction (PopFetcher notes
  §4.1: tuples of a token's selections in consecutive layers; §4.2, Eq. 2
  and Eq. 3, bodies missing: conditional probabilities from the windowed
  tuple counts weight this layer's counts to predict the next layer's).

Readings of points the pages leave open (each is listed in the design notes):
selection on the fp32 logits, ties to the lowest index, weights = softmax over
the k selected logits; capacity C = ceil(cf*T*k/E) clamped to [1, T] (T when
dropless); slots claim capacity in slot order t*k+j (or choice-major); kept
weights are not
renormalised after drops; ReLU'(0) = 0 with the mask taken from the stored h;
the k expert outputs are summed in j order.

Pins: every function here is checked in ``tests/test_oracle.py`` against
brute force, library special cases, closed forms and finite differences.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

F64 = np.float64
F32 = np.float32


# --------------------------------------------------------------------------
# storage precision
# --------------------------------------------------------------------------
def _to_bf16(a: np.ndarray) -> np.ndarray:
    """Round each float64 value to the nearest bf16 value, ties to even, in
    ONE rounding step (no intermediate float32).

    bf16 keeps 8 significant bits over float32's exponent range.  A value
    with 2**(e-1) <= |v| < 2**e is therefore rounded to a multiple of the
    quantum 2**(e-8); below 2**-126 (bf16's subnormals) the quantum is fixed at
    2**-133.  np.rint rounds half-way cases to the even multiple, which is the
    even last significand bit.  Magnitudes that round to 2**128 or beyond are
    infinite; NaN and infinities pass through.  Returned as float32 (exact).
    """
    v = np.array(a, dtype=F64, copy=True)
    fin = np.isfinite(v)
    vf = v[fin]
    _, e = np.frexp(vf)                       # vf = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(vf, -q)), q)  # both scalings are exact
    big = np.abs(r) >= 2.0 ** 128
    r[big] = np.copysign(np.inf, r[big])
    v[fin] = r
    return v.astype(F32)


def round_act(a: np.ndarray, act: str) -> np.ndarray:
    """Round to the activation storage type: 'bf16', 'f32', or 'f64' (none)."""
    if act == "bf16":
        return _to_bf16(a).astype(F64)
    if act == "f32":
        return np.asarray(a, dtype=F64).astype(F32).astype(F64)
    if act == "f64":
        return np.asarray(a, dtype=F64)
    raise ValueError(act)


# --------------------------------------------------------------------------
# gate routing
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_gate: np.ndarray, b_gate: np.ndarray) -> np.ndarray:
    """logits[t, e] = b[e] + sum_i x[t, i] * W_gate[i, e], accumulated in
    float64 and stored as float32.  x: [T, d], W_gate: [d, E], b: [E]."""
    z = np.asarray(x, F64) @ np.asarray(w_gate, F64) + np.asarray(b_gate, F64)[None, :]
    return z.astype(F32)


def topk_gate(logits: np.ndarray, k: int):
    """Top-k experts per token and their renormalised gate weights.

    idx[t, 0..k-1] lists the k largest logits in descending order; among
    equal logits the lowest expert index comes first (float comparison, so
    -0.0 and +0.0 tie).  w[t, j] = exp(L_j - L_0) / sum_i exp(L_i - L_0)
    over the k chosen logits, which equals a softmax over all E followed by
    renormalising the chosen k.  Returns idx int32 [T, k], w float32 [T, k].
    """
    L = np.asarray(logits, dtype=F32)
    if not np.all(np.isfinite(L)):
        raise ValueError("router logits must be finite")
    T, E = L.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    work = L.astype(F64).copy()
    idx = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        # argmax returns the first (lowest-index) maximum; chosen entries
        # are taken out of the running with -inf.
        e = np.argmax(work, axis=1)
        idx[:, j] = e
        work[rows, e] = -np.inf
    sel = L.astype(F64)[rows[:, None], idx]
    p = np.exp(sel - sel[:, :1])
    w = (p / p.sum(axis=1, keepdims=True)).astype(F32)
    return idx, w


def capacity(T: int, k: int, E: int, capacity_factor: float) -> int:
    """C = ceil(cf * T * k / E), the capacity factor times an expert's even
    share of the T*k slots, rounded UP to whole slots (GShard's expert
    capacity, cited in A Survey on Mixture of Experts §5 and the PopFetcher
    notes §2.2; the pages give no formula, so the plainest one is taken).  cf
    is read as a float32 (the type the layer's shape carries it in) and the
    product and quotient are evaluated left to right in float64.  Clamped to
    [1, T]; T when cf <= 0 (dropless: no expert can receive more than T)."""
    cf = float(np.float32(capacity_factor))
    if cf <= 0.0:
        return T
    c = math.ceil(cf * T * k / E)
    return max(1, min(T, c))


# --------------------------------------------------------------------------
# input encode
# --------------------------------------------------------------------------
def priority_order(T: int, k: int, priority: str = "slot") -> List[int]:
    """The order in which slots claim expert capacity.

    "slot": s = t*k + j in increasing order (each expert keeps its earliest
    tokens).  "choice": every token's first choice in token order, then every
    token's second choice, and so on - the GShard gating that the PopFetcher
    notes (§2.2 capacity limit, §8.2 the two routing mechanisms) name beside
    plain top-k.
    """
    if priority == "slot":
        return list(range(T * k))
    if priority == "choice":
        return [t * k + j for j in range(k) for t in range(T)]
    raise ValueError(f"unknown capacity priority {priority!r}")


def assign_slots(idx: np.ndarray, E: int, C: int, priority: str = "slot"
                 ) -> Dict[str, np.ndarray]:
    """Walk the slots in priority order (priority_order); each takes the next
    position in its expert, and is kept iff that position is below the
    capacity C.  Packed rows follow the positions: row = offsets[e] + pos.

    Returns counts_raw [E], counts_kept [E], offsets [E+1] (exclusive prefix
    sum of counts_kept), slot_row [T*k] (row in the packed buffers, -1 when
    dropped) and row_token [S_kept] (token held by each packed row), plus
    "dropped": the dropped slots ordered by expert, then position.
    """
    T, k = idx.shape
    flat = idx.reshape(-1)
    S = flat.size
    seen = [0] * E
    pos = [0] * S
    for s in priority_order(T, k, priority):
        e = int(flat[s])
        pos[s] = seen[e]
        seen[e] += 1
    counts_raw = np.array(seen, dtype=np.int32)
    counts_kept = np.array([min(c, C) for c in seen], dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    run = 0
    for e in range(E):
        offsets[e] = run
        run += int(counts_kept[e])
    offsets[E] = run
    slot_row = np.full(S, -1, dtype=np.int32)
    row_token = np.full(run, -1, dtype=np.int32)
    for s in range(S):
        if pos[s] < C:
            r = int(offsets[flat[s]]) + pos[s]
            slot_row[s] = r
            row_token[r] = s // k
    dropped = sorted((int(flat[s]), pos[s], s) for s in range(S) if pos[s] >= C)
    return {"counts_raw": counts_raw, "counts_kept": counts_kept,
            "offsets": offsets, "slot_row": slot_row, "row_token": row_token,
            "drops": S - run, "dropped": np.array([s for _, _, s in dropped], dtype=np.int32)}


def encode(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """x_perm[r] = x[row_token[r]] (an exact copy of the token's row)."""
    return np.asarray(x)[np.asarray(row_token, dtype=np.int64)]


# --------------------------------------------------------------------------
# expert computation
# --------------------------------------------------------------------------
def expert_ffn(x_perm: np.ndarray, offsets: np.ndarray, w1: np.ndarray,
               w2: np.ndarray, act: str):
    """Per expert e, over packed rows offsets[e]..offsets[e+1]:
    h = round(ReLU(x_perm_e @ W1[e]^T)), O = round(h @ W2[e]^T).
    W1 is [E, F, d] and W2 is [E, d, F] (output x input)."""
    E, F, d = w1.shape
    R = x_perm.shape[0]
    h = np.zeros((R, F), dtype=F64)
    o = np.zeros((R, d), dtype=F64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        xe = np.asarray(x_perm[a:b], F64)
        z = xe @ np.asarray(w1[e], F64).T
        he = round_act(np.maximum(z, 0.0), act)
        h[a:b] = he
        o[a:b] = round_act(he @ np.asarray(w2[e], F64).T, act)
    return h, o


# --------------------------------------------------------------------------
# output decode
# --------------------------------------------------------------------------
def decode(o: np.ndarray, w: np.ndarray, slot_row: np.ndarray, act: str) -> np.ndarray:
    """y[t] = round(sum_j w[t, j] * O[slot_row[t*k + j]]) over kept slots,
    accumulated in j order; a token whose slots were all dropped gets 0."""
    T, k = w.shape
    d = o.shape[1]
    y = np.zeros((T, d), dtype=F64)
    rows = slot_row.reshape(T, k)
    for j in range(k):
        r = rows[:, j]
        kept = r >= 0
        y[kept] += np.asarray(w[kept, j], F64)[:, None] * o[r[kept]]
    return round_act(y, act)


# --------------------------------------------------------------------------
# whole forward
# --------------------------------------------------------------------------
def forward(x, w_gate, b_gate, w1, w2, k: int, capacity_factor: float, act: str,
            logits: Optional[np.ndarray] = None, priority: str = "slot") -> Dict[str, np.ndarray]:
    """The layer forward.  If ``logits`` is given (float32 [T, E]) routing
    starts from those logits instead of computing them.  ``priority`` is the
    capacity priority (priority_order)."""
    T = x.shape[0]
    E = w1.shape[0]
    if logits is None:
        logits = router_logits(x, w_gate, b_gate)
    idx, w = topk_gate(logits, k)
    C = capacity(T, k, E, capacity_factor)
    slots = assign_slots(idx, E, C, priority)
    x_perm = encode(x, slots["row_token"])
    h, o = expert_ffn(x_perm, slots["offsets"], w1, w2, act)
    y = decode(o, w, slots["slot_row"], act)
    out = {"logits": logits, "idx": idx, "w": w, "C": C, "x_perm": x_perm,
           "h": h, "o": o, "y": y}
    out.update(slots)
    return out


# --------------------------------------------------------------------------
# popularity
# --------------------------------------------------------------------------
def popularity_update(ring: np.ndarray, it: int, counts_raw: np.ndarray):
    """Record this iteration's per-expert selections (pre-capacity) in slot
    it % W of the ring and return (ring, window_sum), where window_sum sums
    the last min(it + 1, W) iterations.  Exact integers."""
    ring = np.array(ring, dtype=np.int64, copy=True)
    W = ring.shape[0]
    ring[it % W] = counts_raw
    n = min(it + 1, W)
    total = np.zeros(ring.shape[1], dtype=np.int64)
    for back in range(n):
        total += ring[(it - back) % W]
    return ring.astype(np.int32), total.astype(np.int32)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def _copy_ranges(copies, offsets, E):
    """The packed-row ranges of each expert's copies, checked to tile the
    expert's rows in order: [[(row0, rows), ...] per expert]."""
    start = [int(v) for v in copies["replica_start"]]
    row0 = [int(v) for v in copies["replica_row0"]]
    rows = [int(v) for v in copies["replica_rows"]]
    if len(start) != E + 1:
        raise ValueError("replica_start needs E + 1 entries")
    out = []
    for e in range(E):
        cur, ranges = int(offsets[e]), []
        for p in range(start[e], start[e + 1]):
            if row0[p] != cur or rows[p] < 0:
                raise ValueError(f"copies of expert {e} do not tile its rows in order")
            ranges.append((row0[p], rows[p]))
            cur += rows[p]
        if cur != int(offsets[e + 1]) or not ranges:
            raise ValueError(f"copies of expert {e} do not cover its rows")
        out.append(ranges)
    return out


def backward(dy, fwd: Dict[str, np.ndarray], x, w_gate, w1, w2, act: str, copies=None):
    """Gradients of the layer for output gradient dy, given this module's own
    forward results ``fwd``.

    ``copies`` (optional; ep_plan's replica_start / replica_row0 /
    replica_rows) splits each expert's rows over its copies: the expert's
    weight gradients are then the sum, in copy order, of each copy's
    gradient over its own rows - what the copies' ranks compute and a
    reduction adds up when hot experts are replicated (Fast MoE Inference via
    Predictive Prefetching and Expert Replication, main contributions 2-3).

    Output decode: dO[r] = w[t, j] dy[t] for the kept slot (t, j) held by row
    r, and dg[t, j] = <dy[t], O[r]> (0 for a dropped slot).
    FC2: dh = dO W2[e], dW2[e] = dO^T h; ReLU mask dz = dh * [h > 0];
    FC1: dx_perm = dz W1[e], dW1[e] = dz^T x_perm.
    Input encode: dx_exp[t] = sum of dx_perm over t's kept rows.
    Gate: dlogits[t, idx_j] = w_j (dg_j - sum_i w_i dg_i), 0 elsewhere;
    dW_gate = x^T dlogits, db = sum_t dlogits, dX = dx_exp + dlogits W_gate^T.
    dX is stored in the activation type; weight gradients, db and dlogits
    in float32.
    """
    dy = np.asarray(dy, F64)
    T, d = dy.shape
    idx, w = fwd["idx"], np.asarray(fwd["w"], F64)
    k = idx.shape[1]
    E, F, _ = w1.shape
    slot_row = fwd["slot_row"].reshape(T, k)
    offsets = fwd["offsets"]
    h, o, x_perm = fwd["h"], fwd["o"], np.asarray(fwd["x_perm"], F64)
    R = h.shape[0]

    # output decode backward
    d_o = np.zeros((R, d), dtype=F64)
    for j in range(k):
        r = slot_row[:, j]
        kept = r >= 0
        d_o[r[kept]] = w[kept, j][:, None] * dy[kept]

    # expert backward
    dw1 = np.zeros((E, F, d), dtype=F64)
    dw2 = np.zeros((E, d, F), dtype=F64)
    dx_perm = np.zeros((R, d), dtype=F64)
    ranges = _copy_ranges(copies, offsets, E) if copies is not None else None
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        dO = d_o[a:b]
        he = h[a:b]
        dh = dO @ np.asarray(w2[e], F64)
        dz = dh * (he > 0.0)
        dx_perm[a:b] = dz @ np.asarray(w1[e], F64)
        if ranges is None:
            dw2[e] = dO.T @ he
            dw1[e] = dz.T @ x_perm[a:b]
        else:
            for r0, n in ranges[e]:  # each copy over its own rows, in copy order
                i, j = r0 - a, r0 - a + n
                dw2[e] += dO[i:j].T @ he[i:j]
                dw1[e] += dz[i:j].T @ x_perm[r0:r0 + n]

    # input encode backward (sum over the token's kept rows, in j order)
    dx_exp = np.zeros((T, d), dtype=F64)
    for j in range(k):
        r = slot_row[:, j]
        kept = r >= 0
        dx_exp[kept] += dx_perm[r[kept]]

    # gate backward
    g = gate_backward(dy, fwd, x, w_gate, E)
    dlogits = g["dlogits_f64"]
    dx = dx_exp + dlogits @ np.asarray(w_gate, F64).T
    return {"dx": round_act(dx, act), "dw1": dw1.astype(F32), "dw2": dw2.astype(F32),
            "dw_gate": g["dw_gate"], "db_gate": g["db_gate"],
            "dlogits": g["dlogits"], "dg": g["dg"], "d_o": d_o, "dx_exp": dx_exp,
            "dw1_f64": dw1, "dw2_f64": dw2, "dx_f64": dx}


def gate_backward(dy, fwd: Dict[str, np.ndarray], x, w_gate, E: int):
    """The gate's part of the backward, from the forward's expert outputs:
    dg[t, j] = <dy[t], O[row of slot (t, j)]> (0 for a dropped slot); the
    softmax over the chosen logits gives dsel_j = w_j (dg_j - sum_i w_i dg_i)
    and dlogits[t, idx_j] = dsel_j (0 elsewhere); dW_gate = x^T dlogits and
    db = sum_t dlogits.  float64 throughout; dlogits, dW_gate and db are also
    returned rounded to float32."""
    dy = np.asarray(dy, F64)
    T = dy.shape[0]
    idx, w = fwd["idx"], np.asarray(fwd["w"], F64)
    k = idx.shape[1]
    slot_row = fwd["slot_row"].reshape(T, k)
    o = fwd["o"]
    dg = np.zeros((T, k), dtype=F64)
    for j in range(k):
        r = slot_row[:, j]
        kept = r >= 0
        dg[kept, j] = np.einsum("td,td->t", dy[kept], o[r[kept]])
    s = (w * dg).sum(axis=1, keepdims=True)
    dsel = w * (dg - s)
    dlogits = np.zeros((T, E), dtype=F64)
    rows = np.arange(T)
    for j in range(k):
        dlogits[rows, idx[:, j]] += dsel[:, j]
    dw_gate = np.asarray(x, F64).T @ dlogits
    db = dlogits.sum(axis=0)
    return {"dg": dg, "dlogits_f64": dlogits, "dlogits": dlogits.astype(F32),
            "dw_gate": dw_gate.astype(F32), "db_gate": db.astype(F32)}


# --------------------------------------------------------------------------
# per-token forms used to check single outputs of large problems
# --------------------------------------------------------------------------
def expert_row(xrow: np.ndarray, w1e: np.ndarray, w2e: np.ndarray, act: str):
    """One token through one expert: (h, O) rounded as stored."""
    z = np.asarray(w1e, F64) @ np.asarray(xrow, F64)
    h = round_act(np.maximum(z, 0.0), act)
    return h, round_act(np.asarray(w2e, F64) @ h, act)


def token_output(t: int, x, w, idx, slot_row, w1, w2, act: str) -> np.ndarray:
    """y[t] computed directly from token t's choices, without the packed
    buffers (dense per-token evaluation)."""
    k = idx.shape[1]
    acc = np.zeros(x.shape[1], dtype=F64)
    for j in range(k):
        if slot_row[t * k + j] < 0:
            continue
        e = int(idx[t, j])
        _, o = expert_row(x[t], w1[e], w2[e], act)
        acc += float(w[t, j]) * o
    return round_act(acc, act)


def token_backward(t: int, dy_t, x, w_gate, w1, w2, idx, w, slot_row, act: str):
    """dX[t] and dlogits[t] for one token, evaluated from that token alone
    (no packed buffers): for each kept slot j with expert e, O_j = FFN_e(x_t)
    as stored, dg_j = <dy_t, O_j>, and the expert path adds
    W1[e]^T ((W2[e]^T (w_j dy_t)) * [h_j > 0]); the gate path adds
    sum_j dsel_j W_gate[:, e_j] with dsel_j = w_j (dg_j - sum_i w_i dg_i).
    Returns (dx_t rounded to act, dlogits_t float32 [E])."""
    k = idx.shape[1]
    E = w1.shape[0]
    dy_t = np.asarray(dy_t, F64)
    wt = np.asarray(w[t], F64)
    dg = np.zeros(k)
    dx = np.zeros(x.shape[1])
    for j in range(k):
        if slot_row[t * k + j] < 0:
            continue
        e = int(idx[t, j])
        h, o = expert_row(x[t], w1[e], w2[e], act)
        dg[j] = float(dy_t @ o)
        dz = (np.asarray(w2[e], F64).T @ (wt[j] * dy_t)) * (h > 0.0)
        dx += np.asarray(w1[e], F64).T @ dz
    dsel = wt * (dg - float((wt * dg).sum()))
    dlog = np.zeros(E)
    for j in range(k):
        dlog[int(idx[t, j])] += dsel[j]
        dx += dsel[j] * np.asarray(w_gate, F64)[:, int(idx[t, j])]
    return round_act(dx, act), dlog.astype(F32)


def expert_weight_grad_entries(e: int, rows_f, rows_i, x_perm_e, dy_tok, w_rows, w1e, w2e,
                               act: str):
    """Selected entries of one expert's weight gradients, each summed over all
    of the expert's packed rows r (token t_r, gate weight w_r):
      dW2[e][i][f] = sum_r (w_r dy[t_r, i]) h[r, f]
      dW1[e][f][i] = sum_r dz[r, f] x_perm[r, i],  dz[r, f] = (dO[r] . W2[e][:, f]) [h[r, f] > 0]
    computing only the needed columns of h and dz.  x_perm_e [M, d],
    dy_tok [M, d] (dy of each row's token), w_rows [M].  Returns
    (dW1 entries [len(rows_f), len(rows_i)], dW2 entries [len(rows_i), len(rows_f)])."""
    xp = np.asarray(x_perm_e, F64)
    dO = np.asarray(w_rows, F64)[:, None] * np.asarray(dy_tok, F64)
    fs = list(rows_f)
    h = round_act(np.maximum(xp @ np.asarray(w1e, F64)[fs].T, 0.0), act)   # [M, nf]
    dz = (dO @ np.asarray(w2e, F64)[:, fs]) * (h > 0.0)                    # [M, nf]
    dw1 = dz.T @ xp[:, list(rows_i)]                                        # [nf, ni]
    dw2 = dO[:, list(rows_i)].T @ h                                         # [ni, nf]
    return dw1, dw2


# --------------------------------------------------------------------------
# expert-parallel dispatch plan
# --------------------------------------------------------------------------
def replica_counts(counts, extra: int) -> List[int]:
    """Copies per expert.  Every expert has one; each of the ``extra`` copies
    the memory budget allows goes, one at a time, to the expert with the most
    rows per copy (counts[e] / copies[e], compared exactly; ties to the lowest
    expert index) - demand-based replication under a memory cap."""
    c = [int(v) for v in counts]
    r = [1] * len(c)
    for _ in range(extra):
        best = 0
        for e in range(1, len(c)):
            if c[e] * r[best] > c[best] * r[e]:
                best = e
        r[best] += 1
    return r


def ep_plan(offsets, extra: int, R: int) -> Dict[str, np.ndarray]:
    """Replicas of each expert (replica_counts) over its packed rows
    offsets[e]..offsets[e+1]: copy i of expert e takes rows offsets[e] +
    [floor(i c / r), floor((i+1) c / r)).  Copies are placed on R ranks
    longest first (decreasing rows, ties by copy index p), each on the rank
    with the fewest rows so far (ties to the lowest rank).  Copy p of expert
    e is p = replica_start[e] + i."""
    off = [int(v) for v in offsets]
    E = len(off) - 1
    counts = [off[e + 1] - off[e] for e in range(E)]
    r = replica_counts(counts, extra)
    start = [0]
    for e in range(E):
        start.append(start[-1] + r[e])
    P = start[-1]
    row0 = [0] * P
    rows = [0] * P
    for e in range(E):
        for i in range(r[e]):
            a = (i * counts[e]) // r[e]
            b = ((i + 1) * counts[e]) // r[e]
            row0[start[e] + i] = off[e] + a
            rows[start[e] + i] = b - a
    order = sorted(range(P), key=lambda p: (-rows[p], p))
    load = [0] * R
    rank = [0] * P
    for p in order:
        best = 0
        for q in range(1, R):
            if load[q] < load[best]:
                best = q
        rank[p] = best
        load[best] += rows[p]
    i32 = lambda v: np.array(v, dtype=np.int32)  # noqa: E731
    return {"replica_start": i32(start), "replica_row0": i32(row0), "replica_rows": i32(rows),
            "replica_rank": i32(rank), "rank_rows": i32(load)}


def dispatch_layout(seg_rows, seg_rank, R: int) -> Dict[str, np.ndarray]:
    """All-to-All split sizes of a dispatch (A Survey on Mixture of Experts,
    §5 System Design, first paragraph: the per-expert packed rows are what
    the All-to-All sends).  Segment i - one expert's packed rows, or one
    copy's share of them from ep_plan - holds seg_rows[i] rows bound for rank
    seg_rank[i].  The send buffer holds rank 0's rows, then rank 1's, ...;
    within a rank the segments keep their index order.  Returns send_counts
    [R] (rows per rank: the split sizes), send_offsets [R + 1] (exclusive
    prefix sum) and seg_send_offset [n] (where segment i starts)."""
    rows = [int(v) for v in seg_rows]
    rank = [int(v) for v in seg_rank]
    counts = [0] * R
    for n_i, r in zip(rows, rank):
        counts[r] += n_i
    offsets = [0] * (R + 1)
    for r in range(R):
        offsets[r + 1] = offsets[r] + counts[r]
    filled = list(offsets[:R])
    start = [0] * len(rows)
    for i, (n_i, r) in enumerate(zip(rows, rank)):
        start[i] = filled[r]
        filled[r] += n_i
    i32 = lambda v: np.array(v, dtype=np.int32)  # noqa: E731
    return {"send_counts": i32(counts), "send_offsets": i32(offsets),
            "seg_send_offset": i32(start)}


# --------------------------------------------------------------------------
# cross-layer expert correlation and popularity prediction
# --------------------------------------------------------------------------
def cooccurrence(idx_a: np.ndarray, idx_b: np.ndarray, E_a: int, E_b: int) -> np.ndarray:
    """counts[x][x'] = number of (token, choice in layer j, choice in layer
    j+1) triples with expert x in layer j and x' in layer j+1 (PopFetcher
    notes §4.1: the tuple (x, x') of a token's selections in consecutive
    layers).  Exact integers."""
    T = idx_a.shape[0]
    out = np.zeros((E_a, E_b), dtype=np.int64)
    for t in range(T):
        for x in idx_a[t]:
            for y in idx_b[t]:
                out[int(x), int(y)] += 1
    return out


def window_update(ring: np.ndarray, it: int, current: np.ndarray):
    """Put this iteration's table in slot it % W of the ring and return
    (ring, sum of the last min(it + 1, W) iterations) - the sliding window of
    §4.2 applied to the co-occurrence counts.  Exact integers."""
    ring = np.array(ring, dtype=np.int64, copy=True)
    W = ring.shape[0]
    ring[it % W] = current
    n = min(it + 1, W)
    total = np.zeros_like(ring[0])
    for b in range(n):
        total += ring[(it - b) % W]
    return ring, total


def predict_popularity(counts_a, cooc) -> np.ndarray:
    """Popularity of the next layer's experts from this layer's selections
    (PopFetcher notes §4.2, Eq. 2 and Eq. 3, whose bodies are missing from the
    page; the reading taken): P(x' | x) = cooc[x][x'] / sum_x'' cooc[x][x''];
    pred[x'] = sum over x in index order of counts_a[x] * P(x' | x), each
    product and sum one float64 operation (x with an all-zero row adds
    nothing)."""
    E_a, E_b = cooc.shape
    pred = [0.0] * E_b
    for h in range(E_b):
        acc = 0.0
        for i in range(E_a):
            row = int(np.sum(cooc[i]))
            if row == 0:
                continue
            p = float(int(cooc[i][h])) / float(row)
            acc = acc + float(int(counts_a[i])) * p
        pred[h] = acc
    return np.array(pred, dtype=np.float64)


def rank_experts(pred) -> np.ndarray:
    """Experts by decreasing predicted popularity, ties to the lower index."""
    return np.array(sorted(range(len(pred)), key=lambda h: (-pred[h], h)), dtype=np.int32)


def top_hit_rate(pred, actual, n: int = 5) -> float:
    """Share of the n experts predicted most popular that are among the n
    actually most popular (both ranked with ties to the lower index)."""
    a = set(rank_experts(pred)[:n].tolist())
    b = set(rank_experts(np.asarray(actual, dtype=np.float64))[:n].tolist())
    return len(a & b) / n
