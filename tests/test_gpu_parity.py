"""GPU parity of every step against the CPU reference, element by element,
at sizes the reference finishes in seconds.  Shapes are scaled-down copies
of the five workloads (same E, k, skew and dtype) that still cover several
permutation tiles, several GEMM tiles and ragged tails in M and N.

Protocol: every input comes from the seeded generators or from the
reference; no expected value comes from the GPU.  Routing steps are fed the
reference's float32 logits (so both sides decide on the same numbers) and
must match bit for bit; permutation results are bit-exact; float outputs
are within 2e-2 (bf16) or 1e-5 (float32) of the largest reference entry.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu

from gpu_helpers import (TOL, act_code, ambiguous_tokens, assert_close,  # noqa: E402
                         assert_close_per_expert, down, relu_kink_flips, up, up_i32,
                         upload_case)

if torch.cuda.is_available():
    from mixture_experts_layer_33_amd.layer import MoeLayer

WL = workloads.workloads()

# scaled copies: T not a multiple of the 256-slot tiles or the 128-row GEMM
# tiles, F not a multiple of the 128-column GEMM tiles
SMALL = {
    "tiny_fp32": WL["tiny_fp32"],
    # float32 throughout at a size that spans many row blocks, with drops
    "fp32_cf100": workloads.scaled(WL["tiny_fp32"], T=1000, d=128, F=320, capacity_factor=1.0),
    "uniform_cf125": workloads.scaled(WL["uniform_cf125"], T=1000, d=256, F=320),
    "uniform_cf100": workloads.scaled(WL["uniform_cf125"], T=1000, d=256, F=320,
                                      capacity_factor=1.0),
    "uniform_cf050": workloads.scaled(WL["uniform_cf125"], T=700, d=128, F=192,
                                      capacity_factor=0.5),
    "skewed_zipf12": workloads.scaled(WL["skewed_zipf12"], T=1500, d=256, F=448),
    "mixtral_shaped": workloads.scaled(WL["mixtral_shaped"], T=1200, d=256, F=448),
    "fine_grained": workloads.scaled(WL["fine_grained"], T=2100, d=256, F=128),
    # GShard's choice-major capacity priority
    "uniform_cf100_choice": workloads.scaled(WL["uniform_cf125"], T=1000, d=256, F=320,
                                             capacity_factor=1.0, priority="choice"),
    "skewed_cf080_choice": workloads.scaled(WL["skewed_zipf12"], T=1500, d=128, F=192,
                                            capacity_factor=0.8, priority="choice"),
    # top-1 (Switch-style) routing: one weight of 1 per token, with and without drops
    "uniform_top1_cf100": workloads.scaled(WL["uniform_cf125"], T=1000, d=256, F=320, k=1,
                                           capacity_factor=1.0),
    "skewed_top1": workloads.scaled(WL["skewed_zipf12"], T=1500, d=128, F=192, k=1),
    # K = F = 2048 with a partly filled last round of GEMM tiles: the second
    # expert GEMM and the input-gradient GEMM split that round's tiles along K
    "skewed_split_tail": workloads.scaled(WL["skewed_zipf12"], T=700, d=512, F=2048),
    "uniform_cf100_split_tail": workloads.scaled(WL["uniform_cf125"], T=900, d=512, F=2048,
                                                 capacity_factor=1.0),
    # more row tiles than CUs with K = d < 2048: the first GEMM and the masked
    # input gradient walk several tiles per workgroup (1, 2, 3 and 16 k-steps
    # of 64 per tile)
    "uniform_walk_k64": workloads.scaled(WL["uniform_cf125"], T=4096, d=64, F=2048),
    "uniform_walk_k128": workloads.scaled(WL["uniform_cf125"], T=4096, d=128, F=1024),
    "uniform_walk_k192": workloads.scaled(WL["uniform_cf125"], T=3000, d=192, F=2048,
                                          capacity_factor=1.0),
    "skewed_walk_k1024": workloads.scaled(WL["skewed_zipf12"], T=2048, d=1024, F=2048),
    # tile shapes the cases above do not reach: 256 x 128 row tiles in the
    # persistent walk (every product), and 128 x 256 persistent tiles next to
    # 128 x 128 tiles with a split tail, all with the weights read plainly
    "mixtral_tiles_256x128": workloads.scaled(WL["mixtral_shaped"], T=16384, d=128, F=128),
    "skewed_tiles_mixed": workloads.scaled(WL["skewed_zipf12"], T=8192, d=256, F=2048),
    # narrow d, wide F: FC1's weight gradient takes 128 x 256 tiles
    "mixtral_wgrad_128x256": workloads.scaled(WL["mixtral_shaped"], T=2048, d=128, F=8192),
    # K = d = 2048: FC1 (ReLU and keep bits) and the masked input gradient
    # split their last round along K, so their fixups apply those epilogues
    "skewed_split_fc1": workloads.scaled(WL["skewed_zipf12"], T=700, d=2048, F=512),
    # 32 weight-gradient tiles per expert (256 x 128) and even experts: with
    # copies, no expert's rows are worth splitting over them
    "uniform_walk_k512": workloads.scaled(WL["uniform_cf125"], T=4096, d=512, F=2048),
}


def _setup(name, it=0):
    w = SMALL[name]
    inp = workloads.make_inputs(w, it, with_weights=True, with_dy=True)
    dev = upload_case(inp, w.dtype)
    layer = MoeLayer(w.T, w.d, w.F, w.E, w.k, w.capacity_factor, act_code(w.dtype),
                     priority=w.priority)
    return w, inp, dev, layer


@pytest.mark.parametrize("name", list(SMALL))
def test_router_logits(name):
    w, inp, dev, layer = _setup(name)
    layer.route(dev["x"], dev["w_gate"], dev["b_gate"])
    torch.cuda.synchronize()
    ref = orc.router_logits(inp["x"], inp["w_gate"], inp["b_gate"])
    assert_close(down(layer.logits), ref, 1e-5, "logits")


# (T, d, E, k) reaching each launch shape of the matrix-core router: staged
# experts per part (8 for E <= 8, else E rounded up to a power of two >= 16)
# x tokens per workgroup BM in {16, 32, 64, 128} (BM grows with T: 16 below
# 8192 tokens, 32, 64 from 16384, 128 from 32768; at most 64 with 256
# experts), each with the stage depths its table offers (16 experts: 256
# deep with eight wavefronts where d is a multiple of 256 and BM <= 64, else
# 128, else 64; 32: 128, else 64), with ragged token tails; for 32, 64 and
# 128 experts both the padded W_gate layout (E a power of two) and the plain
# one (E below its padded size)
ROUTER_SHAPES = {}
for _ew, _es in (("EW8", (8, 7, 8, 5, 8, 8, 6, 8, 8, 7, 5)),
                 ("EW16", (16, 13, 16, 13, 16, 16, 9, 12, 16, 15, 11))):
    for _i, (_T, _d) in enumerate(((3001, 512), (3001, 320), (9000, 256), (9000, 64),
                                   (20000, 128), (20000, 192), (40000, 128), (40000, 64),
                                   (20000, 256), (3001, 384), (9000, 384))):
        ROUTER_SHAPES[f"{_ew}_T{_T}_d{_d}"] = (_T, _d, _es[_i], 2 if _es[_i] > 1 else 1)
ROUTER_SHAPES.update({
    "EP32_BM16_KD128": (1000, 128, 32, 2),
    "EP32_BM16_KD128_padded": (1000, 128, 24, 2),
    "EP32_BM16_KD64": (1000, 192, 32, 2),
    "EP32_BM16_KD64_padded": (1000, 192, 17, 2),
    "EP32_BM32_KD64": (9001, 64, 32, 2),
    "EP32_BM32_KD128": (9001, 128, 32, 2),
    "EP32_BM32_KD128_padded": (9001, 128, 20, 3),
    "EP32_BM32_KD64_padded": (9001, 64, 20, 3),
    "EP32_BM64_KD128": (17000, 128, 32, 2),
    "EP32_BM64_KD128_padded": (17000, 128, 30, 2),
    "EP32_BM64_KD64": (17000, 64, 32, 2),
    "EP32_BM64_KD64_padded": (17000, 64, 27, 2),
    "EP32_BM128_KD128": (33000, 128, 32, 2),
    "EP32_BM128_KD128_padded": (33000, 128, 31, 4),
    "EP32_BM128_KD64": (33000, 64, 32, 4),
    "EP32_BM128_KD64_padded": (33000, 64, 31, 4),
    "EP64_BM16": (2000, 128, 64, 2),
    "EP64_BM16_padded": (2000, 128, 33, 2),
    "EP64_BM32": (8192, 64, 64, 3),
    "EP64_BM32_padded": (8192, 64, 48, 3),
    "EP64_BM64": (16384, 64, 64, 2),
    "EP64_BM64_padded": (16384, 64, 57, 2),
    "EP64_BM128": (32768, 64, 64, 2),
    "EP64_BM128_top1_padded": (32768, 64, 40, 1),
    "EP128_BM16": (1000, 128, 128, 4),
    "EP128_BM16_padded": (1000, 128, 126, 4),
    "EP128_BM32": (9000, 64, 128, 4),
    "EP128_BM32_padded": (9000, 64, 65, 4),
    "EP128_BM64": (16500, 64, 128, 2),
    "EP128_BM64_padded": (16500, 64, 100, 2),
    "EP128_BM128": (32768, 128, 128, 4),
    "EP128_BM128_padded": (32768, 64, 120, 4),
    "EP256_BM16_padded": (700, 64, 250, 8),
    "EP256_BM32": (8200, 64, 256, 2),
    "EP256_BM64_padded": (16384, 64, 200, 8),
})


def _router_case(T, d, E, k):
    w = workloads.scaled(WL["skewed_zipf12"], T=T, d=d, F=64, E=E, k=k)
    inp = workloads.make_inputs(w, 0, with_weights=False)
    layer = MoeLayer(T, d, 64, E, k, 0.0, act_code("bf16"), backward=False)
    layer.route(up(inp["x"], "bf16"), up(inp["w_gate"]), up(inp["b_gate"]))
    return inp, layer


@pytest.mark.parametrize("name", list(ROUTER_SHAPES))
def test_router_launch_shapes(name):
    """Logits against the reference, and the kernel's own top-k and weights
    against the reference's top-k of those same float32 logits."""
    T, d, E, k = ROUTER_SHAPES[name]
    inp, layer = _router_case(T, d, E, k)
    torch.cuda.synchronize()
    L = down(layer.logits)
    assert_close(L, orc.router_logits(inp["x"], inp["w_gate"], inp["b_gate"]), 1e-5, "logits")
    idx, wt = orc.topk_gate(L, k)
    np.testing.assert_array_equal(down(layer.topk_idx), idx)
    assert_close(down(layer.topk_w), wt, 1e-5, "topk_w")


@pytest.mark.parametrize("name", list(SMALL))
def test_route_bitexact_on_shared_logits(name):
    w, inp, dev, layer = _setup(name)
    L = orc.router_logits(inp["x"], inp["w_gate"], inp["b_gate"])
    layer.route(None, None, None, logits_in=up(L))
    torch.cuda.synchronize()
    idx, wt = orc.topk_gate(L, w.k)
    np.testing.assert_array_equal(down(layer.topk_idx), idx)
    assert_close(down(layer.topk_w), wt, 1e-5, "topk_w")
    np.testing.assert_array_equal(down(layer.counts_raw), np.bincount(idx.reshape(-1), minlength=w.E))


@pytest.mark.parametrize("name", list(SMALL))
def test_permute_bitexact(name):
    w, inp, dev, layer = _setup(name)
    L = orc.router_logits(inp["x"], inp["w_gate"], inp["b_gate"])
    idx, _ = orc.topk_gate(L, w.k)
    ref = orc.assign_slots(idx, w.E, orc.capacity(w.T, w.k, w.E, w.capacity_factor),
                         w.priority)
    layer.permute(dev["x"], topk_idx=up_i32(idx))
    torch.cuda.synchronize()
    for key in ("counts_raw", "counts_kept", "offsets", "slot_row"):
        np.testing.assert_array_equal(down(getattr(layer, key)), ref[key], err_msg=key)
    n = int(ref["offsets"][-1])
    np.testing.assert_array_equal(down(layer.row_token)[:n], ref["row_token"])
    np.testing.assert_array_equal(down(layer.x_perm)[:n], orc.encode(inp["x"], ref["row_token"]))
    # dropped slots listed after the kept rows, by expert then position
    np.testing.assert_array_equal(down(layer.row_token)[n:n + ref["drops"]], ref["dropped"])
    if name.startswith("uniform_cf0") or name == "uniform_cf100":
        assert ref["drops"] > 0


@pytest.mark.parametrize("name", list(SMALL))
def test_expert_ffn(name):
    w, inp, dev, layer = _setup(name)
    L = orc.router_logits(inp["x"], inp["w_gate"], inp["b_gate"])
    idx, _ = orc.topk_gate(L, w.k)
    s = orc.assign_slots(idx, w.E, orc.capacity(w.T, w.k, w.E, w.capacity_factor),
                         w.priority)
    x_perm = orc.encode(inp["x"], s["row_token"])
    n = x_perm.shape[0]
    xp = torch.zeros(w.T * w.k, w.d, dtype=layer.dtype, device="cuda")
    xp[:n] = up(x_perm, w.dtype)
    layer.expert_ffn(dev["w1"], dev["w2"], x_perm=xp, offsets=up_i32(s["offsets"]))
    torch.cuda.synchronize()
    h, o = orc.expert_ffn(x_perm, s["offsets"], inp["w1"], inp["w2"], w.dtype)
    tol = TOL[w.dtype]
    for e in range(w.E):
        a, b = s["offsets"][e], s["offsets"][e + 1]
        if a == b:
            continue
        assert_close(down(layer.h[a:b]), h[a:b], tol, f"h[{e}]")
        assert_close(down(layer.out_perm[a:b]), o[a:b], tol, f"O[{e}]")


@pytest.mark.parametrize("name", list(SMALL))
def test_combine(name):
    w, inp, dev, layer = _setup(name)
    L = orc.router_logits(inp["x"], inp["w_gate"], inp["b_gate"])
    idx, wt = orc.topk_gate(L, w.k)
    s = orc.assign_slots(idx, w.E, orc.capacity(w.T, w.k, w.E, w.capacity_factor),
                         w.priority)
    x_perm = orc.encode(inp["x"], s["row_token"])
    _, o = orc.expert_ffn(x_perm, s["offsets"], inp["w1"], inp["w2"], w.dtype)
    n = o.shape[0]
    op = torch.zeros(w.T * w.k, w.d, dtype=layer.dtype, device="cuda")
    op[:n] = up(o.astype(np.float32), w.dtype)
    layer.combine(out_perm=op, topk_w=up(wt), slot_row=up_i32(s["slot_row"]))
    torch.cuda.synchronize()
    y = orc.decode(o, wt, s["slot_row"], w.dtype)
    assert_close(down(layer.y), y, TOL[w.dtype], "y")
    dropped_all = (s["slot_row"].reshape(w.T, w.k) < 0).all(axis=1)
    assert not np.any(down(layer.y)[dropped_all])


def _end_to_end(name, it=0):
    w, inp, dev, layer = _setup(name, it)
    layer.forward(dev["x"], dev["w_gate"], dev["b_gate"], dev["w1"], dev["w2"])
    layer.backward(dev["dy"], dev["x"], dev["w_gate"], dev["w1"], dev["w2"])
    torch.cuda.synchronize()
    fwd = orc.forward(inp["x"], inp["w_gate"], inp["b_gate"], inp["w1"], inp["w2"], w.k,
                      w.capacity_factor, w.dtype, priority=w.priority)
    bwd = orc.backward(inp["dy"], fwd, inp["x"], inp["w_gate"], inp["w1"], inp["w2"], w.dtype)
    return w, inp, layer, fwd, bwd


def compare_end_to_end(w, layer, fwd, bwd, w1=None):
    """Compare the fused GPU forward/backward with the reference's own run
    on the same inputs.  Each side routes on its own logits, so a token may
    legitimately route differently when its top-k is a near-tie within the
    logits tolerance; every such disagreement must be a near-tie, and those
    tokens (and the experts they touch) are left out of the comparisons that
    depend on them.  Likewise each side masks the ReLU with its own stored h:
    with w1 (the reference's W1) given, mask disagreements must be near-kinks
    (float32 rounding of a pre-activation at zero), and the FC1 weight-
    gradient rows and the tokens they touch are left out of those two
    comparisons.  Everything else must match: integers bit-exact, floats
    within tolerance.  The numbers set aside are printed (run with -s to see
    them) and bounded: a near-kink flip needs a pre-activation within float32
    rounding of zero, so at most 0.1% of the dW1 rows and of the tokens (and
    a handful in tiny cases) may be set aside for it."""
    tol = TOL[w.dtype]
    assert_close(down(layer.logits), fwd["logits"], 1e-5, "logits")
    gidx = down(layer.topk_idx)
    mism = np.where((gidx != fwd["idx"]).any(axis=1))[0]
    amb = set(ambiguous_tokens(fwd["logits"], w.k).tolist())
    assert set(mism.tolist()) <= amb, "routing differs on tokens that are not near-ties"
    touched = set(fwd["idx"][mism].reshape(-1).tolist()) | set(gidx[mism].reshape(-1).tolist())
    keep_t = np.ones(w.T, bool)
    keep_t[mism] = False
    keep_e = np.array([e not in touched for e in range(w.E)])
    if mism.size == 0:
        for key in ("counts_raw", "counts_kept", "offsets", "slot_row"):
            np.testing.assert_array_equal(down(getattr(layer, key)), fwd[key], err_msg=key)
    else:
        np.testing.assert_array_equal(down(layer.counts_raw)[keep_e], fwd["counts_raw"][keep_e])
    assert_close(down(layer.y)[keep_t], fwd["y"][keep_t], tol, "y")
    dw1_g, dw1_r = down(layer.dw1), np.array(bwd["dw1"])
    keep_dx = keep_t.copy()
    pairs = []
    if w1 is not None and w.dtype == "bf16":
        og, orf = down(layer.offsets), fwd["offsets"]
        rows_g = {e: (int(og[e]), int(og[e + 1])) for e in range(w.E)}
        rows_r = {e: (int(orf[e]), int(orf[e + 1])) for e in range(w.E)}
        pairs, rows = relu_kink_flips(down(layer.h), fwd["h"], fwd["x_perm"], w1, rows_g, rows_r,
                                      [e for e in range(w.E) if keep_e[e]])
        for e, c in pairs:
            dw1_g[e, c] = dw1_r[e, c] = 0.0
        keep_dx[fwd["row_token"][rows]] = False
    kink_tokens = int(keep_t.sum() - keep_dx.sum())
    print(f"set aside T={w.T} E={w.E} F={w.F}: {mism.size} near-tie tokens "
          f"({int((~keep_e).sum())} experts), {len(pairs)} near-kink dW1 rows, "
          f"{kink_tokens} near-kink dX tokens", flush=True)
    assert len(pairs) <= max(4, w.E * w.F // 1000), f"{len(pairs)} dW1 rows set aside"
    assert kink_tokens <= max(4, w.T // 1000), f"{kink_tokens} dX tokens set aside"
    assert_close(down(layer.dx)[keep_dx], bwd["dx"][keep_dx], tol, "dx")
    assert_close(down(layer.dlogits)[keep_t], bwd["dlogits"][keep_t], tol, "dlogits")
    assert_close_per_expert(dw1_g[keep_e], dw1_r[keep_e], tol, "dw1")
    assert_close_per_expert(down(layer.dw2)[keep_e], bwd["dw2"][keep_e], tol, "dw2")
    assert_close(down(layer.dw_gate)[:, keep_e], bwd["dw_gate"][:, keep_e], tol, "dw_gate")
    assert_close(down(layer.db_gate)[keep_e], bwd["db_gate"][keep_e], tol, "db_gate")
    return mism


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_backward_end_to_end(name):
    w, inp, layer, fwd, bwd = _end_to_end(name)
    mism = compare_end_to_end(w, layer, fwd, bwd, inp["w1"])
    assert mism.size <= 3


@pytest.mark.parametrize("name", ["tiny_fp32", "skewed_zipf12", "uniform_cf050",
                                  "skewed_split_tail", "uniform_walk_k128"])
def test_bitwise_repeatable(name):
    w, inp, dev, layer = _setup(name)
    outs = []
    for _ in range(2):
        layer.forward(dev["x"], dev["w_gate"], dev["b_gate"], dev["w1"], dev["w2"])
        layer.backward(dev["dy"], dev["x"], dev["w_gate"], dev["w1"], dev["w2"])
        torch.cuda.synchronize()
        outs.append([getattr(layer, n).clone() for n in
                     ("y", "logits", "topk_w", "slot_row", "x_perm", "h", "dx", "dw1", "dw2",
                      "dw_gate", "db_gate", "dlogits")])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["skewed_zipf12", "uniform_cf050"])
def test_forward_equals_its_entry_points(name):
    """moe_route (no counts) + moe_permute + moe_expert_ffn + moe_combine give
    bit-for-bit what moe_forward gives."""
    w, inp, dev, layer = _setup(name)
    names = ("y", "logits", "topk_idx", "topk_w", "counts_raw", "counts_kept", "offsets",
             "slot_row", "row_token", "x_perm", "h", "out_perm")
    layer.forward(dev["x"], dev["w_gate"], dev["b_gate"], dev["w1"], dev["w2"])
    torch.cuda.synchronize()
    ref = {n: getattr(layer, n).clone() for n in names}
    for n in names:
        getattr(layer, n).fill_(-7)
    layer.route(dev["x"], dev["w_gate"], dev["b_gate"], counts=False)
    layer.permute(dev["x"])
    layer.expert_ffn(dev["w1"], dev["w2"])
    layer.combine()
    torch.cuda.synchronize()
    S = int(ref["offsets"][-1].item())
    for n in names:
        a, b = getattr(layer, n), ref[n]
        if n in ("x_perm", "h", "out_perm"):
            a, b = a[:S], b[:S]
        if n == "row_token":
            a, b = a[:w.T * w.k], b[:w.T * w.k]
        assert torch.equal(a, b), n


@pytest.mark.parametrize("name", ["skewed_zipf12", "uniform_cf050", "skewed_split_fc1"])
def test_forward_relu_bits_and_backward_with_or_without_them(name):
    """The keep bits the forward writes are exactly [h > 0] over the kept
    rows, and the backward gives bit-for-bit the same results whether it is
    handed them or derives the mask from h itself."""
    w, inp, dev, layer = _setup(name)
    layer.forward(dev["x"], dev["w_gate"], dev["b_gate"], dev["w1"], dev["w2"])
    torch.cuda.synchronize()
    n = int(layer.offsets[-1].item())
    h = down(layer.h)[:n]
    bits = down(layer.relu_bits)[:n].view(np.uint32)
    expect = np.packbits((h > 0).reshape(n, -1, 32), axis=-1, bitorder="little")
    np.testing.assert_array_equal(bits, expect.reshape(n, -1, 4).view(np.uint32)[..., 0])
    names = ("dx", "dw1", "dw2", "dw_gate", "db_gate", "dlogits")
    layer.backward(dev["dy"], dev["x"], dev["w_gate"], dev["w1"], dev["w2"])
    torch.cuda.synchronize()
    ref = {k: getattr(layer, k).clone() for k in names}
    layer.relu_bits_used = False
    layer.backward(dev["dy"], dev["x"], dev["w_gate"], dev["w1"], dev["w2"])
    torch.cuda.synchronize()
    for k in names:
        assert torch.equal(getattr(layer, k), ref[k]), k


def test_popularity_window():
    E, W = 32, 4
    layer = MoeLayer(8, 64, 64, E, 2, 0.0, act_code("f32"), window=W, backward=False)
    rng = np.random.default_rng(5)
    ring = np.zeros((W, E), np.int32)
    for it in range(10):
        c = rng.integers(0, 5000, E).astype(np.int32)
        layer.popularity(it, counts_raw=up_i32(c))
        torch.cuda.synchronize()
        ring, ref = orc.popularity_update(ring, it, c)
        np.testing.assert_array_equal(down(layer.window_sum), ref)
        np.testing.assert_array_equal(down(layer.ring), ring)


@pytest.mark.parametrize("name", ["skewed_split_tail", "uniform_cf050"])
def test_side_stream_gives_the_same_bits(name):
    """Every entry point enqueues on the stream it is given: forward and
    backward on a second (default-priority) stream reproduce the
    current-stream results bit for bit once that stream is synchronised."""
    w, inp, dev, layer = _setup(name)
    names = ("y", "topk_idx", "slot_row", "h", "out_perm", "dx", "dw1", "dw2", "dw_gate",
             "db_gate")
    layer.forward(dev["x"], dev["w_gate"], dev["b_gate"], dev["w1"], dev["w2"])
    layer.backward(dev["dy"], dev["x"], dev["w_gate"], dev["w1"], dev["w2"])
    torch.cuda.synchronize()
    ref = {n: getattr(layer, n).clone() for n in names}
    for n in names:
        getattr(layer, n).fill_(-3)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    layer.forward(dev["x"], dev["w_gate"], dev["b_gate"], dev["w1"], dev["w2"], stream=side)
    layer.backward(dev["dy"], dev["x"], dev["w_gate"], dev["w1"], dev["w2"], stream=side)
    side.synchronize()
    n_kept = int(layer.offsets[-1].item())
    for n in names:
        a, b = getattr(layer, n), ref[n]
        if n in ("h", "out_perm"):  # rows past the kept ones are not written
            a, b = a[:n_kept], b[:n_kept]
        assert torch.equal(a, b), n


# Experts whose last row tile is short: a few rows up to a whole tile.
# Shapes whose two products take 256 x 128 tiles (both), 128 x 256 then
# 128 x 128, and 128 x 128 then 128 x 256 (the tile picker's choices for at
# most T*k rows; K < 2048, so every tile is whole and no K split changes the
# summation), with expert row counts around a quarter, a half and all of a
# tile's rows.
SHORT_TILE_CASES = {
    "tiles_256x128": (16384, 128, 128, [1, 31, 33, 64, 65, 127, 129, 200]),
    "tiles_128x256_128x128": (4096, 128, 512,
                              [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 160, 0, 5, 96, 97, 250]),
    "tiles_128x128_128x256": (8192, 256, 512, [2, 30, 40, 64, 100, 128, 130, 255]),
}


@pytest.mark.parametrize("case", list(SHORT_TILE_CASES))
def test_expert_ffn_short_last_tiles(case):
    """h, O and the ReLU keep bits against the reference per expert, and bit
    for bit against the same rows computed inside whole tiles (each expert's
    rows padded with other rows to a multiple of 256)."""
    T, d, F, counts = SHORT_TILE_CASES[case]
    E, k = len(counts), 2
    rng = np.random.default_rng(7)
    S = sum(counts)
    x = workloads.round_to_bf16(rng.standard_normal((S, d), dtype=np.float32))
    w1 = workloads.round_to_bf16(0.05 * rng.standard_normal((E, F, d), dtype=np.float32))
    w2 = workloads.round_to_bf16(0.05 * rng.standard_normal((E, d, F), dtype=np.float32))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dw1, dw2 = up(w1, "bf16"), up(w2, "bf16")

    def run(xp_np, offs):
        layer = MoeLayer(T, d, F, E, k, 0.0, act_code("bf16"), backward=False)
        xp = torch.zeros(T * k, d, dtype=layer.dtype, device="cuda")
        xp[:xp_np.shape[0]] = up(xp_np, "bf16")
        layer.expert_ffn(dw1, dw2, x_perm=xp, offsets=up_i32(offs))
        torch.cuda.synchronize()
        n = int(offs[-1])
        return (down(layer.h)[:n], down(layer.out_perm)[:n],
                layer.relu_bits[:n].cpu().numpy().view(np.uint32))

    h_g, o_g, bits_g = run(x, offsets)
    h_r, o_r = orc.expert_ffn(x, offsets, w1, w2, "bf16")
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        assert_close(h_g[a:b], h_r[a:b], TOL["bf16"], f"h[{e}]")
        assert_close(o_g[a:b], o_r[a:b], TOL["bf16"], f"O[{e}]")
    keep = (h_g > 0).reshape(S, F // 32, 32)
    np.testing.assert_array_equal(bits_g, (keep * (1 << np.arange(32, dtype=np.uint64))).sum(-1))

    # the same rows inside whole tiles: expert e's rows, then filler rows
    pad = [-(-c // 256) * 256 for c in counts]
    assert sum(pad) <= T * k
    offs2 = np.concatenate([[0], np.cumsum(pad)]).astype(np.int32)
    x2 = workloads.round_to_bf16(rng.standard_normal((sum(pad), d), dtype=np.float32))
    src = np.concatenate([np.arange(offs2[e], offs2[e] + counts[e]) for e in range(E)])
    x2[src] = x
    h2, o2, bits2 = run(x2, offs2)
    np.testing.assert_array_equal(workloads.bf16_bits(h_g), workloads.bf16_bits(h2[src]))
    np.testing.assert_array_equal(workloads.bf16_bits(o_g), workloads.bf16_bits(o2[src]))
    np.testing.assert_array_equal(bits_g, bits2[src])
