"""Throughput of one GPU's MoE layer: route + permute + grouped FFN + combine,
the popularity window and the full backward, on seeded synthetic inputs.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = moe_forward + moe_popularity_update + moe_backward over one batch
of T tokens.  Prints ONE JSON line on stdout (progress goes to stderr).

value      = T * K / (time of K back-to-back steps), inputs resident in HBM
roofline   = the grouped expert GEMM (moe_expert_ffn: FC1 + FC2 launches),
             algorithmic 4*d*F*S_kept flops per call over its HIP-event time
cpu_baseline = the CPU reference on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="uniform_cf125", choices=list(workloads.workloads()))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-reps", type=int, default=20)
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


def cpu_baseline(w: workloads.Workload, inp, budget_s: float = 20.0):
    """The CPU reference, as it stands, on a token sample of the workload:
    forward + backward on the first n tokens (same weights), n doubled until
    one run takes a few seconds or the whole batch is done."""
    from oracle import moe_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    n = min(w.T, 256)
    total_t, total_tok, runs = 0.0, 0, 0
    while True:
        x = inp["x"][:n]
        dy = inp["dy"][:n]
        t0 = time.perf_counter()
        fwd = orc.forward(x, inp["w_gate"], inp["b_gate"], inp["w1"], inp["w2"], w.k,
                          w.capacity_factor, w.dtype)
        orc.backward(dy, fwd, x, inp["w_gate"], inp["w1"], inp["w2"], w.dtype)
        dt = time.perf_counter() - t0
        total_t += dt
        total_tok += n
        runs += 1
        log(f"cpu baseline: {n} tokens fwd+bwd in {dt:.2f} s")
        if total_t > budget_s or n >= w.T or dt > budget_s / 4:
            break
        n = min(w.T, n * 2)
    return {"value": total_tok / total_t, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{runs} runs of forward+backward on the first 256..{n} of {w.T} tokens "
                      f"({w.name}), float64 NumPy, {total_t:.1f} s total"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import mixture_experts_layer_33_amd as moe
    from mixture_experts_layer_33_amd.layer import MoeLayer

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs an MI355X GPU")
    moe.lib()  # fails loudly when libmoe.so is missing
    w = workloads.workloads()[args.workload]
    log(f"workload {w.name}: {w.description}")
    inp = workloads.make_inputs(w, 0, with_weights=True, with_dy=True)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a, act=True):
        t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return t.to(dt) if act else t

    x, dy = up(inp["x"]), up(inp["dy"])
    w_gate, b_gate = up(inp["w_gate"], False), up(inp["b_gate"], False)
    w1, w2 = up(inp["w1"]), up(inp["w2"])
    act = moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32
    layer = MoeLayer(w.T, w.d, w.F, w.E, w.k, w.capacity_factor, act, window=w.window)
    stream = torch.cuda.current_stream()

    it_counter = [0]

    def step():
        layer.forward(x, w_gate, b_gate, w1, w2, logits_out=False)
        layer.popularity(it_counter[0])
        layer.backward(dy, x, w_gate, w1, w2, dlogits=False)
        it_counter[0] += 1

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps
    value = w.T / (ms / 1e3)
    s_kept = int(layer.offsets[-1].item())
    log(f"step {ms:.3f} ms ({value:,.0f} tokens/s), wall {t_wall:.3f} s, S_kept {s_kept}")

    # per-part event timings (same inputs, after the timed region)
    def time_it(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = args.kernel_reps
    t_fwd = time_it(lambda: layer.forward(x, w_gate, b_gate, w1, w2, logits_out=False), reps)
    t_bwd = time_it(lambda: layer.backward(dy, x, w_gate, w1, w2, dlogits=False), reps)
    t_ffn = time_it(lambda: layer.expert_ffn(w1, w2), reps)
    t_comb = time_it(lambda: layer.combine(), reps)
    flops_ffn = 4.0 * w.d * w.F * s_kept
    achieved = flops_ffn / (t_ffn / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    comb_bytes = s_kept * w.d * (2 if w.dtype == "bf16" else 4) + \
        w.T * w.d * (2 if w.dtype == "bf16" else 4) + 8 * w.T * w.k
    log(f"forward {t_fwd:.3f} ms, backward {t_bwd:.3f} ms, expert FFN {t_ffn:.3f} ms "
        f"({achieved:.1f} TFLOP/s), combine {t_comb*1e3:.1f} us "
        f"({comb_bytes / (t_comb / 1e3) / 1e9:.0f} GB/s)")

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    out = {
        "metric": "MoE-layer tokens/sec (route+permute+grouped FFN+combine, with popularity "
                  "window and backward); % MFMA roofline of the grouped GEMM",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d, "d_ff": w.F, "E": w.E,
                   "k": w.k, "capacity_factor": w.capacity_factor,
                   "step": "forward + popularity window + backward", "S_kept": s_kept},
        "roofline": {"bound": "mfma", "kernel": "grouped expert GEMM (FC1+FC2 per call)",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None},
        "parts_ms": {"forward": t_fwd, "backward": t_bwd, "expert_ffn": t_ffn,
                     "combine": t_comb},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (CPU reference) ...")
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
