"""Throughput of one GPU's MoE layer: route + permute + grouped FFN + combine,
the popularity window and the full backward, on seeded synthetic inputs.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = moe_route, moe_permute, moe_expert_ffn, moe_combine (the kernels of
moe_forward, in its order), moe_popularity_update and moe_backward over one
batch of T tokens.  Prints ONE JSON line on stdout (progress goes to stderr).

value        = T * K / (time of K back-to-back steps), inputs resident in HBM
roofline     = the grouped expert GEMM kernel (rows_gemm_kernel; its FC1 and FC2
               launches in moe_expert_ffn, 2*d*F*S_kept flops each), averaged
               over the launches of the timed steps with HIP events recorded on
               the launch stream around each moe_expert_ffn call
traffic      = HBM bytes per launch of that kernel from the FETCH_SIZE and
               WRITE_SIZE counters (profiles/rows_gemm_<workload>_hbm_traffic.md),
               or null when the GEMM source changed since they were taken
cpu_baseline = the CPU reference on a bounded sample of the same workload
warm_ms      = median, p10 and p90 of the timed steps
parts_ms     = each entry point and next-row step, warm (calls back to back)
               and cold (after writing 512 MiB and then reading another
               512 MiB, so the caches hold clean lines of other data)
hbm_parts    = route, permute and combine, cold, against their algorithmic
               bytes; also timed after the write alone, whose dirty lines'
               write-back then lands inside the timed call
probes       = a 1 GiB device copy and the vendor dense GEMM of the same flops,
               measured in the same run, with the run's fractions of them

    python bench.py --summarize-traffic FETCH_CSV WRITE_CSV [--workload NAME]

(no GPU) turns the counter files of two rocprofv3 --pmc runs of
``bench.py --copy-calibration`` into that traffic summary, and

    python bench.py --summarize-mfma COUNTER_CSV AGENT_CSV BENCH_JSON [--workload NAME]

(no GPU) turns one rocprofv3 --pmc run of bench.py with the MFMA counters
(SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE; its
JSON line saved as BENCH_JSON) into the per-kernel MFMA utilization of the six
expert GEMM launches of a step.
"""
from __future__ import annotations

import argparse
import json
import os
import re
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
    p.add_argument("--workload", default="mixtral_shaped", choices=list(workloads.workloads()))
    p.add_argument("--priority", default=None, choices=["slot", "choice"],
                   help="capacity priority (default: the workload's)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-reps", type=int, default=20)
    p.add_argument("--cold-reps", type=int, default=20,
                   help="repetitions of the cache-flushed forward / backward timings")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the HBM traffic summary from two counter runs (no GPU)")
    p.add_argument("--summarize-mfma", nargs=3, metavar=("COUNTER_CSV", "AGENT_CSV", "BENCH_JSON"),
                   help="write the MFMA utilization summary from one counter run (no GPU)")
    p.add_argument("--summarize-kernels", metavar="KERNEL_STATS_CSV",
                   help="write the per-kernel time summary of one rocprofv3 --kernel-trace "
                        "--stats run of bench.py (no GPU)")
    p.add_argument("--command", default="",
                   help="the command lines that produced the counter files (recorded)")
    return p.parse_args()


CSRC = os.path.join(ROOT, "mixture_experts_layer_33_amd", "csrc")
GEMM_SRC = os.path.join(CSRC, "gemm.hip")
GEMM_KERNEL = "rows_gemm_kernel"
FIXUP_KERNEL = "rows_fixup_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def _rows_kernel(b_k, epi, row_map):
    """rows_gemm_kernel<BM, BN, B_K, EPI, MAP, PERSIST, STREAM_B> of one product"""
    return GEMM_KERNEL + rf"<\d+, \d+, {b_k}, {epi}, {row_map}, (?:true|false), (?:true|false)>"


def traffic_path(name):
    return os.path.join(ROOT, "profiles", f"rows_gemm_{name}_hbm_traffic.md")


# headers the kernels include: a change there changes the kernels too
SHARED_HEADERS = ["common.hpp", "buffer.hpp"]


def gemm_source_hash():
    """sha256 over gemm.hip and the headers it shares with the other kernels"""
    import hashlib
    h = hashlib.sha256()
    for path in [GEMM_SRC] + [os.path.join(CSRC, f) for f in SHARED_HEADERS]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _counter_rows(path, counter):
    import csv
    with open(path, newline="") as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def summarize_traffic(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the FC1 and FC2 launches,
    each scaled by the same counter's reading for a 1 GiB device copy."""
    w = workloads.workloads()[args.workload]
    out = {}
    lines = []
    all_kib, all_n = {}, {}
    for counter, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.summarize_traffic):
        rows = _counter_rows(path, counter)
        sums = {}
        for r in rows:
            acc = sums.setdefault(r["Kernel_Name"], [0.0, 0])
            acc[0] += float(r["Counter_Value"])
            acc[1] += 1
        all_kib[counter] = {k: v[0] / v[1] for k, v in sums.items()}
        all_n.update({k: v[1] for k, v in sums.items()})
        copies = [float(r["Counter_Value"]) for r in rows
                  if r["Kernel_Name"].startswith(COPY_KERNEL)
                  and float(r["Counter_Value"]) > COPY_BYTES / 1024 / 2]
        if not copies:
            raise SystemExit(f"{path}: no 1 GiB copy dispatch (run with --copy-calibration)")
        scale = (COPY_BYTES / 1024) / (sum(copies) / len(copies))
        per_kernel = {}
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        for i, r in enumerate(rows):
            # forward launches: K-contiguous weights, epilogue ReLU (FC1) or store
            # (FC2), packed rows; a split-tail fixup dispatched right after one
            # belongs to that launch
            if re.search(_rows_kernel("true", "[01]", 0), r["Kernel_Name"]):
                v = float(r["Counter_Value"])
                if i + 1 < len(rows) and FIXUP_KERNEL in rows[i + 1]["Kernel_Name"]:
                    v += float(rows[i + 1]["Counter_Value"])
                per_kernel.setdefault(r["Kernel_Name"], []).append(v)
        if len(per_kernel) != 2:
            raise SystemExit(f"{path}: expected the FC1 and FC2 forward GEMM kernels, "
                             f"found {sorted(per_kernel)}")
        out[counter] = {"copy_kib": sum(copies) / len(copies), "scale": scale,
                        "kernels": {k: sum(v) / len(v) for k, v in per_kernel.items()},
                        "dispatches": {k: len(v) for k, v in per_kernel.items()}}
    names = sorted(out["FETCH_SIZE"]["kernels"])
    per_launch = {}
    for k in names:
        fb = out["FETCH_SIZE"]["kernels"][k] * 1024 * out["FETCH_SIZE"]["scale"]
        wb = out["WRITE_SIZE"]["kernels"][k] * 1024 * out["WRITE_SIZE"]["scale"]
        per_launch[k] = {"fetch_bytes": fb, "write_bytes": wb}
    mean = sum(v["fetch_bytes"] + v["write_bytes"] for v in per_launch.values()) / len(per_launch)
    rec = {"workload": w.name, "gemm_source_sha256": gemm_source_hash(),
           "traffic_bytes_per_launch": mean,
           "fetch_scale": out["FETCH_SIZE"]["scale"], "write_scale": out["WRITE_SIZE"]["scale"],
           "per_kernel": per_launch}
    lines.append(f"# HBM traffic of rows_gemm_kernel (expert FFN forward), {w.name}")
    lines.append("")
    lines.append(f"Workload: {w.description}.")
    lines.append("")
    lines.append("Commands (run from the repository root on one MI355X):")
    lines.append("")
    lines.append("```")
    lines.append(args.command.strip() or "(not recorded)")
    lines.append("```")
    lines.append("")
    lines.append("Counters are KiB per launch (the GEMM dispatch plus the split-tail fixup "
                 "dispatched right after it, if any), averaged over the launches of each "
                 "kernel; each is scaled by 1 GiB / (the same counter's reading for the 1 GiB "
                 f"device copy `{COPY_KERNEL}`).")
    lines.append("")
    lines.append("| counter | copy reading (KiB) | scale |")
    lines.append("|---|---|---|")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f"| {c} | {out[c]['copy_kib']:.0f} | {out[c]['scale']:.4f} |")
    lines.append("")
    lines.append("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) |")
    lines.append("|---|---|---|---|---|")
    for k in names:
        pl = per_launch[k]
        lines.append(f"| `{k}` | {out['FETCH_SIZE']['dispatches'][k]} | "
                     f"{out['FETCH_SIZE']['kernels'][k]:.0f} | "
                     f"{out['WRITE_SIZE']['kernels'][k]:.0f} | "
                     f"{pl['fetch_bytes'] + pl['write_bytes']:.4g} |")
    lines.append("")
    lines.append(f"Mean over the two launches: {mean:.4g} bytes per launch.")
    lines.append("")
    lines.append("traffic-json: " + json.dumps(rec))
    os.makedirs(os.path.dirname(traffic_path(w.name)), exist_ok=True)
    with open(traffic_path(w.name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(traffic_path(w.name))
    summarize_parts_traffic(args, all_kib, {c: out[c]["scale"] for c in out}, all_n)


# the expert GEMM launches of one step: kernel-name pattern -> product
GEMM_ROLES = [
    (_rows_kernel("true", 0, 0), "FC1 forward (ReLU)"),
    (_rows_kernel("true", 1, 0), "FC2 forward"),
    (_rows_kernel("false", 2, 0), "FC2 input gradient (masked)"),
    (_rows_kernel("false", 1, 0), "FC1 input gradient"),
    (r"wgrad_kernel<\d+, \d+, false>", "FC2 weight gradient"),
    (r"wgrad_kernel<\d+, \d+, true>", "FC1 weight gradient (+ gate)"),
]


def mfma_path(name):
    return os.path.join(ROOT, "profiles", f"expert_gemms_{name}_mfma_utilization.md")


def summarize_mfma(args):
    """MFMA busy fraction, clock and executed flops per expert GEMM launch.

    SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD; GRBM_GUI_ACTIVE over
    the XCDs, so busy / (SIMDs * GRBM_GUI_ACTIVE / XCDs) is the fraction of
    SIMD cycles the matrix pipe was busy, and GRBM_GUI_ACTIVE / XCDs over the
    dispatch's duration the average clock.  SQ_INSTS_VALU_MFMA_MOPS_BF16
    counts units of 512 flops."""
    import csv
    w = workloads.workloads()[args.workload]
    cpath, apath, bpath = args.summarize_mfma
    with open(apath, newline="") as f:
        agents = [r for r in csv.DictReader(f) if r.get("Name", "").startswith("gfx")]
    if not agents:
        raise SystemExit(f"{apath}: no GPU agent")
    simds, xcds = int(agents[0]["Simd_Count"]), int(agents[0]["Num_Xcc"])
    disp = {}
    with open(cpath, newline="") as f:
        for r in csv.DictReader(f):
            d = disp.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "c": {},
                                                   "ns": int(r["End_Timestamp"]) -
                                                   int(r["Start_Timestamp"])})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + \
                float(r["Counter_Value"])
    need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")
    with open(bpath) as f:
        cfg = json.loads(f.read().strip().splitlines()[-1])["config"]
    if cfg["workload"] != w.name:
        raise SystemExit(f"{bpath}: workload {cfg['workload']}, not {w.name}")
    alg = 2.0 * cfg["d_model"] * cfg["d_ff"] * cfg["S_kept"]
    rows = []
    for pat, role in GEMM_ROLES:
        ds = [d for d in disp.values() if re.search(pat, d["name"])]
        if not ds:
            continue
        for d in ds:
            missing = [c for c in need if c not in d["c"]]
            if missing:
                raise SystemExit(f"{cpath}: {d['name']} lacks {missing}")
        n = len(ds)
        us = sum(d["ns"] for d in ds) / n / 1e3
        busy = sum(d["c"][need[0]] for d in ds) / n
        flops = sum(d["c"][need[1]] for d in ds) / n * 512
        gui = sum(d["c"][need[2]] for d in ds) / n
        cyc = gui / xcds
        rows.append({"role": role, "kernel": ds[0]["name"], "dispatches": n, "us": us,
                     "busy": busy / (simds * cyc), "ghz": cyc / (us * 1e3),
                     "flops": flops, "alg": alg})
    if len(rows) != len(GEMM_ROLES):
        raise SystemExit(f"{cpath}: found {[r['role'] for r in rows]}, expected all six products")
    L = [f"# MFMA utilization of the expert GEMMs, {w.name}", "",
         f"Workload: {w.description}.", "",
         "Commands (run from the repository root on one MI355X):", "", "```",
         args.command.strip() or "(not recorded)", "```", "",
         f"Counters per dispatch, averaged over each kernel's dispatches ({simds} SIMDs, "
         f"{xcds} XCDs).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x "
         "GRBM_GUI_ACTIVE / XCDs): the share of SIMD cycles the matrix pipe was busy, at "
         "the clock the dispatch ran at (GRBM_GUI_ACTIVE / XCDs / duration).  Executed "
         "flops = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 (rows padded up to whole tiles "
         f"included); algorithmic = 2 d F S_kept = {alg / 1e9:.1f} GFLOP per product.  "
         "Durations are from the counter run (dispatches serialized), so they run a "
         "little longer than in the timed steps.", "",
         "| product | kernel | dispatches | µs | MFMA busy | clock GHz | executed / algorithmic "
         "flops | algorithmic TFLOP/s |",
         "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        L.append(f"| {r['role']} | `{r['kernel'][:70]}` | {r['dispatches']} | {r['us']:.1f} | "
                 f"{r['busy']:.1%} | {r['ghz']:.2f} | {r['flops'] / r['alg']:.3f} | "
                 f"{r['alg'] / (r['us'] * 1e-6) / 1e12:.0f} |")
    # the router's dispatches (matrix-core kernel), if the run has them
    rds = [d for d in disp.values() if "route_tile_kernel" in d["name"]
           and all(c in d["c"] for c in need)]
    router = None
    if rds:
        n = len(rds)
        us = sum(d["ns"] for d in rds) / n / 1e3
        cyc = sum(d["c"][need[2]] for d in rds) / n / xcds
        ep = 16
        while ep < cfg["E"]:
            ep *= 2
        method = 2.0 * cfg["T"] * cfg["d_model"] * cfg["E"]
        router = {"kernel": rds[0]["name"], "dispatches": n, "us": us,
                  "busy": sum(d["c"][need[0]] for d in rds) / n / (simds * cyc),
                  "ghz": cyc / (us * 1e3),
                  "flops": sum(d["c"][need[1]] for d in rds) / n * 512,
                  "three_pass": 3.0 * 2.0 * cfg["T"] * cfg["d_model"] * ep, "method": method}
        L += ["", "Router (`route_tile_kernel`, warm and cold calls alike): executed flops "
              "against three bf16 passes over E rounded up to a power of two >= 16 "
              f"({router['three_pass'] / 1e9:.1f} GFLOP) and against the method's 2 T d E "
              f"({method / 1e9:.2f} GFLOP).", "",
              "| kernel | dispatches | µs | MFMA busy | clock GHz | executed / three-pass | "
              "executed / method |", "|---|---|---|---|---|---|---|",
              f"| `{router['kernel'][:70]}` | {n} | {us:.1f} | {router['busy']:.1%} | "
              f"{router['ghz']:.2f} | {router['flops'] / router['three_pass']:.3f} | "
              f"{router['flops'] / method:.2f} |"]
    L.append("")
    L.append("mfma-json: " + json.dumps({"workload": w.name, "gemm_source_sha256":
                                         gemm_source_hash(), "rows": rows, "router": router}))
    os.makedirs(os.path.dirname(mfma_path(w.name)), exist_ok=True)
    with open(mfma_path(w.name), "w") as f:
        f.write("\n".join(L) + "\n")
    print(mfma_path(w.name))


# the HBM-bound steps: kernels per call, and the sources they are built from
PART_KERNELS = {
    "route": ["route_tile_kernel", "route_kernel"],
    "permute": ["rank_hist_kernel", "scan_kernel", "gather_kernel"],
    "combine": ["combine_kernel"],
}
PART_SOURCES = ["route.hip", "permute.hip", "combine.hip", "common.hpp", "buffer.hpp"]


def parts_hbm_bytes(w, s_kept):
    """Algorithmic bytes per call: route T*d*s + 4*d*E + 8*T*k (logits not
    written); permute T*d*s + S_kept*d*s + 12*T*k; combine S_kept*d*s +
    T*d*s + 8*T*k (s = bytes per activation element)."""
    sx = 2 if w.dtype == "bf16" else 4
    return {"route": w.T * w.d * sx + 4 * w.d * w.E + 8 * w.T * w.k,
            "permute": w.T * w.d * sx + s_kept * w.d * sx + 12 * w.T * w.k,
            "combine": s_kept * w.d * sx + w.T * w.d * sx + 8 * w.T * w.k}


def parts_traffic_path(name):
    return os.path.join(ROOT, "profiles", f"route_permute_combine_{name}_hbm_traffic.md")


def parts_source_hashes():
    import hashlib
    out = {}
    for f in PART_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            out[f] = hashlib.sha256(fh.read()).hexdigest()
    return out


def summarize_parts_traffic(args, per_kernel_kib, scales, dispatches):
    """Counter bytes per call of route, permute and combine: for each step the
    mean FETCH_SIZE and WRITE_SIZE of each of its kernels over that kernel's
    dispatches, scaled by the calibration copy, summed over the step's
    kernels; against the step's algorithmic bytes."""
    w = workloads.workloads()[args.workload]
    alg = parts_hbm_bytes(w, w.T * w.k)  # the measured workloads drop no slot
    rows, rec = [], {}
    for part, kernels in PART_KERNELS.items():
        total, found = 0.0, []
        for kn in kernels:
            # (names may be mangled: "13gather_kernelIDF16b..."; no listed name is
            # a substring of another kernel's)
            names = [n for n in per_kernel_kib["FETCH_SIZE"]
                     if kn in n and n in per_kernel_kib["WRITE_SIZE"]]
            for n in names:
                fb = per_kernel_kib["FETCH_SIZE"][n] * 1024 * scales["FETCH_SIZE"]
                wb = per_kernel_kib["WRITE_SIZE"][n] * 1024 * scales["WRITE_SIZE"]
                found.append((n, dispatches[n], fb, wb))
        if not found:
            continue
        # a kernel name can appear in several instantiations: weight them by
        # their dispatch counts, then add the step's kernels up
        by_kernel = {}
        for n, nd, fb, wb in found:
            base = next(kn for kn in kernels if kn in n)
            acc = by_kernel.setdefault(base, [0.0, 0.0, 0])
            acc[0] += fb * nd
            acc[1] += wb * nd
            acc[2] += nd
        for base, (fb, wb, nd) in by_kernel.items():
            rows.append((part, base, nd, fb / nd, wb / nd))
            total += (fb + wb) / nd
        rec[part] = total
    L = [f"# HBM traffic of route, permute and combine, {w.name}", "",
         f"Workload: {w.description}.", "",
         "Commands (run from the repository root on one MI355X):", "", "```",
         args.command.strip() or "(not recorded)", "```", "",
         "FETCH_SIZE and WRITE_SIZE per dispatch (KiB), averaged over each kernel's "
         "dispatches in the run (warm and cold calls alike), scaled by 1 GiB / (the same "
         f"counter's reading for the 1 GiB device copy `{COPY_KERNEL}`).  A step's bytes are "
         "the sum over its kernels.  Algorithmic bytes: route T*d*s + 4*d*E + 8*T*k, permute "
         "T*d*s + S*d*s + 12*T*k, combine S*d*s + T*d*s + 8*T*k (S = T*k slots, all kept "
         "here), s = bytes per activation element.", "",
         "| step | kernel | dispatches | fetch bytes | write bytes |", "|---|---|---|---|---|"]
    for part, base, nd, fb, wb in rows:
        L.append(f"| {part} | `{base}` | {nd} | {fb:.4g} | {wb:.4g} |")
    L += ["", "| step | counter bytes per call | algorithmic bytes | ratio |", "|---|---|---|---|"]
    for part, b in rec.items():
        L.append(f"| {part} | {b:.4g} | {alg[part]:.4g} | {b / alg[part]:.3f} |")
    L.append("")
    L.append("parts-traffic-json: " + json.dumps({"workload": w.name,
                                                  "sources_sha256": parts_source_hashes(),
                                                  "bytes_per_call": rec,
                                                  "algorithmic_bytes": alg}))
    os.makedirs(os.path.dirname(parts_traffic_path(w.name)), exist_ok=True)
    with open(parts_traffic_path(w.name), "w") as f:
        f.write("\n".join(L) + "\n")
    print(parts_traffic_path(w.name))


def load_parts_traffic(name):
    """Counter bytes per call of route/permute/combine from the committed
    summary, or None when there is none or a source changed since."""
    try:
        with open(parts_traffic_path(name)) as f:
            for line in f:
                if line.startswith("parts-traffic-json: "):
                    rec = json.loads(line[len("parts-traffic-json: "):])
                    if rec["sources_sha256"] == parts_source_hashes():
                        return rec["bytes_per_call"]
                    log("route/permute/combine traffic summary is stale: counter_bytes = null")
    except OSError:
        pass
    return None


def kernels_path(name):
    return os.path.join(ROOT, "profiles", f"kernels_{name}_kernel_stats.md")


def summarize_kernels(args):
    """Per-kernel averages of a rocprofv3 --kernel-trace --stats run of
    bench.py: every kernel of the run (timed steps, part timings, probes),
    sorted by total time, with the expert GEMM launches' TFLOP/s."""
    import csv
    w = workloads.workloads()[args.workload]
    with open(args.summarize_kernels, newline="") as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    alg = 2.0 * w.d * w.F * w.T * w.k  # every slot kept in the measured workloads
    L = [f"# Kernel times, {w.name} (rocprofv3 --kernel-trace --stats)", "",
         f"Workload: {w.description}.", "",
         "Command (run from the repository root on one MI355X):", "", "```",
         args.command.strip() or "(not recorded)", "```", "",
         "All kernels of the run: the timed steps plus the per-part warm and cold timings "
         "(cold ones after a 512 MiB fill and a 512 MiB sum) and the probes; averages over each "
         f"kernel's dispatches.  Expert GEMM TFLOP/s: 2 d F S = {alg / 1e9:.1f} GFLOP per "
         "product over the kernel's average duration.", "",
         "| kernel | calls | average µs | total ms | share | GEMM TFLOP/s |",
         "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        avg = float(r["AverageNs"]) / 1e3
        tf = ""
        if re.search(r"rows_gemm_kernel|wgrad_kernel<", name):
            tf = f"{alg / (avg * 1e-6) / 1e12:.0f}"
        short = name if len(name) <= 90 else name[:87] + "..."
        L.append(f"| `{short}` | {r['Calls']} | {avg:.1f} | "
                 f"{float(r['TotalDurationNs']) / 1e6:.2f} | "
                 f"{float(r['TotalDurationNs']) / total:.1%} | {tf} |")
    os.makedirs(os.path.dirname(kernels_path(w.name)), exist_ok=True)
    with open(kernels_path(w.name), "w") as f:
        f.write("\n".join(L) + "\n")
    print(kernels_path(w.name))


def load_traffic(name):
    """Bytes per launch from the committed counter summary, or None when there
    is none or the GEMM source has changed since it was taken."""
    try:
        with open(traffic_path(name)) as f:
            for line in f:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec["gemm_source_sha256"] == gemm_source_hash():
                        return rec["traffic_bytes_per_launch"]
                    log("traffic summary is stale (GEMM source changed): traffic = null")
    except OSError:
        pass
    return None


def cpu_baseline(w: workloads.Workload, inp, budget_s: float = 12.0):
    """The CPU reference, as it stands, on a token sample of the workload:
    forward + backward on the first n tokens (same weights), n doubled until
    a run takes a quarter of the budget or covers the whole batch; that run is
    then repeated until about budget_s seconds of CPU work are done."""
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
                          w.capacity_factor, w.dtype, priority=w.priority)
        orc.backward(dy, fwd, x, inp["w_gate"], inp["w1"], inp["w2"], w.dtype)
        dt = time.perf_counter() - t0
        total_t += dt
        total_tok += n
        runs += 1
        log(f"cpu baseline: {n} tokens fwd+bwd in {dt:.2f} s")
        if total_t > budget_s:
            break
        if n < w.T and dt < budget_s / 4:
            n = min(w.T, n * 2)
    return {"value": total_tok / total_t, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{runs} runs of forward+backward on the first 256..{n} of {w.T} tokens "
                      f"({w.name}, {total_tok} tokens in all), float64 NumPy, "
                      f"{total_t:.1f} s total"}


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.summarize_kernels:
        summarize_kernels(args)
        return
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
    if args.priority is not None and args.priority != w.priority:
        w = workloads.scaled(w, priority=args.priority,
                             description=f"{w.description}, {args.priority}-major capacity")
    log(f"workload {w.name}: {w.description}")
    inp = workloads.make_inputs(w, 0, with_weights=True, with_dy=True)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a, act=True):
        t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return t.to(dt) if act else t

    x, dy = up(inp["x"]), up(inp["dy"])
    w_gate, b_gate = up(inp["w_gate"], False), up(inp["b_gate"], False)
    w1, w2 = up(inp["w1"]), up(inp["w2"])
    # a drifting workload cycles through its iterations' tokens, output
    # gradients and gate biases (the weights stay fixed)
    per_iter = [(x, dy, b_gate)]
    for it in range(1, w.iters):
        nxt = workloads.make_inputs(w, it, with_weights=False, with_dy=True)
        per_iter.append((up(nxt["x"]), up(nxt["dy"]), up(nxt["b_gate"], False)))
    if w.iters > 1:
        log(f"{w.iters} drifting iterations resident")
    act = moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32
    layer = MoeLayer(w.T, w.d, w.F, w.E, w.k, w.capacity_factor, act, window=w.window,
                     priority=w.priority)
    stream = torch.cuda.current_stream()

    it_counter = [0]
    ev = []  # (before, after) moe_expert_ffn in each timed step

    def step(mark=None):
        xi, dyi, bi = per_iter[it_counter[0] % len(per_iter)]
        layer.route(xi, w_gate, bi, logits_out=False, counts=False)
        layer.permute(xi)
        if mark is not None:
            mark[0].record(stream)
        layer.expert_ffn(w1, w2)
        if mark is not None:
            mark[1].record(stream)
        layer.combine()
        layer.popularity(it_counter[0])
        layer.backward(dyi, xi, w_gate, w1, w2, dlogits=False)
        it_counter[0] += 1

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(ev[i])
        step_end[i].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps
    value = w.T / (ms / 1e3)
    s_kept = int(layer.offsets[-1].item())
    # the GEMM kernel: two launches (FC1, FC2) per moe_expert_ffn call
    gemm_launch_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps / 2
    log(f"step {ms:.3f} ms ({value:,.0f} tokens/s), wall {t_wall:.3f} s, S_kept {s_kept}, "
        f"GEMM launch {gemm_launch_ms * 1e3:.1f} us")

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
    # cold cache: 512 MiB written, then 512 MiB of another buffer read before
    # each repetition (evicts the 256 MB last-level cache and every L2 and
    # leaves them holding clean lines: after the write alone, up to 256 MB of
    # dirty lines would be written back during the timed call); warm: calls
    # back to back on the same inputs (working sets under 256 MB then come
    # from the caches)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flush_rd = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def pct(ts):
        q = np.percentile(ts, [10, 50, 90])
        return {"median": float(q[1]), "p10": float(q[0]), "p90": float(q[2])}

    def warm(fn, reps=args.cold_reps):
        """one call's time, calls back to back with caches warm"""
        fn()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record(stream)
        for r in range(reps):
            fn()
            evs[r + 1].record(stream)
        torch.cuda.synchronize()
        return pct([evs[r].elapsed_time(evs[r + 1]) for r in range(reps)])

    def cold(fn, reps=args.cold_reps, clean=True):
        ts = []
        for r in range(reps):
            flush.fill_(r & 255)
            if clean:
                flush_rd.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return pct(ts)

    # in the order of the layer, so each part reads what the one before wrote
    part_fns = {
        "route": lambda: layer.route(x, w_gate, b_gate, logits_out=False, counts=False),
        "permute": lambda: layer.permute(x),
        "expert_ffn": lambda: layer.expert_ffn(w1, w2),
        "combine": lambda: layer.combine(),
        "forward_fused": lambda: layer.forward_fused(x, w_gate, b_gate, w1, w2, logits_out=False),
        "forward": lambda: layer.forward(x, w_gate, b_gate, w1, w2, logits_out=False),
        "backward": lambda: layer.backward(dy, x, w_gate, w1, w2, dlogits=False),
    }
    parts = {}
    for name, fn in part_fns.items():
        parts[name] = {"warm": warm(fn), "cold": cold(fn)}
        if name in ("route", "permute", "combine"):
            parts[name]["cold_after_write_only"] = cold(fn, clean=False)
        log(f"{name}: warm {parts[name]['warm']['median'] * 1e3:.1f} us, cold "
            f"{parts[name]['cold']['median'] * 1e3:.1f} us (medians)")
    t_ffn = parts["expert_ffn"]["warm"]["median"]
    # dispatch plan for 8 ranks with one extra copy per expert (not part of
    # the step: the planning that would feed an All-to-All)
    R_plan, extra_plan = 8, w.E
    zi = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")  # noqa: E731
    plan = [zi(w.E + 1), zi(w.E + extra_plan), zi(w.E + extra_plan), zi(w.E + extra_plan),
            zi(R_plan)]
    t_plan = time_it(lambda: moe.moe_ep_plan(w.E, R_plan, extra_plan, layer.offsets, *plan), reps)
    rank_rows = plan[4].cpu().numpy()
    plan_balance = float(rank_rows.max() / max(rank_rows.mean(), 1e-9))
    # All-to-All split sizes of that plan's copies
    lay_out = [zi(R_plan), zi(R_plan + 1), zi(w.E + extra_plan)]
    t_layout = time_it(lambda: moe.moe_dispatch_layout(w.E + extra_plan, R_plan, plan[2], plan[3],
                                                       *lay_out), reps)
    # the backward with each expert's weight gradients split over that plan's
    # copies (bf16 only), after a forward that leaves its saved tensors
    rep_ms = None
    if w.dtype == "bf16":
        P_plan = w.E + extra_plan
        rep_ws = torch.empty(moe.moe_backward_replicated_workspace_bytes(layer.shape, P_plan),
                             dtype=torch.uint8, device="cuda")
        layer.forward(x, w_gate, b_gate, w1, w2, logits_out=False)
        moe.moe_ep_plan(w.E, R_plan, extra_plan, layer.offsets, *plan)

        def bwd_rep():
            moe.moe_backward_replicated(layer.shape, dy, x, w_gate, w1, w2, layer.topk_idx,
                                        layer.topk_w, layer.slot_row, layer.row_token,
                                        layer.offsets, layer.x_perm, layer.h, layer.out_perm,
                                        layer.relu_bits, P_plan, plan[0], plan[1], plan[2],
                                        layer.dx, layer.dw1, layer.dw2, layer.dw_gate,
                                        layer.db_gate, None, rep_ws)
        rep_ms = {"warm": warm(bwd_rep), "cold": cold(bwd_rep),
                  "copies": P_plan, "experts_with_copies": int(
                      (plan[0][1:] - plan[0][:-1] > 1).sum().item())}
        log(f"backward over the plan's copies: warm {rep_ms['warm']['median'] * 1e3:.1f} us, "
            f"cold {rep_ms['cold']['median'] * 1e3:.1f} us")
        del rep_ws
    # cross-layer co-occurrence window and next-layer popularity prediction,
    # with this layer's routing as layer j and seeded successor choices as j+1
    idx_b = torch.from_numpy(workloads.next_layer_choices(layer.topk_idx.cpu().numpy(), w.E,
                                                          w.k, 0)).cuda()
    co_ring = torch.zeros((w.window, w.E, w.E), dtype=torch.int32, device="cuda")
    co_sum = torch.zeros((w.E, w.E), dtype=torch.int32, device="cuda")
    co_it = [0]

    def co_update():
        moe.moe_cooccurrence_update(w.E, w.E, w.k, w.k, w.T, w.window, co_it[0], layer.topk_idx,
                                    idx_b, co_ring, co_sum)
        co_it[0] += 1

    t_co = time_it(co_update, reps)
    pred = torch.empty(w.E, dtype=torch.float64, device="cuda")
    order = torch.empty(w.E, dtype=torch.int32, device="cuda")
    t_pred = time_it(lambda: moe.moe_predict_popularity(w.E, w.E, layer.counts_raw, co_sum, pred,
                                                        order), reps)
    flops_launch = 2.0 * w.d * w.F * s_kept
    # FC1 and FC2 move the same bytes: E*d*F weights, S_kept rows of d and F
    gemm_bytes = float((2 if w.dtype == "bf16" else 4) * (w.E * w.d * w.F + s_kept * (w.d + w.F)))
    achieved = flops_launch / (gemm_launch_ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    log(f"expert FFN {t_ffn:.3f} ms warm ({achieved:.1f} TFLOP/s per GEMM launch in the steps)")

    # HBM-bound steps against their algorithmic bytes, from the cold-cache
    # medians (HBM) and the warm ones (cache-resident working sets).  The
    # router is also priced against its matrix-core work: three bf16 passes
    # of 2*T*d*E flops each (W_gate split exactly into three bf16 parts).
    hbm_bytes = parts_hbm_bytes(w, s_kept)
    counters = load_parts_traffic(w.name)
    hbm = {}
    for name in ("route", "permute", "combine"):
        tc, tw = parts[name]["cold"]["median"], parts[name]["warm"]["median"]
        gbs = hbm_bytes[name] / (tc / 1e3) / 1e9
        rec = {"bytes": hbm_bytes[name], "cold_ms": tc, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS,
               "warm_ms": tw, "warm_GB/s (cache-resident)": hbm_bytes[name] / (tw / 1e3) / 1e9,
               "counter_bytes": None if counters is None else counters.get(name),
               "cold_after_write_only_ms": parts[name]["cold_after_write_only"]["median"]}
        if name == "route":
            bound_us = max(hbm_bytes[name] / PEAK_HBM_GBS / 1e3,
                           3 * 2.0 * w.T * w.d * w.E / PEAK_BF16_TFLOPS / 1e6)
            rec.update({"bound_us (max of HBM, 3-pass MFMA)": bound_us,
                        "frac_of_bound": bound_us / (tc * 1e3)})
        hbm[name] = rec
    t_fwd_c, t_fwd_w = parts["forward"]["cold"]["median"], parts["forward"]["warm"]["median"]
    fwd_tok = {"cold": w.T / (t_fwd_c / 1e3), "warm": w.T / (t_fwd_w / 1e3)}
    log(f"forward: {fwd_tok['cold']:,.0f} tokens/s cold, {fwd_tok['warm']:,.0f} warm; "
        + ", ".join(f"{k} {v['frac']:.0%} of HBM cold" for k, v in hbm.items()))

    step_ms = [(start if i == 0 else step_end[i - 1]).elapsed_time(step_end[i])
               for i in range(args.steps)]
    warm_ms = {"step": pct(step_ms)}

    # Probes measured on the same GPU in the same run: a plain 1 GiB device
    # copy (read + write) and the vendor dense GEMM (torch.mm in bf16) with the
    # first expert GEMM's flops (all kept rows times one expert's weights); the
    # roofline and the HBM-bound steps are also given as fractions of them.
    def probe_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    copy_gbs = 2.0 * (1 << 30) / (probe_ms(lambda: dst.copy_(src)) * 1e-3) / 1e9
    # the same copy once, after the cold-cache flush the parts are timed after
    copy_cold_gbs = 2.0 * (1 << 30) / (cold(lambda: dst.copy_(src))["median"] * 1e-3) / 1e9
    del src, dst, flush, flush_rd
    probes = {"copy_1GiB_GB/s": copy_gbs, "copy_1GiB_cold_GB/s": copy_cold_gbs,
              "hbm_parts_cold_frac_of_copy": {k: v["GB/s"] / copy_gbs for k, v in hbm.items()},
              "hbm_parts_cold_frac_of_cold_copy": {k: v["GB/s"] / copy_cold_gbs
                                                   for k, v in hbm.items()}}
    if w.dtype == "bf16":
        pa = torch.randn(s_kept, w.d, device="cuda").to(torch.bfloat16)
        pb = (torch.randn(w.d, w.F, device="cuda") * 0.02).to(torch.bfloat16)
        mm_tflops = flops_launch / (probe_ms(lambda: torch.mm(pa, pb)) * 1e-3) / 1e12
        probes.update({"dense_gemm_shape": [s_kept, w.d, w.F], "dense_gemm_TFLOP/s": mm_tflops,
                       "roofline_frac_of_dense_gemm": achieved / mm_tflops})
        del pa, pb
    log(f"probes: copy {copy_gbs:.0f} GB/s ({copy_cold_gbs:.0f} cold), dense GEMM "
        f"{probes.get('dense_gemm_TFLOP/s', float('nan')):.0f} TFLOP/s")

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    out = {
        "metric": "MoE-layer tokens/sec (route+permute+grouped FFN+combine); "
                  "% MFMA/HBM roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d, "d_ff": w.F, "E": w.E,
                   "k": w.k, "capacity_factor": w.capacity_factor,
                   "capacity_priority": w.priority,
                   "step": "forward + popularity window + backward", "S_kept": s_kept,
                   "iterations": w.iters},
        "roofline": {"bound": "mfma",
                     "kernel": "rows_gemm_kernel (grouped expert GEMM, FC1 and FC2 launches)",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": load_traffic(w.name),
                     "flops_per_launch": flops_launch,
                     "launch_us": gemm_launch_ms * 1e3,
                     # attainable roofline of one launch: max(flops / peak,
                     # algorithmic bytes / 8 TB/s); bytes = one expert weight
                     # tensor + the packed rows in (d or F wide) and out
                     "bytes_per_launch": gemm_bytes,
                     "attainable_frac": max(flops_launch / (peak * 1e12),
                                            gemm_bytes / (PEAK_HBM_GBS * 1e9))
                                        / (gemm_launch_ms / 1e3)},
        "forward_tokens_per_s": fwd_tok,
        "parts_ms": {**{k: {"warm": v["warm"], "cold": v["cold"]} for k, v in parts.items()},
                     "ep_plan_8_ranks": t_plan, "dispatch_layout_8_ranks": t_layout,
                     "backward_replicated_8_ranks": rep_ms,
                     "cooccurrence_update": t_co, "predict_popularity": t_pred},
        "ep_plan": {"ranks": R_plan, "extra_copies": extra_plan,
                    "max_over_mean_rank_rows": plan_balance},
        "hbm_parts": hbm,
        "warm_ms": warm_ms,
        "probes": probes,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (CPU reference) ...")
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
