"""Derive the gate-bias exponent of the Mixtral-shaped workload.

The workload asks for a skewed gate whose most popular expert receives about
35% of all routing slots.  The bias is b[e] = -s * ln(rank(e)); this script
bisects s on the workload's own seeded x and W_gate, routing with the CPU
reference only, until the top expert's share of the T*k slots is 0.35 to
within 0.005, and writes s to workloads/calibration.json.

Run:  python -m oracle.calibrate
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import workloads  # noqa: E402
from oracle import moe_oracle as orc  # noqa: E402

TARGET, TOL = 0.35, 0.005


def top_share(w, x, w_gate, s):
    b = workloads.gate_bias(w, 0, zipf_s=s)
    logits = orc.router_logits(x, w_gate, b)
    idx, _ = orc.topk_gate(logits, w.k)
    slots = orc.assign_slots(idx, w.E, orc.capacity(w.T, w.k, w.E, 0.0))
    return slots["counts_raw"].max() / float(w.T * w.k), slots["counts_raw"]


def main():
    w = workloads.scaled(workloads.workloads()["mixtral_shaped"], zipf_s=None)
    x = workloads.make_x(w)
    w_gate = workloads.make_w_gate(w)
    lo, hi = 0.0, 4.0
    s = None
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        share, counts = top_share(w, x, w_gate, mid)
        print(f"s={mid:.5f} top share={share:.4f}", flush=True)
        if abs(share - TARGET) <= TOL / 4:
            s = mid
            break
        if share < TARGET:
            lo = mid
        else:
            hi = mid
    if s is None:
        s = mid
    s = round(s, 4)
    share, counts = top_share(w, x, w_gate, s)
    assert abs(share - TARGET) <= TOL, share
    path = os.path.join(os.path.dirname(workloads.__file__), "calibration.json")
    with open(path, "w") as f:
        json.dump({"mixtral_shaped_zipf_s": s, "top_share": round(float(share), 5),
                   "counts_raw": [int(c) for c in counts],
                   "written_by": "python -m oracle.calibrate"}, f, indent=1)
        f.write("\n")
    print("wrote", path, s, share)


if __name__ == "__main__":
    main()
