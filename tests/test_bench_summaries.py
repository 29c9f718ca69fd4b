"""bench.py without a GPU: its counter summaries on synthetic rocprofv3 CSV
files (the HBM-traffic scaling by the calibration copy, the MFMA utilization
arithmetic: busy share of SIMD cycles, clock, executed flops), and the
refusal of more than one GPU."""
import csv
import json
import types

import pytest

import bench

COUNTER_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
                  "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
                  "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
                  "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]

KERNELS = [
    "void moe::rows_gemm_kernel<128, 256, true, 0, 0, true, true>(moe::RowsArgs)",
    "void moe::rows_gemm_kernel<128, 256, true, 1, 0, false, true>(moe::RowsArgs)",
    "void moe::rows_gemm_kernel<128, 256, false, 2, 0, true, false>(moe::RowsArgs)",
    "void moe::rows_gemm_kernel<128, 256, false, 1, 0, false, false>(moe::RowsArgs)",
    "void moe::wgrad_kernel<256, 256, false>(moe::WgradArgs)",
    "void moe::wgrad_kernel<256, 256, true>(moe::WgradArgs)",
]


def write_counters(path, dispatches):
    """dispatches: list of (kernel name, duration ns, {counter: value})"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        t = 1000
        for i, (name, ns, counters) in enumerate(dispatches):
            for c, v in counters.items():  # one row per dispatch and counter
                w.writerow({k: 0 for k in COUNTER_FIELDS} | {
                    "Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": c,
                    "Counter_Value": v, "Start_Timestamp": t, "End_Timestamp": t + ns})
            t += ns + 500


@pytest.fixture
def out_root(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_mfma_summary_arithmetic(tmp_path, out_root):
    simds, xcds = 1024, 8
    ns, ghz, busy_share, pad = 100_000, 2.2, 0.30, 1.109
    cfg = {"workload": "uniform_cf125", "d_model": 1024, "d_ff": 4096, "S_kept": 8192}
    alg = 2.0 * 1024 * 4096 * 8192
    cycles = ns * ghz  # per XCD
    counters = {"GRBM_GUI_ACTIVE": cycles * xcds,
                "SQ_VALU_MFMA_BUSY_CYCLES": busy_share * simds * cycles,
                "SQ_INSTS_VALU_MFMA_MOPS_BF16": alg * pad / 512}
    other = {"GRBM_GUI_ACTIVE": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 0.0,
             "SQ_INSTS_VALU_MFMA_MOPS_BF16": 0.0}
    # the gather/scatter-fused forward's launches must not be counted
    disp = [(k, ns, counters) for k in KERNELS for _ in range(2)]
    disp.append(("void moe::rows_gemm_kernel<128, 256, true, 0, 1, true, true>(moe::RowsArgs)", 7, other))
    cpath, apath, bpath = tmp_path / "c.csv", tmp_path / "a.csv", tmp_path / "b.json"
    write_counters(cpath, disp)
    with open(apath, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Simd_Count", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Name": "cpu", "Simd_Count": 0, "Num_Xcc": 0})
        w.writerow({"Name": "gfx950", "Simd_Count": simds, "Num_Xcc": xcds})
    bpath.write_text("progress\n" + json.dumps({"config": cfg}) + "\n")
    bench.summarize_mfma(types.SimpleNamespace(summarize_mfma=[str(cpath), str(apath), str(bpath)],
                                               workload="uniform_cf125", command="cmd"))
    text = (out_root / "profiles" / "expert_gemms_uniform_cf125_mfma_utilization.md").read_text()
    rec = json.loads(text.split("mfma-json: ")[1])
    assert [r["role"] for r in rec["rows"]] == [role for _, role in bench.GEMM_ROLES]
    for r in rec["rows"]:
        assert r["dispatches"] == 2
        assert r["busy"] == pytest.approx(busy_share)
        assert r["ghz"] == pytest.approx(ghz)
        assert r["flops"] / r["alg"] == pytest.approx(pad)
        assert r["us"] == pytest.approx(ns / 1e3)
    assert "| FC1 forward (ReLU) |" in text and "30.0%" in text


def test_mfma_summary_needs_all_six_products(tmp_path, out_root):
    counters = {"GRBM_GUI_ACTIVE": 8.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1.0,
                "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1.0}
    cpath, apath, bpath = tmp_path / "c.csv", tmp_path / "a.csv", tmp_path / "b.json"
    write_counters(cpath, [(k, 1000, counters) for k in KERNELS[:4]])
    apath.write_text("Name,Simd_Count,Num_Xcc\ngfx950,1024,8\n")
    bpath.write_text(json.dumps({"config": {"workload": "uniform_cf125", "d_model": 64,
                                            "d_ff": 64, "S_kept": 64}}) + "\n")
    with pytest.raises(SystemExit):
        bench.summarize_mfma(types.SimpleNamespace(
            summarize_mfma=[str(cpath), str(apath), str(bpath)], workload="uniform_cf125",
            command=""))


def test_traffic_summary_scales_by_the_copy(tmp_path, out_root):
    copy = "__amd_rocclr_copyBuffer"
    fc1, fc2 = KERNELS[0], KERNELS[1]
    fix = "void moe::rows_fixup_kernel<128, 256, 1, 0>(moe::RowsArgs)"
    gib_kib = (1 << 30) / 1024

    def run(counter, copy_reading, fc1_v, fc2_v, fix_v):
        disp = [(copy, 10, {counter: copy_reading}),
                (fc1, 10, {counter: fc1_v}), (fc2, 10, {counter: fc2_v}), (fix, 10, {counter: fix_v}),
                (fc1, 10, {counter: fc1_v}), (fc2, 10, {counter: fc2_v}), (fix, 10, {counter: fix_v})]
        p = tmp_path / f"{counter}.csv"
        write_counters(p, disp)
        return str(p)

    # FETCH_SIZE reads 60% of a copy's bytes (scale 1/0.6), WRITE_SIZE all of them
    fs = 1 / 0.6
    fpath = run("FETCH_SIZE", gib_kib * 0.6, 1000.0, 2000.0, 100.0)
    wpath = run("WRITE_SIZE", gib_kib, 300.0, 400.0, 50.0)
    # route / permute / combine kernels in the same runs (two dispatches each,
    # readings differing, so the per-call mean is checked)
    part_kernels = {"void moe::route_tile_kernel<64, 16, 8, 1, 1, 4, 128, 7>(...)": (10.0, 1.0),
                    "moe::rank_hist_kernel(...)": (2.0, 3.0),
                    "moe::scan_kernel(...)": (0.5, 0.25),
                    "_ZN3moe13gather_kernelIDF16bEEvPKT_PKi": (20.0, 30.0),
                    "_ZN3moe14combine_kernelIDF16bEEvPKT_PKfPKiPS1_iiib": (40.0, 8.0)}
    for counter, path, col in (("FETCH_SIZE", fpath, 0), ("WRITE_SIZE", wpath, 1)):
        rows = list(csv.DictReader(open(path, newline="")))
        extra = []
        for name, vals in part_kernels.items():
            extra += [(name, 10, {counter: vals[col]}), (name, 10, {counter: 3 * vals[col]})]
        write_counters(path, [(r["Kernel_Name"], 10, {counter: float(r["Counter_Value"])})
                              for r in rows] + extra)
    bench.summarize_traffic(types.SimpleNamespace(summarize_traffic=[fpath, wpath],
                                                  workload="uniform_cf125", command="cmd"))
    text = (out_root / "profiles" / "rows_gemm_uniform_cf125_hbm_traffic.md").read_text()
    rec = json.loads(text.split("traffic-json: ")[1])
    assert rec["fetch_scale"] == pytest.approx(fs)
    assert rec["write_scale"] == pytest.approx(1.0)
    b1 = (1000.0 * fs + 300.0) * 1024
    b2 = ((2000.0 + 100.0) * fs + 400.0 + 50.0) * 1024  # FC2 owns the fixup after it
    assert rec["traffic_bytes_per_launch"] == pytest.approx((b1 + b2) / 2)
    assert rec["gemm_source_sha256"] == bench.gemm_source_hash()
    assert bench.load_traffic("uniform_cf125") == pytest.approx((b1 + b2) / 2)
    ptext = (out_root / "profiles" / "route_permute_combine_uniform_cf125_hbm_traffic.md").read_text()
    prec = json.loads(ptext.split("parts-traffic-json: ")[1])
    per = {n: 2 * (v[0] * fs + v[1]) * 1024 for n, v in part_kernels.items()}  # mean of 1x and 3x
    keys = list(part_kernels)
    want = {"route": per[keys[0]], "permute": per[keys[1]] + per[keys[2]] + per[keys[3]],
            "combine": per[keys[4]]}
    for k, v in want.items():
        assert prec["bytes_per_call"][k] == pytest.approx(v), k
    assert bench.load_parts_traffic("uniform_cf125") == pytest.approx(prec["bytes_per_call"])


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
