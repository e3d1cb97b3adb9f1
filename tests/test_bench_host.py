"""Host logic of bench.py: algorithmic work figures, the labelling of
profiler dispatches by the library's launch trace, and the counter summary
round trip.  No GPU, no oracle arithmetic."""
import csv
import json
import os

import pytest

import bench
import synth


def test_algorithmic_flops_match_stated_totals():
    # GEMM work of the workloads: 2B-Flash mlp1 1340 GFLOP and mlp2 2457 GFLOP
    # with both projectors on every tile; 4B mlp1 907 GFLOP; 38B 9771 GFLOP
    c3 = dict(synth.config("internvl35_2b_flash"), ln_fold=1)
    a = bench.algorithmic(c3, route_first=False)
    mlp1 = a["mlp1_gemm1"]["flops"] + a["mlp1_gemm2"]["flops"]
    mlp2 = sum(a[k]["flops"] for k in ("mlp2_gemm1", "mlp2_gemm2", "mlp2_gemm3"))
    assert round(mlp1 / 1e9) == 1340
    assert round(mlp2 / 1e9) == 2457
    c2 = synth.config("internvl35_4b_std")
    a2 = bench.algorithmic(c2)
    assert round((a2["mlp1_gemm1"]["flops"] + a2["mlp1_gemm2"]["flops"]) / 1e9) == 907
    c5 = synth.config("internvl3_38b")
    a5 = bench.algorithmic(c5)
    assert round((a5["mlp1_gemm1"]["flops"] + a5["mlp1_gemm2"]["flops"]) / 1e9) == 9771
    assert "mlp2_gemm1" not in a2 and "pool_folded" not in a5


def test_algorithmic_route_first_splits_tiles():
    c3 = dict(synth.config("internvl35_2b_flash"), ln_fold=1)
    T = c3["T"]
    both = bench.algorithmic(c3, route_first=False)
    rf = bench.algorithmic(c3, n64=104, route_first=True)
    assert rf["mlp1_gemm1"]["flops"] == pytest.approx(both["mlp1_gemm1"]["flops"] * (T - 104) / T)
    assert rf["mlp2_gemm3"]["flops"] == pytest.approx(both["mlp2_gemm3"]["flops"] * 104 / T)
    # one pass over the 208 x 1024 x 1024 bf16 tokens per pooling layer
    assert rf["pool_folded"]["bytes"] == 208 * 1024 * 1024 * 2


def test_kernel_names():
    sym = "void ivc::k_gemm_dma8<1, true>(ivc::GemmOps, float const*, unsigned short*)"
    assert bench.kernel_base(sym) == "k_gemm_dma8"
    assert bench.kernel_template(sym) == "k_gemm_dma8<1, true>"
    assert bench.kernel_base("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    fn, sha = bench.source_sha("k_gemm_dma8")
    assert fn == "k_gemm_dma.hip" and len(sha) == 64
    assert bench.source_sha("k_no_such_kernel") == (None, None)


# A profiled run: the connector's set-up kernels, a torch kernel, the traced
# launches (compaction issues four kernels), then the calibration copies.
_DISPATCHES = [
    ("void ivc::k_widen(void const*, int, float*, long long)", 256),
    ("void ivc::k_ln_fold_weights(unsigned short const*)", 256),
    ("void at::native::elementwise_kernel<128, 4>(int)", 128),
    ("void ivc::k_tile_offsets(int const*, int, int*, int*)", 1024),
    ("void ivc::k_token_stats<1024>(unsigned short const*)", 512),
    ("void ivc::k_ln_stats(float const*)", 256),
    ("void ivc::k_gemm_dma8<1, true>(ivc::GemmOps)", 512),
    ("void ivc::k_gemm_dma8<0, false>(ivc::GemmOps)", 512),
    ("void ivc::k_compact_count(int const*)", 256),
    ("void ivc::k_compact_plan(int const*)", 1024),
    ("void ivc::k_compact_map(int const*)", 256),
    ("void ivc::k_compact_copy<8>(long long const*)", 256),
] + [("__amd_rocclr_copyBuffer", 512)] * 4
_LAUNCHES = ["tile_offsets", "token_stats", "ln_stats", "mlp1_gemm1", "mlp1_gemm2", "compact"]


def _write_pass(d, counters):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size",
                    "Counter_Name", "Counter_Value"])
        for i, (sym, wg) in enumerate(_DISPATCHES):
            for cn, fn in counters.items():
                w.writerow([i + 1, wg * 100, sym, wg, cn, fn(i, sym)])


def _write_trace(d, dur_ns):
    """A kernel-trace pass of the same dispatches, dispatch i lasting dur_ns(i, sym)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size_X", "Kernel_Name", "Workgroup_Size_X",
                    "Start_Timestamp", "End_Timestamp"])
        t = 1000
        for i, (sym, wg) in enumerate(_DISPATCHES):
            w.writerow([i + 1, wg * 100, sym, wg, t, t + dur_ns(i, sym)])
            t += dur_ns(i, sym) + 500


def _write_log(path):
    with open(path, "w") as f:
        f.write("[ivc] create dtype=1 C=1024\n")
        for n in _LAUNCHES:
            f.write(f"[ivc]   launch {n} stream=0x1234\n")


def test_label_dispatches_assigns_aux_kernels_to_their_launch(tmp_path):
    _write_pass(str(tmp_path / "fetch"), {"FETCH_SIZE": lambda i, s: 1.0})
    _write_log(str(tmp_path / "fetch.log"))
    disp = bench._read_dispatches(str(tmp_path / "fetch" / "p_counter_collection.csv"))
    labels = bench.label_dispatches(disp, bench._read_launches(str(tmp_path / "fetch.log")))
    got = {bench.kernel_template(disp[i]["symbol"]): lab for i, lab in labels.items()}
    assert got == {"k_tile_offsets": "tile_offsets", "k_token_stats<1024>": "token_stats",
                   "k_ln_stats": "ln_stats", "k_gemm_dma8<1, true>": "mlp1_gemm1",
                   "k_gemm_dma8<0, false>": "mlp1_gemm2", "k_compact_count": "compact",
                   "k_compact_plan": "compact", "k_compact_map": "compact",
                   "k_compact_copy<8>": "compact"}
    # a launch whose first kernel is of another family is an alignment error
    bad = list(_LAUNCHES)
    bad[3], bad[2] = bad[2], bad[3]
    with pytest.raises(ValueError):
        bench.label_dispatches(disp, bad)
    with pytest.raises(ValueError):
        bench.label_dispatches(disp, _LAUNCHES * 3)


def test_label_dispatches_split_compaction():
    # forward_compact: the index kernels right after the decision, the row copy
    # after the products, as a launch of its own
    disp = {i + 1: {"symbol": sym, "counters": {}} for i, sym in enumerate([
        "void ivc::k_widen(void const*, int, float*, long long)",
        "void ivc::k_quantile_decide(float const*)",
        "void ivc::k_compact_count(int const*)",
        "void ivc::k_compact_plan(int const*)",
        "void ivc::k_compact_map(int const*)",
        "void ivc::k_gemm_dma8<1, true>(ivc::GemmOps)",
        "void ivc::k_compact_copy<4>(long long const*)",
        "void ivc::k_compact_count(int const*)",
        "void ivc::k_compact_plan(int const*)",
        "void ivc::k_compact_map(int const*)",
        "void ivc::k_compact_copy<4>(long long const*)",
    ])}
    launches = ["quantile_decide", "compact_index", "mlp1_gemm1", "compact_copy", "compact"]
    labels = bench.label_dispatches(disp, launches)
    assert [labels.get(i) for i in sorted(disp)] == [
        None, "quantile_decide", "compact_index", "compact_index", "compact_index", "mlp1_gemm1",
        "compact_copy", "compact", "compact", "compact", "compact"]


def test_counter_summary_round_trip(tmp_path):
    wdir = tmp_path / "internvl35_4b_std"
    # fetch reads half of a copy's bytes (scale 2), write reads them all (scale 1)
    _write_pass(str(wdir / "fetch"), {
        "FETCH_SIZE": lambda i, s: 262144.0 if "copyBuffer" in s else 100.0 * (i + 1)})
    _write_pass(str(wdir / "write"), {
        "WRITE_SIZE": lambda i, s: 524288.0 if "copyBuffer" in s else 10.0,
        "SQ_INSTS_VALU_MFMA_MOPS_BF16": lambda i, s: 1000.0 if "gemm" in s else 0.0,
        "SQ_VALU_MFMA_BUSY_CYCLES": lambda i, s: 8192.0 * 512 if "gemm" in s else 0.0,
        "GRBM_GUI_ACTIVE": lambda i, s: 8 * 8192.0})
    # the GEMMs last 100 us in the trace pass, everything else 10 us
    _write_trace(str(wdir / "trace"), lambda i, s: 100000 if "gemm" in s else 10000)
    for p in ("fetch", "write", "trace"):
        _write_log(str(wdir / (p + ".log")))
    cfg = synth.config("internvl35_4b_std")
    with open(wdir / "algorithmic.json", "w") as f:
        json.dump({"workload": "internvl35_4b_std",
                   "launches": bench.algorithmic(dict(cfg, ln_fold=1)),
                   "commands": []}, f)
    s = bench.summarize_workload(str(wdir))
    assert s["fetch_scale"] == pytest.approx(2.0) and s["write_scale"] == pytest.approx(1.0)
    k = {(e["launch"], e["kernel"]): e for e in s["kernels"]}
    g1 = k[("mlp1_gemm1", "k_gemm_dma8<1, true>")]
    # dispatch 7 (index 6): fetch 700 KiB x 2 + write 10 KiB
    assert g1["traffic_bytes"] == pytest.approx((700 * 2 + 10) * 1024)
    assert g1["mfma_flops"] == 512000.0
    assert g1["mfma_util"] == pytest.approx(0.5)
    # 8192 active cycles per XCD over 100 us: 0.08192 GHz; launches shorter
    # than 50 us carry no clock
    assert g1["duration_us"] == pytest.approx(100.0)
    assert g1["clock_ghz"] == pytest.approx(8192 / 100e3)
    assert "clock_ghz" not in k[("ln_stats", "k_ln_stats")]
    assert g1["workgroups"] == 100
    assert s["commands"][0].startswith(
        'B="python3 $R/bench.py --profile-workload internvl35_4b_std --profile-out')
    L = s["launches"]
    # the compaction's four kernels (dispatches 9..12) add up in its launch row
    assert L["compact"]["traffic_bytes"] == pytest.approx(
        sum((100 * i * 2 + 10) * 1024 for i in (9, 10, 11, 12)))
    assert L["mlp1_gemm1"]["traffic_over_algorithmic"] == pytest.approx(
        g1["traffic_bytes"] / bench.algorithmic(dict(cfg, ln_fold=1))["mlp1_gemm1"]["bytes"])
    md = tmp_path / "counters.md"
    bench.write_counters_md(s, str(md))
    c = bench.committed_counters("internvl35_4b_std", str(md))
    assert c["mlp1_gemm1"]["traffic_bytes"] == pytest.approx(g1["traffic_bytes"])
    assert c["mlp1_gemm1"]["clock_ghz"] == pytest.approx(g1["clock_ghz"])
    assert c["compact"]["traffic_bytes"] == pytest.approx(L["compact"]["traffic_bytes"])
    # a launch whose kernel source hash no longer matches drops out
    md.write_text(md.read_text().replace(g1["source_sha256"], "0" * 64))
    c2 = bench.committed_counters("internvl35_4b_std", str(md))
    assert "mlp1_gemm1" not in c2 and "mlp1_gemm2" not in c2 and "compact" in c2


def test_gpus_above_one_exits_with_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_roofline_at_the_measured_clock():
    kern = {"mlp2_gemm1": {"ms_per_step": 0.7, "ms_avg": 0.7},
            "pool_folded": {"ms_per_step": 0.3, "ms_avg": 0.1}}
    alg = {"mlp2_gemm1": {"flops": 875e9, "bytes": 4e8}}
    r = bench.roofline_of(kern, alg, {"mlp2_gemm1": {"clock_ghz": 1.8, "traffic_bytes": 1e9}})
    assert r["kernel"] == "mlp2_gemm1" and r["bound"] == "mfma"
    assert r["achieved"] == pytest.approx(1250.0)
    assert r["frac"] == pytest.approx(0.5)
    # the peak scaled to 1.8 of the 2.4 GHz it is quoted at: 1875 TFLOP/s
    assert r["frac_at_clock"] == pytest.approx(1250.0 / 1875.0)
    assert r["traffic"] == 1e9
    # no counter summary: no clock figures
    r2 = bench.roofline_of(kern, alg, None)
    assert "clock_ghz" not in r2 and "frac_at_clock" not in r2
