"""Throughput of the InternVL visual-token compression connector on one MI355X.

A step is one pass of the whole hot path over one batch of the 2B-Flash
workload (16 images x 13 tiles = 208 tiles of 1025 x 1024 bf16 ViT rows,
D = 2048, a 53,760-token prompt): ragged tile offsets, the connector run
(pixel_shuffle + LayerNorm, mlp1, mlp2), the router (pooling, gating,
quantile decision) and the sequence compaction.  Inputs and weights are
synthetic (seeded) and resident in HBM before timing starts.

Prints one JSON line.  ``value`` is tiles per second; ``roofline`` describes
the dominant kernel, timed with HIP events on the launch stream inside the
timed region; ``cpu_baseline`` times the CPU oracle on a bounded sample;
``compact_batch`` times the variable-length batch compaction on 64 prompts of
the same layout packed back to back (3.4M tokens), outside the step.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "connector tiles/s (+visual tokens/s) at 1 GPU; % of MFMA / HBM peak"
WORKLOAD = "internvl35_2b_flash"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def gemm_flops(cfg: dict) -> dict:
    """Algorithmic flops per launch of each GEMM kernel name (2 M N K; per
    launch, summed over the launches of one step when a name repeats)."""
    T, C, D = cfg["T"], cfg["C"], cfg["D"]
    S, S64, N = cfg["S"], cfg["S64"], cfg["N"]
    H1, H2, L = cfg["mlp1_hidden"], cfg["mlp2_hidden"], cfg["pool_layers"]
    return {
        "mlp1_gemm1": 2.0 * T * S * H1 * 4 * C,
        "mlp1_gemm2": 2.0 * T * S * D * H1,
        "mlp2_gemm1": 2.0 * T * S64 * H2 * 16 * C,
        "mlp2_gemm2": 2.0 * T * S64 * H2 * H2,
        "mlp2_gemm3": 2.0 * T * S64 * D * H2,
        "pool_kv_gemm": 2.0 * T * N * 2 * L * C * C,
    }


def hbm_bytes(cfg: dict, L_seq: int, Lp: int) -> dict:
    """Algorithmic HBM bytes per launch of the bandwidth-bound kernels."""
    T, C, D, N = cfg["T"], cfg["C"], cfg["D"], cfg["N"]
    e = 2
    x_read = T * N * C * e  # CLS rows are skipped
    return {
        "shuffle_ln": x_read + T * cfg["S"] * 4 * C * e + T * cfg["S64"] * 16 * C * e,
        "pool_attn": T * N * 2 * C * e,  # one layer's K and V
        "pool_folded": T * N * C * e,  # one layer's pass over the tokens
        "token_stats": x_read + T * N * 8,  # per-token LayerNorm moments
        "ln_stats": T * N * 8 + T * (cfg["S"] + cfg["S64"]) * 8,
        "compact": 2 * Lp * D * e + L_seq * 4 * 2 + Lp * 4 * 2,
    }


# source file of each timed kernel name (the committed traffic figures of a
# kernel are valid only for the source they were measured on)
KERNEL_SOURCE = {
    "mlp1_gemm1": "k_gemm_dma.hip", "mlp1_gemm2": "k_gemm_dma.hip",
    "mlp2_gemm1": "k_gemm_dma.hip", "mlp2_gemm2": "k_gemm_dma.hip",
    "mlp2_gemm3": "k_gemm_dma.hip", "pool_folded": "k_pool_folded.hip",
    "shuffle_ln": "k_loader.hip", "compact": "k_compact.hip", "token_stats": "k_pool_folded.hip",
    "ln_stats": "k_loader.hip",
}


def committed_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from its committed rocprofv3 counter
    summary (profiles/traffic_<kernel>_<workload>.md: FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy's counter reading), or None when there is none or
    the kernel's source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{WORKLOAD}.md")
    src = KERNEL_SOURCE.get(kernel)
    if src is None or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    with open(os.path.join(ROOT, "vlm_visual_token_amd", "csrc", src), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if fields.get("source_sha256") != sha:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, w, seq, n_tiles: int) -> dict:
    """The CPU oracle as it stands, on a bounded sample: the per-tile steps
    (connector run + router pooling and gating) on ``n_tiles`` tiles, plus
    the batch-wide steps (quantile, decision, compaction) on the whole batch;
    scaled to tiles/s for a whole batch."""
    import synth
    from oracle import connector as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    tiles = list(range(n_tiles))
    x = synth.make_vit_tiles(cfg, tiles)
    t0 = time.perf_counter()
    O.connector_run(x, cfg, w)
    gate, _, _, _ = O.connector_route(x, cfg, w)
    t1 = time.perf_counter()
    per_tile = (t1 - t0) / n_tiles
    # batch-wide steps over the whole batch (gate values / features of the
    # right shape; the work does not depend on their values)
    T = cfg["T"]
    g0 = np.resize(gate[:, 0], T).astype(np.float32)
    ids, emb = seq
    o256 = np.zeros((T, cfg["S"], cfg["D"]), np.float32)
    o64 = np.zeros((T, cfg["S64"], cfg["D"]), np.float32)
    t2 = time.perf_counter()
    thr, use = O.decide(g0, cfg)
    O.compact(ids, emb, synth.IMG_CONTEXT, use, o256, o64, cfg["S"], cfg["S64"])
    t3 = time.perf_counter()
    batch_s = per_tile * T + (t3 - t2)
    return {"value": T / batch_s, "unit": "tiles/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_tiles} tiles of run+route ({per_tile:.3f} s/tile) plus quantile, "
                      f"decision and compaction over the full {T}-tile batch "
                      f"({t3 - t2:.2f} s); scaled to one {T}-tile batch"}


def compact_batch_stress(con, cfg, n_prompts, use64_one, torch, synth, ivc) -> dict:
    """Batched compaction at serving scale: n_prompts prompts of this
    workload's layout packed back to back (each with its own tiles, routed as
    the timed batch was), one ivc_connector_compact_batch call per step.
    Rows are copies, so the embedding and feature buffers are zero-filled."""
    B = n_prompts
    ids, _, cu, to = synth.make_batch_sequences(cfg, [cfg["tiles"]] * B, 0, with_embeds=False)
    L, T, D, S, S64 = len(ids), int(to[-1]), cfg["D"], cfg["S"], cfg["S64"]
    use = np.tile(use64_one, B).astype(np.uint8)
    dev = "cuda"
    ids_d = torch.from_numpy(ids).to(dev)
    cu_d = torch.from_numpy(cu).to(dev)
    to_d = torch.from_numpy(to).to(dev)
    use_d = torch.from_numpy(use).to(dev)
    emb = torch.zeros((L, D), dtype=torch.bfloat16, device=dev)
    o256 = torch.zeros((T, S, D), dtype=torch.bfloat16, device=dev)
    o64 = torch.zeros((T, S64, D), dtype=torch.bfloat16, device=dev)
    n = ivc.ivc_connector_compact_batch_workspace_bytes(con.h, T, L, B)
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    out = None
    stream = torch.cuda.current_stream()
    for _ in range(2):
        out = con.compact_batch(ids_d, cu_d, emb, to_d, use_d, o256, o64, synth.IMG_CONTEXT,
                                stream=stream, out=out, ws=ws)
    torch.cuda.synchronize()
    reps = 10
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        con.compact_batch(ids_d, cu_d, emb, to_d, use_d, o256, o64, synth.IMG_CONTEXT,
                          stream=stream, out=out, ws=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    Lp = int(out["cu"][-1].item())
    assert int(out["status"].item()) == 0 and Lp == L - (S - S64) * int(use.sum())
    byts = 2 * Lp * D * 2 + L * 4 * 2 + Lp * 4 * 2
    gbs = byts / (ms / 1e3) / 1e9
    res = {"prompts": B, "tiles": T, "L": L, "L_out": Lp, "ms": ms, "gbs": gbs,
           "frac_hbm": gbs / PEAK_HBM_GBS, "algorithmic_bytes": byts}
    del emb, o256, o64, ws, out
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--ln-fold", type=int, default=1,
                    help="1: fold the projectors' LayerNorm into their first product")
    ap.add_argument("--mall-flush-steps", type=int, default=10,
                    help="also time this many single steps, each after writing 1 GiB to evict "
                         "the memory-side cache (median reported; 0: skip)")
    ap.add_argument("--compact-prompts", type=int, default=64,
                    help="prompts in the batched-compaction measurement (0: skip)")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--pool-mode", type=int, default=1,
                    help="0: K/V projection + attention, 1: folded pooling (same mathematics)")
    ap.add_argument("--run-mode", choices=["routed", "both"], default="routed",
                    help="routed: decide first, then run only each tile's chosen projector (one forward call); "
                         "both: run mlp1 and mlp2 on every tile, as the pages do")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tiles", type=int, default=32)
    ap.add_argument("--kernel-events", choices=["timed", "separate"], default="separate",
                    help="separate: the timed region runs without per-kernel events (the two "
                         "projector chains overlap on two streams) and a second pass of the same "
                         "steps records them (chains serialised, each kernel timed alone); "
                         "timed: events inside the timed region")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run 4 device-to-device copies of 512 MiB (calibration "
                         "for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(tiles are independent, so several GPUs would each run a whole-image tile range; "
              f"that sharding is not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from vlm_visual_token_amd import Connector, ivc

    with open(os.path.join(ROOT, "tests", "golden", "gate_bias.json")) as f:
        bias = json.load(f)["gate_bias0"][WORKLOAD]
    cfg = dict(synth.config(WORKLOAD), pool_mode=args.pool_mode, ln_fold=args.ln_fold)
    T = cfg["T"]
    w = synth.make_weights(cfg, gate_bias0=bias)
    wd = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in w.items()}
    ids, emb = synth.make_sequence(cfg)
    L = len(ids)
    con = Connector(cfg, wd, max_tiles=T, max_seq_len=L)
    del wd
    x = torch.empty((T, cfg["rows"], cfg["C"]), dtype=torch.bfloat16, device="cuda")
    for t0 in range(0, T, 16):
        x[t0:t0 + 16].copy_(torch.from_numpy(synth.make_vit_tiles(cfg, range(t0, min(T, t0 + 16)))).to(torch.bfloat16))
    ids_d = torch.from_numpy(ids).cuda()
    emb_d = torch.from_numpy(emb).to(torch.bfloat16).cuda()
    tiles_d = torch.tensor(cfg["tiles"], dtype=torch.int32, device="cuda")
    off_d = torch.empty(len(cfg["tiles"]) + 1, dtype=torch.int32, device="cuda")
    st_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    o256 = torch.empty((T, cfg["S"], cfg["D"]), dtype=torch.bfloat16, device="cuda")
    o64 = torch.empty((T, cfg["S64"], cfg["D"]), dtype=torch.bfloat16, device="cuda")
    rbuf = None
    cbuf = None
    stream = torch.cuda.current_stream()

    def step():
        nonlocal rbuf, cbuf
        ivc.ivc_tile_offsets(tiles_d, len(cfg["tiles"]), off_d, st_d, stream)
        if args.run_mode == "routed":
            # route + route-first run in one call (the LayerNorm statistics
            # pass runs beside the router)
            if rbuf is None:
                rbuf = dict(gate=torch.empty((T, 2), dtype=torch.float32, device="cuda"),
                            thr=torch.empty(1, dtype=torch.float64, device="cuda"),
                            use64=torch.empty(T, dtype=torch.uint8, device="cuda"), pooled=None,
                            status=torch.zeros(1, dtype=torch.int32, device="cuda"),
                            out256=o256, out64=o64)
            rbuf = con.forward(x, with_pooled=False, stream=stream, out=rbuf)
        else:
            rbuf = con.route(x, with_pooled=False, stream=stream, out=rbuf)
            con.run(x, o256, o64, stream=stream)
        cbuf = con.compact(ids_d, emb_d, rbuf["use64"], o256, o64, synth.IMG_CONTEXT,
                           stream=stream, out=cbuf)

    print(f"# warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(kernel_events: bool):
        ivc.ivc_profile_reset()
        ivc.ivc_profile_enable(kernel_events)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        ivc.ivc_profile_enable(False)
        return ev0.elapsed_time(ev1), ivc.ivc_profile_read()

    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    if args.kernel_events == "timed":
        ms, prof = timed(True)
        ms_ev = None
    else:
        ms, _ = timed(False)
        print(f"# per-kernel event pass ({args.steps} steps)", file=sys.stderr, flush=True)
        ms_ev, prof = timed(True)
    ms_step = ms / args.steps

    # the same steps with the 256 MB memory-side cache (MALL) evicted before
    # each one (a 1 GiB buffer written between steps, outside the timed spans):
    # weights and activations then come from HBM at every step
    ms_cold = None
    if args.mall_flush_steps > 0:
        print(f"# {args.mall_flush_steps} steps after a cache flush each", file=sys.stderr, flush=True)
        junk = torch.empty(512 << 20, dtype=torch.int16, device="cuda")
        evs = []
        for i in range(args.mall_flush_steps):  # all enqueued, one synchronisation
            junk.fill_(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms_cold = float(np.median([a.elapsed_time(b) for a, b in evs]))
        del junk
        torch.cuda.empty_cache()

    use64 = rbuf["use64"].cpu().numpy()
    Lp = int(cbuf["len"].item())
    emitted = int((use64 == 0).sum()) * cfg["S"] + int(use64.sum()) * cfg["S64"]
    tiles_per_s = T / (ms_step / 1e3)

    # roofline of the dominant kernel (largest share of the step's kernel time)
    flops = gemm_flops(cfg)
    hbm = hbm_bytes(cfg, L, Lp)
    if args.run_mode == "routed":
        # each projector runs on its own path's tiles only
        n64 = int(use64.sum())
        for k in ("mlp1_gemm1", "mlp1_gemm2"):
            flops[k] *= (T - n64) / T
        for k in ("mlp2_gemm1", "mlp2_gemm2", "mlp2_gemm3"):
            flops[k] *= n64 / T
        # the loader writes only the chosen path's rows
        e, C = 2, cfg["C"]
        hbm["shuffle_ln"] = (T * cfg["N"] * C * e + (T - n64) * cfg["S"] * 4 * C * e
                             + n64 * cfg["S64"] * 16 * C * e)
    if args.ln_fold:  # the loader reads the rows and writes 8 bytes of statistics per LN row
        e, C = 2, cfg["C"]
        hbm["shuffle_ln"] = T * cfg["N"] * C * e + T * (cfg["S"] + cfg["S64"]) * 8
    kern = {k: {"ms_avg": v[0] / v[1], "launches_per_step": v[1] / args.steps,
                "ms_per_step": v[0] / args.steps} for k, v in prof.items()}
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
    d = kern[dom]
    if dom in flops:
        ach = flops[dom] / (d["ms_avg"] / 1e3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": None}
    else:
        ach = hbm.get(dom, 0.0) / (d["ms_avg"] / 1e3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": None}
    for k, v in kern.items():
        if k in flops:
            v["tflops"] = flops[k] / (v["ms_avg"] / 1e3) / 1e12
        if k in hbm:
            v["gbs"] = hbm[k] / (v["ms_avg"] / 1e3) / 1e9

    roof["traffic"] = committed_traffic(dom)

    cb = None
    if args.compact_prompts > 0:
        print(f"# batched compaction, {args.compact_prompts} prompts", file=sys.stderr, flush=True)
        cb = compact_batch_stress(con, cfg, args.compact_prompts, use64, torch, synth, ivc)

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print(f"# cpu baseline ({args.cpu_tiles} tiles)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, w, (ids, emb), args.cpu_tiles)

    out = {
        "metric": METRIC,
        "value": tiles_per_s,
        "unit": "tiles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded ViT rows, random-init weights, synthetic prompt ids)",
        "config": {"workload": WORKLOAD, "tiles": T, "images": len(cfg["tiles"]),
                   "vit_tokens_per_tile": cfg["N"], "vit_width": cfg["C"], "llm_width": cfg["D"],
                   "seq_len": L, "pool_mode": "kv" if args.pool_mode == 0 else "folded",
                   "run_mode": args.run_mode, "ln_fold": bool(args.ln_fold),
                   "parallelism": "single GPU"},
        "visual_tokens_per_s": emitted / (ms_step / 1e3),
        "input_vit_tokens_per_s": T * cfg["N"] / (ms_step / 1e3),
        "routed_to_64": int(use64.sum()),
        "compacted_len": Lp,
        "compact_batch": cb,
        "roofline": roof,
        "kernels": kern,
        "kernel_events": ("separate pass, projector chains serialised"
                          if args.kernel_events == "separate" else "inside the timed region"),
        "cpu_baseline": cpu,
    }
    if ms_ev is not None:
        out["ms_per_step_event_pass"] = ms_ev / args.steps
    if ms_cold is not None:
        out["ms_per_step_mall_flushed"] = ms_cold
        out["tiles_per_s_mall_flushed"] = T / (ms_cold / 1e3)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
