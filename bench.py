"""Throughput of the InternVL visual-token compression connector on one MI355X.

A step is one pass of the whole hot path over one batch of the 2B-Flash
workload (16 images x 13 tiles = 208 tiles of 1025 x 1024 bf16 ViT rows,
D = 2048, a 53,760-token prompt): ragged tile offsets, the router (pooling,
gating, quantile decision), the route-first connector run (LayerNorm
statistics, mlp1 or mlp2 per tile) and the sequence compaction.  Inputs and
weights are synthetic (seeded) and resident in HBM before timing starts.

Prints one JSON line.  ``value`` is tiles per second of that step (wall clock
around exactly K steps, synchronised on both sides); ``roofline`` describes
the dominant kernel (HIP events on its launch stream; HBM traffic and MFMA
work from the committed rocprofv3 counter summary); ``cpu_baseline`` times the
CPU oracle on a bounded sample (single-threaded per stage, and one
single-threaded process per core); ``configs`` times the standard connectors
(4B, 14B ragged, 38B; ``run`` with the LayerNorm fold); ``compact_batch`` the
variable-length batch compaction on 64 prompts of the 2B-Flash layout packed
back to back (3.4M tokens), outside the step.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--configs 4b,14b,38b | none]
    python bench.py --profile-workload WL --profile-out DIR   # one workload, for rocprofv3
    python bench.py --counters-summary DIR                    # rocprofv3 CSVs -> profiles/*.md
    python bench.py --stats-summary DIR                       # kernel trace of the step -> profiles/
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "connector tiles/s (+visual tokens/s) at 1 GPU; % of MFMA / HBM peak"
WORKLOAD = "internvl35_2b_flash"
STD_CONFIGS = {"4b": "internvl35_4b_std", "14b": "internvl3_14b_ragged", "38b": "internvl3_38b"}
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_CLOCK_GHZ = 2.4  # the clock the MFMA peak is quoted at
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "vlm_visual_token_amd", "csrc")
CALIB_COPY_KIB = 524288  # one calibration copy: 512 MiB read and 512 MiB written


# ---------------------------------------------------------------------------
# algorithmic work per kernel launch
# ---------------------------------------------------------------------------
def algorithmic(cfg: dict, n64: int | None = None, L_seq: int = 0, Lp: int = 0,
                route_first: bool = True, placed: bool = False) -> dict:
    """{launch name: {"flops": F, "bytes": B}} per launch (None where a kernel
    has no stated figure).  Flops are 2 M N K of the products; bytes are the
    operands read once and the results written once, bf16 activations and
    weights, fp32 statistics (8 bytes per row: mean and rstd).  On the
    route-first Flash step each projector runs on its own tiles only
    (``n64`` tiles take the 64-token path); ``placed``: each chain's last
    product also writes its rows into the compacted sequence (forward_compact)."""
    T, C, D, N = cfg["T"], cfg["C"], cfg["D"], cfg["N"]
    S, S64 = cfg["S"], cfg["S64"]
    H1, H2 = cfg["mlp1_hidden"], cfg["mlp2_hidden"]
    e = 2
    if not cfg["flash"]:
        n64, n256 = 0, T
    elif not route_first:  # both projectors on every tile
        n64, n256 = T, T
    else:
        n256 = T - n64
    x_read = T * N * C * e  # CLS rows are never read
    out = {
        "mlp1_gemm1": dict(flops=2.0 * n256 * S * H1 * 4 * C,
                           bytes=n256 * N * C * e + H1 * 4 * C * e + n256 * S * H1 * e
                           + (n256 * S * 8 if cfg.get("ln_fold") else 0)),
        "mlp1_gemm2": dict(flops=2.0 * n256 * S * D * H1,
                           bytes=n256 * S * H1 * e + D * H1 * e
                           + (2 if placed else 1) * n256 * S * D * e),
        "token_stats": dict(flops=None, bytes=x_read + T * N * 8),
        "ln_stats": dict(flops=None, bytes=T * N * 8 + (n256 * S + n64 * S64) * 8),
        # with the LayerNorm fold the loader only writes each row's statistics
        "shuffle_ln": dict(flops=None, bytes=x_read + (
            (n256 * S + n64 * S64) * 8 if cfg.get("ln_fold")
            else n256 * S * 4 * C * e + n64 * S64 * 16 * C * e)),
        "tile_offsets": dict(flops=None, bytes=None),
    }
    if cfg["flash"]:
        G = cfg["gate_hidden"] * cfg["gate_expansion"]
        out.update({
            "mlp2_gemm1": dict(flops=2.0 * n64 * S64 * H2 * 16 * C,
                               bytes=n64 * N * C * e + H2 * 16 * C * e + n64 * S64 * H2 * e
                               + (n64 * S64 * 8 if cfg.get("ln_fold") else 0)),
            "mlp2_gemm2": dict(flops=2.0 * n64 * S64 * H2 * H2,
                               bytes=2 * n64 * S64 * H2 * e + H2 * H2 * e),
            "mlp2_gemm3": dict(flops=2.0 * n64 * S64 * D * H2,
                               bytes=n64 * S64 * H2 * e + D * H2 * e
                               + (2 if placed else 1) * n64 * S64 * D * e),
            # folded pooling: one pass over a tile's tokens per layer; the first
            # layer's pass also writes each token's LayerNorm moments
            "pool_folded_stats": dict(flops=None, bytes=x_read + T * N * 8),
            "pool_folded": dict(flops=None, bytes=x_read),
            # the query and value folds and the gating products stream their weights
            "pool_query_fold": dict(flops=None, bytes=2 * C * C * e),
            "pool_fold_value": dict(flops=None, bytes=2 * C * C * e),
            # a layer's value fold and the next layer's query fold in one launch
            "pool_fold_value_query": dict(flops=None, bytes=4 * C * C * e),
            "gate_ln_fc1": dict(flops=None, bytes=G * cfg["gate_hidden"] * e),
            "gate_fc1": dict(flops=None, bytes=G * cfg["gate_hidden"] * e),
            "gate_fc2": dict(flops=None, bytes=G * cfg["gate_hidden"] * e),
            # the one-launch Gating: the pooling's last value fold and output
            # projection and the eight block products stream their weights once
            "gating": dict(flops=None, bytes=(2 * C * C + 8 * G * cfg["gate_hidden"]) * e),
            "compact": dict(flops=None, bytes=2 * Lp * D * e + L_seq * 4 * 2 + Lp * 4 * 2),
            # its halves when forward_compact runs it: the index work (ids read;
            # ids, positions and keep map written; a source code per output row)
            # and the row copy
            "compact_index": dict(flops=None, bytes=L_seq * 4 * 4 + Lp * 8),
            "compact_copy": dict(flops=None, bytes=2 * Lp * D * e + Lp * 8),
            # the text rows alone (every output row's source code read): the
            # image rows are the last products' second store
            "compact_copy_text": dict(flops=None, bytes=2 * max(Lp - n256 * S - n64 * S64, 0)
                                      * D * e + Lp * 8),
        })
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _usable_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_tiles(cfg, w, x, O):
    """run (shuffle + LN + mlp1 + mlp2) and route (pooling + gating) of each
    tile in x, one tile at a time; returns per-tile seconds of each."""
    run_s, route_s = [], []
    for i in range(x.shape[0]):
        t0 = time.perf_counter()
        O.connector_run(x[i:i + 1], cfg, w)
        t1 = time.perf_counter()
        O.gating(O.cross_attention_pooling(x[i:i + 1], cfg, w), cfg, w)
        t2 = time.perf_counter()
        run_s.append(t1 - t0)
        route_s.append(t2 - t1)
    return run_s, route_s


def _cpu_worker(bias, tiles, barrier, q):
    """One single-threaded oracle process of the all-core measurement: set-up
    (weights, tiles) untimed, then its tiles timed from a common barrier."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        import synth
        from oracle import connector as O
        cfg = synth.config(WORKLOAD)
        w = synth.make_weights(cfg, gate_bias0=bias)
        x = synth.make_vit_tiles(cfg, tiles)
        barrier.wait()
        t0 = time.perf_counter()
        _oracle_tiles(cfg, w, x, O)
        q.put(time.perf_counter() - t0)


def cpu_baseline(bias: float, n_single: int, per_proc: int, procs: int) -> dict:
    """Single core: run and route timed apart on ``n_single`` sampled tiles,
    the batch-wide steps (quantile, decision, compaction) once over the whole
    batch.  All cores: ``procs`` single-threaded processes on disjoint tiles
    (``per_proc`` each), timed from a common start.  Both scaled to one
    208-tile batch (tile work x T + the batch-wide steps)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import synth
    from oracle import connector as O

    cfg = synth.config(WORKLOAD)
    T = cfg["T"]
    with threadpool_limits(1):
        w = synth.make_weights(cfg, gate_bias0=bias)
        tiles = synth.sample_tiles(T, seed=0, n=max(2, n_single))[:n_single]
        x = synth.make_vit_tiles(cfg, tiles)
        run_s, route_s = _oracle_tiles(cfg, w, x, O)
        del x
        # batch-wide steps over the full batch (gates of the right shape; the
        # work does not depend on their values)
        g0 = np.random.default_rng(0).random(T).astype(np.float32)
        ids, emb = synth.make_sequence(cfg)
        o256 = np.zeros((T, cfg["S"], cfg["D"]), np.float32)
        o64 = np.zeros((T, cfg["S64"], cfg["D"]), np.float32)
        t0 = time.perf_counter()
        _, use = O.decide(g0, cfg)
        O.compact(ids, emb, synth.IMG_CONTEXT, use, o256, o64, cfg["S"], cfg["S64"])
        batch_s = time.perf_counter() - t0
        del o256, o64, emb, w
    tile_s = float(np.mean(run_s) + np.mean(route_s))
    single = T / (tile_s * T + batch_s)

    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(procs)
    q = ctx.Queue()
    ps = []
    for p in range(procs):
        mine = [(p * per_proc + i) % T for i in range(per_proc)]
        ps.append(ctx.Process(target=_cpu_worker, args=(bias, mine, barrier, q)))
    for pr in ps:
        pr.start()
    el = [q.get() for _ in ps]
    for pr in ps:
        pr.join()
    agg_rate = procs * per_proc / max(el)  # tiles/s of run + route on all cores
    aggregate = T / (T / agg_rate + batch_s)
    return {
        "value": aggregate, "unit": "tiles/s", "cores": procs, "kind": "oracle",
        "sample": (f"{procs}-core aggregate: {procs} single-threaded oracle processes x "
                   f"{per_proc} tiles of run (shuffle, LayerNorm, mlp1 and mlp2) + route "
                   f"(pooling, gating), plus the batch-wide quantile, decision and compaction "
                   f"over the full {T}-tile batch ({batch_s:.2f} s, one core); scaled to one "
                   f"{T}-tile batch"),
        "single_core": {"value": single, "unit": "tiles/s", "tiles_sampled": len(tiles),
                        "run_s_per_tile": float(np.mean(run_s)),
                        "route_s_per_tile": float(np.mean(route_s)),
                        "batch_steps_s": batch_s},
        "all_core_tile_rate": agg_rate,
        "nproc": os.cpu_count(), "usable_cores": _usable_cores(), "cpu_model": _cpu_model(),
        "oracle": "numpy float64 (BLAS products, single-threaded via threadpoolctl)",
    }


# ---------------------------------------------------------------------------
# GPU workloads
# ---------------------------------------------------------------------------
def gpu_vit(cfg: dict, torch, seed: int = 0):
    """Seeded ViT rows on the device: z * s_c with z ~ N(0,1) and one
    lognormal(0, 0.5) scale per channel (the standard connectors' recipe)."""
    T, rows, C = cfg["T"], cfg["rows"], cfg["C"]
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    scale = torch.exp(0.5 * torch.randn(C, generator=g, device="cuda"))
    x = torch.empty((T, rows, C), dtype=torch.bfloat16, device="cuda")
    for t0 in range(0, T, 16):
        n = min(16, T - t0)
        x[t0:t0 + n].copy_(torch.randn((n, rows, C), generator=g, device="cuda") * scale)
    return x


def weights_on_gpu(cfg, torch, synth, bias=None):
    w = synth.make_weights(cfg, gate_bias0=bias)
    return {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in w.items()}


class FlashStep:
    """The 2B-Flash step: tile offsets, route + route-first run, compaction."""

    def __init__(self, args, torch, synth, ivc, Connector):
        self.torch, self.ivc, self.synth = torch, ivc, synth
        with open(os.path.join(ROOT, "tests", "golden", "gate_bias.json")) as f:
            bias = json.load(f)["gate_bias0"][WORKLOAD]
        cfg = dict(synth.config(WORKLOAD), pool_mode=args.pool_mode, ln_fold=args.ln_fold)
        self.cfg, self.args = cfg, args
        T = cfg["T"]
        ids, emb = synth.make_sequence(cfg)
        self.L = len(ids)
        self.con = Connector(cfg, weights_on_gpu(cfg, torch, synth, bias), max_tiles=T,
                             max_seq_len=self.L)
        self.x = torch.empty((T, cfg["rows"], cfg["C"]), dtype=torch.bfloat16, device="cuda")
        for t0 in range(0, T, 16):
            self.x[t0:t0 + 16].copy_(torch.from_numpy(
                synth.make_vit_tiles(cfg, range(t0, min(T, t0 + 16)))).to(torch.bfloat16))
        self.ids_d = torch.from_numpy(ids).cuda()
        self.emb_d = torch.from_numpy(emb).to(torch.bfloat16).cuda()
        self.tiles_d = torch.tensor(cfg["tiles"], dtype=torch.int32, device="cuda")
        self.off_d = torch.empty(len(cfg["tiles"]) + 1, dtype=torch.int32, device="cuda")
        self.st_d = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.o256 = torch.empty((T, cfg["S"], cfg["D"]), dtype=torch.bfloat16, device="cuda")
        self.o64 = torch.empty((T, cfg["S64"], cfg["D"]), dtype=torch.bfloat16, device="cuda")
        self.rbuf = None
        self.cbuf = None
        self.stream = torch.cuda.current_stream()

    def step(self):
        torch, cfg, T = self.torch, self.cfg, self.cfg["T"]
        self.ivc.ivc_tile_offsets(self.tiles_d, len(cfg["tiles"]), self.off_d, self.st_d,
                                  self.stream)
        if self.args.run_mode == "routed":
            # route + route-first run + compaction in one call: the compaction's
            # index work and text rows run beside the projector chains, whose
            # last products write the image rows into the compacted sequence
            if self.rbuf is None:
                self.rbuf = dict(
                    gate=torch.empty((T, 2), dtype=torch.float32, device="cuda"),
                    thr=torch.empty(1, dtype=torch.float64, device="cuda"),
                    use64=torch.empty(T, dtype=torch.uint8, device="cuda"), pooled=None,
                    status=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    out256=self.o256, out64=self.o64,
                    ids=torch.empty(self.L, dtype=torch.int32, device="cuda"),
                    pos=torch.empty(self.L, dtype=torch.int32, device="cuda"),
                    keep_map=torch.empty(self.L, dtype=torch.int32, device="cuda"),
                    embeds=torch.empty((self.L, cfg["D"]), dtype=torch.bfloat16, device="cuda"),
                    len=torch.zeros(1, dtype=torch.int64, device="cuda"))
            self.rbuf = self.con.forward_compact(self.x, self.ids_d, self.emb_d,
                                                 self.synth.IMG_CONTEXT, with_pooled=False,
                                                 stream=self.stream, out=self.rbuf)
            self.cbuf = self.rbuf
        else:
            self.rbuf = self.con.route(self.x, with_pooled=False, stream=self.stream,
                                       out=self.rbuf)
            self.con.run(self.x, self.o256, self.o64, stream=self.stream)
            self.cbuf = self.con.compact(self.ids_d, self.emb_d, self.rbuf["use64"], self.o256,
                                         self.o64, self.synth.IMG_CONTEXT, stream=self.stream,
                                         out=self.cbuf)

    def algorithmic(self):
        use64 = self.rbuf["use64"].cpu().numpy()
        Lp = int(self.cbuf["len"].item())
        routed = self.args.run_mode == "routed"
        return algorithmic(self.cfg, int(use64.sum()), self.L, Lp, route_first=routed,
                           placed=routed)

    def close(self):
        self.con.close()


class StdRun:
    """A standard connector's run (a1-a6: tile offsets, LayerNorm statistics,
    mlp1), LayerNorm folded into mlp1's first product."""

    def __init__(self, name, torch, synth, ivc, Connector):
        self.torch, self.ivc = torch, ivc
        cfg = dict(synth.config(name), ln_fold=1)
        self.cfg, self.name = cfg, name
        T = cfg["T"]
        self.con = Connector(cfg, weights_on_gpu(cfg, torch, synth), max_tiles=T)
        self.x = gpu_vit(cfg, torch)
        self.tiles_d = torch.tensor(cfg["tiles"], dtype=torch.int32, device="cuda")
        self.off_d = torch.empty(len(cfg["tiles"]) + 1, dtype=torch.int32, device="cuda")
        self.st_d = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.o256 = torch.empty((T, cfg["S"], cfg["D"]), dtype=torch.bfloat16, device="cuda")
        self.stream = torch.cuda.current_stream()

    def step(self):
        self.ivc.ivc_tile_offsets(self.tiles_d, len(self.cfg["tiles"]), self.off_d, self.st_d,
                                  self.stream)
        self.con.run(self.x, self.o256, None, stream=self.stream)

    def algorithmic(self):
        return algorithmic(self.cfg)

    def close(self):
        self.con.close()


def timed_wall(work, steps, torch):
    """Wall-clock ms of exactly ``steps`` steps, synchronised on both sides."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        work.step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def span_median(work, n, torch, flush=None):
    """Median HIP-event span of n single steps (each after ``flush`` if given)."""
    evs = []
    for i in range(n):
        if flush is not None:
            flush.fill_(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(work.stream)
        work.step()
        e1.record(work.stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def kernel_events(work, steps, torch, ivc, mode: int = 1):
    """Per launch name: mean ms per launch and launches per step, from HIP
    events recorded around each launch on its own stream.  mode 1: the
    projector chains run one after the other (each kernel alone); mode 2:
    they keep their two streams, as in the timed steps.  Returns the table
    and the wall-clock ms per step of the pass."""
    ivc.ivc_profile_reset()
    ivc.ivc_profile_enable(mode)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        work.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    ivc.ivc_profile_enable(0)
    prof = ivc.ivc_profile_read()
    return {k: {"ms_avg": v[0] / v[1], "launches_per_step": v[1] / steps,
                "ms_per_step": v[0] / steps} for k, v in prof.items()}, ms


def annotate(kern: dict, alg: dict, counters: dict | None):
    """Adds TFLOP/s and GB/s from the algorithmic figures, and the committed
    counter readings (traffic, counted MFMA flops) where present."""
    for k, v in kern.items():
        a = alg.get(k, {})
        sec = v["ms_avg"] / 1e3
        if a.get("flops"):
            v["tflops"] = a["flops"] / sec / 1e12
            v["frac_mfma"] = v["tflops"] / PEAK_BF16_TFLOPS
        if a.get("bytes"):
            v["gbs"] = a["bytes"] / sec / 1e9
            v["frac_hbm"] = v["gbs"] / PEAK_HBM_GBS
            v["algorithmic_bytes"] = a["bytes"]
        if counters and k in counters:
            c = counters[k]
            if c.get("traffic_bytes") is not None:
                v["traffic_bytes"] = c["traffic_bytes"]
            if c.get("mfma_flops"):
                v["mfma_flops_counted"] = c["mfma_flops"]
            if c.get("mfma_util") is not None:
                v["mfma_busy"] = c["mfma_util"]
            if c.get("clock_ghz") is not None:
                v["clock_ghz"] = c["clock_ghz"]
            if c.get("duration_us") is not None:
                v["rocprof_us"] = c["duration_us"]


def roofline_of(kern: dict, alg: dict, counters: dict | None) -> dict:
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
    d = kern[dom]
    a = alg.get(dom, {})
    sec = d["ms_avg"] / 1e3
    c = (counters or {}).get(dom, {})
    if a.get("flops"):
        ach = a["flops"] / sec / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                "traffic": c.get("traffic_bytes"),
                "algorithmic_flops_per_launch": a["flops"],
                "mfma_flops_counted": c.get("mfma_flops")}
        if c.get("clock_ghz"):
            # the clock the kernel ran at (counter pass) and the fraction of the
            # peak at that clock (the published peak assumes 2.4 GHz)
            roof["clock_ghz"] = c["clock_ghz"]
            roof["frac_at_clock"] = ach / (PEAK_BF16_TFLOPS * c["clock_ghz"] / PEAK_CLOCK_GHZ)
    else:
        ach = (a.get("bytes") or 0.0) / sec / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": c.get("traffic_bytes")}
    roof["algorithmic_bytes_per_launch"] = a.get("bytes")
    roof["ms_avg"] = d["ms_avg"]
    roof["rocprof_avg_us"] = c.get("duration_us")  # kernel-trace pass of the committed summary
    return roof


class CompactBatch:
    """Batched compaction at serving scale: n_prompts prompts of this
    workload's layout packed back to back (each with its own tiles, routed as
    use64_one routes one batch), one ivc_connector_compact_batch call per
    step.  Rows are copies, so the embedding and feature buffers are
    zero-filled."""

    def __init__(self, con, cfg, n_prompts, use64_one, torch, synth, ivc):
        self.con, self.synth, self.torch = con, synth, torch
        B = n_prompts
        ids, _, cu, to = synth.make_batch_sequences(cfg, [cfg["tiles"]] * B, 0,
                                                    with_embeds=False)
        L, T, D = len(ids), int(to[-1]), cfg["D"]
        self.B, self.L, self.T, self.D, self.S, self.S64 = B, L, T, D, cfg["S"], cfg["S64"]
        self.use = np.tile(use64_one, B).astype(np.uint8)
        dev = "cuda"
        self.ids_d = torch.from_numpy(ids).to(dev)
        self.cu_d = torch.from_numpy(cu).to(dev)
        self.to_d = torch.from_numpy(to).to(dev)
        self.use_d = torch.from_numpy(self.use).to(dev)
        self.emb = torch.zeros((L, D), dtype=torch.bfloat16, device=dev)
        self.o256 = torch.zeros((T, cfg["S"], D), dtype=torch.bfloat16, device=dev)
        self.o64 = torch.zeros((T, cfg["S64"], D), dtype=torch.bfloat16, device=dev)
        n = ivc.ivc_connector_compact_batch_workspace_bytes(con.h, T, L, B)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.out = None
        self.stream = torch.cuda.current_stream()

    def step(self):
        self.out = self.con.compact_batch(self.ids_d, self.cu_d, self.emb, self.to_d, self.use_d,
                                          self.o256, self.o64, self.synth.IMG_CONTEXT,
                                          stream=self.stream, out=self.out, ws=self.ws)

    def out_len(self) -> int:
        return int(self.out["cu"][-1].item())

    def algorithmic(self) -> dict:
        Lp = self.out_len()
        return {"compact_batch": dict(flops=None, bytes=2 * Lp * self.D * 2 + self.L * 4 * 2
                                      + Lp * 4 * 2)}

    def close(self):
        del self.emb, self.o256, self.o64, self.ws, self.out
        self.torch.cuda.empty_cache()


class CompactBatchWork(CompactBatch):
    """The batched compaction of bench.py's figure on a connector of its own
    (for the profiler): 64 prompts of the 2B-Flash layout, every other tile
    routed (half the tiles, as the timed batch routes them)."""

    def __init__(self, args, torch, synth, ivc, Connector, n_prompts=64):
        cfg = dict(synth.config(WORKLOAD), pool_mode=args.pool_mode, ln_fold=args.ln_fold)
        with open(os.path.join(ROOT, "tests", "golden", "gate_bias.json")) as f:
            bias = json.load(f)["gate_bias0"][WORKLOAD]
        self.own = Connector(cfg, weights_on_gpu(cfg, torch, synth, bias), max_tiles=cfg["T"])
        use_one = (np.arange(cfg["T"]) % 2).astype(np.uint8)
        super().__init__(self.own, cfg, n_prompts, use_one, torch, synth, ivc)

    def close(self):
        super().close()
        self.own.close()


def compact_batch_stress(con, cfg, n_prompts, use64_one, torch, synth, ivc) -> dict:
    """The batched compaction timed: 2 warm-up calls, then 10 between events."""
    work = CompactBatch(con, cfg, n_prompts, use64_one, torch, synth, ivc)
    for _ in range(2):
        work.step()
    torch.cuda.synchronize()
    reps = 10
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(work.stream)
    for _ in range(reps):
        work.step()
    ev1.record(work.stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    L, T, S, S64 = work.L, work.T, work.S, work.S64
    Lp = work.out_len()
    assert int(work.out["status"].item()) == 0 and Lp == L - (S - S64) * int(work.use.sum())
    byts = work.algorithmic()["compact_batch"]["bytes"]
    gbs = byts / (ms / 1e3) / 1e9
    res = {"prompts": work.B, "tiles": T, "L": L, "L_out": Lp, "ms": ms, "gbs": gbs,
           "frac_hbm": gbs / PEAK_HBM_GBS, "algorithmic_bytes": byts}
    # the counter reading of a call of the same shape (64 prompts of this
    # layout, half the tiles routed: profile workload compact_batch)
    cc = committed_counters("compact_batch")
    if cc and "compact_batch" in cc and work.B == 64:
        res["traffic_bytes"] = cc["compact_batch"]["traffic_bytes"]
        res["rocprof_us"] = cc["compact_batch"]["duration_us"]
    work.close()
    return res


def std_config_result(name, args, torch, synth, ivc, Connector) -> dict:
    work = StdRun(name, torch, synth, ivc, Connector)
    cfg, T = work.cfg, work.cfg["T"]
    for _ in range(args.warmup):
        work.step()
    ms_wall = timed_wall(work, args.config_steps, torch) / args.config_steps
    ms_med = span_median(work, args.config_steps, torch)
    ms_cold = None
    if args.mall_flush_steps > 0:
        junk = torch.empty(512 << 20, dtype=torch.int16, device="cuda")
        ms_cold = span_median(work, args.mall_flush_steps, torch, flush=junk)
        del junk
    kern, _ = kernel_events(work, min(args.config_steps, 10), torch, ivc)
    alg = work.algorithmic()
    annotate(kern, alg, committed_counters(name))
    flops = sum(a["flops"] for a in alg.values() if a.get("flops"))
    res = {
        "workload": name, "tiles": T, "images": len(cfg["tiles"]), "vit_width": cfg["C"],
        "llm_width": cfg["D"], "ln_fold": True, "steps": args.config_steps,
        "ms_per_run_wall": ms_wall, "ms_per_run_median": ms_med,
        "tiles_per_s": T / (ms_med / 1e3),
        "visual_tokens_per_s": T * cfg["S"] / (ms_med / 1e3),
        "input_vit_tokens_per_s": T * cfg["N"] / (ms_med / 1e3),
        "gemm_tflops": flops / (ms_med / 1e3) / 1e12,
        "kernels": kern,
    }
    if ms_cold is not None:
        res["ms_per_run_mall_flushed"] = ms_cold
        res["tiles_per_s_mall_flushed"] = T / (ms_cold / 1e3)
    work.close()
    del work
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries
# ---------------------------------------------------------------------------
# kernels a launch issues after its first one (merges, scans' later phases,
# the compaction copy): their dispatches belong to the launch before them
AUX_KERNELS = {"k_pool_folded_merge", "k_pool_merge", "k_splitk_reduce", "k_compact_plan",
               "k_compact_map", "k_compact_copy", "k_cbatch_bounds", "k_cbatch_plan",
               "k_cbatch_map", "k_fill_i32"}
# kernels after which the row copy belongs to the same compaction launch
COPY_AFTER = {"k_compact_map", "k_cbatch_map", "k_cbatch_plan"}
# the kernel family each launch name may start with (a check of the alignment)
LAUNCH_FAMILY = {
    "tile_offsets": ("k_tile_offsets",), "token_stats": ("k_token_stats",),
    "ln_stats": ("k_ln_stats",), "shuffle_ln": ("k_shuffle_ln",),
    "mlp1_gemm1": ("k_gemm",), "mlp1_gemm2": ("k_gemm",), "mlp2_gemm1": ("k_gemm",),
    "mlp2_gemm2": ("k_gemm",), "mlp2_gemm3": ("k_gemm",), "pool_kv_gemm": ("k_gemm",),
    "pool_q_proj": ("k_gemm",), "pool_o_proj": ("k_gemm",),
    "pool_query": ("k_broadcast_rows",), "pool_query_fold": ("k_fold_query",),
    "pool_fold_query": ("k_gemm_f32a", "k_fold_query"), "pool_fold_pad": ("k_zero_heads",),
    "pool_folded": ("k_pool_folded",), "pool_folded_stats": ("k_pool_folded",),
    "pool_fold_value": ("k_fold_value", "k_gemm"), "pool_attn": ("k_pool_attn",),
    "pool_fold_value_query": ("k_fold_value_query",),
    "gate_fc1": ("k_gemm",), "gate_ln_fc1": ("k_gemm_f32a", "k_f32a_ln_rows"),
    "gate_fc2": ("k_gemm",), "gate_res_ln": ("k_residual_ln", "k_f32a_ln_rows"),
    "gate_res_ln_head": ("k_residual_ln", "k_f32a_ln_rows"),
    "gating": ("k_gating_fused",),
    "quantile_decide": ("k_quantile_decide",), "route_lists": ("k_route_lists",),
    "compact": ("k_compact_count", "k_set_i64"), "compact_batch": ("k_compact_count",),
    "compact_index": ("k_compact_count", "k_set_i64"), "compact_copy": ("k_compact_copy",),
    "compact_copy_text": ("k_compact_copy_text",),
}


def kernel_base(symbol: str) -> str:
    """'void ivc::k_gemm_dma8<1, true>(...)' -> 'k_gemm_dma8'."""
    s = symbol.split("(")[0]
    s = re.sub(r"<.*", "", s)
    return s.split("::")[-1].split()[-1]


def kernel_template(symbol: str) -> str:
    """'void ivc::k_gemm_dma8<1, true>(...)' -> 'k_gemm_dma8<1, true>'."""
    s = symbol.split("(")[0].strip()
    if s.startswith("void "):
        s = s[5:]
    return s.replace("ivc::", "")


def source_sha(base: str) -> tuple[str, str] | tuple[None, None]:
    """(file, sha256) of the .hip file that defines kernel ``base``, hashed
    together with the local headers it includes."""
    for fn in sorted(os.listdir(CSRC)):
        if not fn.endswith(".hip"):
            continue
        with open(os.path.join(CSRC, fn), "rb") as f:
            src = f.read()
        if re.search(rb"__global__[^;{]*?\b" + base.encode() + rb"\s*\(", src) is None:
            continue
        h = hashlib.sha256(src)
        for inc in re.findall(rb'#include\s+"([^"]+)"', src):
            p = os.path.join(CSRC, inc.decode())
            if os.path.exists(p):
                with open(p, "rb") as f:
                    h.update(f.read())
        return fn, h.hexdigest()
    return None, None


def _read_dispatches(path: str) -> dict:
    """{dispatch id: {"symbol", "grid", "counters": {name: value}, "start", "end"}}
    from a rocprofv3 counter_collection.csv or kernel_trace.csv."""
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            did = int(row["Dispatch_Id"])
            d = out.setdefault(did, {
                "symbol": row["Kernel_Name"], "counters": {},
                "grid": int(row.get("Grid_Size") or row.get("Grid_Size_X") or 0),
                "wg": int(row.get("Workgroup_Size") or row.get("Workgroup_Size_X") or 0)})
            if "Counter_Name" in row:
                d["counters"][row["Counter_Name"]] = float(row["Counter_Value"])
            if "Start_Timestamp" in row:
                d["start"] = int(row["Start_Timestamp"])
                d["end"] = int(row["End_Timestamp"])
    return out


def _read_launches(path: str) -> list[str]:
    names = []
    with open(path, errors="replace") as f:
        for line in f:
            m = re.match(r"\[ivc\]\s+launch (\S+) stream=", line)
            if m:
                names.append(m.group(1))
    return names


def label_dispatches(disp: dict, launches: list[str]) -> dict:
    """Labels each library dispatch with the launch it belongs to: the
    library's trace names every launch in host order, and a launch's first
    dispatch is a kernel outside AUX_KERNELS.  Dispatches of the connector's
    set-up (before the first traced launch) are the surplus at the front."""
    ids = sorted(k for k, d in disp.items() if "ivc::" in d["symbol"])

    def is_head(n: int) -> bool:
        base = kernel_base(disp[ids[n]]["symbol"])
        if base not in AUX_KERNELS:
            return True
        # the row copy is a launch of its own unless the index kernels of its
        # compaction come right before it
        return (base == "k_compact_copy" and n > 0
                and kernel_base(disp[ids[n - 1]]["symbol"]) not in COPY_AFTER)

    heads = [ids[n] for n in range(len(ids)) if is_head(n)]
    skip = len(heads) - len(launches)
    if skip < 0:
        raise ValueError(f"{len(launches)} traced launches but only {len(heads)} dispatches")
    head_label = {}
    for i, name in zip(heads[skip:], launches):
        base = kernel_base(disp[i]["symbol"])
        fam = LAUNCH_FAMILY.get(name)
        if fam is not None and not base.startswith(fam):
            raise ValueError(f"dispatch {i} ({base}) does not fit launch {name}")
        head_label[i] = name
    labels, cur = {}, None
    first = heads[skip] if skip < len(heads) else None
    head_set = set(heads)
    for i in ids:
        if i in head_label:
            cur = head_label[i]
        elif first is None or i < first or i in head_set:
            continue
        labels[i] = cur
    return labels


def _calibration(disp: dict, counter: str) -> float | None:
    """KiB per copy that ``counter`` reads on the trailing 512 MiB
    device-to-device copies (the runtime's copy kernel)."""
    cp = sorted(k for k, d in disp.items() if "copyBuffer" in d["symbol"]
                and counter in d["counters"])
    if not cp:
        return None
    return float(np.median([disp[k]["counters"][counter] for k in cp[-4:]]))


def _find(d: str, suffix: str) -> str | None:
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    return None


def summarize_workload(wdir: str) -> dict:
    """Per (launch, kernel): medians over the dispatches of each pass; per
    launch: the sums over its kernels against the launch's algorithmic
    figures."""
    with open(os.path.join(wdir, "algorithmic.json")) as f:
        meta = json.load(f)
    rows: dict = {}
    passes = {}
    for pname in ("fetch", "write", "trace"):
        pdir = os.path.join(wdir, pname)
        csvp = _find(pdir, "counter_collection.csv") if pname != "trace" else \
            _find(pdir, "kernel_trace.csv")
        logp = os.path.join(wdir, pname + ".log")
        if csvp is None or not os.path.exists(logp):
            continue
        disp = _read_dispatches(csvp)
        labels = label_dispatches(disp, _read_launches(logp))
        passes[pname] = disp
        for i, lab in labels.items():
            d = disp[i]
            key = (lab, kernel_template(d["symbol"]))
            r = rows.setdefault(key, {"n": {}, "vals": {}})
            r["n"][pname] = r["n"].get(pname, 0) + 1
            for cn, cv in d["counters"].items():
                r["vals"].setdefault(cn, []).append(cv)
            if pname == "trace":
                r["vals"].setdefault("duration_ns", []).append(d["end"] - d["start"])
            r["workgroups"] = d["grid"] // d["wg"] if d["wg"] else None
    fetch_cal = _calibration(passes.get("fetch", {}), "FETCH_SIZE")
    write_cal = _calibration(passes.get("write", {}), "WRITE_SIZE")
    fs = CALIB_COPY_KIB / fetch_cal if fetch_cal else None
    ws = CALIB_COPY_KIB / write_cal if write_cal else None
    out = {"workload": meta["workload"], "fetch_scale": fs, "write_scale": ws,
           "calibration_kib": {"FETCH_SIZE": fetch_cal, "WRITE_SIZE": write_cal},
           "kernels": [], "launches": {}}
    for (lab, tmpl), r in sorted(rows.items(), key=lambda kv: kv[0]):
        v = {k: float(np.median(x)) for k, x in r["vals"].items()}
        src, sha = source_sha(kernel_base(tmpl))
        ent = {"launch": lab, "kernel": tmpl, "workgroups": r.get("workgroups"),
               "dispatches": r["n"], "source": src, "source_sha256": sha}
        if "FETCH_SIZE" in v:
            ent["fetch_kib"] = v["FETCH_SIZE"]
        if "WRITE_SIZE" in v:
            ent["write_kib"] = v["WRITE_SIZE"]
        if fs and ws and "fetch_kib" in ent and "write_kib" in ent:
            ent["traffic_bytes"] = (ent["fetch_kib"] * fs + ent["write_kib"] * ws) * 1024
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in v:
            ent["mfma_flops"] = v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        if "SQ_VALU_MFMA_BUSY_CYCLES" in v and v.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; 1024 SIMDs
            ent["mfma_util"] = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / 8 * 1024)
        if "duration_ns" in v:
            ent["duration_us"] = v["duration_ns"] / 1e3
            if v.get("GRBM_GUI_ACTIVE") and v["duration_ns"] >= 50e3:
                # shader clock over the dispatch: GRBM_GUI_ACTIVE (summed over the
                # 8 XCDs) of the counter pass over the kernel-trace duration (for
                # launches of 50 us or more: the counter also covers the dispatch's
                # own start and end, which dominate shorter ones)
                ent["clock_ghz"] = v["GRBM_GUI_ACTIVE"] / 8 / v["duration_ns"]
        out["kernels"].append(ent)
    alg, ev = meta["launches"], meta.get("events", {})
    for ent in out["kernels"]:
        L = out["launches"].setdefault(ent["launch"], {"kernels": [], "sources": {}})
        L["kernels"].append(ent["kernel"])
        L["sources"][ent["kernel"]] = [ent["source"], ent["source_sha256"]]
        for k in ("duration_us", "traffic_bytes", "mfma_flops"):
            if k in ent:
                L[k] = L.get(k, 0.0) + ent[k]
        if ent.get("mfma_util") is not None and ent.get("duration_us", 0) >= \
                L.get("_util_us", -1.0):
            L["mfma_util"], L["_util_us"] = ent["mfma_util"], ent.get("duration_us", 0)
            if ent.get("clock_ghz") is not None:
                L["clock_ghz"] = ent["clock_ghz"]
    for lab, L in out["launches"].items():
        L.pop("_util_us", None)
        a = alg.get(lab, {})
        if lab in ev:
            L["events_us"] = ev[lab] * 1e3
        if a.get("bytes"):
            L["algorithmic_bytes"] = a["bytes"]
            if L.get("traffic_bytes"):
                L["traffic_over_algorithmic"] = L["traffic_bytes"] / a["bytes"]
            if L.get("duration_us"):
                L["gbs"] = a["bytes"] / L["duration_us"] / 1e3
        if a.get("flops"):
            L["algorithmic_flops"] = a["flops"]
            if L.get("duration_us"):
                L["tflops"] = a["flops"] / L["duration_us"] / 1e6
    out["commands"] = [c.replace("{WL}", meta["workload"]) for c in PROFILE_COMMANDS]
    return out


def write_counters_md(summary: dict, path: str) -> None:
    wl = summary["workload"]
    L = [f"# rocprofv3 counters and durations per launch: {wl}", ""]
    L.append("Medians over the profiled dispatches of each pass.  HBM-side traffic: "
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the same counters "
             "read for a 512 MiB device-to-device copy.  MFMA work: "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops; MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES "
             "over (GRBM_GUI_ACTIVE / 8 XCDs) x 1024 SIMDs; GHz: GRBM_GUI_ACTIVE / 8 over the "
             "kernel-trace duration (the shader clock the launch ran at; peaks assume 2.4).  "
             "Durations: the kernel-trace pass "
             "(`us`) and HIP events around each launch in the same run (`us ev`); both passes "
             "run the two projector chains one after the other, so each kernel has the chip "
             "to itself.  Launch names come from the library's own trace (IVC_TRACE=1), "
             "aligned with the dispatches in order; a launch's row sums its kernels.  "
             "FETCH_SIZE counts L2 misses, which the 256 MB memory-side cache may serve "
             "before HBM.")
    L.append("")
    L.append("Commands (`$R` is the repository path, `$OUT` an output directory with "
             "`$OUT/pmc/<workload>` created beforehand; `cd /tmp && export TMPDIR=/tmp` first "
             "for the profiler's own files):")
    L.append("")
    L.append("```")
    L.extend(summary["commands"])
    L.append("```")
    L.append("")
    cal = summary["calibration_kib"]
    L.append(f"Calibration: a 512 MiB copy reads FETCH_SIZE {cal['FETCH_SIZE']} KiB and "
             f"WRITE_SIZE {cal['WRITE_SIZE']} KiB; scale factors "
             f"{summary['fetch_scale']:.4f} (fetch), {summary['write_scale']:.4f} (write).")
    L.append("")

    def f(x, sc=1.0, nd=1):
        return "" if x is None else f"{x * sc:.{nd}f}"
    hdr = ["launch", "kernels", "us", "us ev", "traffic MB", "alg. MB", "traffic/alg",
           "GB/s (alg)", "MFMA GFLOP", "alg. GFLOP", "TFLOP/s", "MFMA busy", "GHz"]
    L.append("| " + " | ".join(hdr) + " |")
    L.append("|" + "---|" * len(hdr))
    order = sorted(summary["launches"].items(), key=lambda kv: -(kv[1].get("duration_us") or 0))
    for lab, x in order:
        util = x.get("mfma_util")
        L.append("| " + " | ".join([
            lab, ", ".join(f"`{k}`" for k in x["kernels"]), f(x.get("duration_us")),
            f(x.get("events_us")), f(x.get("traffic_bytes"), 1e-6),
            f(x.get("algorithmic_bytes"), 1e-6), f(x.get("traffic_over_algorithmic"), 1, 2),
            f(x.get("gbs"), 1, 0), f(x.get("mfma_flops"), 1e-9),
            f(x.get("algorithmic_flops"), 1e-9), f(x.get("tflops"), 1, 0),
            "" if not util else f"{100 * util:.0f}%", f(x.get("clock_ghz"), 1, 2)]) + " |")
    L.append("")
    L.append("Per kernel:")
    L.append("")
    hdr = ["launch", "kernel", "WGs", "us", "fetch KiB", "write KiB", "MFMA GFLOP", "source"]
    L.append("| " + " | ".join(hdr) + " |")
    L.append("|" + "---|" * len(hdr))
    for k in summary["kernels"]:
        L.append("| " + " | ".join([
            k["launch"], f"`{k['kernel']}`", str(k.get("workgroups") or ""),
            f(k.get("duration_us")), f(k.get("fetch_kib"), 1, 0), f(k.get("write_kib"), 1, 0),
            f(k.get("mfma_flops"), 1e-9), k.get("source") or ""]) + " |")
    L.append("")
    L.append("Machine-readable (read by bench.py while each kernel's source, with the local "
             "headers it includes, has the SHA-256 recorded here):")
    L.append("")
    L.append("```json")
    L.append(json.dumps(summary, indent=1, sort_keys=True))
    L.append("```")
    with open(path, "w") as fh:
        fh.write("\n".join(L) + "\n")


def counters_summary(d: str) -> None:
    for wl in sorted(os.listdir(d)):
        wdir = os.path.join(d, wl)
        if not os.path.exists(os.path.join(wdir, "algorithmic.json")):
            continue
        s = summarize_workload(wdir)
        path = os.path.join(ROOT, "profiles", f"counters_{s['workload']}.md")
        write_counters_md(s, path)
        print(f"wrote {path} ({len(s['launches'])} launches)")


def committed_counters(workload: str, path: str | None = None) -> dict | None:
    """{launch name: {"traffic_bytes", "mfma_flops", "mfma_util", "duration_us",
    "clock_ghz"}}
    from the committed summary profiles/counters_<workload>.md, for the
    launches whose kernels' sources are unchanged since the counters were
    taken; None when there is no summary."""
    path = path or os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if m is None:
        return None
    s = json.loads(m.group(1))
    out = {}
    for lab, x in s["launches"].items():
        fresh = all(source_sha(kernel_base(k))[1] == sha
                    for k, (_, sha) in x["sources"].items())
        if fresh:
            out[lab] = {k: x.get(k) for k in ("traffic_bytes", "mfma_flops", "mfma_util",
                                             "duration_us", "clock_ghz")}
    return out


BENCH_STATS_COMMANDS = [
    "timeout -s KILL 300 rocprofv3 --kernel-trace --stats -f csv -d $OUT/bstats -o p "
    "-- python3 $R/bench.py --no-cpu-baseline --mall-flush-steps 0 --compact-prompts 0 "
    "--configs none > $OUT/bstats/bench.json",
    "python3 $R/bench.py --stats-summary $OUT/bstats",
]


def bench_stats_summary(d: str) -> None:
    """profiles/kernel_stats_<workload>_bench.md from a kernel-trace run of
    bench.py's timed step: per (kernel, workgroups) the calls and durations,
    the launch names the committed per-workload summaries give that kernel,
    and the dominant kernel's mean span against bench.py's own event figure."""
    disp = _read_dispatches(_find(d, "kernel_trace.csv"))
    groups: dict = {}
    for x in disp.values():
        key = (kernel_template(x["symbol"]), x["grid"] // x["wg"] if x["wg"] else 0)
        groups.setdefault(key, []).append((x["end"] - x["start"]) / 1e3)
    names: dict = {}
    pdir = os.path.join(ROOT, "profiles")
    summ = None
    for fn in sorted(os.listdir(pdir)):
        if not (fn.startswith("counters_") and fn.endswith(".md")):
            continue
        with open(os.path.join(pdir, fn)) as f:
            m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
        js = json.loads(m.group(1))
        if js["workload"] == WORKLOAD:
            summ = js
        for k in js["kernels"]:
            names.setdefault((k["kernel"], k["workgroups"]), set()).add(
                f"{js['workload']}: {k['launch']}")
    with open(os.path.join(d, "bench.json")) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    roof = line["roofline"]
    L = [f"# rocprofv3 kernel trace of bench.py's timed step: {WORKLOAD}", ""]
    L.append("Every dispatch of the command below grouped by kernel (template instance) "
             "and workgroup count; durations from `--kernel-trace` (the `--stats` file "
             "groups by kernel name only, which merges different products of one GEMM "
             "kernel).  The run times the step as bench.py's default run does (warm-up, "
             "the timed steps, the kernels-alone event pass) and skips the CPU baseline, "
             "the cache-flush pass, the batched compaction and the other workloads.")
    L.append("")
    L.append("`$R` is the repository path, `$OUT` an output directory (`$OUT/bstats` created "
             "beforehand).")
    L.append("")
    L.append("```")
    L.extend(BENCH_STATS_COMMANDS)
    L.append("```")
    L.append("")
    if summ is not None:
        ks = [k for k in summ["kernels"] if k["launch"] == roof["kernel"]]
        W, K = line["warmup"], line["steps"]
        if ks:
            key = (ks[0]["kernel"], ks[0]["workgroups"])
            ids = sorted(i for i, x in disp.items()
                         if (kernel_template(x["symbol"]), x["grid"] // max(x["wg"], 1)) == key)
            du = [(disp[i]["end"] - disp[i]["start"]) / 1e3 for i in ids]
            L.append(f"Dominant kernel `{roof['kernel']}` (`{key[0]}`, {key[1]} workgroups), "
                     f"{len(du)} dispatches: {W} warm-up steps, {K} timed steps, then {K} "
                     f"steps with every kernel alone between HIP events.")
            L.append("")
            if len(du) == W + 2 * K:
                iso = float(np.mean(du[W + K:]))
                L.append(f"- kernels-alone pass: rocprofv3 mean {iso:.1f} us; bench.py's "
                         f"events in the same run {roof['ms_avg'] * 1e3:.1f} us -> "
                         f"{roof['achieved']:.0f} {roof['unit']} "
                         f"({100 * roof['frac']:.1f}% of peak)")
                L.append(f"- timed steps (the two projector chains overlap): rocprofv3 mean "
                         f"{float(np.mean(du[W:W + K])):.1f} us")
            else:
                L.append(f"- all dispatches: rocprofv3 mean {float(np.mean(du)):.1f} us; "
                         f"bench.py's events {roof['ms_avg'] * 1e3:.1f} us")
            L.append(f"- the step: {line['ms_per_step'] * 1e3:.0f} us wall per timed step, "
                     f"{line['value']:.0f} tiles/s")
            L.append("")
    hdr = ["kernel", "WGs", "calls", "mean us", "min us", "max us", "total ms", "launch"]
    L.append("| " + " | ".join(hdr) + " |")
    L.append("|" + "---|" * len(hdr))
    for (k, wg), du in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        L.append("| " + " | ".join([
            f"`{k}`", str(wg), str(len(du)), f"{np.mean(du):.1f}", f"{np.min(du):.1f}",
            f"{np.max(du):.1f}", f"{sum(du) / 1e3:.2f}",
            "; ".join(sorted(names.get((k, wg), [])))]) + " |")
    path = os.path.join(pdir, f"kernel_stats_{WORKLOAD}_bench.md")
    with open(path, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print(f"wrote {path}")


# ---------------------------------------------------------------------------
def calibrate_copy(torch):
    """4 device-to-device copies of 512 MiB (the counters' calibration)."""
    src = torch.empty(256 << 20, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


PROFILE_COMMANDS = [
    "B=\"python3 $R/bench.py --profile-workload {WL} --profile-out $OUT/pmc/{WL}\"",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/pmc/{WL}/fetch "
    "-o p -- $B --steps 2 --warmup 1 2> $OUT/pmc/{WL}/fetch.log",
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE SQ_INSTS_VALU_MFMA_MOPS_BF16 "
    "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -f csv -d $OUT/pmc/{WL}/write -o p "
    "-- $B --steps 2 --warmup 1 2> $OUT/pmc/{WL}/write.log",
    "timeout -s KILL 180 rocprofv3 --kernel-trace --stats -f csv -d $OUT/pmc/{WL}/trace "
    "-o p -- $B --steps 20 --warmup 5 2> $OUT/pmc/{WL}/trace.log",
    "python3 $R/bench.py --counters-summary $OUT/pmc",
]


def profile_workload(args, torch, synth, ivc, Connector):
    """One workload, for the profiler: warm-up, the timed steps, the copy
    calibration, and the algorithmic figures written next to the counters.
    The library's trace (IVC_TRACE=1, on stderr) names every launch."""
    wl = args.profile_workload
    if wl == WORKLOAD:
        work = FlashStep(args, torch, synth, ivc, Connector)
    elif wl == "compact_batch":
        work = CompactBatchWork(args, torch, synth, ivc, Connector)
    else:
        work = StdRun(wl, torch, synth, ivc, Connector)
    for _ in range(args.warmup):
        work.step()
    # per-launch events on: the two projector chains run one after the other,
    # as in the counter passes, so every kernel's span is its own
    kern, ms = kernel_events(work, args.steps, torch, ivc)
    alg = work.algorithmic()
    calibrate_copy(torch)
    os.makedirs(args.profile_out, exist_ok=True)
    with open(os.path.join(args.profile_out, "algorithmic.json"), "w") as f:
        json.dump({"workload": wl, "steps": args.steps, "warmup": args.warmup,
                   "launches": alg, "events": {k: v["ms_avg"] for k, v in kern.items()},
                   "commands": PROFILE_COMMANDS}, f, indent=1)
    work.close()
    print(json.dumps({"workload": wl, "ms_per_step_serialised": ms}))


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default="4b,14b,38b",
                    help="standard connectors also timed (comma list of 4b, 14b, 38b; none)")
    ap.add_argument("--config-steps", type=int, default=50)
    ap.add_argument("--pool-mode", type=int, default=1,
                    help="0: K/V projection + attention, 1: folded pooling (same mathematics)")
    ap.add_argument("--run-mode", choices=["routed", "both"], default="routed",
                    help="routed: decide first, then run only each tile's chosen projector "
                         "(one forward call); both: run mlp1 and mlp2 on every tile, as the "
                         "pages do")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tiles", type=int, default=4,
                    help="tiles timed single-threaded (run and route apart)")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="single-threaded oracle processes of the all-core figure "
                         "(0: the usable cores, at most 16)")
    ap.add_argument("--cpu-tiles-per-proc", type=int, default=2)
    ap.add_argument("--profile-workload", default=None,
                    help="run one workload for rocprofv3 (no other measurement)")
    ap.add_argument("--profile-out", default=None)
    ap.add_argument("--counters-summary", default=None, metavar="DIR",
                    help="write profiles/counters_<workload>.md from rocprofv3 output in DIR")
    ap.add_argument("--stats-summary", default=None, metavar="DIR",
                    help="write profiles/kernel_stats_<workload>_bench.md from a kernel-trace "
                         "run of bench.py in DIR")
    args = ap.parse_args()
    if args.counters_summary:
        counters_summary(args.counters_summary)
        return
    if args.stats_summary:
        bench_stats_summary(args.stats_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(tiles are independent, so several GPUs would each run a whole-image tile range; "
              f"that sharding is not built).",
              file=sys.stderr)
        sys.exit(2)

    # the CPU baseline runs before anything touches the GPU, so its worker
    # processes start from a process without a GPU context
    cpu = None
    if not args.no_cpu_baseline and args.profile_workload is None:
        with open(os.path.join(ROOT, "tests", "golden", "gate_bias.json")) as f:
            bias = json.load(f)["gate_bias0"][WORKLOAD]
        procs = args.cpu_procs or min(16, _usable_cores())
        print(f"# cpu baseline: {args.cpu_tiles} tiles single-threaded, {procs} processes x "
              f"{args.cpu_tiles_per_proc} tiles", file=sys.stderr, flush=True)
        cpu = cpu_baseline(bias, args.cpu_tiles, args.cpu_tiles_per_proc, procs)

    if args.profile_workload is not None:
        os.environ["IVC_TRACE"] = "1"  # read once, at the library's first traced call
    import torch

    import synth
    from vlm_visual_token_amd import Connector, ivc

    if args.profile_workload is not None:
        profile_workload(args, torch, synth, ivc, Connector)
        return

    work = FlashStep(args, torch, synth, ivc, Connector)
    cfg, T, L = work.cfg, work.cfg["T"], work.L
    print(f"# warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        work.step()
    torch.cuda.synchronize()

    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(work.stream)
    for _ in range(args.steps):
        work.step()
    ev1.record(work.stream)
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) * 1e3
    ms_events = ev0.elapsed_time(ev1)
    ms_step = ms_wall / args.steps
    # per-kernel spans: the same steps again with an event pair around every
    # launch and the two projector chains one after the other, so every
    # kernel has the chip to itself (events between overlapping kernels would
    # slow the step and split shared time arbitrarily)
    print(f"# per-kernel events, kernels alone, {args.steps} steps", file=sys.stderr, flush=True)
    kern, ms_iso = kernel_events(work, args.steps, torch, ivc, mode=1)

    # the same steps with the 256 MB memory-side cache (MALL) evicted before
    # each one (a 1 GiB buffer written between steps, outside the timed spans):
    # weights and activations then come from HBM at every step
    ms_cold = None
    if args.mall_flush_steps > 0:
        print(f"# {args.mall_flush_steps} steps after a cache flush each", file=sys.stderr,
              flush=True)
        junk = torch.empty(512 << 20, dtype=torch.int16, device="cuda")
        ms_cold = span_median(work, args.mall_flush_steps, torch, flush=junk)
        del junk
        torch.cuda.empty_cache()

    use64 = work.rbuf["use64"].cpu().numpy()
    Lp = int(work.cbuf["len"].item())
    emitted = int((use64 == 0).sum()) * cfg["S"] + int(use64.sum()) * cfg["S64"]
    alg = work.algorithmic()
    counters = committed_counters(WORKLOAD)  # taken with every kernel alone, too
    annotate(kern, alg, counters)
    roof = roofline_of(kern, alg, counters)

    cb = None
    if args.compact_prompts > 0:
        print(f"# batched compaction, {args.compact_prompts} prompts", file=sys.stderr,
              flush=True)
        cb = compact_batch_stress(work.con, cfg, args.compact_prompts, use64, torch, work.synth,
                                  ivc)
    work.close()
    del work
    torch.cuda.empty_cache()

    configs = {}
    names = [] if args.configs in ("", "none") else args.configs.split(",")
    for n in names:
        print(f"# standard connector {STD_CONFIGS[n]}", file=sys.stderr, flush=True)
        configs[STD_CONFIGS[n]] = std_config_result(STD_CONFIGS[n], args, torch, synth, ivc,
                                                    Connector)

    out = {
        "metric": METRIC,
        "value": T / (ms_step / 1e3),
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
        "ms_per_step_events": ms_events / args.steps,
        "visual_tokens_per_s": emitted / (ms_step / 1e3),
        "input_vit_tokens_per_s": T * cfg["N"] / (ms_step / 1e3),
        "gemm_tflops": sum(a["flops"] for a in alg.values() if a.get("flops"))
        / (ms_step / 1e3) / 1e12,
        "routed_to_64": int(use64.sum()),
        "compacted_len": Lp,
        "roofline": roof,
        "kernels": kern,
        "kernel_events": ("the timed steps again, each launch between a HIP event pair on its "
                          "own stream, projector chains one after the other (every kernel "
                          "alone on the chip)"),
        "ms_per_step_kernel_events": ms_iso,
        "counters_summary": (f"profiles/counters_{WORKLOAD}.md" if counters is not None
                             else None),
        "compact_batch": cb,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    if ms_cold is not None:
        out["ms_per_step_mall_flushed"] = ms_cold
        out["tiles_per_s_mall_flushed"] = T / (ms_cold / 1e3)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
