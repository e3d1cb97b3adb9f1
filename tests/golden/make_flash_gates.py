"""Writes tests/golden/flash_gates.json: the CPU oracle's gate probabilities
for every tile of the 2B-Flash workload (16 images x 13 tiles, seed 0, the
class-0 bias of gate_bias.json), its rel_quantile threshold and its own
routing decisions.

The GPU parity tests compare the library's gates with these on all 208 tiles
(|dp| <= 2e-3) and its decisions with the oracle's independent ones on every
tile farther than 1e-3 from either threshold ([4B-Flash] section 4, inference
decision; [2B-Flash] routing decision).  It runs only the oracle, one process
per worker with BLAS limited to one thread.

    python tests/golden/make_flash_gates.py [--workers 8]
"""
import argparse
import json
import os
import sys

os.environ.setdefault("OMP_NUM_THREADS", "1")
os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")
os.environ.setdefault("MKL_NUM_THREADS", "1")

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import connector as O  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "flash_gates.json")
WORKLOAD = "internvl35_2b_flash"


def _bias() -> float:
    with open(os.path.join(HERE, "gate_bias.json")) as f:
        return json.load(f)["gate_bias0"][WORKLOAD]


def _gates(tiles):
    cfg = synth.config(WORKLOAD, 0)
    w = synth.make_weights(cfg, 0, gate_bias0=_bias())
    x = synth.make_vit_tiles(cfg, tiles, 0)
    return O.gating(O.cross_attention_pooling(x, cfg, w), cfg, w)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    cfg = synth.config(WORKLOAD, 0)
    T = cfg["T"]
    chunks = [list(range(t0, min(T, t0 + 4))) for t0 in range(0, T, 4)]
    if args.workers > 1:
        from multiprocessing import get_context
        with get_context("spawn").Pool(args.workers) as pool:
            parts = pool.map(_gates, chunks)
    else:
        parts = [_gates(c) for c in chunks]
    gate = np.concatenate(parts, axis=0).astype(np.float32)  # the form the GPU emits
    thr, use = O.decide(gate[:, 0], cfg)
    out = {"workload": WORKLOAD, "seed": 0, "gate_bias0": _bias(), "T": T,
           "rel_quantile": cfg["rel_quantile"], "abs_threshold": cfg["abs_threshold"],
           "threshold": float(thr), "use64": [int(u) for u in use],
           "gate": [[float(a), float(b)] for a, b in gate]}
    with open(OUT, "w") as f:
        json.dump(out, f)
        f.write("\n")
    print(f"{T} tiles, threshold {thr:.6f}, routed {int(use.sum())}")


if __name__ == "__main__":
    main()
