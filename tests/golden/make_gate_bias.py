"""Writes tests/golden/gate_bias.json: the gating classifier's class-0 bias for
each Flash workload, chosen so that about half of the tiles have
gate[:, 0] >= 0.5.

It runs only the CPU oracle: with the class-0 bias at 0 it computes the logit
gap z0 - z1 = log(p0 / p1) of every tile and stores minus its median.

    python tests/golden/make_gate_bias.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import connector as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gate_bias.json")


def gap_median(name: str, seed: int = 0) -> float:
    cfg = synth.config(name, seed)
    w = synth.make_weights(cfg, seed, gate_bias0=0.0)
    gaps = []
    for t0 in range(0, cfg["T"], 8):
        x = synth.make_vit_tiles(cfg, range(t0, min(cfg["T"], t0 + 8)), seed)
        p = O.gating(O.cross_attention_pooling(x, cfg, w), cfg, w)
        gaps.extend(np.log(p[:, 0] / p[:, 1]).tolist())
    return float(np.median(gaps))


def main():
    out = {}
    for name in ("tiny_flash_f32", "internvl35_2b_flash"):
        out[name] = -gap_median(name)
        print(name, out[name], flush=True)
    with open(OUT, "w") as f:
        json.dump({"seed": 0, "gate_bias0": out}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
