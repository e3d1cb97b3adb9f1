"""Helpers for the GPU parity tests: upload seeded workloads, compare results."""
import json
import os
import sys

import numpy as np
import torch

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gate_bias(name):
    with open(os.path.join(GOLDEN, "gate_bias.json")) as f:
        return json.load(f)["gate_bias0"].get(name)


def workload(name, seed=0, **over):
    cfg = dict(synth.config(name, seed))
    cfg.update(over)
    if over:
        P = cfg["P"]
        cfg["N"] = P * P
        cfg["rows"] = cfg["has_cls"] + P * P
        cfg["S"] = (P // 2) ** 2
        cfg["S64"] = (P // 4) ** 2 if cfg["flash"] else 0
    return cfg


def host_gate_bias(cfg):
    return gate_bias(cfg["name"]) if cfg["flash"] else None


def host_weights(cfg, seed=0):
    return synth.make_weights(cfg, seed, gate_bias0=gate_bias(cfg["name"]) if cfg["flash"] else None)


def dev_weights(cfg, w):
    dt = TORCH_DT[cfg["dtype"]]
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(dt).cuda() for k, v in w.items()}


def dev_vit(cfg, seed=0, chunk=16):
    dt = TORCH_DT[cfg["dtype"]]
    T = cfg["T"]
    out = torch.empty((T, cfg["rows"], cfg["C"]), dtype=dt, device="cuda")
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        x = synth.make_vit_tiles(cfg, range(t0, t1), seed)
        out[t0:t1].copy_(torch.from_numpy(x).to(dt))
    return out


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def float_report(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    err = g - o
    rms = float(np.sqrt(np.mean(o * o)))
    return dict(rel_l2=float(np.linalg.norm(err) / max(np.linalg.norm(o), 1e-300)),
                max_abs_over_rms=float(np.abs(err).max() / max(rms, 1e-300)))


# tolerances (relative L2, max |err| / RMS): bf16 outputs 1e-2 and 5e-2; the
# fp32 path (no bf16 rounding of inputs or intermediates, fp32 accumulation
# over K <= 16384) 1e-5 and 1e-4
TOL = {"bf16": (1e-2, 5e-2), "f32": (1e-5, 1e-4)}


def log_margin(what, **vals):
    """Appends one JSON line (test, quantity, measured values) to the file named
    by IVC_PARITY_LOG, if set: the record of how close each parity check sits
    to its bar."""
    path = os.environ.get("IVC_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps(dict(test=test, what=what, **vals)) + "\n")


def assert_close(g, o, dtype, what):
    rep = float_report(g, o)
    rel, mx = TOL[dtype]
    say(f"  {what}: rel_l2={rep['rel_l2']:.3e} max_abs/rms={rep['max_abs_over_rms']:.3e}")
    log_margin(what, dtype=dtype, **rep)
    assert np.isfinite(np.asarray(g)).all(), what + " has non-finite values"
    assert rep["rel_l2"] <= rel, (what, rep)
    assert rep["max_abs_over_rms"] <= mx, (what, rep)
