"""The merged router launches against the separate launches of the same
arithmetic: a layer's value fold with the next layer's query fold in one
launch, and the last layer's value fold as the one-launch Gating's first
phase (IVC_FOLD_MERGED=0 selects the separate launches).  Gates, threshold,
decisions and pooled vectors must be bit-identical, on batch sizes that leave
ragged row blocks, with padding masks, with 64- and 32-wide heads, with the
Gating in one launch and launch per product, and on consecutive calls that
share a workspace (the counters of an earlier call never count).  Parity of
either form with the oracle is covered by the route tests."""
import os

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_vit, dev_weights, host_weights, say, workload

pytestmark = pytest.mark.gpu

_KNOBS = ("IVC_FOLD_MERGED", "IVC_GATING_FUSED")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vlm_visual_token_amd import ivc
    ivc.load()
    yield
    for k in _KNOBS:
        os.environ.pop(k, None)
    torch.cuda.synchronize()


def _route(con, xd, valid, env):
    for k in _KNOBS:
        os.environ.pop(k, None)
    os.environ.update(env)
    try:
        r = con.route(xd, valid=valid)
        torch.cuda.synchronize()
    finally:
        for k in _KNOBS:
            os.environ.pop(k, None)
    return {k: v.cpu().numpy() for k, v in r.items() if v is not None}


def _same(a, b):
    for k in ("gate", "thr", "use64", "pooled", "status"):
        assert np.array_equal(a[k], b[k]), k
    assert int(a["status"][0]) == 0


def _vit(cfg, T):
    if T <= 100:
        return dev_vit(cfg)
    # values need not come from synth: both forms read the same device tensor
    g = torch.Generator(device="cuda")
    g.manual_seed(T)
    return torch.randn((T, cfg["rows"], cfg["C"]), generator=g, device="cuda").to(torch.bfloat16)


@pytest.mark.parametrize("gating_one_launch", [True, False])
@pytest.mark.parametrize("T,padded", [(1, False), (13, True), (100, False), (208, False),
                                      (600, False)])
def test_fold_merged_matches_separate(T, padded, gating_one_launch):
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    cfg["tiles"], cfg["T"] = [T], T
    say(f"merged folds: T={T} padded={padded} gating one launch={gating_one_launch}")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T)
    xd = _vit(cfg, T)
    valid = (torch.from_numpy(synth.make_valid_tokens(cfg, seed=T)).cuda() if padded else None)
    env = {} if gating_one_launch else {"IVC_GATING_FUSED": "0"}
    merged = _route(con, xd, valid, env)
    apart = _route(con, xd, valid, dict(env, IVC_FOLD_MERGED="0"))
    _same(merged, apart)
    # again on the same workspace: this call's counters start from what the
    # previous one left
    _same(_route(con, xd, valid, env), apart)
    say(f"  routed {int(merged['use64'].sum())}/{T}, thr {float(merged['thr'][0]):.6f}")


@pytest.mark.parametrize("H", [16, 8])
def test_fold_merged_head_widths(H):
    """C = 512: heads of 32 (H = 16) and 64 (H = 8) channels."""
    from vlm_visual_token_amd import Connector
    cfg = workload("tiny_flash_f32", dtype="bf16", C=512, D=256, mlp1_hidden=256,
                   mlp2_hidden=256, pool_heads=H, gate_hidden=512, pool_mode=1)
    cfg["name"] = "small_bf16_router"
    say(f"merged folds: C=512 H={H} T={cfg['T']}")
    w = synth.make_weights(cfg)
    con = Connector(cfg, dev_weights(cfg, w), max_tiles=cfg["T"])
    xd = torch.from_numpy(synth.make_vit(cfg)).to(torch.bfloat16).cuda()
    merged = _route(con, xd, None, {})
    apart = _route(con, xd, None, {"IVC_FOLD_MERGED": "0"})
    _same(merged, apart)


def test_fold_merged_smaller_call_after_larger():
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    T = 64
    cfg["tiles"], cfg["T"] = [T], T
    say("merged folds: T=64 then T=7 on one workspace")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T)
    xd = dev_vit(cfg)
    big = _route(con, xd, None, {})
    small = _route(con, xd[:7].contiguous(), None, {})
    _same(small, _route(con, xd[:7].contiguous(), None, {"IVC_FOLD_MERGED": "0"}))
    _same(big, _route(con, xd, None, {"IVC_FOLD_MERGED": "0"}))
