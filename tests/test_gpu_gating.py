"""The one-launch Gating (the pooling's last output projection, the four
residual blocks and the classifier head in one kernel) against the
launch-per-product form of the same arithmetic: gates, threshold, decisions
and pooled vectors bit-identical, on batch sizes that leave ragged row tiles,
with padding masks, on both pooling forms, and on consecutive calls that
share a workspace (the phase counters of an earlier call never count).
Parity of either form with the oracle is covered by the route tests."""
import os

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_vit, host_weights, say, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vlm_visual_token_amd import ivc
    ivc.load()
    yield
    os.environ.pop("IVC_GATING_FUSED", None)
    torch.cuda.synchronize()


def _route(con, xd, valid, fused: bool):
    if fused:
        os.environ.pop("IVC_GATING_FUSED", None)
    else:
        os.environ["IVC_GATING_FUSED"] = "0"
    try:
        r = con.route(xd, valid=valid)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("IVC_GATING_FUSED", None)
    return {k: v.cpu().numpy() for k, v in r.items() if v is not None}


def _same(a, b):
    for k in ("gate", "thr", "use64", "pooled", "status"):
        assert np.array_equal(a[k], b[k]), k
    assert int(a["status"][0]) == 0


@pytest.mark.parametrize("T,padded,pool_mode", [
    (1, False, 1), (13, True, 1), (100, False, 1), (208, False, 1), (13, False, 0),
    (17, True, 0)])
def test_gating_one_launch_matches_per_product(T, padded, pool_mode):
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=pool_mode)
    cfg["tiles"], cfg["T"] = [T], T
    say(f"one-launch gating: T={T} padded={padded} pool_mode={pool_mode}")
    w = host_weights(cfg)
    from tests.gpu_util import dev_weights
    con = Connector(cfg, dev_weights(cfg, w), max_tiles=T)
    xd = dev_vit(cfg)
    valid = (torch.from_numpy(synth.make_valid_tokens(cfg, seed=T)).cuda() if padded else None)
    one = _route(con, xd, valid, True)
    per = _route(con, xd, valid, False)
    _same(one, per)
    # again on the same workspace: this call's counters start from what the
    # previous one left
    again = _route(con, xd, valid, True)
    _same(again, per)
    say(f"  routed {int(one['use64'].sum())}/{T}, thr {float(one['thr'][0]):.6f}")


def test_gating_one_launch_smaller_call_after_larger():
    from vlm_visual_token_amd import Connector
    from tests.gpu_util import dev_weights
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    T = 64
    cfg["tiles"], cfg["T"] = [T], T
    say("one-launch gating: T=64 then T=7 on one workspace")
    w = host_weights(cfg)
    con = Connector(cfg, dev_weights(cfg, w), max_tiles=T)
    xd = dev_vit(cfg)
    big = _route(con, xd, None, True)
    small = _route(con, xd[:7].contiguous(), None, True)
    small_ref = _route(con, xd[:7].contiguous(), None, False)
    _same(small, small_ref)
    big_ref = _route(con, xd, None, False)
    _same(big, big_ref)


def test_gating_one_launch_large_batch():
    """600 tiles (38 row blocks, the last one ragged; 6,072 workgroups over
    ten phases): many more workgroups than fit on the chip at once."""
    from vlm_visual_token_amd import Connector
    from tests.gpu_util import dev_weights
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    T = 600
    cfg["tiles"], cfg["T"] = [T], T
    say("one-launch gating: T=600")
    w = host_weights(cfg)
    con = Connector(cfg, dev_weights(cfg, w), max_tiles=T)
    g = torch.Generator(device="cuda")
    g.manual_seed(600)
    # values need not come from synth: both forms read the same device tensor
    xd = torch.randn((T, cfg["rows"], cfg["C"]), generator=g, device="cuda").to(torch.bfloat16)
    one = _route(con, xd, None, True)
    per = _route(con, xd, None, False)
    _same(one, per)

