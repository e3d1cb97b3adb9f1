"""LayerNorm-folded calls larger than the folded products' address range run
as consecutive sub-batches.  With the cap lowered (IVC_FOLD_CHUNK_BYTES) a
small batch takes that path: a Flash connector's forward (route-first run,
moments from the first token pass) must give the same gates, decisions and
chosen rows bit for bit; a standard connector's run the same rows up to the
summation order of the last round's K pieces, whose split depends on the
number of tiles in a call.  Parity with the oracle is covered by the
ln_fold tests."""
import os

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_vit, dev_weights, host_weights, say, workload

pytestmark = pytest.mark.gpu

_KNOB = "IVC_FOLD_CHUNK_BYTES"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vlm_visual_token_amd import ivc
    ivc.load()
    yield
    os.environ.pop(_KNOB, None)
    torch.cuda.synchronize()


def _tile_bytes(cfg):
    return cfg["rows"] * cfg["C"] * 2


def _with_cap(cap, fn):
    os.environ[_KNOB] = str(cap)
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        os.environ.pop(_KNOB, None)
    return out


def _clone(d):
    return {k: (v.clone() if v is not None else None) for k, v in d.items()}


@pytest.mark.parametrize("per", [9, 1])
def test_forward_sub_batches_bit_identical(per):
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=1)
    T = 24
    cfg["tiles"], cfg["T"] = [T], T
    cap = per * _tile_bytes(cfg) + 1  # sub-batches of `per` tiles
    say(f"forward in sub-batches of {per} tiles (T={T})")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T)
    xd = dev_vit(cfg)
    whole = _clone(con.forward(xd))
    torch.cuda.synchronize()
    parts = _with_cap(cap, lambda: _clone(con.forward(xd)))
    for k in ("gate", "thr", "use64", "pooled", "status"):
        assert torch.equal(whole[k], parts[k]), k
    use = whole["use64"].cpu().numpy().astype(bool)
    assert 0 < use.sum() < T
    for t in np.nonzero(~use)[0]:
        assert torch.equal(whole["out256"][t], parts["out256"][t]), f"out256 tile {t}"
    for t in np.nonzero(use)[0]:
        assert torch.equal(whole["out64"][t], parts["out64"][t]), f"out64 tile {t}"


def test_run_sub_batches_standard_connector():
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_4b_std", ln_fold=1)
    T = 24
    cfg["tiles"], cfg["T"] = [T], T
    cap = 9 * _tile_bytes(cfg) + 1
    say(f"4B run in sub-batches of 9 tiles (T={T})")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T)
    xd = dev_vit(cfg)
    whole = con.run(xd)[0].clone()
    torch.cuda.synchronize()
    parts = _with_cap(cap, lambda: con.run(xd)[0].clone())
    a, b = whole.float(), parts.float()
    assert torch.isfinite(b).all()
    rel = ((a - b).norm() / a.norm()).item()
    mx = ((a - b).abs().max() / a.pow(2).mean().sqrt()).item()
    say(f"  rel-L2 {rel:.2e}, max-abs/rms {mx:.2e}")
    assert rel < 2e-3 and mx < 5e-2


def test_forward_compact_sub_batches_bit_identical():
    """forward_compact with the run half in sub-batches (the compaction's index
    work beside the first one): the same outputs bit for bit."""
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=1)
    T = 24
    cfg["tiles"], cfg["T"] = [T], T
    ids, emb = synth.make_sequence(cfg)
    say(f"forward_compact in sub-batches of 10 tiles (T={T}, L={len(ids)})")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T, max_seq_len=len(ids))
    xd = dev_vit(cfg)
    ids_d = torch.from_numpy(ids).cuda()
    emb_d = torch.from_numpy(emb).to(torch.bfloat16).cuda()
    img = synth.IMG_CONTEXT
    whole = _clone(con.forward_compact(xd, ids_d, emb_d, img))
    torch.cuda.synchronize()
    parts = _with_cap(10 * _tile_bytes(cfg) + 1,
                      lambda: _clone(con.forward_compact(xd, ids_d, emb_d, img)))
    for k in ("gate", "thr", "use64", "status", "ids", "pos", "keep_map", "len"):
        assert torch.equal(whole[k], parts[k]), k
    n = int(whole["len"].item())
    assert torch.equal(whole["embeds"][:n], parts["embeds"][:n])


def test_forward_compact_placed_rows_in_sub_batches():
    """The 208-tile 2B-Flash batch in two sub-batches of 104: mlp1's last
    product places its rows in the compacted sequence itself in both, mlp2's
    (104 x 64 rows) runs on the smaller-tile kernel and leaves its rows to the
    row copy after the join.  Everything bit for bit as in one call, where
    both last products place their rows."""
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=1)
    T = cfg["T"]
    ids, emb = synth.make_sequence(cfg)
    say(f"forward_compact in sub-batches of 104 tiles (T={T}, L={len(ids)})")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T, max_seq_len=len(ids))
    xd = dev_vit(cfg)
    ids_d = torch.from_numpy(ids).cuda()
    emb_d = torch.from_numpy(emb).to(torch.bfloat16).cuda()
    img = synth.IMG_CONTEXT
    whole = _clone(con.forward_compact(xd, ids_d, emb_d, img))
    torch.cuda.synchronize()
    parts = _with_cap(104 * _tile_bytes(cfg) + 1,
                      lambda: _clone(con.forward_compact(xd, ids_d, emb_d, img)))
    for k in ("gate", "thr", "use64", "status", "ids", "pos", "keep_map", "len"):
        assert torch.equal(whole[k], parts[k]), k
    n = int(whole["len"].item())
    assert torch.equal(whole["embeds"][:n], parts["embeds"][:n])
    use = whole["use64"].cpu().numpy().astype(bool)
    assert 0 < use.sum() < T
    for t in np.nonzero(~use)[0]:
        assert torch.equal(whole["out256"][t], parts["out256"][t]), f"out256 tile {t}"
    for t in np.nonzero(use)[0]:
        assert torch.equal(whole["out64"][t], parts["out64"][t]), f"out64 tile {t}"
