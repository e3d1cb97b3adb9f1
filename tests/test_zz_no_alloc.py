"""ivc_connector_compact_noalloc (compaction with its scratch in the library's
fixed device array, no workspace, nothing allocated) against
ivc_connector_compact on the same inputs: every output bit-exact, on two
calls in a row, the second with a smaller input, then a call past the
array's stated limits (rejected on the host)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def con():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vlm_visual_token_amd import Connector, ivc
    ivc.load()
    cfg = synth.config("tiny_flash_f32")
    w = synth.make_weights(cfg)
    c = Connector(cfg, {k: torch.from_numpy(v).cuda() for k, v in w.items()}, max_tiles=4096,
                  max_seq_len=262144)
    yield c
    torch.cuda.synchronize()
    c.close()


def _case(cfg, T, n_text, seed):
    """A prompt of T tiles' IMG_CONTEXT runs (S slots each) with n_text text
    tokens spread before, between and after them; random features; about
    half of the tiles routed."""
    rng = np.random.default_rng(seed)
    S, S64, D = cfg["S"], cfg["S64"], cfg["D"]
    cuts = np.sort(rng.integers(0, n_text + 1, size=T))
    parts, prev = [], 0
    for t in range(T):
        parts.append(rng.integers(0, 151936, size=cuts[t] - prev))
        parts.append(np.full(S, synth.IMG_CONTEXT))
        prev = cuts[t]
    parts.append(rng.integers(0, 151936, size=n_text - prev))
    ids = np.concatenate(parts).astype(np.int32)
    L = len(ids)
    d = dict(ids=torch.from_numpy(ids).cuda(),
             emb=torch.randn((L, D), generator=torch.Generator().manual_seed(seed)).cuda(),
             o256=torch.randn((T, S, D), generator=torch.Generator().manual_seed(seed + 1)).cuda(),
             o64=torch.randn((T, S64, D), generator=torch.Generator().manual_seed(seed + 2)).cuda(),
             use=torch.from_numpy((rng.random(T) < 0.5).astype(np.uint8)).cuda())
    return L, T, d


def _outs(L, D):
    return dict(ids=torch.full((L,), -7, dtype=torch.int32, device="cuda"),
                pos=torch.full((L,), -7, dtype=torch.int32, device="cuda"),
                keep=torch.full((L,), -7, dtype=torch.int32, device="cuda"),
                emb=torch.full((L, D), float("nan"), device="cuda"),
                len=torch.full((1,), -7, dtype=torch.int64, device="cuda"),
                st=torch.zeros(1, dtype=torch.int32, device="cuda"))


def _noalloc(con, L, T, d, o, stream):
    from vlm_visual_token_amd import ivc
    ivc.ivc_connector_compact_noalloc(con.h, d["ids"], d["emb"], L, synth.IMG_CONTEXT, d["use"],
                                      d["o256"], d["o64"], T, o["ids"], o["pos"], o["keep"],
                                      o["emb"], o["len"], o["st"], stream)


def _with_ws(con, L, T, d, o, stream):
    from vlm_visual_token_amd import ivc
    ivc.ivc_connector_compact(con.h, d["ids"], d["emb"], L, synth.IMG_CONTEXT, d["use"], d["o256"],
                              d["o64"], T, o["ids"], o["pos"], o["keep"], o["emb"], o["len"],
                              o["st"], con.ws, con.ws_bytes, stream)


def _same(a, b, what):
    for k in ("ids", "pos", "keep", "len", "st"):
        assert torch.equal(a[k], b[k]), (what, k)
    n = int(b["len"].item())
    assert torch.equal(a["emb"][:n].view(torch.int32), b["emb"][:n].view(torch.int32)), (what, "emb")


def test_noalloc_matches_workspace_form_two_calls(con):
    cfg = con.cfg
    stream = torch.cuda.current_stream()
    L1, T1, d1 = _case(cfg, 3000, 150000, 11)  # 198,000 tokens
    L2, T2, d2 = _case(cfg, 37, 500, 12)       # a smaller second call
    say(f"compact_noalloc: call 1 L={L1} T={T1}, call 2 L={L2} T={T2}")
    a1, b1 = _outs(L1, cfg["D"]), _outs(L1, cfg["D"])
    a2, b2 = _outs(L2, cfg["D"]), _outs(L2, cfg["D"])
    _noalloc(con, L1, T1, d1, a1, stream)
    _noalloc(con, L2, T2, d2, a2, stream)
    torch.cuda.synchronize()
    _with_ws(con, L1, T1, d1, b1, stream)
    _with_ws(con, L2, T2, d2, b2, stream)
    torch.cuda.synchronize()
    _same(a1, b1, "call 1")
    _same(a2, b2, "call 2")
    for o, (L, T, d) in ((a1, (L1, T1, d1)), (a2, (L2, T2, d2))):
        routed = int(d["use"].sum().item())
        assert int(o["st"].item()) == 0
        assert int(o["len"].item()) == L - (cfg["S"] - cfg["S64"]) * routed
    # and again after the workspace form ran in between (the array keeps the
    # last call's contents; each call writes what it reads first)
    c1 = _outs(L1, cfg["D"])
    _noalloc(con, L1, T1, d1, c1, stream)
    torch.cuda.synchronize()
    _same(c1, b1, "call 1 repeated")


def test_noalloc_rejects_beyond_its_limits(con):
    from vlm_visual_token_amd import ivc
    cfg = con.cfg
    L, T, d = _case(cfg, 4, 10, 13)
    o = _outs(L, cfg["D"])
    with pytest.raises(ivc.IvcError) as e:
        ivc.ivc_connector_compact_noalloc(con.h, d["ids"], d["emb"], 262145, synth.IMG_CONTEXT,
                                          d["use"], d["o256"], d["o64"], T, o["ids"], o["pos"],
                                          o["keep"], o["emb"], o["len"], o["st"], None)
    assert e.value.status == 2
    with pytest.raises(ivc.IvcError) as e:
        ivc.ivc_connector_compact_noalloc(con.h, d["ids"], d["emb"], L, synth.IMG_CONTEXT,
                                          d["use"], d["o256"], d["o64"], 4097, o["ids"], o["pos"],
                                          o["keep"], o["emb"], o["len"], o["st"], None)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert int(o["len"].item()) == -7  # nothing was enqueued
