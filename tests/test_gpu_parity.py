"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: permutation, routing decisions, compaction indices and positions are
bit-exact (decisions compared on the GPU's own gate values); bf16 float
outputs within relative L2 1e-2 and max-abs 5e-2 x RMS; fp32 outputs within
1e-5 / 1e-4 x RMS; gate probabilities within 2e-3 absolute.  Large workloads
are checked on 16 sampled tiles (first, last and 14 drawn), the batch-wide
steps (quantile, decisions, compaction) on every tile.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import connector as O
from tests.gpu_util import (GOLDEN, TORCH_DT, assert_close, dev_vit, dev_weights, host_gate_bias,
                            host_weights, log_margin, say, to_np, workload)

pytestmark = pytest.mark.gpu

GATE_TOL = 2e-3
BAND = 1e-3  # tiles whose gate[:,0] is this close to a threshold are not compared for decisions


def assert_gates(gate, e_gate, what="gate"):
    """Gate probabilities within GATE_TOL absolute of the oracle's."""
    dg = float(np.abs(np.asarray(gate, np.float64) - np.asarray(e_gate, np.float64)).max())
    say(f"  {what} max abs diff {dg:.3e}")
    log_margin(what, max_abs=dg, tol=GATE_TOL)
    assert dg <= GATE_TOL, (what, dg)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vlm_visual_token_amd import ivc
    ivc.load()
    yield
    torch.cuda.synchronize()


def _connector(cfg, w_host, max_tiles, max_seq=0):
    from vlm_visual_token_amd import Connector
    return Connector(cfg, dev_weights(cfg, w_host), max_tiles=max_tiles, max_seq_len=max_seq)


# ---------------------------------------------------------------------------
# pixel shuffle: bit-exact permutation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,P,C,T,has_cls", [
    ("f32", 8, 64, 5, 1), ("bf16", 8, 64, 3, 0), ("bf16", 32, 1024, 3, 1), ("bf16", 32, 3200, 2, 1),
    ("f32", 4, 4, 7, 1), ("bf16", 16, 8, 9, 1)])
@pytest.mark.parametrize("r", [2, 4])
def test_pixel_shuffle_bit_exact(dtype, P, C, T, has_cls, r):
    from vlm_visual_token_amd import ivc
    say(f"pixel_shuffle dtype={dtype} P={P} C={C} T={T} cls={has_cls} r={r}")
    g = torch.Generator().manual_seed(P * 1000 + C + r)
    x = torch.randn((T, has_cls + P * P, C), generator=g).to(TORCH_DT[dtype])
    xd = x.cuda()
    Q = P // r
    out = torch.full((T, Q * Q, r * r * C), float("nan"), dtype=xd.dtype, device="cuda")
    ivc.ivc_pixel_shuffle(1 if dtype == "bf16" else 0, xd, T, P, C, has_cls, r, out)
    torch.cuda.synchronize()
    exp = O.pixel_shuffle(O.token_grid(x.float().numpy(), P, has_cls), r)
    got = out.float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), exp.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("dtype,P,C,T,has_cls", [("f32", 8, 4, 5, 1), ("bf16", 32, 1024, 2, 1),
                                                  ("bf16", 16, 8, 3, 0)])
@pytest.mark.parametrize("r,version,order", [(2, 1, "direct"), (4, 1, "direct"), (4, 2, "twice_r2"),
                                             (4, 1, "twice_r2")])
def test_pixel_shuffle_variants_bit_exact(dtype, P, C, T, has_cls, r, version, order):
    from vlm_visual_token_amd import ivc
    say(f"pixel_shuffle variant dtype={dtype} P={P} C={C} T={T} r={r} v{version} {order}")
    g = torch.Generator().manual_seed(7 * P + C + r + version)
    x = torch.randn((T, has_cls + P * P, C), generator=g).to(TORCH_DT[dtype])
    xd = x.cuda()
    Q = P // r
    out = torch.full((T, Q * Q, r * r * C), float("nan"), dtype=xd.dtype, device="cuda")
    ivc.ivc_pixel_shuffle(1 if dtype == "bf16" else 0, xd, T, P, C, has_cls, r, out,
                          ps_version=version, shuffle64_order=ivc.SHUFFLE64_ORDERS.index(order))
    torch.cuda.synchronize()
    G = O.token_grid(x.float().numpy(), P, has_cls)
    exp = O.pixel_shuffle(G, 2, version) if r == 2 else O.shuffle64(G, order, version)
    got = out.float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), exp.astype(np.float32).view(np.uint32))


# ---------------------------------------------------------------------------
# tiny Flash workload, fp32: everything, every tile
# ---------------------------------------------------------------------------
def _tiny_all(valid=None, poison=False):
    cfg = workload("tiny_flash_f32")
    w = host_weights(cfg)
    x = synth.make_vit(cfg)
    if poison:
        x[:, 0, :] = np.nan
        if valid is not None:
            for t in range(cfg["T"]):
                x[t, 1 + valid[t]:, :] = np.nan
    return cfg, w, x


def test_tiny_run_matches_oracle():
    cfg, w, x = _tiny_all()
    say("tiny run")
    con = _connector(cfg, w, cfg["T"])
    o256, o64 = con.run(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    e256, e64 = O.connector_run(x, cfg, w)
    assert_close(to_np(o256), e256, "f32", "out256")
    assert_close(to_np(o64), e64, "f32", "out64")


@pytest.mark.parametrize("version,order", [(1, "direct"), (2, "twice_r2"), (1, "twice_r2")])
def test_tiny_run_index_variants_match_oracle(version, order):
    cfg = workload("tiny_flash_f32", ps_version=version, shuffle64_order=order)
    w = host_weights(cfg)
    x = synth.make_vit(cfg)
    say(f"tiny run ps_version={version} order={order}")
    con = _connector(cfg, w, cfg["T"])
    o256, o64 = con.run(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    e256, e64 = O.connector_run(x, cfg, w)
    assert_close(to_np(o256), e256, "f32", "out256")
    assert_close(to_np(o64), e64, "f32", "out64")


@pytest.mark.parametrize("padded", [False, True])
def test_tiny_route_matches_oracle(padded):
    cfg = workload("tiny_flash_f32")
    valid = synth.make_valid_tokens(cfg, seed=4) if padded else None
    cfg, w, x = _tiny_all(valid, poison=padded)
    say(f"tiny route padded={padded}")
    con = _connector(cfg, w, cfg["T"])
    vd = torch.from_numpy(valid).cuda() if padded else None
    r = con.route(torch.from_numpy(x).cuda(), valid=vd)
    torch.cuda.synchronize()
    assert int(r["status"].item()) == 0
    gate = r["gate"].cpu().numpy()
    e_gate, e_thr, e_use, e_pooled = O.connector_route(x, cfg, w, valid)
    assert_close(to_np(r["pooled"]), e_pooled, "f32", "pooled")
    assert_gates(gate, e_gate)
    # decisions on the GPU's own gates: bit-exact
    thr, use = O.decide(gate[:, 0], cfg)
    assert float(r["thr"].item()) == thr
    assert np.array_equal(r["use64"].cpu().numpy(), use)
    # and on independent gates, away from the thresholds
    far = (np.abs(e_gate[:, 0] - e_thr) > 1e-3) & (np.abs(e_gate[:, 0] - 0.5) > 1e-3)
    assert np.array_equal(r["use64"].cpu().numpy()[far], e_use[far])


def test_tiny_compact_matches_oracle():
    cfg, w, x = _tiny_all()
    say("tiny compact")
    ids, emb = synth.make_sequence(cfg)
    con = _connector(cfg, w, cfg["T"], len(ids))
    xd = torch.from_numpy(x).cuda()
    o256, o64 = con.run(xd)
    r = con.route(xd)
    c = con.compact(torch.from_numpy(ids).cuda(), torch.from_numpy(emb).cuda(), r["use64"], o256,
                    o64, synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    use = r["use64"].cpu().numpy()
    assert 0 < use.sum() < cfg["T"], "workload should route some but not all tiles"
    _check_compact(cfg, ids, emb, use, o256, o64, c)


def _check_compact(cfg, ids, emb, use, o256, o64, c):
    ref = O.compact(ids, emb, synth.IMG_CONTEXT, use, to_np(o256), to_np(o64), cfg["S"], cfg["S64"])
    assert int(c["status"].item()) == 0 and ref["status"] == 0
    n = int(c["len"].item())
    assert n == ref["out_len"] == len(ids) - (cfg["S"] - cfg["S64"]) * int(use.sum())
    assert np.array_equal(c["ids"].cpu().numpy(), ref["out_ids"])
    assert np.array_equal(c["pos"].cpu().numpy(), ref["out_pos"])
    assert np.array_equal(c["keep_map"].cpu().numpy(), ref["keep_map"])
    got = c["embeds"][:n].float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref["out_embeds"][:n].astype(np.float32).view(np.uint32))


# ---------------------------------------------------------------------------
# bf16 tiny shapes: MFMA GEMMs with ragged row tails
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 5, 11])
def test_bf16_small_ragged_run(T):
    cfg = workload("tiny_flash_f32", dtype="bf16")
    cfg = dict(cfg, T=T, tiles=[T], name="tiny_bf16")
    w = synth.make_weights(cfg)
    x = synth.make_vit_tiles(cfg, range(T))
    say(f"bf16 small run T={T}")
    con = _connector(cfg, w, T)
    o256, o64 = con.run(torch.from_numpy(x).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    e256, e64 = O.connector_run(x, cfg, w)
    assert_close(to_np(o256), e256, "bf16", "out256")
    assert_close(to_np(o64), e64, "bf16", "out64")


# ---------------------------------------------------------------------------
# full-size workloads, sampled tiles
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["internvl35_4b_std", "internvl3_14b_ragged", "internvl3_38b"])
def test_standard_connector_sampled(name):
    cfg = workload(name)
    say(f"{name}: T={cfg['T']} C={cfg['C']} D={cfg['D']}")
    w = host_weights(cfg)
    con = _connector(cfg, w, cfg["T"])
    xd = dev_vit(cfg)
    o256, _ = con.run(xd)
    torch.cuda.synchronize()
    tiles = synth.sample_tiles(cfg["T"])
    x = synth.make_vit_tiles(cfg, tiles)
    e256, _ = O.connector_run(x, cfg, w)
    assert_close(to_np(o256[tiles]), e256, "bf16", f"{name} out256")


def test_ragged_tile_offsets():
    from vlm_visual_token_amd import ivc
    cfg = workload("internvl3_14b_ragged")
    tiles = np.array(cfg["tiles"], np.int32)
    say(f"tile offsets B={len(tiles)}")
    td = torch.from_numpy(tiles).cuda()
    off = torch.empty(len(tiles) + 1, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ivc.ivc_tile_offsets(td, len(tiles), off, st)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), O.tile_offsets(tiles))
    assert int(st.item()) == 0
    assert int(off[-1].item()) == cfg["T"]
    big = torch.full((3000,), 5, dtype=torch.int32, device="cuda")
    off = torch.empty(3001, dtype=torch.int32, device="cuda")
    ivc.ivc_tile_offsets(big, 3000, off, st)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), np.arange(3001) * 5)
    neg = torch.tensor([3, -1, 2], dtype=torch.int32, device="cuda")
    ivc.ivc_tile_offsets(neg, 3, off, st)
    torch.cuda.synchronize()
    assert int(st.item()) & ivc.IVC_DEV_ERR_TILE_COUNT


def test_flash_workload_end_to_end():
    cfg = workload("internvl35_2b_flash")
    say(f"2B-Flash: T={cfg['T']}")
    w = host_weights(cfg)
    ids, emb = synth.make_sequence(cfg)
    con = _connector(cfg, w, cfg["T"], len(ids))
    xd = dev_vit(cfg)
    o256, o64 = con.run(xd)
    r = con.route(xd)
    c = con.compact(torch.from_numpy(ids).cuda(), torch.from_numpy(emb).to(torch.bfloat16).cuda(),
                    r["use64"], o256, o64, synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    say("  gpu done")
    gate = r["gate"].cpu().numpy()
    use = r["use64"].cpu().numpy()
    # batch-wide steps on every tile, on the GPU's gates: bit-exact
    thr, e_use = O.decide(gate[:, 0], cfg)
    assert float(r["thr"].item()) == thr
    assert np.array_equal(use, e_use)
    frac = use.mean()
    say(f"  routed fraction {frac:.3f}")
    assert 0.2 < frac < 0.8
    emb_bf = synth.to_bf16_exact(emb)
    _check_compact(cfg, ids, emb_bf, use, o256, o64, c)
    # float outputs on sampled tiles, plus the tiles nearest each threshold
    g0 = gate[:, 0].astype(np.float64)
    near = {int(np.argmin(np.abs(g0 - thr))), int(np.argmin(np.abs(g0 - 0.5)))}
    tiles = sorted(set(synth.sample_tiles(cfg["T"], n=12)) | near)
    x = synth.make_vit_tiles(cfg, tiles)
    e256, e64 = O.connector_run(x, cfg, w)
    assert_close(to_np(o256[tiles]), e256, "bf16", "out256")
    assert_close(to_np(o64[tiles]), e64, "bf16", "out64")
    e_gate, _, _, e_pooled = O.connector_route(x, cfg, w)
    assert_close(to_np(r["pooled"][tiles]), e_pooled, "bf16", "pooled")
    assert_gates(gate[tiles], e_gate)


@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 13, 100, 208, 999, 1024, 1025, 5000])
def test_route_decide_bit_exact(T):
    # the quantile + decision step on many gate sets, ties included
    from vlm_visual_token_amd import ivc
    say(f"route_decide T={T}")
    rng = np.random.default_rng(T)
    for trial in range(4):
        p0 = rng.random(T).astype(np.float32)
        if trial == 1:
            p0 = (np.round(p0 * 8) / 8).astype(np.float32)   # many ties
        if trial == 2:
            p0[:] = np.float32(0.5)
        if trial == 3:
            p0 = (0.5 + (p0 - 0.5) * 1e-6).astype(np.float32)  # values straddling 0.5
        gate = np.stack([p0, 1 - p0], axis=1).astype(np.float32)
        gd = torch.from_numpy(gate).cuda()
        thr_d = torch.empty(1, dtype=torch.float64, device="cuda")
        use_d = torch.empty(T, dtype=torch.uint8, device="cuda")
        ivc.ivc_route_decide(gd, T, 0.1, 0.5, thr_d, use_d)
        torch.cuda.synchronize()
        thr, use = O.decide(p0, {"rel_quantile": 0.1, "abs_threshold": 0.5})
        assert float(thr_d.item()) == thr, (trial, float(thr_d.item()), thr)
        assert np.array_equal(use_d.cpu().numpy(), use), trial


# ---------------------------------------------------------------------------
# folded pooling (key/value projections folded out of the token pass)
# ---------------------------------------------------------------------------
def _small_bf16_router(pool_mode, C=512, H=8):
    cfg = workload("tiny_flash_f32", dtype="bf16", C=C, D=256, mlp1_hidden=256,
                   mlp2_hidden=256, pool_heads=H, gate_hidden=C, pool_mode=pool_mode)
    cfg["name"] = "small_bf16_router"
    return cfg


# Gating with a wider hidden layer (expansion 2: W1 [2h, h], W2 [h, 2h], each
# stored with its own padded row stride), folded and K/V pooling
@pytest.mark.parametrize("pool_mode", [1, 0])
def test_router_gate_expansion(pool_mode):
    cfg = dict(_small_bf16_router(pool_mode), gate_expansion=2)
    w = synth.make_weights(cfg)
    x = synth.make_vit(cfg)
    say(f"router gate expansion 2, pool_mode {pool_mode}")
    r = _connector(cfg, w, cfg["T"]).route(torch.from_numpy(x).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    assert int(r["status"].item()) == 0
    e_gate, _, _, e_pooled = O.connector_route(x, cfg, w)
    assert_close(to_np(r["pooled"]), e_pooled, "bf16", "pooled")
    assert_gates(r["gate"].cpu().numpy(), e_gate)
    thr, use = O.decide(r["gate"].cpu().numpy()[:, 0], cfg)
    assert float(r["thr"].item()) == thr
    assert np.array_equal(r["use64"].cpu().numpy(), use)


# (C, H): head widths 64, 32 and 128 of the fused query projection + key fold;
# head width 256 takes the separate query projection and key-fold products
@pytest.mark.parametrize("C,H", [(512, 8), (512, 16), (1024, 8), (1024, 4)])
@pytest.mark.parametrize("padded", [False, True])
def test_folded_pool_small_matches_oracle_and_kv(padded, C, H):
    cfg = _small_bf16_router(1, C, H)
    w = synth.make_weights(cfg)
    x = synth.make_vit(cfg)
    valid = synth.make_valid_tokens(cfg, seed=9) if padded else None
    if padded:
        x[:, 0, :] = np.nan
        for t in range(cfg["T"]):
            x[t, 1 + valid[t]:, :] = np.nan
    say(f"folded small padded={padded} C={C} H={H}")
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    vd = torch.from_numpy(valid).cuda() if padded else None
    rf = _connector(cfg, w, cfg["T"]).route(xd, valid=vd)
    rk = _connector(dict(cfg, pool_mode=0), w, cfg["T"]).route(xd, valid=vd)
    torch.cuda.synchronize()
    assert int(rf["status"].item()) == 0
    e_gate, _, _, e_pooled = O.connector_route(x, cfg, w, valid)
    assert_close(to_np(rf["pooled"]), e_pooled, "bf16", "folded pooled")
    assert_close(to_np(rk["pooled"]), e_pooled, "bf16", "kv pooled")
    assert_gates(rf["gate"].cpu().numpy(), e_gate, "gate (folded)")
    gate = rf["gate"].cpu().numpy()
    thr, use = O.decide(gate[:, 0], cfg)
    assert float(rf["thr"].item()) == thr
    assert np.array_equal(rf["use64"].cpu().numpy(), use)


def test_folded_pool_flash_workload():
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    say(f"2B-Flash folded route: T={cfg['T']}")
    w = host_weights(cfg)
    con = _connector(cfg, w, cfg["T"])
    xd = dev_vit(cfg)
    r = con.route(xd)
    torch.cuda.synchronize()
    gate = r["gate"].cpu().numpy()
    thr, use = O.decide(gate[:, 0], cfg)
    assert float(r["thr"].item()) == thr
    assert np.array_equal(r["use64"].cpu().numpy(), use)
    g0 = gate[:, 0].astype(np.float64)
    near = {int(np.argmin(np.abs(g0 - thr))), int(np.argmin(np.abs(g0 - 0.5)))}
    tiles = sorted(set(synth.sample_tiles(cfg["T"], n=12)) | near)
    x = synth.make_vit_tiles(cfg, tiles)
    e_gate, _, _, e_pooled = O.connector_route(x, cfg, w)
    assert_close(to_np(r["pooled"][tiles]), e_pooled, "bf16", "pooled")
    assert_gates(gate[tiles], e_gate)


# Every tile of the 2B-Flash workload against the oracle's gates, stored by
# tests/golden/make_flash_gates.py (the oracle alone, all 208 tiles): gates
# within 2e-3; the GPU's decisions equal to the oracle's own, independently
# computed ones on every tile whose gate[:,0] is at least 1e-3 from both
# thresholds on both sides ([4B-Flash] section 4, inference decision;
# [2B-Flash] routing decision); and bit-exact on the GPU's own gates.
def _flash_fixture():
    import json
    import os
    with open(os.path.join(GOLDEN, "flash_gates.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("path", ["kv", "folded", "forward"])
def test_flash_gates_all_tiles_vs_oracle(path):
    fx = _flash_fixture()
    cfg = workload("internvl35_2b_flash", pool_mode=0 if path == "kv" else 1,
                   ln_fold=1 if path == "forward" else 0)
    T = cfg["T"]
    assert fx["T"] == T and fx["gate_bias0"] == host_gate_bias(cfg)
    say(f"2B-Flash all-tile gates: path={path} T={T}")
    w = host_weights(cfg)
    con = _connector(cfg, w, T)
    xd = dev_vit(cfg)
    r = con.forward(xd) if path == "forward" else con.route(xd)
    torch.cuda.synchronize()
    gate = r["gate"].cpu().numpy()
    use = r["use64"].cpu().numpy()
    g_thr = float(r["thr"].item())
    e_gate = np.asarray(fx["gate"], np.float64)
    e_use = np.asarray(fx["use64"], np.uint8)
    e_thr = float(fx["threshold"])
    assert_gates(gate, e_gate, f"gate all {T} tiles ({path})")
    # the threshold is an interpolation between order statistics, and order
    # statistics of two sets move by at most the largest element change
    dthr = abs(g_thr - e_thr)
    log_margin(f"threshold ({path})", max_abs=dthr, tol=GATE_TOL)
    assert dthr <= GATE_TOL
    # bit-exact decisions on the GPU's own gates
    thr, own = O.decide(gate[:, 0], cfg)
    assert g_thr == thr
    assert np.array_equal(use, own)
    # independent decisions away from both thresholds (either side's values)
    g0, e0 = gate[:, 0].astype(np.float64), e_gate[:, 0]
    near = np.zeros(T, bool)
    for v in (g0, e0):
        for t in (g_thr, e_thr, cfg["abs_threshold"]):
            near |= np.abs(v - t) < BAND
    far = ~near
    mism = int((use[far] != e_use[far]).sum())
    say(f"  decisions compared on {int(far.sum())}/{T} tiles, {int(near.sum())} in the band, "
        f"{mism} differ; routed gpu {int(use.sum())} oracle {int(e_use.sum())}")
    log_margin(f"decisions ({path})", compared=int(far.sum()), band=int(near.sum()),
               mismatches=mism)
    assert far.sum() >= T - 8
    assert mism == 0


# Batch sizes that split a tile's tokens over many token-pass workgroups (T = 3:
# 64 per tile, T = 13: up to 17, the value fold then reads a merged xbar) or
# over up to four (T = 100: the value fold merges the partials in its operand
# load), with padding masks (odd layers walk each workgroup's range backwards,
# skipping the padded chunks from the other end).
@pytest.mark.parametrize("T,padded", [(3, False), (13, True), (100, True)])
def test_folded_pool_batch_sizes(T, padded):
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    cfg["tiles"], cfg["T"] = [T], T
    say(f"2B-Flash folded route: T={T} padded={padded}")
    w = host_weights(cfg)
    con = _connector(cfg, w, T)
    xd = dev_vit(cfg)
    valid = synth.make_valid_tokens(cfg, seed=T) if padded else None
    r = con.route(xd, valid=torch.from_numpy(valid).cuda() if padded else None)
    torch.cuda.synchronize()
    assert int(r["status"].item()) == 0
    gate = r["gate"].cpu().numpy()
    thr, use = O.decide(gate[:, 0], cfg)
    assert float(r["thr"].item()) == thr
    assert np.array_equal(r["use64"].cpu().numpy(), use)
    tiles = sorted(set(synth.sample_tiles(T, n=6)))
    x = synth.make_vit_tiles(cfg, tiles)
    e_gate, _, _, e_pooled = O.connector_route(x, cfg, w, valid[tiles] if padded else None)
    assert_close(to_np(r["pooled"][tiles]), e_pooled, "bf16", "pooled")
    assert_gates(gate[tiles], e_gate)


# ---------------------------------------------------------------------------
# route-first run: only the chosen path per tile
# ---------------------------------------------------------------------------
def _check_routed(con, cfg, xd, use_d):
    use = use_d.cpu().numpy()
    f256, f64 = con.run(xd)
    r256 = torch.full_like(f256, float("nan"))
    r64 = torch.full_like(f64, float("nan"))
    con.run_routed(xd, use_d, r256, r64)
    torch.cuda.synchronize()
    keep256 = torch.from_numpy(use == 0).cuda()
    keep64 = torch.from_numpy(use != 0).cuda()
    # chosen path: bit-identical to the full run (same K order per output
    # element: a Flash connector's products keep one tile per workgroup)
    assert torch.equal(r256[keep256], f256[keep256])
    assert torch.equal(r64[keep64], f64[keep64])
    # other path: untouched
    assert torch.isnan(r256[~keep256].float()).all()
    assert torch.isnan(r64[~keep64].float()).all()
    return f256, f64, r256, r64


@pytest.mark.parametrize("pattern", ["route", "none", "all", "alternate"])
def test_run_routed_tiny(pattern):
    cfg, w, x = _tiny_all()
    say(f"run_routed tiny pattern={pattern}")
    con = _connector(cfg, w, cfg["T"])
    xd = torch.from_numpy(x).cuda()
    if pattern == "route":
        use_d = con.route(xd)["use64"]
    else:
        use = {"none": np.zeros(cfg["T"]), "all": np.ones(cfg["T"]),
               "alternate": np.arange(cfg["T"]) % 2}[pattern].astype(np.uint8)
        use_d = torch.from_numpy(use).cuda()
    _check_routed(con, cfg, xd, use_d)


def test_run_routed_flash_workload_and_compaction():
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    say(f"2B-Flash run_routed: T={cfg['T']}")
    w = host_weights(cfg)
    ids, emb = synth.make_sequence(cfg)
    con = _connector(cfg, w, cfg["T"], len(ids))
    xd = dev_vit(cfg)
    r = con.route(xd)
    f256, f64, r256, r64 = _check_routed(con, cfg, xd, r["use64"])
    ids_d = torch.from_numpy(ids).cuda()
    emb_d = torch.from_numpy(emb).to(torch.bfloat16).cuda()
    cf = con.compact(ids_d, emb_d, r["use64"], f256, f64, synth.IMG_CONTEXT)
    cf = {k: v.clone() for k, v in cf.items()}
    cr = con.compact(ids_d, emb_d, r["use64"], r256, r64, synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    n = int(cf["len"].item())
    assert n == int(cr["len"].item())
    for k in ("ids", "pos", "keep_map"):
        assert torch.equal(cf[k], cr[k]), k
    assert torch.equal(cf["embeds"][:n], cr["embeds"][:n])
    assert not torch.isnan(cr["embeds"][:n].float()).any()


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_edge_cases():
    cfg = workload("tiny_flash_f32")
    w = host_weights(cfg)
    con = _connector(cfg, w, cfg["T"], 200)
    x = torch.from_numpy(synth.make_vit(cfg)).cuda()
    say("edge: T=0 run/route are no-ops")
    con.run(x[:0])
    con.route(x[:0])
    say("edge: T=1 route compresses nothing")
    r = con.route(x[:1])
    torch.cuda.synchronize()
    assert int(r["use64"].item()) == 0
    assert float(r["thr"].item()) == float(r["gate"][0, 0].item())
    say("edge: valid_tokens out of range sets the status bit")
    bad = torch.tensor([0, 64, 65, 1, 2, 3, 4, 5], dtype=torch.int32, device="cuda")
    r = con.route(x, valid=bad)
    torch.cuda.synchronize()
    assert int(r["status"].item()) & 2
    say("edge: IMG_CONTEXT count mismatch sets the status bit")
    ids, emb = synth.make_sequence(cfg)
    o256, o64 = con.run(x)
    use = torch.zeros(cfg["T"], dtype=torch.uint8, device="cuda")
    ids_bad = ids.copy()
    ids_bad[np.flatnonzero(ids == synth.IMG_CONTEXT)[3]] = 5
    c = con.compact(torch.from_numpy(ids_bad).cuda(), torch.from_numpy(emb).cuda(), use, o256, o64,
                    synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    assert int(c["status"].item()) == 1 and int(c["len"].item()) == 0
    say("edge: empty sequence")
    c = con.compact(torch.from_numpy(ids[:0]).cuda(), torch.from_numpy(emb[:0]).cuda(), use[:0],
                    o256, o64, synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    assert int(c["len"].item()) == 0
    say("edge: nothing routed keeps every slot")
    c = con.compact(torch.from_numpy(ids).cuda(), torch.from_numpy(emb).cuda(), use, o256, o64,
                    synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    assert int(c["len"].item()) == len(ids)
    assert np.array_equal(c["ids"].cpu().numpy(), ids)


def test_deterministic():
    cfg = workload("tiny_flash_f32")
    w = host_weights(cfg)
    con = _connector(cfg, w, cfg["T"])
    x = torch.from_numpy(synth.make_vit(cfg)).cuda()
    say("determinism")
    a = [t.clone() for t in con.run(x)] + [con.route(x)["gate"].clone()]
    b = [t.clone() for t in con.run(x)] + [con.route(x)["gate"].clone()]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ---------------------------------------------------------------------------
# batched, ragged compaction (B prompts packed back to back)
# ---------------------------------------------------------------------------
def _compact_model(name):
    """A connector whose compaction geometry (P, D, dtype) is the named
    workload's, with small projector widths (compaction reads none of them)."""
    if name == "tiny_flash_f32":
        return workload(name)
    return workload(name, C=64, mlp1_hidden=256, mlp2_hidden=256, gate_hidden=64, pool_heads=4)


def _batch_case(cfg, images, seed):
    ids, emb, cu, to = synth.make_batch_sequences(cfg, images, seed)
    T = int(to[-1])
    dt = TORCH_DT[cfg["dtype"]]
    g = torch.Generator().manual_seed(seed)
    o256 = torch.randn((T, cfg["S"], cfg["D"]), generator=g).to(dt)
    o64 = torch.randn((T, cfg["S64"], cfg["D"]), generator=g).to(dt)
    use = (torch.rand(T, generator=g) < 0.5).to(torch.uint8).numpy()
    return ids, emb, cu, to, use, o256, o64


def _run_batch(con, cfg, ids, emb_d, cu, to, use, o256, o64):
    return con.compact_batch(torch.from_numpy(ids).cuda(), torch.from_numpy(cu).cuda(), emb_d,
                             torch.from_numpy(to).cuda(), torch.from_numpy(use).cuda(),
                             o256.cuda(), o64.cuda(), synth.IMG_CONTEXT)


@pytest.mark.parametrize("name,images,seed", [
    ("tiny_flash_f32", [[1, 2], [], [3], [1], [], [2]], 1),
    ("tiny_flash_f32", [[1]], 2),
    ("tiny_flash_f32", [[], []], 3),
    ("internvl35_2b_flash", [[13, 1], [], [4, 4, 1], [13], [2]], 4),
])
def test_compact_batch_matches_oracle(name, images, seed):
    cfg = _compact_model(name)
    say(f"compact_batch {name} images={images}")
    ids, emb, cu, to, use, o256, o64 = _batch_case(cfg, images, seed)
    con = _connector(cfg, host_weights(cfg), 1)
    emb_d = torch.from_numpy(emb).to(TORCH_DT[cfg["dtype"]]).cuda()
    c = _run_batch(con, cfg, ids, emb_d, cu, to, use, o256, o64)
    torch.cuda.synchronize()
    ref = O.compact_batch(ids, cu, emb, synth.IMG_CONTEXT, to, use, to_np(o256), to_np(o64),
                          cfg["S"], cfg["S64"])
    assert int(c["status"].item()) == 0 and ref["status"] == 0
    assert np.array_equal(c["cu"].cpu().numpy(), ref["out_cu"])
    n = int(ref["out_cu"][-1])
    assert n == len(ids) - (cfg["S"] - cfg["S64"]) * int(use.sum())
    assert np.array_equal(c["ids"].cpu().numpy(), ref["out_ids"])
    assert np.array_equal(c["pos"].cpu().numpy(), ref["out_pos"])
    assert np.array_equal(c["keep_map"].cpu().numpy(), ref["keep_map"])
    got = c["embeds"][:n].float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref["out_embeds"][:n].astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("bad", ["slot_count", "cu_end", "tile_order"])
def test_compact_batch_errors(bad):
    cfg = workload("tiny_flash_f32")
    say(f"compact_batch error case {bad}")
    ids, emb, cu, to, use, o256, o64 = _batch_case(cfg, [[1], [2], [1]], 5)
    if bad == "slot_count":
        p = int(np.flatnonzero(ids[cu[1]:cu[2]] == synth.IMG_CONTEXT)[0]) + int(cu[1])
        ids = np.delete(ids, p)
        emb = np.delete(emb, p, axis=0)
        cu = cu.copy()
        cu[2:] -= 1
    elif bad == "cu_end":
        cu = cu.copy()
        cu[-1] -= 1
    else:
        to = to.copy()
        to[1] = to[2] + 1
    con = _connector(cfg, host_weights(cfg), 1)
    c = _run_batch(con, cfg, ids, torch.from_numpy(emb).cuda(), cu, to, use, o256, o64)
    torch.cuda.synchronize()
    ref = O.compact_batch(ids, cu, emb, synth.IMG_CONTEXT, to, use, to_np(o256), to_np(o64),
                          cfg["S"], cfg["S64"])
    st = int(c["status"].item())
    assert st == ref["status"] == (O.STATUS_IMG_COUNT if bad == "slot_count" else O.STATUS_SEQ_LAYOUT)
    assert np.array_equal(c["cu"].cpu().numpy(), ref["out_cu"])
    assert np.array_equal(c["keep_map"].cpu().numpy(), ref["keep_map"])
    n = int(ref["out_cu"][-1])
    assert np.array_equal(c["ids"].cpu().numpy(), ref["out_ids"])
    assert np.array_equal(c["pos"].cpu().numpy(), ref["out_pos"])
    got = c["embeds"][:n].float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref["out_embeds"][:n].astype(np.float32).view(np.uint32))


def test_compact_batch_flash_layout_16_prompts():
    # 16 prompts, each the 2B-Flash batch layout (16 images x 13 tiles), D = 2048:
    # L = 860k.  Index outputs bit-exact against the oracle; every embedding row
    # checked against the source row the oracle assigns it (the oracle runs
    # on one-column stand-ins that name each source row).
    cfg = _compact_model("internvl35_2b_flash")
    B = 16
    ids, _, cu, to = synth.make_batch_sequences(cfg, [cfg["tiles"]] * B, 6, with_embeds=False)
    L, T, S, S64, D = len(ids), int(to[-1]), cfg["S"], cfg["S64"], cfg["D"]
    say(f"compact_batch 2B-Flash layout x{B}: L={L} T={T}")
    g = torch.Generator(device="cuda").manual_seed(6)
    emb_d = torch.randn((L, D), generator=g, device="cuda").to(torch.bfloat16)
    o256 = torch.randn((T, S, D), generator=g, device="cuda").to(torch.bfloat16)
    o64 = torch.randn((T, S64, D), generator=g, device="cuda").to(torch.bfloat16)
    use = (np.random.default_rng(6).random(T) < 0.5).astype(np.uint8)
    con = _connector(cfg, host_weights(cfg), 1)
    c = con.compact_batch(torch.from_numpy(ids).cuda(), torch.from_numpy(cu).cuda(), emb_d,
                          torch.from_numpy(to).cuda(), torch.from_numpy(use).cuda(), o256, o64,
                          synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    code_e = np.arange(L, dtype=np.float64)[:, None]
    code_256 = (L + np.arange(T * S, dtype=np.float64)).reshape(T, S, 1)
    code_64 = (L + T * S + np.arange(T * S64, dtype=np.float64)).reshape(T, S64, 1)
    ref = O.compact_batch(ids, cu, code_e, synth.IMG_CONTEXT, to, use, code_256, code_64, S, S64)
    assert int(c["status"].item()) == 0 and ref["status"] == 0
    assert np.array_equal(c["cu"].cpu().numpy(), ref["out_cu"])
    n = int(ref["out_cu"][-1])
    assert n == L - (S - S64) * int(use.sum())
    assert np.array_equal(c["ids"].cpu().numpy(), ref["out_ids"])
    assert np.array_equal(c["pos"].cpu().numpy(), ref["out_pos"])
    assert np.array_equal(c["keep_map"].cpu().numpy(), ref["keep_map"])
    code = torch.from_numpy(ref["out_embeds"][:n, 0].astype(np.int64)).cuda()
    want = torch.empty((n, D), dtype=torch.bfloat16, device="cuda")
    m = code < L
    want[m] = emb_d[code[m]]
    m2 = (code >= L) & (code < L + T * S)
    want[m2] = o256.view(-1, D)[code[m2] - L]
    m3 = code >= L + T * S
    want[m3] = o64.view(-1, D)[code[m3] - L - T * S]
    assert torch.equal(c["embeds"][:n].view(torch.int16), want.view(torch.int16))


# ---------------------------------------------------------------------------
# LayerNorm folded into the first product of each projector (ln_fold)
# ---------------------------------------------------------------------------
def _tiny_bf16(T, **over):
    cfg = workload("tiny_flash_f32", dtype="bf16", **over)
    return dict(cfg, T=T, tiles=[T], name="tiny_bf16")


@pytest.mark.parametrize("T,version,order,shift", [
    (1, 2, "direct", 0.0), (5, 2, "direct", 0.0), (11, 2, "direct", 3.0), (5, 1, "direct", 0.0),
    (5, 2, "twice_r2", 0.0), (7, 1, "twice_r2", 3.0)])
def test_ln_fold_small_matches_oracle(T, version, order, shift):
    # shift: LayerNorm ignores a constant added to a row, so a large common
    # offset (mean >> spread) must cancel exactly in the folded epilogue
    cfg = _tiny_bf16(T, ln_fold=1, ps_version=version, shuffle64_order=order)
    w = synth.make_weights(cfg)
    x = synth.to_bf16_exact(synth.make_vit_tiles(cfg, range(T)) + np.float32(shift))
    say(f"ln_fold small T={T} v{version} {order} shift={shift}")
    con = _connector(cfg, w, T)
    o256, o64 = con.run(torch.from_numpy(x).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    e256, e64 = O.connector_run(x, cfg, w)
    assert_close(to_np(o256), e256, "bf16", "out256")
    assert_close(to_np(o64), e64, "bf16", "out64")


@pytest.mark.parametrize("pattern", ["none", "all", "alternate"])
def test_ln_fold_run_routed_small(pattern):
    T = 9
    cfg = _tiny_bf16(T, ln_fold=1)
    w = synth.make_weights(cfg)
    x = synth.make_vit_tiles(cfg, range(T))
    say(f"ln_fold run_routed small pattern={pattern}")
    con = _connector(cfg, w, T)
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    use = {"none": np.zeros(T), "all": np.ones(T), "alternate": np.arange(T) % 2}[pattern]
    _check_routed(con, cfg, xd, torch.from_numpy(use.astype(np.uint8)).cuda())


@pytest.mark.parametrize("name", ["internvl35_4b_std", "internvl3_14b_ragged", "internvl3_38b"])
def test_ln_fold_standard_connector_sampled(name):
    # standard (non-Flash) connectors: the statistics pass for r = 2 only, C = 1024 and 3200
    cfg = workload(name, ln_fold=1)
    say(f"{name} ln_fold: T={cfg['T']} C={cfg['C']} D={cfg['D']}")
    w = host_weights(cfg)
    con = _connector(cfg, w, cfg["T"])
    o256, _ = con.run(dev_vit(cfg))
    torch.cuda.synchronize()
    tiles = synth.sample_tiles(cfg["T"])
    x = synth.make_vit_tiles(cfg, tiles)
    e256, _ = O.connector_run(x, cfg, w)
    assert_close(to_np(o256[tiles]), e256, "bf16", f"{name} out256 (ln_fold)")


def test_ln_fold_flash_workload_sampled():
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=1)
    say(f"2B-Flash ln_fold run_routed: T={cfg['T']}")
    w = host_weights(cfg)
    con = _connector(cfg, w, cfg["T"])
    xd = dev_vit(cfg)
    r = con.route(xd)
    use_d = r["use64"]
    f256, f64, r256, r64 = _check_routed(con, cfg, xd, use_d)
    use = use_d.cpu().numpy()
    tiles = synth.sample_tiles(cfg["T"])
    x = synth.make_vit_tiles(cfg, tiles)
    e256, e64 = O.connector_run(x, cfg, w)
    t256 = [i for i, t in enumerate(tiles) if use[t] == 0]
    t64 = [i for i, t in enumerate(tiles) if use[t] != 0]
    assert t256 and t64
    assert_close(to_np(r256[[tiles[i] for i in t256]]), e256[t256], "bf16", "out256 (ln_fold)")
    assert_close(to_np(r64[[tiles[i] for i in t64]]), e64[t64], "bf16", "out64 (ln_fold)")


# ---------------------------------------------------------------------------
# forward = route + route-first run in one call
# ---------------------------------------------------------------------------
def _check_forward(cfg, w, xd, valid=None):
    con = _connector(cfg, w, cfg["T"])
    r = con.route(xd, valid=valid)
    r = {k: (v.clone() if v is not None else None) for k, v in r.items()}
    r256 = torch.full((cfg["T"], cfg["S"], cfg["D"]), float("nan"), dtype=xd.dtype, device="cuda")
    r64 = torch.full((cfg["T"], cfg["S64"], cfg["D"]), float("nan"), dtype=xd.dtype, device="cuda")
    con.run_routed(xd, r["use64"], r256, r64)
    f = con.forward(xd, valid=valid)
    torch.cuda.synchronize()
    for k in ("gate", "thr", "use64", "pooled", "status"):
        assert torch.equal(f[k], r[k]), k
    use = r["use64"].cpu().numpy()
    keep256 = torch.from_numpy(use == 0).cuda()
    keep64 = torch.from_numpy(use != 0).cuda()
    assert torch.equal(f["out256"][keep256], r256[keep256])
    assert torch.equal(f["out64"][keep64], r64[keep64])
    return f


def test_forward_matches_route_then_run_tiny():
    cfg, w, x = _tiny_all()
    say("forward tiny fp32")
    _check_forward(cfg, w, torch.from_numpy(x).cuda())


@pytest.mark.parametrize("version,order", [(2, "direct"), (1, "twice_r2")])
def test_forward_matches_route_then_run_ln_fold_small(version, order):
    T = 9
    cfg = _tiny_bf16(T, ln_fold=1, ps_version=version, shuffle64_order=order)
    w = synth.make_weights(cfg)
    x = synth.make_vit_tiles(cfg, range(T))
    say(f"forward ln_fold small v{version} {order}")
    _check_forward(cfg, w, torch.from_numpy(x).to(torch.bfloat16).cuda())


# C = 512: LayerNorm statistics through per-token moments (from the first
# token pass in forward, from their own kernel in run_routed), every index
# variant; outputs bit-equal between the two calls and close to the oracle
@pytest.mark.parametrize("version,order", [(2, "direct"), (1, "direct"), (2, "twice_r2"),
                                           (1, "twice_r2")])
def test_forward_ln_fold_token_stats_small(version, order):
    cfg = workload("tiny_flash_f32", dtype="bf16", C=512, D=256, mlp1_hidden=256,
                   mlp2_hidden=256, pool_heads=8, gate_hidden=512, pool_mode=1, ln_fold=1,
                   ps_version=version, shuffle64_order=order)
    cfg["name"] = "small_bf16_ln_fold"
    w = synth.make_weights(cfg)
    x = synth.make_vit(cfg)
    say(f"forward token stats small v{version} {order}")
    f = _check_forward(cfg, w, torch.from_numpy(x).to(torch.bfloat16).cuda())
    use = f["use64"].cpu().numpy()
    e256, e64 = O.connector_run(x, cfg, w)
    t256, t64 = np.flatnonzero(use == 0), np.flatnonzero(use != 0)
    if len(t256):
        assert_close(to_np(f["out256"][t256]), e256[t256], "bf16", "out256 (forward)")
    if len(t64):
        assert_close(to_np(f["out64"][t64]), e64[t64], "bf16", "out64 (forward)")


def test_forward_flash_workload_ln_fold():
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=1)
    say(f"2B-Flash forward (ln_fold): T={cfg['T']}")
    w = host_weights(cfg)
    f = _check_forward(cfg, w, dev_vit(cfg))
    use = f["use64"].cpu().numpy()
    assert 0 < use.sum() < cfg["T"]
