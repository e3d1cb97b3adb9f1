"""ivc_connector_forward_compact against ivc_connector_forward followed by
ivc_connector_compact on the same inputs: gates, threshold, decisions,
pooled vectors, the chosen path's projector rows, and the compacted ids,
positions, keep map, length and embedding rows, bit for bit.  Parity of
forward and compact with the oracle is covered by their own tests.  Also
the forked path (bf16, the index work and text rows on a stream of its own
beside both projector chains; at 208 tiles both chains' last products write
their rows into the compacted sequence themselves), the unforked one (fp32),
a padding mask, T = 0, a sequence with the wrong slot count (nothing placed),
and a workspace that is too small (reported before anything is enqueued)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_vit, dev_weights, host_weights, say, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vlm_visual_token_amd import ivc
    ivc.load()
    yield
    torch.cuda.synchronize()


def _clone(d):
    return {k: (v.clone() if v is not None else None) for k, v in d.items()}


def _both(con, xd, ids_d, emb_d, valid=None):
    f = _clone(con.forward(xd, valid=valid))
    c = _clone(con.compact(ids_d, emb_d, f["use64"], f["out256"], f["out64"], synth.IMG_CONTEXT))
    fc = _clone(con.forward_compact(xd, ids_d, emb_d, synth.IMG_CONTEXT, valid=valid))
    torch.cuda.synchronize()
    return f, c, fc


def _same(f, c, fc):
    for k in ("gate", "thr", "use64", "pooled", "status"):
        assert torch.equal(f[k], fc[k]), k
    assert int(fc["status"].item()) == 0
    use = f["use64"].cpu().numpy().astype(bool)
    # forward writes only the chosen path's rows
    for t in np.nonzero(~use)[0]:
        assert torch.equal(f["out256"][t], fc["out256"][t]), f"out256 tile {t}"
    for t in np.nonzero(use)[0]:
        assert torch.equal(f["out64"][t], fc["out64"][t]), f"out64 tile {t}"
    n = int(c["len"].item())
    assert n == int(fc["len"].item())
    for k in ("ids", "pos", "keep_map"):
        assert torch.equal(c[k], fc[k]), k
    assert torch.equal(c["embeds"][:n], fc["embeds"][:n])
    return n


@pytest.mark.parametrize("ln_fold", [1, 0])
def test_forward_compact_flash_workload(ln_fold):
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=ln_fold)
    ids, emb = synth.make_sequence(cfg)
    say(f"forward_compact 2B-Flash: T={cfg['T']} L={len(ids)} ln_fold={ln_fold}")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=cfg["T"],
                    max_seq_len=len(ids))
    ids_d = torch.from_numpy(ids).cuda()
    emb_d = torch.from_numpy(emb).to(torch.bfloat16).cuda()
    f, c, fc = _both(con, dev_vit(cfg), ids_d, emb_d)
    n = _same(f, c, fc)
    use = f["use64"].cpu().numpy()
    assert 0 < use.sum() < cfg["T"]
    assert n == len(ids) - (cfg["S"] - cfg["S64"]) * int(use.sum())
    say(f"  routed {int(use.sum())}/{cfg['T']}, L' = {n}")


def test_forward_compact_flash_padded():
    """bf16 with a padding mask: the chains fork, and the moments come from the
    statistics pass (the token pass does not read every token)."""
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=1)
    T = 24
    cfg["tiles"], cfg["T"] = [T], T
    ids, emb = synth.make_sequence(cfg)
    say(f"forward_compact 2B-Flash padded: T={T} L={len(ids)}")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T, max_seq_len=len(ids))
    vd = torch.from_numpy(synth.make_valid_tokens(cfg, seed=5)).cuda()
    f, c, fc = _both(con, dev_vit(cfg), torch.from_numpy(ids).cuda(),
                     torch.from_numpy(emb).to(torch.bfloat16).cuda(), vd)
    _same(f, c, fc)


@pytest.mark.parametrize("name,padded", [("tiny_flash_f32", False), ("tiny_flash_f32", True)])
def test_forward_compact_tiny(name, padded):
    """fp32: the chains do not fork, the index work runs on the caller's stream."""
    from vlm_visual_token_amd import Connector
    cfg = workload(name)
    ids, emb = synth.make_sequence(cfg)
    say(f"forward_compact {name}: T={cfg['T']} L={len(ids)} padded={padded}")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=cfg["T"],
                    max_seq_len=len(ids))
    x = synth.make_vit(cfg)
    valid = synth.make_valid_tokens(cfg, seed=3) if padded else None
    xd = torch.from_numpy(x).cuda()
    vd = torch.from_numpy(valid).cuda() if padded else None
    f, c, fc = _both(con, xd, torch.from_numpy(ids).cuda(), torch.from_numpy(emb).cuda(), vd)
    _same(f, c, fc)


def test_forward_compact_no_tiles_and_small_workspace():
    from vlm_visual_token_amd import Connector, ivc
    cfg = workload("internvl35_2b_flash", pool_mode=1)
    T = 4
    cfg["tiles"], cfg["T"] = [T], T
    ids, emb = synth.make_sequence(cfg)
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T, max_seq_len=len(ids))
    xd = dev_vit(cfg)
    ids_d = torch.from_numpy(ids).cuda()
    emb_d = torch.from_numpy(emb).to(torch.bfloat16).cuda()
    say("forward_compact: T = 0 (text only)")
    text = ids_d[ids_d != synth.IMG_CONTEXT].contiguous()
    temb = emb_d[(ids_d != synth.IMG_CONTEXT)].contiguous()
    r = con.forward_compact(xd[:0], text, temb, synth.IMG_CONTEXT)
    torch.cuda.synchronize()
    L0 = text.shape[0]
    assert int(r["len"].item()) == L0 and int(r["status"].item()) == 0
    assert torch.equal(r["ids"], text)
    assert torch.equal(r["pos"], torch.arange(L0, dtype=torch.int32, device="cuda"))
    assert torch.equal(r["embeds"], temb)
    say("forward_compact: workspace one byte short")
    need = ivc.ivc_connector_forward_compact_workspace_bytes(con.h, T, len(ids))
    assert need <= con.ws_bytes
    out = con.forward_compact(xd, ids_d, emb_d, synth.IMG_CONTEXT)  # buffers to reuse
    torch.cuda.synchronize()
    sentinel = {k: v.clone() for k, v in out.items() if v is not None}
    with pytest.raises(ivc.IvcError) as e:
        ivc.ivc_connector_forward_compact(
            con.h, xd, None, T, out["gate"], out["thr"], out["use64"], out["pooled"],
            out["status"], out["out256"], out["out64"], ids_d, emb_d, len(ids), synth.IMG_CONTEXT,
            out["ids"], out["pos"], out["keep_map"], out["embeds"], out["len"], con.ws,
            need - 1)
    assert e.value.status == 4  # IVC_ERR_WORKSPACE
    torch.cuda.synchronize()
    for k, v in sentinel.items():  # nothing was enqueued (bytes: unwritten rows may hold NaN)
        assert torch.equal(out[k].view(torch.uint8), v.view(torch.uint8)), k


@pytest.mark.parametrize("change", ["one_short", "one_extra"])
def test_forward_compact_wrong_slot_count_places_nothing(change):
    """A sequence whose IMG_CONTEXT count is not 256 per tile compacts to
    length 0 with status bit 1 ([4B-Flash] section 4 compaction; the single
    prompt rule).  At 208 tiles the projectors' last products place their
    rows themselves, so they must place none here: the embedding rows keep
    what the caller left in them."""
    from vlm_visual_token_amd import Connector
    cfg = workload("internvl35_2b_flash", pool_mode=1, ln_fold=1)
    T = cfg["T"]
    ids, emb = synth.make_sequence(cfg)
    img = synth.IMG_CONTEXT
    at = np.nonzero(ids == img)[0]
    if change == "one_short":
        keep = np.ones(len(ids), dtype=bool)
        keep[at[len(at) // 2]] = False
        ids2, emb2 = ids[keep], emb[keep]
    else:
        ids2 = np.insert(ids, at[-1] + 1, img)
        emb2 = np.insert(emb, at[-1] + 1, emb[at[-1]], axis=0)
    say(f"forward_compact, {change}: T={T} L={len(ids2)} (slots {int((ids2 == img).sum())})")
    con = Connector(cfg, dev_weights(cfg, host_weights(cfg)), max_tiles=T, max_seq_len=len(ids2))
    xd = dev_vit(cfg)
    ids_d = torch.from_numpy(ids2).cuda()
    emb_d = torch.from_numpy(emb2).to(torch.bfloat16).cuda()
    out = con.forward_compact(xd, ids_d, emb_d, img)
    torch.cuda.synchronize()
    out["embeds"].fill_(7.0)  # exact in bf16
    out["status"].zero_()  # the library only ORs bits in
    r = con.forward_compact(xd, ids_d, emb_d, img, out=out)
    torch.cuda.synchronize()
    assert int(r["len"].item()) == 0
    assert int(r["status"].item()) & 1
    assert torch.all(r["embeds"] == 7.0)
    f = _clone(con.forward(xd))
    torch.cuda.synchronize()
    for k in ("gate", "thr", "use64"):
        assert torch.equal(f[k], r[k]), k
