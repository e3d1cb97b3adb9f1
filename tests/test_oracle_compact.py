"""Pins for the oracle's compaction and tile offsets (no GPU).

Compaction is tied to a brute-force delete written independently (find every
IMG_CONTEXT position, cut the sequence into runs of S slots, delete slots
S64..S-1 of each routed run with numpy.delete), to the closed-form length
L' = L - 192 * routed the pages state, and to invariants (positions are
0..L'-1, text tokens survive in order).
"""
import numpy as np
import pytest

import synth
from oracle import connector as O

IMG = synth.IMG_CONTEXT


def _brute(ids, emb, use64, o256, o64, S, S64):
    ids = np.asarray(ids)
    L = len(ids)
    src = [("e", p, 0) for p in range(L)]
    img_pos = np.flatnonzero(ids == IMG)
    for k, p in enumerate(img_pos):
        t, loc = divmod(k, S)
        src[p] = ("64" if use64[t] else "256", t, loc)
    drop = []
    for t in range(len(use64)):
        if use64[t]:
            drop.extend(img_pos[t * S + S64:(t + 1) * S].tolist())
    keep_idx = np.delete(np.arange(L), drop)
    rows = []
    for p in keep_idx:
        kind, a, b = src[p]
        rows.append(emb[a] if kind == "e" else (o64 if kind == "64" else o256)[a][b])
    return ids[keep_idx], keep_idx, np.array(rows)


def _case(T, S, S64, D, seed, n_text=(3, 5)):
    r = np.random.default_rng(seed)
    parts = []
    tiles_left = T
    while tiles_left:
        nt = int(r.integers(1, tiles_left + 1))
        parts += [r.integers(0, 1000, int(r.integers(*n_text))), [IMG - 2], [IMG] * (nt * S), [IMG - 1]]
        tiles_left -= nt
    parts.append(r.integers(0, 1000, 2))
    ids = np.concatenate([np.asarray(p, np.int64) for p in parts]).astype(np.int32)
    L = len(ids)
    emb = r.standard_normal((L, D))
    emb[ids == IMG] = np.nan
    o256 = r.standard_normal((T, S, D))
    o64 = r.standard_normal((T, S64, D))
    use64 = (r.random(T) < 0.5).astype(np.uint8)
    return ids, emb, use64, o256, o64


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("T,S,S64", [(1, 16, 4), (5, 16, 4), (13, 256, 64), (3, 4, 1)])
def test_compact_matches_brute_force(seed, T, S, S64):
    ids, emb, use64, o256, o64 = _case(T, S, S64, 3, seed)
    got = O.compact(ids, emb, IMG, use64, o256, o64, S, S64)
    bids, bkeep, brows = _brute(ids, emb, use64, o256, o64, S, S64)
    n = got["out_len"]
    assert got["status"] == O.STATUS_OK
    assert n == len(bids)
    assert np.array_equal(got["out_ids"][:n], bids)
    assert np.array_equal(np.flatnonzero(got["keep_map"] >= 0), bkeep)
    assert np.array_equal(got["keep_map"][bkeep], np.arange(n))
    assert np.array_equal(got["out_embeds"][:n], brows)
    assert not np.isnan(got["out_embeds"][:n]).any()
    assert np.array_equal(got["out_pos"][:n], np.arange(n))
    assert (got["out_pos"][n:] == -1).all() and (got["out_ids"][n:] == -1).all()


def test_compact_length_closed_form(golden):
    g = golden("routing.txt")
    S, S64, drop = int(g["slots_per_tile"][0]), int(g["slots_kept"][0]), int(g["slots_deleted"][0])
    assert S - S64 == drop
    ids, emb, use64, o256, o64 = _case(13, S, S64, 2, 11)
    got = O.compact(ids, emb, IMG, use64, o256, o64, S, S64)
    assert got["out_len"] == len(ids) - drop * int(use64.sum())
    # text tokens survive, in order
    txt = ids[ids != IMG]
    out = got["out_ids"][:got["out_len"]]
    assert np.array_equal(out[out != IMG], txt)
    # per routed tile exactly S64 slots remain, per unrouted tile S
    assert int((out == IMG).sum()) == int(S64 * use64.sum() + S * (13 - use64.sum()))


def test_compact_nothing_routed_is_identity_on_ids():
    ids, emb, use64, o256, o64 = _case(4, 16, 4, 2, 3)
    got = O.compact(ids, emb, IMG, np.zeros(4, np.uint8), o256, o64, 16, 4)
    assert got["out_len"] == len(ids)
    assert np.array_equal(got["out_ids"], ids)
    assert np.array_equal(got["keep_map"], np.arange(len(ids)))


def test_compact_rejects_wrong_slot_count():
    ids, emb, use64, o256, o64 = _case(4, 16, 4, 2, 3)
    got = O.compact(ids[:-3] if ids[-3] == IMG else np.append(ids, IMG), emb, IMG, use64, o256, o64, 16, 4)
    assert got["status"] == O.STATUS_IMG_COUNT


def test_tile_offsets():
    assert O.tile_offsets([]).tolist() == [0]
    assert O.tile_offsets([13] * 16).tolist() == [13 * i for i in range(17)]
    r = np.random.default_rng(0)
    t = r.integers(1, 13, 32) + 1
    assert np.array_equal(O.tile_offsets(t), np.concatenate([[0], np.cumsum(t)]))
