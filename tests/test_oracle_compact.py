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


# ---------------------------------------------------------------------------
# batched, ragged compaction: B prompts packed back to back
# ---------------------------------------------------------------------------
def _batch_case(tiles, S, S64, D, seed):
    """Sequences with the given per-sequence tile counts (0 = text only),
    concatenated; returns the packed inputs and the per-sequence pieces."""
    seqs = [_case(t, S, S64, D, seed * 100 + b) if t else None for b, t in enumerate(tiles)]
    r = np.random.default_rng(seed)
    pieces = []
    for t, c in zip(tiles, seqs):
        if c is None:
            n = int(r.integers(0, 4))  # text-only sequence, possibly empty
            c = (r.integers(0, 1000, n).astype(np.int32), r.standard_normal((n, D)),
                 np.zeros(0, np.uint8), np.zeros((0, S, D)), np.zeros((0, S64, D)))
        pieces.append(c)
    ids = np.concatenate([c[0] for c in pieces])
    emb = np.concatenate([c[1] for c in pieces])
    use64 = np.concatenate([c[2] for c in pieces])
    o256 = np.concatenate([c[3] for c in pieces])
    o64 = np.concatenate([c[4] for c in pieces])
    cu = np.concatenate([[0], np.cumsum([len(c[0]) for c in pieces])])
    to = np.concatenate([[0], np.cumsum(tiles)])
    return ids, emb, use64, o256, o64, cu, to, pieces


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("tiles,S,S64", [([2, 0, 3, 1], 16, 4), ([1], 16, 4), ([0, 0], 4, 1),
                                         ([3, 1, 0, 2, 5], 4, 1)])
def test_compact_batch_matches_brute_force(seed, tiles, S, S64):
    ids, emb, use64, o256, o64, cu, to, pieces = _batch_case(tiles, S, S64, 3, seed)
    got = O.compact_batch(ids, cu, emb, IMG, to, use64, o256, o64, S, S64)
    assert got["status"] == O.STATUS_OK
    j = 0
    for b, (sid, semb, suse, s256, s64) in enumerate(pieces):
        bids, bkeep, brows = _brute(sid, semb, suse, s256, s64, S, S64)
        n = len(bids)
        assert got["out_cu"][b] == j and got["out_cu"][b + 1] == j + n
        assert np.array_equal(got["out_ids"][j:j + n], bids)
        assert np.array_equal(got["out_pos"][j:j + n], np.arange(n))
        if n:
            assert np.array_equal(got["out_embeds"][j:j + n], brows)
        km = got["keep_map"][cu[b]:cu[b + 1]]
        assert np.array_equal(np.flatnonzero(km >= 0), bkeep)
        assert np.array_equal(km[bkeep], j + np.arange(n))
        j += n
    L = len(ids)
    assert j == L - (S - S64) * int(use64.sum())
    assert (got["out_ids"][j:] == -1).all() and (got["out_pos"][j:] == -1).all()


def test_compact_batch_one_bad_sequence():
    ids, emb, use64, o256, o64, cu, to, pieces = _batch_case([2, 2, 1], 16, 4, 2, 5)
    # drop one IMG_CONTEXT slot from sequence 1: its count no longer matches its tiles
    p = int(np.flatnonzero(ids[cu[1]:cu[2]] == IMG)[0]) + cu[1]
    ids = np.delete(ids, p)
    emb = np.delete(emb, p, axis=0)
    cu = cu.copy()
    cu[2:] -= 1
    got = O.compact_batch(ids, cu, emb, IMG, to, use64, o256, o64, 16, 4)
    assert got["status"] == O.STATUS_IMG_COUNT
    lens = np.diff(got["out_cu"])
    assert lens[1] == 0
    for b in (0, 2):
        sid, semb, suse, s256, s64 = pieces[b]
        assert lens[b] == len(_brute(sid, semb, suse, s256, s64, 16, 4)[0])
    assert (got["keep_map"][cu[1]:cu[2]] == -1).all()


@pytest.mark.parametrize("bad", ["cu_end", "cu_order", "tile_order", "tile_range"])
def test_compact_batch_rejects_bad_layout(bad):
    ids, emb, use64, o256, o64, cu, to, _ = _batch_case([1, 2], 4, 1, 2, 6)
    cu, to = cu.copy(), to.copy()
    if bad == "cu_end":
        cu[-1] -= 1
    elif bad == "cu_order":
        cu[1] = cu[2] + 1
    elif bad == "tile_order":
        to[1] = to[2] + 1
    else:
        to[-1] = len(use64) + 1
    got = O.compact_batch(ids, cu, emb, IMG, to, use64, o256, o64, 4, 1)
    assert got["status"] == O.STATUS_SEQ_LAYOUT
    assert (got["out_cu"] == 0).all() and (got["keep_map"] == -1).all()
