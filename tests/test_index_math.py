"""The kernels' index math on the CPU (libivc_index_check.so: index_math.h
built with bounds checks, walked the way the kernels decompose the work)
against the oracle, element by element:

* the loader's rows for the 256- and 64-token paths, every ps_version and
  64-path channel order, against the oracle's pixel_shuffle / shuffle64 of a
  tensor that holds each row's own index ([14B] pixel_shuffle and v1/v2
  sections; [2B-Flash] three token levels);
* the folded products' gathered A rows (route-first tile lists included),
  against the same, and the sign and range of the 32-bit offsets the DMA
  forms from each product tile's base row;
* the compaction closed form against the oracle's left-to-right walk
  ([4B-Flash] section 4; [14B] token injection).
"""
import ctypes
import os

import numpy as np
import pytest

import synth
from oracle import connector as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "vlm_visual_token_amd", "libivc_index_check.so")

i64p = ctypes.POINTER(ctypes.c_longlong)
i32p = ctypes.POINTER(ctypes.c_int32)
u8p = ctypes.POINTER(ctypes.c_uint8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from vlm_visual_token_amd import build
        build.build_index_check()
    L = ctypes.CDLL(LIB)
    L.ivc_check_loader_rows.restype = ctypes.c_longlong
    L.ivc_check_loader_rows.argtypes = [ctypes.c_int] * 6 + [i64p]
    L.ivc_check_gather.restype = ctypes.c_longlong
    L.ivc_check_gather.argtypes = [ctypes.c_int] * 6 + [i32p, ctypes.c_int, i64p]
    L.ivc_check_compact.restype = ctypes.c_longlong
    L.ivc_check_compact.argtypes = [i32p, ctypes.c_longlong, ctypes.c_int, u8p, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, i32p, i64p]
    L.ivc_index_failures.restype = ctypes.c_longlong
    L.ivc_index_reset()
    yield L
    assert L.ivc_index_failures() == 0


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _oracle_rows(T, P, has_cls, r, version, order):
    """Oracle permutation of a tensor whose single channel is the global row
    index: entry [t, tok, blk] = the ViT row feeding channel block blk."""
    rows = has_cls + P * P
    x = np.arange(T * rows, dtype=np.float64).reshape(T, rows, 1)
    G = O.token_grid(x, P, has_cls)
    if r == 2:
        y = O.pixel_shuffle(G, 2, version)
    else:
        y = O.shuffle64(G, order, version)
    return y.astype(np.int64)


GRIDS = [(P, cls, r, v, o) for P in (4, 8, 12, 16, 24, 32, 40, 48) for cls in (0, 1)
         for r in (2, 4) for v in (1, 2) for o in ("direct", "twice_r2")
         if P % r == 0 and not (o == "twice_r2" and r == 2)]


@pytest.mark.parametrize("P,has_cls,r,version,order", GRIDS)
def test_loader_rows_match_oracle(lib, P, has_cls, r, version, order):
    T = 3
    exp = _oracle_rows(T, P, has_cls, r, version, order)
    got = np.full(exp.size, -1, np.int64)
    n = lib.ivc_check_loader_rows(T, P, has_cls, r, 1 if version == 1 else 0,
                                  1 if order == "twice_r2" else 0, _ptr(got, i64p))
    assert n == exp.size
    assert np.array_equal(got.reshape(exp.shape), exp)


@pytest.mark.parametrize("P,has_cls,r,version,order", GRIDS)
@pytest.mark.parametrize("lst", ["all", "sparse"])
def test_gathered_rows_match_oracle_and_offsets_stay_unsigned(lib, P, has_cls, r, version, order,
                                                              lst):
    T = 7
    exp_all = _oracle_rows(T, P, has_cls, r, version, order)
    tiles = list(range(T)) if lst == "all" else [1, 2, 4, 6]
    exp = exp_all[tiles].reshape(-1)
    got = np.full(exp.size, -1, np.int64)
    ltab = np.asarray(tiles, np.int32)
    bad = lib.ivc_check_gather(P, 64, has_cls, r, 1 if version == 1 else 0,
                               1 if order == "twice_r2" else 0, _ptr(ltab, i32p), len(tiles),
                               _ptr(got, i64p))
    assert bad == 0  # no offset from a product tile's base row is negative or >= 4 GiB
    assert np.array_equal(got, exp)


def test_gather_base_fixes_v1_negative_offsets(lib):
    # the grids where a product tile starts inside a ViT tile under ps_version
    # 1 (the first row's own ViT row is then not the tile's lowest): checked
    # above through the kernel's base; the row-of-m0 base would go negative
    for P, r in ((24, 2), (48, 2), (40, 4)):
        Q = P // r
        S = Q * Q
        starts = [m0 for m0 in range(0, 4 * S, 256) if m0 % S]
        assert starts, (P, r)
        rows_v1 = _oracle_rows(4, P, 1, r, 1, "direct")[:, :, 0].reshape(-1)
        neg = sum(int(rows_v1[m0:m0 + 256].min() < rows_v1[m0]) for m0 in starts)
        assert neg > 0, (P, r)  # the old base was not the minimum on these grids


@pytest.mark.parametrize("name,seed,frac", [("tiny_flash_f32", 0, 0.5), ("tiny_flash_f32", 3, 0.0),
                                            ("tiny_flash_f32", 5, 1.0),
                                            ("internvl35_2b_flash", 0, 0.5)])
def test_compaction_closed_form_matches_oracle_walk(lib, name, seed, frac):
    cfg = synth.config(name)
    ids, _ = synth.make_sequence(cfg, seed, poison=False)
    T, S, S64 = cfg["T"], cfg["S"], cfg["S64"]
    rng = np.random.default_rng(seed)
    use = (rng.random(T) < frac).astype(np.uint8)
    L = len(ids)
    ids32 = np.ascontiguousarray(ids, np.int32)
    km = np.full(L, -7, np.int32)
    code = np.full(L, -7, np.int64)
    Lp = lib.ivc_check_compact(_ptr(ids32, i32p), L, synth.IMG_CONTEXT, _ptr(use, u8p), T, S, S64,
                               _ptr(km, i32p), _ptr(code, i64p))
    D = 1
    o256 = np.arange(T * S, dtype=np.float64).reshape(T, S, D) + 1e6
    o64 = np.arange(T * S64, dtype=np.float64).reshape(T, S64, D) + 2e6
    emb = np.arange(L, dtype=np.float64).reshape(L, D)
    ref = O.compact(ids, emb, synth.IMG_CONTEXT, use, o256, o64, S, S64)
    assert Lp == ref["out_len"]
    assert np.array_equal(km, ref["keep_map"])
    # the source code of each output row names the row the oracle copied
    src = code[:Lp]
    kind, idx = src >> 60, src & ((1 << 60) - 1)
    val = np.where(kind == 0, idx, np.where(kind == 1, idx + 1e6, idx + 2e6)).astype(np.float64)
    assert np.array_equal(val, ref["out_embeds"][:Lp, 0])


def test_compaction_rejects_wrong_slot_count(lib):
    cfg = synth.config("tiny_flash_f32")
    ids, _ = synth.make_sequence(cfg)
    ids = np.ascontiguousarray(ids[:-3], np.int32)  # drop the tail: IMG count still T*S
    img_pos = np.flatnonzero(ids == synth.IMG_CONTEXT)
    ids[img_pos[0]] = 5  # one slot fewer
    use = np.zeros(cfg["T"], np.uint8)
    km = np.zeros(len(ids), np.int32)
    code = np.zeros(len(ids), np.int64)
    Lp = lib.ivc_check_compact(_ptr(ids, i32p), len(ids), synth.IMG_CONTEXT, _ptr(use, u8p),
                               cfg["T"], cfg["S"], cfg["S64"], _ptr(km, i32p), _ptr(code, i64p))
    assert Lp == -1
