"""Pins for the oracle's CLS drop and pixel_shuffle (no GPU).

The index formula is tied to (1) brute-force bijection and an explicit
inverse, (2) torch's own space-to-depth routine ``pixel_unshuffle`` (same
grouping, channels reordered from torch's (c, m, k) to the connector's
(m, k, c)), (3) the head-to-tail concatenation order the 14B page describes,
and (4) the shapes and token counts the pages print.
"""
import numpy as np
import pytest
import torch

from oracle import connector as O


def _grid_ids(T, P, C):
    return np.arange(T * P * P * C, dtype=np.float64).reshape(T, P, P, C)


@pytest.mark.parametrize("P", [4, 8, 32])
@pytest.mark.parametrize("C", [1, 3, 8])
@pytest.mark.parametrize("r", [2, 4])
@pytest.mark.parametrize("version", [1, 2])
def test_bijection(P, C, r, version):
    G = _grid_ids(2, P, C)
    Y = O.pixel_shuffle(G, r, version)
    assert Y.shape == (2, (P // r) ** 2, r * r * C)
    assert np.array_equal(np.sort(Y.ravel()), G.ravel())


@pytest.mark.parametrize("P,C,r", [(8, 3, 2), (8, 2, 4), (32, 4, 2)])
def test_inverse_round_trip(P, C, r):
    G = _grid_ids(1, P, C)
    Y = O.pixel_shuffle(G, r)
    Q = P // r
    back = np.empty_like(G)
    # depth-to-space, written independently: token (a, b), channel block q
    for tok in range(Q * Q):
        a, b = divmod(tok, Q)
        for q in range(r * r):
            m, k = divmod(q, r)
            back[0, r * a + m, r * b + k] = Y[0, tok, q * C:(q + 1) * C]
    assert np.array_equal(back, G)


@pytest.mark.parametrize("P,C,r", [(8, 5, 2), (8, 3, 4), (32, 16, 2), (32, 4, 4)])
def test_matches_torch_pixel_unshuffle(P, C, r):
    rng = np.random.default_rng(1)
    G = rng.standard_normal((3, P, P, C))
    Y = O.pixel_shuffle(G, r)
    # torch: NCHW with H = grid row i, W = grid column j;
    # output channel = c * r^2 + m * r + k at spatial (a, b).
    pu = torch.nn.functional.pixel_unshuffle(torch.from_numpy(G).permute(0, 3, 1, 2), r)
    Q = P // r
    pu = pu.reshape(3, C, r, r, Q, Q).permute(0, 4, 5, 2, 3, 1).reshape(3, Q * Q, r * r * C)
    assert np.array_equal(Y, pu.numpy())


def test_head_to_tail_order():
    # 14B page, pixel_shuffle walkthrough: step 1 joins each 2 consecutive
    # tokens along the inner grid axis head to tail (C -> 2C), step 3 joins 2
    # consecutive ones along the outer axis (2C -> 4C).  So channel block 0 is
    # cell (2a, 2b), block 1 is (2a, 2b+1), block 2 is (2a+1, 2b), block 3 is
    # (2a+1, 2b+1).
    P, C = 4, 2
    G = _grid_ids(1, P, C)
    Y = O.pixel_shuffle(G, 2)
    for a in range(2):
        for b in range(2):
            row = Y[0, a * 2 + b]
            cells = [(2 * a, 2 * b), (2 * a, 2 * b + 1), (2 * a + 1, 2 * b), (2 * a + 1, 2 * b + 1)]
            for blk, (i, j) in enumerate(cells):
                assert np.array_equal(row[blk * C:(blk + 1) * C], G[0, i, j])


def test_cls_drop_and_grid(golden):
    g = golden("shape_walk.txt")
    P = int(g["grid"][0])
    assert int(g["image_size"][0]) // int(g["patch_size"][0]) == P
    assert P * P == int(g["patch_tokens"][0])
    rows = int(g["tokens_with_cls"][0])
    C = 4
    x = np.arange(rows * C, dtype=np.float64).reshape(1, rows, C)
    G = O.token_grid(x, P, 1)
    assert G.shape == (1, P, P, C)
    # CLS (row 0) never appears; grid (i, j) is row 1 + i*P + j
    assert not np.isin(x[0, 0], G).any()
    assert np.array_equal(G[0, 3, 5], x[0, 1 + 3 * P + 5])


def test_page_shapes_and_counts(golden):
    g = golden("shape_walk.txt")
    n, P, _, C = (int(v) for v in g["ps_in"])
    G = np.zeros((n, P, P, C))
    Y = O.pixel_shuffle(G, 2)
    assert (n, int(np.sqrt(Y.shape[1])), int(np.sqrt(Y.shape[1])), Y.shape[2]) == tuple(
        int(v) for v in g["ps_out"])
    assert Y.shape[1:] == (int(g["ef_tokens"][0]), int(g["ef_width"][0]))
    tiles = int(g["tiles_with_thumb"][0])
    assert tiles * P * P == int(g["tokens_before"][0])
    assert tiles * Y.shape[1] == int(g["tokens_after"][0])


def test_token_levels(golden):
    lv = golden("token_levels.txt")
    P, C = int(lv["vit"][1]), int(lv["vit"][3])
    G = np.zeros((1, P, P, 1))
    for name, r in (("std", 2), ("flash", 4)):
        scale, grid, tokens, width = float(lv[name][0]), int(lv[name][1]), int(lv[name][2]), int(lv[name][3])
        assert r == int(round(1 / scale))
        Y = O.pixel_shuffle(G, r)
        assert Y.shape[1] == grid * grid == tokens
        assert Y.shape[2] * C == width


def test_r4_differs_from_twice_r2_only_by_channel_order():
    # The 64-token path's default is the direct r=4 formula.  Two successive
    # r=2 shuffles gather the same 16 cells into each token, in a different
    # channel order.
    P, C = 8, 2
    G = _grid_ids(1, P, C)
    direct = O.pixel_shuffle(G, 4)
    twice = O.pixel_shuffle(O.pixel_shuffle(G, 2).reshape(1, P // 2, P // 2, 4 * C), 2)
    assert direct.shape == twice.shape
    assert np.array_equal(np.sort(direct, axis=-1), np.sort(twice, axis=-1))
    assert not np.array_equal(direct, twice)


def _torch_unshuffle(G, r):
    """torch's pixel_unshuffle with channels reordered to the connector's
    (m, k, c) order, as [T, P/r, P/r, r*r*C] (spatial axes a, b)."""
    T, P, _, C = G.shape
    Q = P // r
    pu = torch.nn.functional.pixel_unshuffle(torch.from_numpy(G).permute(0, 3, 1, 2), r)
    return pu.reshape(T, C, r, r, Q, Q).permute(0, 4, 5, 2, 3, 1).reshape(T, Q, Q, r * r * C).numpy()


@pytest.mark.parametrize("P,C,r", [(8, 5, 2), (8, 3, 4), (32, 4, 2), (32, 2, 4)])
def test_v1_is_transposed_token_grid(P, C, r):
    # 14B page, v1/v2 section: v1 does not swap the two spatial axes back, so
    # its output grid is the transpose of v2's (token (a, b) lands at b, a),
    # channels unchanged.  Checked against torch's space-to-depth.
    rng = np.random.default_rng(2)
    G = rng.standard_normal((2, P, P, C))
    Q = P // r
    want = _torch_unshuffle(G, r).transpose(0, 2, 1, 3).reshape(2, Q * Q, r * r * C)
    assert np.array_equal(O.pixel_shuffle(G, r, 1), want)
    assert not np.array_equal(O.pixel_shuffle(G, r, 1), O.pixel_shuffle(G, r, 2))


def test_shuffle64_orders_worked_example():
    # P = 4, C = 1, cell (i, j) holds 10*i + j; the single 64-path token of
    # the tile, channel by channel.  direct: the 4 x 4 block row by row.
    # twice_r2: the r = 2 shuffle (2 x 2 cells in the order (0,0), (0,1),
    # (1,0), (1,1)) applied to 2 x 2 blocks taken in that same order.
    G = np.array([[10.0 * i + j for j in range(4)] for i in range(4)]).reshape(1, 4, 4, 1)
    direct = [0, 1, 2, 3, 10, 11, 12, 13, 20, 21, 22, 23, 30, 31, 32, 33]
    twice = [0, 1, 10, 11, 2, 3, 12, 13, 20, 21, 30, 31, 22, 23, 32, 33]
    assert O.shuffle64(G, "direct")[0, 0].tolist() == direct
    assert O.shuffle64(G, "twice_r2")[0, 0].tolist() == twice
    for v in (1, 2):  # one token: the transpose changes nothing
        assert O.shuffle64(G, "twice_r2", v)[0, 0].tolist() == twice


@pytest.mark.parametrize("P,C", [(8, 3), (32, 2)])
@pytest.mark.parametrize("version", [1, 2])
def test_shuffle64_twice_matches_torch_twice(P, C, version):
    rng = np.random.default_rng(3)
    G = rng.standard_normal((2, P, P, C))
    Q = P // 4
    twice = _torch_unshuffle(_torch_unshuffle(G, 2), 2)
    if version == 1:
        twice = twice.transpose(0, 2, 1, 3)
    assert np.array_equal(O.shuffle64(G, "twice_r2", version), twice.reshape(2, Q * Q, 16 * C))
    direct = _torch_unshuffle(G, 4)
    if version == 1:
        direct = direct.transpose(0, 2, 1, 3)
    assert np.array_equal(O.shuffle64(G, "direct", version), direct.reshape(2, Q * Q, 16 * C))
