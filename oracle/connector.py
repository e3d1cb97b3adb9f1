"""Plain CPU oracle of InternVL's visual-token compression connector.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check the HIP kernels and to
time a CPU baseline.  It shares no code with ``vlm_visual_token_amd``.

Everything is computed in float64 from the float32/bf16 inputs widened
exactly.  Reductions are plain numpy sums, matrix products use numpy's
``matmul`` as a library primitive, ``sort`` is numpy's; there is no blocking,
fusion or reordering beyond the definitions below.

Pages cited (titles abbreviated):

* [14B] "InternVL3-14B-Instruct: pixel shuffle and MLP connector, line by line"
  (zwxr.cn/news/271642).
* [4B-Flash] "InternVL3_5-4B-Flash Gating and CrossAttentionPooling explained"
  (mrgr.cn/news/14598).
* [2B-Flash] "InternVL3_5-2B-Flash dual-path visual-token compression pipeline"
  (kwkr.cn/news/620108).
* [4B] "InternVL3.5-4B architecture deep dive" (lmnt.cn/news/105786).

Pins (tests that tie each function to something other than itself) live in
``tests/test_oracle_*.py``.  Numeric values of the mlp1/mlp2 outputs and of
the gate probabilities are not printed on any page: those functions are pinned
by closed forms, invariants and library cross-checks, not by page values.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

STATUS_OK = 0
STATUS_IMG_COUNT = 1  # IMG_CONTEXT slots in the sequence != tiles * slots per tile
STATUS_SEQ_LAYOUT = 8  # batch: sequence or tile offsets not an ordered partition


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# a1: ragged tile offsets
# ---------------------------------------------------------------------------
def tile_offsets(tiles_per_image) -> np.ndarray:
    """Exclusive prefix sum over per-image tile counts: off[0] = 0,
    off[i+1] = off[i] + tiles[i].  Splits the batch's tiles into per-image
    lists ([4B-Flash] section 5, the split-and-merge step)."""
    off = [0]
    for n in tiles_per_image:
        off.append(off[-1] + int(n))
    return np.array(off, dtype=np.int64)


# ---------------------------------------------------------------------------
# a2-a3: CLS drop, token grid, pixel shuffle (v2)
# ---------------------------------------------------------------------------
def token_grid(x, P: int, has_cls: int) -> np.ndarray:
    """Drop the CLS row and lay the remaining P*P tokens out as a P x P grid:
    grid (i, j) is row has_cls + i*P + j ([14B] extract_feature walkthrough,
    steps 3-5)."""
    x = f64(x)
    T, rows, C = x.shape
    assert rows == has_cls + P * P
    return x[:, has_cls:, :].reshape(T, P, P, C)


def pixel_shuffle(G, r: int, version: int = 2) -> np.ndarray:
    """Space-to-depth by r, written as explicit index math:

        out[a*(P/r) + b, (r*m + k)*C + c] = G[r*a + m, r*b + k, c]

    for a, b < P/r and m, k < r.  [14B] section on pixel_shuffle: each step
    concatenates neighbouring tokens' feature vectors head to tail along one
    grid axis, then the other; v2 swaps the axes back so the grid is not
    transposed.  r = 2 is downsample ratio 0.5 (256 tokens of 4C); r = 4 is
    ratio 0.25 (64 tokens of 16C, [2B-Flash] three token levels).

    version = 1 is the older ps_version of the same page (section on v1 and
    v2): the axes are not swapped back, so the output token grid is the
    transpose of v2's; channels are unchanged:

        out_v1[b*(P/r) + a] = out_v2[a*(P/r) + b]
    """
    T, P, P2, C = G.shape
    assert P == P2 and P % r == 0 and version in (1, 2)
    Q = P // r
    out = np.empty((T, Q * Q, r * r * C), dtype=G.dtype)
    for a in range(Q):
        for b in range(Q):
            tok = a * Q + b if version == 2 else b * Q + a
            for m in range(r):
                for k in range(r):
                    blk = r * m + k
                    out[:, tok, blk * C:(blk + 1) * C] = G[:, r * a + m, r * b + k, :]
    return out


SHUFFLE64_ORDERS = ("direct", "twice_r2")


def shuffle64(G, order: str = "direct", version: int = 2) -> np.ndarray:
    """The 64-token path's input, [T, (P/4)^2, 16C].

    [2B-Flash] three token levels: scale 0.25 = 0.5 squared, described as
    equivalent to two pixel_shuffles.  Both readings gather the same 4 x 4
    cells into a token and differ only in channel order:

    * "direct": pixel_shuffle(G, 4), the r = 4 formula
      (channel block 4*M + K for cell (M, K) of the 4 x 4 block);
    * "twice_r2": the r = 2 shuffle applied to the 16 x 16 grid of 4C
      tokens that the first r = 2 shuffle makes (channel block
      4*(2*m2 + k2) + (2*m + k) for cell (2*m2 + m, 2*k2 + k)).

    version = 1 transposes the resulting token grid, as for pixel_shuffle.
    """
    assert order in SHUFFLE64_ORDERS
    T, P, _, C = G.shape
    if order == "direct":
        return pixel_shuffle(G, 4, version)
    Y2 = pixel_shuffle(G, 2).reshape(T, P // 2, P // 2, 4 * C)
    return pixel_shuffle(Y2, 2, version)


# ---------------------------------------------------------------------------
# a4-a7: LayerNorm, Linear, GELU, mlp1, mlp2
# ---------------------------------------------------------------------------
def layer_norm(y, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm over the last axis, biased variance, two passes:
    mu = mean(y); var = mean((y - mu)^2); (y - mu) / sqrt(var + eps) * gamma + beta."""
    y = f64(y)
    mu = y.mean(axis=-1, keepdims=True)
    d = y - mu
    var = (d * d).mean(axis=-1, keepdims=True)
    return d / np.sqrt(var + eps) * f64(gamma) + f64(beta)


def linear(x, W, b) -> np.ndarray:
    """torch nn.Linear layout: W is [out, in]; y = x W^T + b."""
    return f64(x) @ f64(W).T + f64(b)


def gelu(z) -> np.ndarray:
    """Exact (erf) GELU: 0.5 z (1 + erf(z / sqrt 2))."""
    z = f64(z)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def mlp1(Y, w: dict, eps: float) -> np.ndarray:
    """LayerNorm(4C) -> Linear(4C -> hidden) -> GELU -> Linear(hidden -> D)
    ([14B] MLP connector section; [4B] layer-2 projector)."""
    h = layer_norm(Y, w["mlp1.ln.w"], w["mlp1.ln.b"], eps)
    h = gelu(linear(h, w["mlp1.l1.w"], w["mlp1.l1.b"]))
    return linear(h, w["mlp1.l2.w"], w["mlp1.l2.b"])


def mlp2(Y, w: dict, eps: float) -> np.ndarray:
    """The deeper projector of the 64-token path: LayerNorm(16C) ->
    Linear(16C -> 4096) -> GELU -> Linear(4096 -> 4096) -> GELU ->
    Linear(4096 -> D).  [2B-Flash] says only "three layers, intermediate
    width 4096"; the LayerNorm and GELU placement mirrors mlp1."""
    h = layer_norm(Y, w["mlp2.ln.w"], w["mlp2.ln.b"], eps)
    h = gelu(linear(h, w["mlp2.l1.w"], w["mlp2.l1.b"]))
    h = gelu(linear(h, w["mlp2.l2.w"], w["mlp2.l2.b"]))
    return linear(h, w["mlp2.l3.w"], w["mlp2.l3.b"])


def shuffled(x, cfg: dict, r: int) -> np.ndarray:
    """The projector input of one path, [T, (P/r)^2, r^2 C]: pixel_shuffle
    (r = 2) or the 64-token shuffle (r = 4) of the token grid, with the
    config's ps_version (default 2) and 64-path channel order (default
    "direct")."""
    G = token_grid(x, cfg["P"], cfg["has_cls"])
    version = cfg.get("ps_version", 2)
    if r == 2:
        return pixel_shuffle(G, 2, version)
    return shuffle64(G, cfg.get("shuffle64_order", "direct"), version)


def shuffled_ln_rows(x, cfg: dict, w: dict, r: int) -> np.ndarray:
    """The LayerNorm'd pixel-shuffled rows (the first projector's input after
    its LayerNorm), [T, (P/r)^2, r^2 C]."""
    key = "mlp1.ln" if r == 2 else "mlp2.ln"
    return layer_norm(shuffled(x, cfg, r), w[key + ".w"], w[key + ".b"], cfg["ln_eps"])


def connector_run(x, cfg: dict, w: dict):
    """extract_feature ([14B]) and, for Flash models, the 64-token branch of
    extract_feature_flash ([2B-Flash] dual pipeline, step 2):

        out256 = mlp1(pixel_shuffle(grid(x), 2))      [T, 256, D]
        out64  = mlp2(shuffle64(grid(x)))             [T, 64, D]  (Flash only)
    """
    out256 = mlp1(shuffled(x, cfg, 2), w, cfg["ln_eps"])
    out64 = mlp2(shuffled(x, cfg, 4), w, cfg["ln_eps"]) if cfg["flash"] else None
    return out256, out64


# ---------------------------------------------------------------------------
# a8-a9: CrossAttentionPooling
# ---------------------------------------------------------------------------
def softmax(z, axis=-1) -> np.ndarray:
    z = f64(z)
    e = np.exp(z - z.max(axis=axis, keepdims=True))
    return e / e.sum(axis=axis, keepdims=True)


def cross_attention_pooling(x, cfg: dict, w: dict, valid=None) -> np.ndarray:
    """One learnable query attends over each tile's tokens, four times.

    [4B-Flash] section 2: a learnable query token reads all of a tile's
    tokens through four multi-head cross-attention layers (attn1..attn4),
    refining itself each round; padded tokens are masked out; the result is
    one vector per tile.  Each layer is standard multi-head attention with
    biased Q/K/V in-projections, scale 1/sqrt(d) with d = C / heads, and a
    biased out-projection; the layer's output is the next layer's query.
    Keys and values are the tile's ViT tokens (CLS dropped).  Only the first
    ``valid[t]`` tokens of tile t are read.
    """
    G = token_grid(x, cfg["P"], cfg["has_cls"])
    T, P, _, C = G.shape
    N = P * P
    H = cfg["pool_heads"]
    d = C // H
    toks = G.reshape(T, N, C)
    out = np.empty((T, C), dtype=np.float64)
    for t in range(T):
        n = N if valid is None else int(valid[t])
        assert 1 <= n <= N
        xs = toks[t, :n]
        q = f64(w["pool.query"])
        for l in range(cfg["pool_layers"]):
            Q = linear(q, w[f"pool.{l}.q.w"], w[f"pool.{l}.q.b"])
            K = linear(xs, w[f"pool.{l}.k.w"], w[f"pool.{l}.k.b"])
            V = linear(xs, w[f"pool.{l}.v.w"], w[f"pool.{l}.v.b"])
            o = np.empty(C, dtype=np.float64)
            for h in range(H):
                sl = slice(h * d, (h + 1) * d)
                s = K[:, sl] @ Q[sl] / math.sqrt(d)
                p = softmax(s)
                o[sl] = p @ V[:, sl]
            q = linear(o, w[f"pool.{l}.o.w"], w[f"pool.{l}.o.b"])
        out[t] = q
    return out


# ---------------------------------------------------------------------------
# a10: Gating
# ---------------------------------------------------------------------------
def gating(pooled, cfg: dict, w: dict) -> np.ndarray:
    """[4B-Flash] section 3: four residual MLP blocks, each
    Linear -> GELU -> Dropout -> Linear -> Dropout -> LayerNorm added back
    onto its input (dropout is the identity at inference), then a
    Linear(hidden, 2) classifier and a softmax.  Returns probabilities [T, 2];
    column 0 is the confidence that the tile can take the 64-token path."""
    x = f64(pooled)
    eps = cfg["ln_eps"]
    for b in range(4):
        y = gelu(linear(x, w[f"gate.{b}.l1.w"], w[f"gate.{b}.l1.b"]))
        y = linear(y, w[f"gate.{b}.l2.w"], w[f"gate.{b}.l2.b"])
        x = x + layer_norm(y, w[f"gate.{b}.ln.w"], w[f"gate.{b}.ln.b"], eps)
    z = linear(x, w["gate.cls.w"], w["gate.cls.b"])
    return softmax(z, axis=-1)


# ---------------------------------------------------------------------------
# a11: quantile threshold and routing decision
# ---------------------------------------------------------------------------
def _lerp(a: float, b: float, t: float) -> float:
    # Linear interpolation, evaluated from whichever end is nearer (the form
    # torch.lerp and numpy's "linear" quantile use).
    if t < 0.5:
        return a + t * (b - a)
    return b - (b - a) * (1.0 - t)


def quantile_linear(values, q: float) -> float:
    """The q-quantile with linear interpolation between order statistics:
    pos = q (n - 1), lo = floor(pos), hi = ceil(pos),
    result = lerp(v[lo], v[hi], pos - lo) over the sorted values, in float64."""
    v = np.sort(f64(values).ravel())
    n = v.shape[0]
    assert n >= 1
    pos = float(q) * (n - 1)
    lo = int(math.floor(pos))
    hi = int(math.ceil(pos))
    return _lerp(float(v[lo]), float(v[hi]), pos - lo)


def route_decision(g0, thr: float, abs_threshold: float) -> np.ndarray:
    """A tile takes the 64-token path when both hold: g0 > the batch's
    relative-threshold quantile, and g0 >= the absolute threshold
    ([4B-Flash] section 4; [2B-Flash] routing decision: "both must hold")."""
    g = f64(g0)
    return ((g > thr) & (g >= abs_threshold)).astype(np.uint8)


def connector_route(x, cfg: dict, w: dict, valid=None):
    """Visual Resolution Router for a batch: pool -> gate -> quantile -> decision.

    Gate probabilities are returned as float32 (the form the GPU emits); the
    quantile and the decision are taken on those float32 values widened to
    float64.  The quantile covers every tile passed in (the decision needs the
    whole batch's gates, [4B-Flash] section 5)."""
    pooled = cross_attention_pooling(x, cfg, w, valid)
    gate = gating(pooled, cfg, w).astype(np.float32)
    thr, use64 = decide(gate[:, 0], cfg)
    return gate, thr, use64, pooled


def decide(g0_f32, cfg: dict):
    """Quantile threshold and per-tile decision from float32 gate[:, 0]."""
    g = f64(np.asarray(g0_f32, dtype=np.float32))
    thr = quantile_linear(g, cfg["rel_quantile"])
    return thr, route_decision(g, thr, cfg["abs_threshold"])


# ---------------------------------------------------------------------------
# a12: compaction of IMG_CONTEXT slots and embedding assembly
# ---------------------------------------------------------------------------
def compact(ids, embeds, img_context_id: int, use64, out256, out64, S: int, S64: int):
    """Walk the sequence left to right; the k-th IMG_CONTEXT slot belongs to
    tile k // S at local slot k % S (the injection order of [14B] section on
    token injection).  A tile routed to the 64-token path keeps only its first
    S64 slots, filled with its 64-token features; its other S - S64 slots are
    deleted and the sequence really shortens ([4B-Flash] section 4;
    [2B-Flash] routing decision).  Positions are renumbered 0..L'-1.

    Returns a dict: out_ids [L] (-1 past out_len), out_pos [L] (-1 past
    out_len), keep_map [L] (new index or -1), out_embeds [L, D] (rows past
    out_len are zero), out_len, status.
    """
    ids = np.asarray(ids)
    L = ids.shape[0]
    T = len(use64)
    D = embeds.shape[1]
    out_ids = np.full(L, -1, dtype=np.int64)
    out_pos = np.full(L, -1, dtype=np.int64)
    keep_map = np.full(L, -1, dtype=np.int64)
    out_emb = np.zeros((L, D), dtype=np.float64)
    n_img = int(np.count_nonzero(ids == img_context_id))
    if n_img != T * S:
        return dict(out_ids=out_ids, out_pos=out_pos, keep_map=keep_map,
                    out_embeds=out_emb, out_len=0, status=STATUS_IMG_COUNT)
    j = 0
    k = 0
    for p in range(L):
        tok = int(ids[p])
        if tok == img_context_id:
            tile, loc = divmod(k, S)
            k += 1
            if use64[tile]:
                if loc >= S64:
                    continue
                row = out64[tile][loc]
            else:
                row = out256[tile][loc]
        else:
            row = embeds[p]
        out_ids[j] = tok
        out_pos[j] = j
        keep_map[p] = j
        out_emb[j] = row
        j += 1
    return dict(out_ids=out_ids, out_pos=out_pos, keep_map=keep_map,
                out_embeds=out_emb, out_len=j, status=STATUS_OK)



def compact_batch(ids, cu_seqlens, embeds, img_context_id: int, tile_offsets, use64, out256,
                  out64, S: int, S64: int):
    """Compaction of B prompts packed back to back (variable-length batch).

    Sequence b is positions cu_seqlens[b] .. cu_seqlens[b+1]-1 of ``ids``
    and its images own tiles tile_offsets[b] .. tile_offsets[b+1]-1 (image
    order within the sequence, as for one prompt).  Every sequence is
    compacted on its own exactly as ``compact`` does for one prompt: its
    k-th IMG_CONTEXT slot is local slot k % S of its (k // S)-th tile, a
    routed tile keeps its first S64 slots ([4B-Flash] section 4), and its
    positions restart at 0.  The compacted sequences are packed back to back:
    out_cu[0] = 0, out_cu[b+1] = out_cu[b] + L'_b, and keep_map holds packed
    indices.  A sequence whose IMG_CONTEXT count differs from S times its
    tile count compacts to length 0 (status STATUS_IMG_COUNT); the others
    are unaffected.  Offsets that are not an ordered partition (cu_seqlens
    from 0 to L, non-decreasing; tile_offsets non-decreasing within [0, T])
    give status STATUS_SEQ_LAYOUT and an empty result.

    Returns a dict like ``compact``'s, with out_pos holding per-sequence
    positions and out_cu [B+1] in place of out_len.
    """
    ids = np.asarray(ids)
    cu = [int(v) for v in cu_seqlens]
    to = [int(v) for v in tile_offsets]
    L = ids.shape[0]
    B = len(cu) - 1
    T = len(use64)
    D = embeds.shape[1]
    out_ids = np.full(L, -1, dtype=np.int64)
    out_pos = np.full(L, -1, dtype=np.int64)
    keep_map = np.full(L, -1, dtype=np.int64)
    out_emb = np.zeros((L, D), dtype=np.float64)
    out_cu = np.zeros(B + 1, dtype=np.int64)
    layout_ok = (len(to) == B + 1 and cu[0] == 0 and cu[B] == L and to[0] >= 0 and to[B] <= T
                 and all(cu[b] <= cu[b + 1] and to[b] <= to[b + 1] for b in range(B)))
    if not layout_ok:
        return dict(out_ids=out_ids, out_pos=out_pos, keep_map=keep_map, out_embeds=out_emb,
                    out_cu=out_cu, status=STATUS_SEQ_LAYOUT)
    status = STATUS_OK
    for b in range(B):
        p0, p1, t0, t1 = cu[b], cu[b + 1], to[b], to[b + 1]
        one = compact(ids[p0:p1], embeds[p0:p1], img_context_id, use64[t0:t1],
                      out256[t0:t1], None if out64 is None else out64[t0:t1], S, S64)
        n = one["out_len"]
        j0 = int(out_cu[b])
        out_cu[b + 1] = j0 + n
        if one["status"] != STATUS_OK:
            status |= one["status"]
            continue
        out_ids[j0:j0 + n] = one["out_ids"][:n]
        out_pos[j0:j0 + n] = one["out_pos"][:n]
        out_emb[j0:j0 + n] = one["out_embeds"][:n]
        kept = one["keep_map"] >= 0
        keep_map[p0:p1][kept] = one["keep_map"][kept] + j0
    return dict(out_ids=out_ids, out_pos=out_pos, keep_map=keep_map, out_embeds=out_emb,
                out_cu=out_cu, status=status)
