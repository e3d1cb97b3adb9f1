"""Seeded, order-independent synthetic workloads with the pages' shapes.

Every tensor is drawn from its own numpy ``Generator`` keyed by
``(seed, tensor_id, index)``: ``tensor_id`` is the CRC-32 of the tensor's
name and ``index`` a tile or layer number, so any tile can be regenerated on
its own (the oracle checks sampled tiles of the large workloads) and the same
bytes come out on every machine with this numpy.

Shapes follow the InternVL pages: a 448x448 tile gives a 32x32 ViT grid plus
one CLS token (InternVL3-14B-Instruct pixel-shuffle page, section on why a
tile has 1024 tokens); images are cut into 1-12 tiles plus a thumbnail
(InternVL3.5-4B architecture page, data-flow overview); the Flash models route
each tile to 256 or 64 IMG_CONTEXT slots (InternVL3_5-2B-Flash page, routing
section).  Value distributions are synthetic stand-ins: there are no trained
weights or images here.

bf16 workloads are returned as float32 arrays whose values are exactly
representable in bfloat16 (rounded to nearest even), so the oracle can widen
them losslessly and the GPU receives the same numbers.
"""
from __future__ import annotations

import zlib

import numpy as np

# Special token ids.  The real ids live in the model's added_tokens.json, which
# is not available; these sit just past the Qwen3 text vocabulary (151,936
# entries, InternVL3.5-4B architecture page, Qwen3-4B layer table) so they
# cannot collide with synthetic text ids drawn from [0, TEXT_VOCAB).
TEXT_VOCAB = 151936
IMG_START = 151936
IMG_END = 151937
IMG_CONTEXT = 151938


def _base(**kw):
    c = dict(
        dtype="bf16",
        P=32,
        has_cls=1,
        C=1024,
        D=2048,
        mlp1_hidden=2048,
        flash=0,
        mlp2_hidden=4096,
        pool_layers=4,
        pool_heads=16,
        gate_hidden=1024,
        gate_expansion=1,
        rel_quantile=0.1,
        abs_threshold=0.5,
        ln_eps=1e-5,
        images=1,
        tiles_per_image=None,  # list[int] or None (uniform 13)
        text_per_image=30,
        x_recipe="lognormal",
    )
    c.update(kw)
    return c


CONFIGS = {
    # Tiny Flash path in fp32: 8 tiles of an 8x8 grid (65 tokens with CLS), C=64.
    "tiny_flash_f32": _base(
        dtype="f32", P=8, C=64, D=128, mlp1_hidden=128, flash=1, mlp2_hidden=256,
        pool_layers=4, pool_heads=4, gate_hidden=64, images=2, tiles_per_image=[4, 4],
        text_per_image=6, x_recipe="normal"),
    # InternVL3.5-4B standard connector: 8 images x 13 tiles, D = 2560.
    "internvl35_4b_std": _base(
        C=1024, D=2560, mlp1_hidden=2560, flash=0, images=8, tiles_per_image=[13] * 8),
    # InternVL3.5-2B-Flash: dual path + router, 16 images x 13 tiles, D = 2048.
    "internvl35_2b_flash": _base(
        C=1024, D=2048, mlp1_hidden=2048, flash=1, mlp2_hidden=4096, pool_layers=4,
        pool_heads=16, gate_hidden=1024, images=16, tiles_per_image=[13] * 16,
        text_per_image=30, x_recipe="structured"),
    # InternVL3-14B: 32 images with U{1..12} tiles + thumbnail each, D = 5120.
    "internvl3_14b_ragged": _base(
        C=1024, D=5120, mlp1_hidden=5120, flash=0, images=32, tiles_per_image="ragged"),
    # InternVL3-38B: InternViT-6B width 3200, 16 images x 13 tiles, D = 5120.
    "internvl3_38b": _base(
        C=3200, D=5120, mlp1_hidden=5120, flash=0, images=16, tiles_per_image=[13] * 16),
}


def _tid(name: str) -> int:
    return zlib.crc32(name.encode("utf-8"))


def _rng(seed: int, name: str, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), _tid(name), int(index)])


def make_tiles_per_image(cfg: dict, seed: int = 0) -> list[int]:
    """Tiles per image: fixed lists, or U{1..12} + 1 thumbnail for the ragged workload."""
    tpi = cfg["tiles_per_image"]
    if tpi == "ragged":
        r = _rng(seed, "tiles_per_image")
        return [int(v) + 1 for v in r.integers(1, 13, size=cfg["images"])]
    return list(tpi)


def config(name: str, seed: int = 0) -> dict:
    """A workload description: model widths, thresholds and batch layout."""
    cfg = dict(CONFIGS[name])
    cfg["name"] = name
    cfg["tiles"] = make_tiles_per_image(cfg, seed)
    cfg["T"] = int(sum(cfg["tiles"]))
    P = cfg["P"]
    cfg["N"] = P * P
    cfg["rows"] = cfg["has_cls"] + P * P
    cfg["S"] = (P // 2) ** 2
    cfg["S64"] = (P // 4) ** 2 if cfg["flash"] else 0
    return cfg


def to_bf16_exact(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); NaN stays NaN.

    Returned as float32 holding bf16-representable values.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def _finish(cfg: dict, a: np.ndarray) -> np.ndarray:
    a = a.astype(np.float32, copy=False)
    return to_bf16_exact(a) if cfg["dtype"] == "bf16" else np.ascontiguousarray(a)


def _normal(seed, name, shape, index=0, std=1.0, mean=0.0):
    g = _rng(seed, name, index)
    return (g.standard_normal(size=shape, dtype=np.float64) * std + mean).astype(np.float32)


def make_weights(cfg: dict, seed: int = 0, gate_bias0: float | None = None) -> dict:
    """All connector parameters in torch ``nn.Linear`` layout ([out, in]).

    Linear weights ~ N(0, 1/fan_in); biases ~ 0.1 N(0,1); LayerNorm
    gamma ~ 1 + 0.1 N(0,1), beta ~ 0.1 N(0,1); the pooling query ~ N(0,1).
    ``gate_bias0`` sets the first class bias of the gating classifier (the
    second stays 0); it is the knob that puts about half of the tiles above
    the absolute threshold.
    """
    C, D = cfg["C"], cfg["D"]
    w: dict[str, np.ndarray] = {}

    def lin(prefix, n_out, n_in):
        w[prefix + ".w"] = _finish(cfg, _normal(seed, prefix + ".w", (n_out, n_in), std=n_in ** -0.5))
        w[prefix + ".b"] = _finish(cfg, _normal(seed, prefix + ".b", (n_out,), std=0.1))

    def ln(prefix, n):
        w[prefix + ".w"] = _finish(cfg, _normal(seed, prefix + ".w", (n,), std=0.1, mean=1.0))
        w[prefix + ".b"] = _finish(cfg, _normal(seed, prefix + ".b", (n,), std=0.1))

    W4 = 4 * C
    ln("mlp1.ln", W4)
    lin("mlp1.l1", cfg["mlp1_hidden"], W4)
    lin("mlp1.l2", D, cfg["mlp1_hidden"])
    if cfg["flash"]:
        W16, H2 = 16 * C, cfg["mlp2_hidden"]
        ln("mlp2.ln", W16)
        lin("mlp2.l1", H2, W16)
        lin("mlp2.l2", H2, H2)
        lin("mlp2.l3", D, H2)
        w["pool.query"] = _finish(cfg, _normal(seed, "pool.query", (C,)))
        for l in range(cfg["pool_layers"]):
            for p in ("q", "k", "v", "o"):
                lin(f"pool.{l}.{p}", C, C)
        h = cfg["gate_hidden"]
        he = h * cfg["gate_expansion"]
        for b in range(4):
            lin(f"gate.{b}.l1", he, h)
            lin(f"gate.{b}.l2", h, he)
            ln(f"gate.{b}.ln", h)
        w["gate.cls.w"] = _finish(cfg, _normal(seed, "gate.cls.w", (2, h), std=h ** -0.5))
        b0 = 0.0 if gate_bias0 is None else float(gate_bias0)
        w["gate.cls.b"] = _finish(cfg, np.array([b0, 0.0], dtype=np.float32))
    return w


def make_vit_tiles(cfg: dict, tiles, seed: int = 0) -> np.ndarray:
    """ViT output rows (CLS first when ``has_cls``) for the listed tile indices.

    Recipes: ``normal``: N(0,1).  ``lognormal``: s_c * z with a per-channel
    scale s_c = exp(0.5 N(0,1)) shared by all tiles and tokens.
    ``structured``: s_c * (mu_t[c] + tau_t * z) with a per-tile channel mean
    mu_t ~ 0.5 N(0,1) and a per-tile spread tau_t ~ U(0.25, 1); it stands in
    for tiles that range from flat background to dense detail, so the router
    has something to rank.
    """
    tiles = [int(t) for t in tiles]
    rows, C = cfg["rows"], cfg["C"]
    out = np.empty((len(tiles), rows, C), dtype=np.float32)
    rec = cfg["x_recipe"]
    if rec != "normal":
        s_c = np.exp(0.5 * _normal(seed, "x.scale", (C,)).astype(np.float64)).astype(np.float32)
    for i, t in enumerate(tiles):
        g = _rng(seed, "x", t)
        z = g.standard_normal(size=(rows, C), dtype=np.float32)
        if rec == "normal":
            x = z
        elif rec == "lognormal":
            x = z * s_c
        elif rec == "structured":
            gt = _rng(seed, "x.tile", t)
            mu = (0.5 * gt.standard_normal(size=(C,))).astype(np.float32)
            tau = np.float32(gt.uniform(0.25, 1.0))
            x = s_c * (mu + tau * z)
        else:
            raise ValueError(rec)
        out[i] = _finish(cfg, x)
    return out


def make_vit(cfg: dict, seed: int = 0) -> np.ndarray:
    """The whole ViT output [T, rows, C] (float32 holding bf16 values for bf16 workloads)."""
    return make_vit_tiles(cfg, range(cfg["T"]), seed)


def make_valid_tokens(cfg: dict, seed: int = 0) -> np.ndarray:
    """Per-tile count of real tokens, U{1..N}: padded tokens sit at the end of a tile."""
    g = _rng(seed, "valid_tokens")
    return g.integers(1, cfg["N"] + 1, size=cfg["T"]).astype(np.int32)


def make_sequence(cfg: dict, seed: int = 0, poison: bool = True):
    """A prompt with every image expanded into IMG_CONTEXT slots.

    Per image: half the text tokens, <img>, S IMG_CONTEXT slots per tile,
    </img>, the other half of the text tokens.  Returns ``(ids int32 [L],
    embeds float32 [L, D])``.  With ``poison`` the embedding rows of
    IMG_CONTEXT positions are NaN: those rows are replaced by visual features
    and must never be read.
    """
    S = cfg["S"]
    n_text = cfg["text_per_image"]
    g = _rng(seed, "seq.ids")
    parts = []
    for i, nt in enumerate(cfg["tiles"]):
        txt = g.integers(0, TEXT_VOCAB, size=n_text).astype(np.int32)
        h = n_text // 2
        parts += [txt[:h], np.array([IMG_START], np.int32),
                  np.full(nt * S, IMG_CONTEXT, np.int32),
                  np.array([IMG_END], np.int32), txt[h:]]
    ids = np.concatenate(parts).astype(np.int32)
    L = ids.shape[0]
    emb = _normal(seed, "seq.embeds", (L, cfg["D"]))
    emb = _finish(cfg, emb)
    if poison:
        emb[ids == IMG_CONTEXT] = np.float32(np.nan)
    return ids, emb


def make_batch_sequences(cfg: dict, images_per_seq, seed: int = 0, poison: bool = True,
                         with_embeds: bool = True):
    """B prompts packed back to back (a variable-length batch).

    ``images_per_seq[b]`` lists the tile counts of sequence b's images (an
    empty list gives a text-only prompt).  Each prompt is laid out as
    ``make_sequence`` lays out one, with its own seeded text.  Returns
    ``(ids int32 [L], embeds float32 [L, D] or None, cu_seqlens int32 [B+1],
    tile_offsets int32 [B+1])``: sequence b is positions cu_seqlens[b] ..
    cu_seqlens[b+1]-1 and owns tiles tile_offsets[b] .. tile_offsets[b+1]-1.
    """
    S = cfg["S"]
    n_text = cfg["text_per_image"]
    parts, lens, tiles = [], [], []
    for b, imgs in enumerate(images_per_seq):
        g = _rng(seed, "batch.ids", b)
        n0 = sum(len(p) for p in parts)
        if not imgs:
            parts.append(g.integers(0, TEXT_VOCAB, size=int(g.integers(0, n_text + 1))).astype(np.int32))
        for nt in imgs:
            txt = g.integers(0, TEXT_VOCAB, size=n_text).astype(np.int32)
            h = n_text // 2
            parts += [txt[:h], np.array([IMG_START], np.int32), np.full(nt * S, IMG_CONTEXT, np.int32),
                      np.array([IMG_END], np.int32), txt[h:]]
        lens.append(sum(len(p) for p in parts) - n0)
        tiles.append(int(sum(imgs)))
    ids = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    to = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int32)
    emb = None
    if with_embeds:
        emb = _finish(cfg, _normal(seed, "batch.embeds", (ids.shape[0], cfg["D"])))
        if poison:
            emb[ids == IMG_CONTEXT] = np.float32(np.nan)
    return ids, emb, cu, to


def sample_tiles(T: int, seed: int = 0, n: int = 16) -> list[int]:
    """Tiles checked element by element on large workloads: the first, the
    last and ``n - 2`` more drawn without replacement."""
    if T <= n:
        return list(range(T))
    g = _rng(seed, "sample_tiles")
    rest = g.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return sorted({0, T - 1, *[int(v) for v in rest]})
