"""The seeded generator: determinism, order independence, shapes, bf16 rounding."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    a = (r.standard_normal(100000) * np.exp(r.standard_normal(100000) * 4)).astype(np.float32)
    a[:5] = [0.0, -0.0, np.inf, -np.inf, 1e-40]
    ours = synth.to_bf16_exact(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(synth.to_bf16_exact(np.array([np.nan], np.float32)))[0]


def test_tiles_are_order_independent():
    cfg = synth.config("internvl35_2b_flash")
    cfg = dict(cfg, P=4, N=16, rows=17)
    a = synth.make_vit_tiles(cfg, [3, 7])
    b = synth.make_vit_tiles(cfg, [7])
    assert np.array_equal(a[1], b[0])
    assert np.array_equal(a, synth.make_vit_tiles(cfg, [3, 7]))


def test_config_shapes():
    c = synth.config("internvl35_2b_flash")
    assert (c["T"], c["N"], c["rows"], c["S"], c["S64"]) == (208, 1024, 1025, 256, 64)
    c = synth.config("tiny_flash_f32")
    assert (c["T"], c["N"], c["rows"], c["S"], c["S64"]) == (8, 64, 65, 16, 4)
    c = synth.config("internvl3_14b_ragged")
    assert len(c["tiles"]) == 32 and all(2 <= t <= 13 for t in c["tiles"])
    ids, emb = synth.make_sequence(synth.config("tiny_flash_f32"))
    assert ids.shape == (144,) and emb.shape == (144, 128)
    assert int((ids == synth.IMG_CONTEXT).sum()) == 8 * 16


def test_bf16_weights_are_bf16_exact():
    cfg = dict(synth.config("tiny_flash_f32"), dtype="bf16")
    w = synth.make_weights(cfg)
    for k, v in w.items():
        assert np.array_equal(synth.to_bf16_exact(v), v), k
