"""Pins for LayerNorm, GELU, Linear, mlp1 and mlp2 of the oracle (no GPU).

The pages print no output values of the projectors, so these are pinned by
closed forms, invariants, torch's own modules composed in the order the pages
list (nn.LayerNorm, nn.Linear, nn.GELU), and the parameter count the 14B page
prints.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import connector as O


def _rng(s=0):
    return np.random.default_rng(s)


def test_layer_norm_invariants():
    r = _rng()
    y = r.standard_normal((7, 96)) * 3.0 + 2.0
    eps = 1e-5
    z = O.layer_norm(y, np.ones(96), np.zeros(96), eps)
    assert np.allclose(z.mean(-1), 0.0, atol=1e-13)
    var = np.var(y, axis=-1)
    assert np.allclose(z.var(-1), var / (var + eps), rtol=1e-12)
    # eps = 0 gives unit variance
    assert np.allclose(O.layer_norm(y, np.ones(96), np.zeros(96), 0.0).var(-1), 1.0, rtol=1e-12)
    # constant rows map to beta
    beta = r.standard_normal(96)
    assert np.allclose(O.layer_norm(np.full((2, 96), 5.0), r.standard_normal(96), beta, eps), beta)


def test_layer_norm_matches_torch():
    r = _rng(1)
    y, g, b = r.standard_normal((5, 64)), r.standard_normal(64), r.standard_normal(64)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(y), (64,), torch.from_numpy(g),
                                         torch.from_numpy(b), 1e-5).numpy()
    assert np.allclose(O.layer_norm(y, g, b, 1e-5), ref, rtol=0, atol=1e-13)


def test_gelu_closed_forms():
    assert O.gelu(0.0) == 0.0
    # GELU(1) = Phi(1), the standard normal CDF at 1
    assert abs(float(O.gelu(1.0)) - 0.8413447460685429) < 1e-15
    x = np.linspace(-6, 6, 101)
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, atol=1e-14)
    assert abs(float(O.gelu(40.0)) / 40.0 - 1.0) < 1e-15
    assert abs(float(O.gelu(-40.0))) < 1e-300 + 1e-15
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(O.gelu(x), ref, rtol=0, atol=1e-15)


def test_linear_layout():
    r = _rng(2)
    x = r.standard_normal((3, 5))
    W = r.standard_normal((4, 5))
    b = r.standard_normal(4)
    assert np.allclose(O.linear(x, np.eye(5), np.zeros(5)), x)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(W), torch.from_numpy(b))
    assert np.allclose(O.linear(x, W, b), ref.numpy(), atol=1e-14)
    # one element by hand: y[1,2] = b[2] + sum_i W[2,i] x[1,i]
    assert abs(O.linear(x, W, b)[1, 2] - (b[2] + sum(W[2, i] * x[1, i] for i in range(5)))) < 1e-13


def _torch_linear(W, b):
    m = torch.nn.Linear(W.shape[1], W.shape[0]).double()
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(np.asarray(W, np.float64)))
        m.bias.copy_(torch.from_numpy(np.asarray(b, np.float64)))
    return m


def _torch_ln(g, b, eps):
    m = torch.nn.LayerNorm(g.shape[0], eps=eps).double()
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(np.asarray(g, np.float64)))
        m.bias.copy_(torch.from_numpy(np.asarray(b, np.float64)))
    return m


def test_mlp1_mlp2_match_torch_sequential():
    cfg = synth.config("tiny_flash_f32")
    w = synth.make_weights(cfg)
    eps = cfg["ln_eps"]
    r = _rng(3)
    Y2 = r.standard_normal((2, 16, 4 * cfg["C"]))
    Y4 = r.standard_normal((2, 4, 16 * cfg["C"]))
    # mlp1 as the 14B page lists it: LayerNorm, Linear, GELU, Linear
    m1 = torch.nn.Sequential(_torch_ln(w["mlp1.ln.w"], w["mlp1.ln.b"], eps),
                             _torch_linear(w["mlp1.l1.w"], w["mlp1.l1.b"]), torch.nn.GELU(),
                             _torch_linear(w["mlp1.l2.w"], w["mlp1.l2.b"]))
    m2 = torch.nn.Sequential(_torch_ln(w["mlp2.ln.w"], w["mlp2.ln.b"], eps),
                             _torch_linear(w["mlp2.l1.w"], w["mlp2.l1.b"]), torch.nn.GELU(),
                             _torch_linear(w["mlp2.l2.w"], w["mlp2.l2.b"]), torch.nn.GELU(),
                             _torch_linear(w["mlp2.l3.w"], w["mlp2.l3.b"]))
    with torch.no_grad():
        r1 = m1(torch.from_numpy(Y2)).numpy()
        r2 = m2(torch.from_numpy(Y4)).numpy()
    assert np.allclose(O.mlp1(Y2, w, eps), r1, rtol=1e-12, atol=1e-12)
    assert np.allclose(O.mlp2(Y4, w, eps), r2, rtol=1e-12, atol=1e-12)


def test_connector_run_matches_torch_pipeline():
    # extract_feature built from torch primitives: drop row 0, reshape to the
    # grid, torch pixel_unshuffle with channels reordered to (m, k, c), mlp.
    cfg = synth.config("tiny_flash_f32")
    w = synth.make_weights(cfg)
    x = synth.make_vit_tiles(cfg, [0, 5])
    out256, out64 = O.connector_run(x, cfg, w)
    P, C, eps = cfg["P"], cfg["C"], cfg["ln_eps"]
    g = torch.from_numpy(x.astype(np.float64))[:, 1:, :].reshape(2, P, P, C).permute(0, 3, 1, 2)

    def shuf(r):
        Q = P // r
        pu = torch.nn.functional.pixel_unshuffle(g, r)
        return pu.reshape(2, C, r, r, Q, Q).permute(0, 4, 5, 2, 3, 1).reshape(2, Q * Q, r * r * C)

    with torch.no_grad():
        h = torch.nn.functional.layer_norm(shuf(2), (4 * C,), torch.tensor(w["mlp1.ln.w"], dtype=torch.float64),
                                           torch.tensor(w["mlp1.ln.b"], dtype=torch.float64), eps)
        h = _torch_linear(w["mlp1.l2.w"], w["mlp1.l2.b"])(
            torch.nn.functional.gelu(_torch_linear(w["mlp1.l1.w"], w["mlp1.l1.b"])(h)))
    assert np.allclose(out256, h.numpy(), rtol=1e-12, atol=1e-12)
    assert out64.shape == (2, 4, cfg["D"])


def test_mlp1_parameter_count(golden):
    g = golden("mlp1_params.txt")
    cfg = synth.config("internvl3_14b_ragged")
    assert 4 * cfg["C"] == int(g["in_width"][0]) and cfg["D"] == int(g["llm_width"][0])
    # weight shapes the oracle's mlp1 consumes ([out, in]); count only, no draw
    shapes = {"mlp1.l1.w": (cfg["mlp1_hidden"], 4 * cfg["C"]), "mlp1.l2.w": (cfg["D"], cfg["mlp1_hidden"])}
    n = sum(int(np.prod(s)) for s in shapes.values())
    assert n == int(g["weight_params"][0])
    assert round(n / 1e6, 1) == float(g["rounded_millions"][0])


def test_mlp_dims_follow_token_levels(golden):
    lv = golden("token_levels.txt")
    cfg = synth.config("tiny_flash_f32")
    w = synth.make_weights(cfg)
    assert w["mlp1.l1.w"].shape[1] == 4 * cfg["C"]
    assert w["mlp2.l1.w"].shape[1] == 16 * cfg["C"]
    assert int(lv["std"][3]) == 4 * int(lv["vit"][3]) and int(lv["flash"][3]) == 16 * int(lv["vit"][3])
