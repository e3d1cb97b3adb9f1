"""Pins for CrossAttentionPooling, Gating, the quantile and the decision (no GPU).

Pooling is tied to torch's nn.MultiheadAttention (four layers chained, with
key_padding_mask), and to closed forms: one valid token, a zero query
projection (uniform attention), and invariance to poisoned padding.  Gating is
tied to torch modules composed as the 4B-Flash page lists them and to softmax
identities.  The quantile is tied bit for bit to numpy's and torch's linear
quantile; the decision to a truth table and a counting bound.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import connector as O


def _cfg():
    return synth.config("tiny_flash_f32")


def _mha(w, l, C, H):
    m = torch.nn.MultiheadAttention(C, H, bias=True, batch_first=True).double().eval()
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.from_numpy(np.concatenate(
            [w[f"pool.{l}.{p}.w"] for p in "qkv"]).astype(np.float64)))
        m.in_proj_bias.copy_(torch.from_numpy(np.concatenate(
            [w[f"pool.{l}.{p}.b"] for p in "qkv"]).astype(np.float64)))
        m.out_proj.weight.copy_(torch.from_numpy(w[f"pool.{l}.o.w"].astype(np.float64)))
        m.out_proj.bias.copy_(torch.from_numpy(w[f"pool.{l}.o.b"].astype(np.float64)))
    return m


@pytest.mark.parametrize("padded", [False, True])
def test_pool_matches_torch_mha(padded):
    cfg = _cfg()
    w = synth.make_weights(cfg)
    x = synth.make_vit(cfg)
    T, C, H, N = cfg["T"], cfg["C"], cfg["pool_heads"], cfg["N"]
    valid = synth.make_valid_tokens(cfg, seed=3) if padded else None
    got = O.cross_attention_pooling(x, cfg, w, valid)
    toks = torch.from_numpy(x[:, 1:, :].astype(np.float64))
    mask = None
    if padded:
        mask = torch.arange(N)[None, :] >= torch.from_numpy(valid.astype(np.int64))[:, None]
    q = torch.from_numpy(w["pool.query"].astype(np.float64)).expand(T, 1, C)
    with torch.no_grad():
        for l in range(cfg["pool_layers"]):
            q, _ = _mha(w, l, C, H)(q, toks, toks, key_padding_mask=mask, need_weights=False)
    assert np.allclose(got, q[:, 0].numpy(), rtol=1e-11, atol=1e-11)


def test_pool_single_valid_token_closed_form():
    # With one key, softmax gives it weight 1: every layer outputs
    # Wo (Wv x0 + bv) + bo whatever its query.
    cfg = _cfg()
    w = synth.make_weights(cfg)
    x = synth.make_vit(cfg)
    valid = np.ones(cfg["T"], np.int32)
    got = O.cross_attention_pooling(x, cfg, w, valid)
    l = cfg["pool_layers"] - 1
    x0 = x[:, 1, :].astype(np.float64)
    v = x0 @ w[f"pool.{l}.v.w"].T.astype(np.float64) + w[f"pool.{l}.v.b"]
    exp = v @ w[f"pool.{l}.o.w"].T.astype(np.float64) + w[f"pool.{l}.o.b"]
    assert np.allclose(got, exp, rtol=1e-12, atol=1e-12)


def test_pool_zero_query_projection_is_mean_of_values():
    # Wq = 0, bq = 0 for one layer: all scores are 0, attention is uniform,
    # and the layer outputs Wo (mean_n V_n) + bo.
    cfg = dict(_cfg(), pool_layers=1)
    w = synth.make_weights(_cfg())
    w["pool.0.q.w"] = np.zeros_like(w["pool.0.q.w"])
    w["pool.0.q.b"] = np.zeros_like(w["pool.0.q.b"])
    x = synth.make_vit(cfg)
    got = O.cross_attention_pooling(x, cfg, w)
    xs = x[:, 1:, :].astype(np.float64)
    V = xs @ w["pool.0.v.w"].T.astype(np.float64) + w["pool.0.v.b"]
    exp = V.mean(axis=1) @ w["pool.0.o.w"].T.astype(np.float64) + w["pool.0.o.b"]
    assert np.allclose(got, exp, rtol=1e-12, atol=1e-12)


def test_pool_ignores_padding_contents():
    cfg = _cfg()
    w = synth.make_weights(cfg)
    x = synth.make_vit(cfg)
    valid = synth.make_valid_tokens(cfg, seed=5)
    a = O.cross_attention_pooling(x, cfg, w, valid)
    xp = x.copy()
    for t in range(cfg["T"]):
        xp[t, 1 + valid[t]:, :] = np.nan
    xp[:, 0, :] = np.nan  # CLS is dropped as well
    b = O.cross_attention_pooling(xp, cfg, w, valid)
    assert np.array_equal(a, b)


def _torch_gating(w, cfg):
    h = cfg["gate_hidden"]
    he = h * cfg["gate_expansion"]
    blocks = []
    for b in range(4):
        l1 = torch.nn.Linear(h, he).double()
        l2 = torch.nn.Linear(he, h).double()
        ln = torch.nn.LayerNorm(h, eps=cfg["ln_eps"]).double()
        with torch.no_grad():
            for mod, key in ((l1, f"gate.{b}.l1"), (l2, f"gate.{b}.l2"), (ln, f"gate.{b}.ln")):
                mod.weight.copy_(torch.from_numpy(w[key + ".w"].astype(np.float64)))
                mod.bias.copy_(torch.from_numpy(w[key + ".b"].astype(np.float64)))
        blocks.append(torch.nn.Sequential(l1, torch.nn.GELU(), torch.nn.Dropout(0.1), l2,
                                          torch.nn.Dropout(0.1), ln).eval())
    cls = torch.nn.Linear(h, 2).double()
    with torch.no_grad():
        cls.weight.copy_(torch.from_numpy(w["gate.cls.w"].astype(np.float64)))
        cls.bias.copy_(torch.from_numpy(w["gate.cls.b"].astype(np.float64)))

    def f(x):
        for blk in blocks:
            x = x + blk(x)
        return torch.softmax(cls(x), dim=-1)
    return f


def test_gating_matches_torch_modules():
    cfg = _cfg()
    w = synth.make_weights(cfg, gate_bias0=0.3)
    r = np.random.default_rng(7)
    pooled = r.standard_normal((9, cfg["C"]))
    with torch.no_grad():
        ref = _torch_gating(w, cfg)(torch.from_numpy(pooled)).numpy()
    got = O.gating(pooled, cfg, w)
    assert np.allclose(got, ref, rtol=0, atol=1e-14)
    assert np.allclose(got.sum(-1), 1.0, atol=1e-15)
    assert (got >= 0).all() and (got <= 1).all()


def test_gating_softmax_identities():
    cfg = _cfg()
    w = synth.make_weights(cfg)
    # identical classifier rows and biases: p0 = p1 = 0.5 exactly
    w2 = dict(w)
    w2["gate.cls.w"] = np.stack([w["gate.cls.w"][0]] * 2)
    w2["gate.cls.b"] = np.zeros(2, np.float32)
    pooled = np.random.default_rng(8).standard_normal((5, cfg["C"]))
    assert np.array_equal(O.gating(pooled, cfg, w2), np.full((5, 2), 0.5))
    # p0 = sigmoid(z0 - z1): a bias shift of +b on class 0 moves the logit gap by b
    p_a = O.gating(pooled, cfg, w)
    w3 = dict(w)
    w3["gate.cls.b"] = w["gate.cls.b"] + np.array([1.5, 0.0], np.float32)
    p_b = O.gating(pooled, cfg, w3)
    gap_a = np.log(p_a[:, 0] / p_a[:, 1])
    gap_b = np.log(p_b[:, 0] / p_b[:, 1])
    assert np.allclose(gap_b - gap_a, 1.5, atol=1e-12)


@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 11, 100, 208, 257])
@pytest.mark.parametrize("ties", [False, True])
def test_quantile_matches_numpy_and_torch(T, ties):
    r = np.random.default_rng(T + 1000 * ties)
    v = r.random(T).astype(np.float32).astype(np.float64)
    if ties:
        v = np.round(v * 4) / 4
    for q in (0.1, 0.0, 0.5, 0.9, 1.0):
        got = O.quantile_linear(v, q)
        assert got == float(np.quantile(v, q, method="linear"))
        # torch evaluates the same lerp with a fused multiply-add: within 2 ulp
        tq = float(torch.quantile(torch.from_numpy(v), q))
        assert abs(got - tq) <= 2 * np.spacing(max(abs(got), abs(tq)))


def test_quantile_small_cases():
    assert O.quantile_linear([0.7], 0.1) == 0.7
    a, b = 0.25, 0.75
    assert O.quantile_linear([b, a], 0.1) == a + 0.1 * (b - a)


def test_decision_truth_table(golden):
    g = golden("routing.txt")
    q, absthr = float(g["relative_threshold"][0]), float(g["absolute_threshold"][0])
    thr = 0.55
    g0 = np.array([0.9, 0.55, 0.5, 0.56, 0.4, 0.549999])
    # > thr and >= 0.5: strict on the quantile, inclusive on the absolute bound
    assert O.route_decision(g0, thr, absthr).tolist() == [1, 0, 0, 1, 0, 0]
    assert O.route_decision([0.5, 0.5], 0.45, absthr).tolist() == [1, 1]
    assert O.route_decision([0.49999], 0.1, absthr).tolist() == [0]
    assert q == 0.1


@pytest.mark.parametrize("T", [1, 2, 8, 208])
def test_decision_bound(T):
    # the lo+1 smallest gates are <= the quantile, so at most T - lo - 1 tiles compress
    r = np.random.default_rng(T)
    g0 = r.random(T).astype(np.float32)
    thr, use64 = O.decide(g0, {"rel_quantile": 0.1, "abs_threshold": 0.5})
    lo = math.floor(0.1 * (T - 1))
    assert int(use64.sum()) <= T - lo - 1
    if T == 1:
        assert use64.sum() == 0
