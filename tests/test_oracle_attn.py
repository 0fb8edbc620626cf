"""Pins of the attention-block oracle against things other than itself: a hand-derived golden,
a library matmul, PyTorch's own scaled-dot-product attention, closed forms and invariants.
unite.ai PowerInfer, section "Adaptive sparse predictor": every layer also predicts for its
self-attention block; the unit predicted is read as a head."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_block(rng, d, H, G, e, S, dt=np.float16):
    f = lambda *s: (rng.standard_normal(s) * 0.5).astype(dt)
    return dict(w_q=f(H * e, d), w_k=f(G * e, d), w_v=f(G * e, d), w_o_t=f(H * e, d),
                Kc=f(G, S, e), Vc=f(G, S, e), x=f(d))


def test_attn_golden():
    g = json.load(open(os.path.join(GOLD, "attn_tiny.json")))
    h16 = lambda a: np.ascontiguousarray(np.array(a, np.float16))
    layer = dict(w_q=h16(g["w_q"]), w_k=h16(g["w_k"]), w_v=h16(g["w_v"]),
                 w_o_t=h16(g["w_o_t"]), head_dim=g["head_dim"])
    Kc, Vc, x, t = h16(g["k_cache"]), h16(g["v_cache"]), h16(g["x"]), g["t"]
    k, v = oracle.attn_kv(layer["w_k"], layer["w_v"], x, g["head_dim"])
    assert np.array_equal(k, g["k_new"]) and np.array_equal(v, g["v_new"])
    for case in g["cases"]:
        mask = np.array(case["mask"] if case["mask"] is not None else [1, 1], np.uint8)
        y, pred, Kn, Vn = oracle.attn_token(layer, Kc, Vc, x, t, mask)
        assert pred is None
        np.testing.assert_allclose(y, case["y"], rtol=1e-14, atol=1e-14)
        assert np.array_equal(Kn[0, t], g["k_new"]) and np.array_equal(Vn[0, t], g["v_new"])
        assert np.array_equal(Kn[0, 2], Kc[0, 2]) and np.array_equal(Kc[0, 1], [-5, -5])
        _, o = oracle.attn(layer["w_q"], layer["w_o_t"], Kn, Vn, x, t,
                           None if case["mask"] is None else mask)
        np.testing.assert_allclose(o, case["o"], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_attn_kv_is_the_matmul(dt):
    rng = np.random.default_rng(1)
    b = _rand_block(rng, 40, 4, 2, 8, 3, dt)
    k, v = oracle.attn_kv(b["w_k"], b["w_v"], b["x"], 8)
    x = b["x"].astype(np.float64)
    np.testing.assert_allclose(k, b["w_k"].astype(np.float64) @ x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v, b["w_v"].astype(np.float64) @ x, rtol=1e-12, atol=1e-12)


def test_attn_one_position_returns_the_value():
    """t = 0: the softmax over one position is exactly 1, so o_h is the value row itself and y is
    W_o_t^T o (W_o_t not square, so a transposed use would not even fit)."""
    rng = np.random.default_rng(2)
    d, H, G, e = 24, 4, 2, 8
    b = _rand_block(rng, d, H, G, e, 5)
    y, o = oracle.attn(b["w_q"], b["w_o_t"], b["Kc"], b["Vc"], b["x"], 0)
    for h in range(H):
        assert np.array_equal(o[h], b["Vc"][h // (H // G), 0].astype(np.float64))
    ref = b["w_o_t"].astype(np.float64).T @ o.reshape(-1)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("H,G,t", [(4, 4, 6), (6, 3, 9), (4, 1, 0), (2, 2, 30)])
def test_attn_matches_torch_sdpa(H, G, t):
    """Every head active: each head's output equals PyTorch's scaled_dot_product_attention (fp64,
    default scale 1/sqrt(e)) over the cache's positions 0..t of its key/value head; positions
    past t hold NaN, which would poison any read of them."""
    rng = np.random.default_rng(3 + H + G + t)
    d, e, S = 32, 16, t + 4
    b = _rand_block(rng, d, H, G, e, S)
    b["Kc"][:, t + 1:] = np.nan
    b["Vc"][:, t + 1:] = np.nan
    y, o = oracle.attn(b["w_q"], b["w_o_t"], b["Kc"], b["Vc"], b["x"], t)
    q = (b["w_q"].astype(np.float64) @ b["x"].astype(np.float64)).reshape(H, e)
    for h in range(H):
        g = h // (H // G)
        K = torch.from_numpy(b["Kc"][g, :t + 1].astype(np.float64))[None]
        V = torch.from_numpy(b["Vc"][g, :t + 1].astype(np.float64))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h])[None, None], K, V)[0, 0].numpy()
        np.testing.assert_allclose(o[h], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(y, b["w_o_t"].astype(np.float64).T @ o.reshape(-1), rtol=1e-11,
                               atol=1e-12)


def test_attn_heads_add_up_and_inactive_heads_are_never_read():
    rng = np.random.default_rng(4)
    d, H, G, e, t = 32, 6, 2, 8, 5
    b = _rand_block(rng, d, H, G, e, t + 1)
    mask = np.array([1, 0, 1, 1, 0, 0], np.uint8)
    y, _ = oracle.attn(b["w_q"], b["w_o_t"], b["Kc"], b["Vc"], b["x"], t, mask)
    parts = np.zeros(d)
    for h in np.flatnonzero(mask):
        one = np.zeros(H, np.uint8)
        one[h] = 1
        parts += oracle.attn(b["w_q"], b["w_o_t"], b["Kc"], b["Vc"], b["x"], t, one)[0]
    np.testing.assert_allclose(y, parts, rtol=1e-12, atol=1e-13)
    wq, wo = b["w_q"].copy(), b["w_o_t"].copy()
    for h in np.flatnonzero(mask == 0):
        wq[h * e:(h + 1) * e] = np.nan
        wo[h * e:(h + 1) * e] = np.nan
    y2, _ = oracle.attn(wq, wo, b["Kc"], b["Vc"], b["x"], t, mask)
    assert np.array_equal(y, y2)


def test_attn_uniform_keys_average_the_values():
    rng = np.random.default_rng(5)
    d, H, G, e, t = 16, 2, 1, 4, 7
    b = _rand_block(rng, d, H, G, e, t + 1)
    b["Kc"][0, :] = b["Kc"][0, 0]
    _, o = oracle.attn(b["w_q"], b["w_o_t"], b["Kc"], b["Vc"], b["x"], t)
    mean = b["Vc"][0, :t + 1].astype(np.float64).mean(axis=0)
    for h in range(H):
        np.testing.assert_allclose(o[h], mean, rtol=1e-13, atol=1e-14)


def test_attn_large_scores_stay_finite():
    """Scores near 1e4 (exp would overflow without the max shift): the largest one takes all the
    weight, so o is that position's value row."""
    d, H, G, e, t = 8, 1, 1, 4, 3
    w_q = np.zeros((e, d), np.float16)
    w_q[0, 0] = 1000.0
    x = np.zeros(d, np.float16)
    x[0] = 1.0
    Kc = np.zeros((1, t + 1, e), np.float16)
    Kc[0, :, 0] = [20.0, 21.0, 19.0, 20.5]          # scores 1e4, 1.05e4, 0.95e4, 1.025e4
    Vc = np.arange((t + 1) * e, dtype=np.float16).reshape(1, t + 1, e)
    w_o_t = np.eye(e, d, dtype=np.float16)
    y, o = oracle.attn(w_q, w_o_t, Kc, Vc, x, t)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o[0], Vc[0, 1].astype(np.float64), rtol=0, atol=1e-12)


def test_attn_token_head_predictor_uses_the_ffn_predictor():
    """The head set comes from the same two-stage predictor as the FFN's (pinned in
    test_oracle.py), over heads instead of neurons; its density follows the generator's
    calibration."""
    cfg = synth.AttnConfig("t", d=64, heads=32, kv_heads=8, head_dim=16, rank=16, density=0.5,
                           context=4)
    L = {k: (v.numpy() if isinstance(v, torch.Tensor) else v)
         for k, v in synth.make_attn_layer(cfg).items()}
    K, V = (a.numpy() for a in synth.make_kv_cache(cfg))
    xs = synth.make_attn_tokens(cfg, 64).numpy()
    counts = []
    for x in xs:
        y, pred, Kn, Vn = oracle.attn_token(L, K, V, x, cfg.context)
        ref = oracle.predictor(L["p1"], L["p2"], None, L["c2"], x, cfg.tau)
        assert np.array_equal(pred["active"], ref["active"])
        y2, _ = oracle.attn(L["w_q"], L["w_o_t"], Kn, Vn, x, cfg.context, ref["active"])
        assert np.array_equal(y, y2)
        counts.append(pred["count"])
    assert 0.4 < np.mean(counts) / 32 < 0.6
