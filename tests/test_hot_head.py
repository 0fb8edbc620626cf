"""Pins of the hot-head reading (no GPU needed): neurons ordered by profiled firing frequency,
the first n_hot always active, the rest predicted (unite.ai PowerInfer, sections "Offline stage"
and "Neuron placement and management").

The oracle's ``predictor_hot`` is pinned by brute force on tiny predictors, by its two extremes
(n_hot = 0 is the plain predictor, n_hot = ffn activates everything), and the generator's
hot-first ordering by the invariants a neuron permutation must keep: the dense FFN, and every
neuron's own predictor decision.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import oracle_layer


def _tiny(rng, d, r, F):
    p1 = rng.standard_normal((r, d)).astype(np.float32)
    p2 = rng.standard_normal((F, r)).astype(np.float32)
    c1 = rng.standard_normal(r).astype(np.float32)
    c2 = rng.standard_normal(F).astype(np.float32)
    x = rng.standard_normal(d).astype(np.float32)
    return p1, p2, c1, c2, x


@pytest.mark.parametrize("n_hot", [0, 32, 64, 96])
def test_predictor_hot_bruteforce(n_hot):
    rng = np.random.default_rng(11 + n_hot)
    p1, p2, c1, c2, x = _tiny(rng, 16, 8, 96)
    res = oracle.predictor_hot(p1, p2, c1, c2, x, 0.5, n_hot)
    z = p1.astype(np.float64) @ x + c1
    s = p2.astype(np.float64) @ z + c2
    want = [i for i in range(96) if i < n_hot or s[i] > 0]       # sigmoid(s) > 1/2  <=>  s > 0
    assert res["idx"].tolist() == want
    assert res["count"] == len(want)
    assert np.all(np.isnan(res["s"][:n_hot]))
    assert np.allclose(res["s"][n_hot:], s[n_hot:], rtol=1e-12, atol=1e-12)


def test_predictor_hot_extremes():
    rng = np.random.default_rng(5)
    p1, p2, c1, c2, x = _tiny(rng, 24, 8, 64)
    base = oracle.predictor(p1, p2, c1, c2, x, 0.7)
    none = oracle.predictor_hot(p1, p2, c1, c2, x, 0.7, 0)
    assert np.array_equal(none["active"], base["active"])
    assert np.array_equal(none["s"], base["s"])
    full = oracle.predictor_hot(p1, p2, c1, c2, x, 0.7, 64)
    assert full["count"] == 64 and full["idx"].tolist() == list(range(64))


def _layer(act, w_dtype="f32"):
    cfg = synth.small_config(d=64, ffn=256, rank=16, act=act, w_dtype=w_dtype, x_dtype="f32",
                             p_dtype="f32", density=0.1, bias_gate=act != "relu",
                             bias_up=True, bias_down=True)
    return cfg, synth.make_layer(cfg, layer=1)


@pytest.mark.parametrize("act", ["relu", "reglu", "drelu"])
def test_hot_first_keeps_the_dense_ffn_and_each_decision(act):
    cfg, L = _layer(act)
    H = synth.hot_first(L)
    order = H["order"]
    assert sorted(order.tolist()) == list(range(cfg.ffn))
    assert np.all(np.diff(H["probs"]) <= 0)                     # hottest first
    OL, OH = oracle_layer(L), oracle_layer(H)
    x = synth.make_tokens(cfg, 2, layer=1).numpy()
    for t in range(2):
        y0, h0 = oracle.ffn(OL, x[t])
        y1, h1 = oracle.ffn(OH, x[t])
        assert np.allclose(y1, y0, rtol=1e-12, atol=1e-12)       # only the summation order moved
        assert np.array_equal(h1, h0[order])                     # each neuron's h is its own
        p0 = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], x[t], OL["tau"])
        p1 = oracle.predictor(OH["p1"], OH["p2"], OH["c1"], OH["c2"], x[t], OH["tau"])
        assert np.array_equal(p1["active"], p0["active"][order])
        assert np.array_equal(p1["s"], p0["s"][order])


def test_hot_first_int4_rows_move_with_their_scales():
    cfg, L = _layer("drelu", "i4g32")
    H = synth.hot_first(L)
    order = torch.from_numpy(H["order"])
    for k in ("w_up", "s_up", "w_gate", "s_gate", "w_down_t", "s_down_t"):
        assert torch.equal(H[k], L[k][order])


@pytest.mark.parametrize("name,expect", [("llama2_7b_reglu_f16", 256),
                                         ("falcon_40b_relu_f16", 1312)])
def test_hot_head_size_is_the_capped_set(name, expect):
    """The head is the neurons at the generator's firing cap (0.99), rounded down to a multiple
    of 32: about 2.5% of the Llama-2-shaped layer's neurons and a quarter of its firings."""
    cfg = synth.CONFIGS[name]
    probs = synth.zipf_probs(cfg.ffn, cfg.density, cfg.zipf_s, cfg.cap, synth._seed(cfg, 0, 0, 0))
    L = {"cfg": cfg, "probs": probs}
    n = synth.hot_head_size(L)
    assert n == expect and n % 32 == 0
    H = synth.hot_first(L)
    assert np.all(H["probs"][:n] >= cfg.cap * (1 - 1e-12))
    assert 0.2 < H["probs"][:n].sum() / probs.sum() < 0.3
