"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test fixes part of the oracle with an independent fact: hand-worked fixtures under
tests/golden (each cites the page passage it follows), closed forms, invariants that follow from
the operator's definition, library routines (numpy float16 decoding, numpy matmul) on special
cases, and brute force on tiny layers.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, np.float32))


def _act(name, u, g):
    if name == "relu":
        return np.maximum(u, 0.0)
    if name == "reglu":
        return np.maximum(g, 0.0) * u
    return np.maximum(g, 0.0) * np.maximum(u, 0.0)


def _rand_layer(rng, d, F, act, dtype=np.float32, bias=True, bias_down=True):
    def w(shape, scale=0.5):
        return np.ascontiguousarray((rng.standard_normal(shape) * scale).astype(dtype))
    L = {"act": act, "w_up": w((F, d)), "w_down_t": w((F, d)),
         "w_gate": w((F, d)) if act != "relu" else None}
    L["b_up"] = _f32(rng.standard_normal(F) * 0.3) if bias else None
    L["b_gate"] = _f32(rng.standard_normal(F) * 0.3) if (bias and act != "relu") else None
    L["b_down"] = _f32(rng.standard_normal(d) * 0.3) if bias_down else None
    return L


def _brute(L, x, mask):
    """numpy float64 evaluation of the FFN definition, written independently of the C oracle."""
    X = np.asarray(x, np.float64)
    Wu = np.asarray(L["w_up"], np.float64)
    u = Wu @ X + (0 if L.get("b_up") is None else np.asarray(L["b_up"], np.float64))
    g = None
    if L["act"] != "relu":
        Wg = np.asarray(L["w_gate"], np.float64)
        g = Wg @ X + (0 if L.get("b_gate") is None else np.asarray(L["b_gate"], np.float64))
    h = _act(L["act"], u, g)
    if mask is not None:
        h = np.where(np.asarray(mask) != 0, h, 0.0)
    y = np.asarray(L["w_down_t"], np.float64).T @ h
    if L.get("b_down") is not None:
        y = y + np.asarray(L["b_down"], np.float64)
    return y, h, u, g


# ---------------------------------------------------------------- fp16 decoding
def test_half_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_half_decode_golden():
    for c in _load("half_bits.json")["cases"]:
        v = oracle.half_to_double(c["bits"])
        exp = math.inf if c["value"] == "inf" else c["value"]
        assert v == exp, c
        assert math.copysign(1.0, v) == math.copysign(1.0, exp), c


# ---------------------------------------------------------------- hand-worked FFN fixtures
@pytest.mark.parametrize("fixture", ["ffn_tiny.json", "relu_bias_tiny.json"])
def test_ffn_golden(fixture):
    G = _load(fixture)
    for c in G["cases"]:
        L = {"act": c["act"], "w_up": _f32(G["w_up"]), "w_gate": _f32(G.get("w_gate")),
             "w_down_t": _f32(G["w_down_t"]), "b_up": _f32(G.get("b_up")),
             "b_gate": _f32(G.get("b_gate")), "b_down": _f32(G.get("b_down"))}
        mask = None if c["mask"] is None else np.array(c["mask"], np.uint8)
        y, h = oracle.ffn(L, _f32(G["x"]), mask)
        assert np.array_equal(h, np.array(c["h"])), (fixture, c)
        assert np.array_equal(y, np.array(c["y"])), (fixture, c)


def test_ffn_golden_f16_storage_is_exact():
    """The same fixture stored as fp16 (every value is exactly representable) gives the same y."""
    G = _load("ffn_tiny.json")
    for c in G["cases"]:
        L = {"act": c["act"], "w_up": _f32(G["w_up"]).astype(np.float16),
             "w_gate": _f32(G["w_gate"]).astype(np.float16),
             "w_down_t": _f32(G["w_down_t"]).astype(np.float16),
             "b_gate": _f32(G["b_gate"]), "b_down": _f32(G["b_down"])}
        mask = None if c["mask"] is None else np.array(c["mask"], np.uint8)
        y, _ = oracle.ffn(L, _f32(G["x"]).astype(np.float16), mask)
        assert np.array_equal(y, np.array(c["y"]))


def test_predictor_golden():
    G = _load("predictor_tiny.json")
    for c in G["cases"]:
        r = oracle.predictor(_f32(G["p1"]), _f32(G["p2"]), _f32(G["c1"]), _f32(G["c2"]),
                             _f32(G["x"]), c["tau"])
        assert np.array_equal(r["z"], np.array(G["z"]))
        assert np.array_equal(r["s"], np.array(G["s"]))
        assert np.allclose(r["p"], np.array(G["p"]), rtol=0, atol=1e-15)
        assert r["idx"].tolist() == c["idx"], c
        assert r["count"] == len(c["idx"])


def test_int4_golden():
    G = _load("int4_tiny.json")
    d = G["d"]
    packed = np.zeros((1, d // 2), np.uint8)
    for k, v in G["bytes_nonzero"].items():
        packed[0, int(k)] = v
    scales = np.array([G["scales_f16_bits"]], np.uint16).view(np.float16)
    dec = oracle.decode_matrix(packed, scales, d)[0]
    want = np.zeros(d)
    for k, v in G["decoded_nonzero"].items():
        want[int(k)] = v
    assert np.array_equal(dec, want)
    L = {"act": "relu", "w_up": packed, "s_up": scales, "w_down_t": packed, "s_down_t": scales,
         "b_up": _f32([G["ffn"]["b_up"]])}
    y, h = oracle.ffn(L, np.ones(d, np.float32))
    assert h[0] == G["ffn"]["h"]
    wy = np.zeros(d)
    for k, v in G["ffn"]["y_nonzero"].items():
        wy[int(k)] = v
    assert np.array_equal(y, wy)


def test_router_golden():
    G = _load("router_tiny.json")
    R = _f32(G["R"]).astype(np.float16)
    for c in G["cases"]:
        ids, w, _ = oracle.router(R, _f32(c["x"]).astype(np.float16), 2)
        assert ids.tolist() == c["ids"], c
        assert np.allclose(w, c["w"], rtol=0, atol=1e-15), c


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("act", ["relu", "reglu", "drelu"])
@pytest.mark.parametrize("shape", [(8, 32), (32, 8)])
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_bruteforce_small_layers(act, shape, dtype):
    d, F = shape
    rng = np.random.default_rng(hash((act, shape, str(dtype))) & 0xFFFF)
    L = _rand_layer(rng, d, F, act, dtype)
    for trial in range(4):
        x = rng.standard_normal(d).astype(dtype)
        mask = None if trial == 0 else (rng.random(F) < 0.5).astype(np.uint8)
        y, h = oracle.ffn(L, x, mask)
        yb, hb, _, _ = _brute(L, x, mask)
        assert np.allclose(h, hb, rtol=1e-13, atol=1e-13)
        assert np.allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_predictor_bruteforce():
    rng = np.random.default_rng(7)
    for (d, r, F) in [(8, 4, 32), (32, 8, 8), (16, 16, 64)]:
        p1 = rng.standard_normal((r, d)).astype(np.float32)
        p2 = rng.standard_normal((F, r)).astype(np.float32)
        c1 = rng.standard_normal(r).astype(np.float32)
        c2 = rng.standard_normal(F).astype(np.float32)
        x = rng.standard_normal(d).astype(np.float32)
        res = oracle.predictor(p1, p2, c1, c2, x, 0.5)
        z = p1.astype(np.float64) @ x + c1
        s = p2.astype(np.float64) @ z + c2
        assert np.allclose(res["z"], z, rtol=1e-13, atol=1e-13)
        assert np.allclose(res["s"], s, rtol=1e-12, atol=1e-12)
        assert res["idx"].tolist() == np.nonzero(s > 0)[0].tolist()


# ---------------------------------------------------------------- invariants from the pages
@pytest.mark.parametrize("act", ["relu", "reglu", "drelu"])
def test_true_positive_mask_equals_dense(act):
    """Neurons whose activation is exactly zero contribute nothing (citnews, 'Dynamic neuron
    cache'), so the FFN over the true positive set equals the dense FFN."""
    rng = np.random.default_rng(11)
    d, F = 24, 96
    L = _rand_layer(rng, d, F, act)
    for _ in range(5):
        x = rng.standard_normal(d).astype(np.float32)
        _, hb, u, g = _brute(L, x, None)
        if act == "relu":
            true = u > 0
        elif act == "reglu":
            true = g > 0
        else:
            true = (g > 0) & (u > 0)
        assert 0 < true.sum() < F
        y_dense, _ = oracle.ffn(L, x, None)
        y_true, _ = oracle.ffn(L, x, true.astype(np.uint8))
        assert np.array_equal(y_dense, y_true)
        y_ones, _ = oracle.ffn(L, x, np.ones(F, np.uint8))
        assert np.array_equal(y_dense, y_ones)


def test_fig8_split_is_additive():
    """nearauto.com Fig. 8: hot neurons {3,5,7} live on one device, the rest on another; at run
    time {3,4,5} fire.  One side computes {3,5}, the other {4}, and the sum is merged; neuron 7,
    though hot, does not fire and contributes nothing."""
    rng = np.random.default_rng(8)
    d, F = 6, 8
    L = _rand_layer(rng, d, F, "relu", bias=False, bias_down=False)
    x = rng.standard_normal(d).astype(np.float32)
    u = np.asarray(L["w_up"], np.float64) @ x
    b = np.where(np.isin(np.arange(F), [3, 4, 5]), 5.0 + np.abs(u), -5.0 - np.abs(u))
    L["b_up"] = b.astype(np.float32)

    def m(ids):
        a = np.zeros(F, np.uint8)
        a[list(ids)] = 1
        return a
    y_all, h = oracle.ffn(L, x, m([3, 4, 5]))
    y_gpu, _ = oracle.ffn(L, x, m([3, 5]))
    y_cpu, _ = oracle.ffn(L, x, m([4]))
    assert np.allclose(y_gpu + y_cpu, y_all, rtol=1e-14, atol=1e-14)
    y_hot7, h7 = oracle.ffn(L, x, m([3, 4, 5, 7]))
    assert h7[7] == 0.0 and np.array_equal(y_hot7, y_all)
    y_dense, _ = oracle.ffn(L, x, None)
    assert np.array_equal(y_dense, y_all)
    assert (h[[3, 4, 5]] > 0).all()


def test_permutation_invariance():
    rng = np.random.default_rng(12)
    d, F = 16, 40
    L = _rand_layer(rng, d, F, "drelu")
    x = rng.standard_normal(d).astype(np.float32)
    mask = (rng.random(F) < 0.4).astype(np.uint8)
    y, h = oracle.ffn(L, x, mask)
    perm = rng.permutation(F)
    P = {k: (np.ascontiguousarray(v[perm]) if isinstance(v, np.ndarray) and v.shape[0] == F
             else v) for k, v in L.items()}
    yp, hp = oracle.ffn(P, x, np.ascontiguousarray(mask[perm]))
    assert np.allclose(yp, y, rtol=1e-13, atol=1e-13)
    assert np.array_equal(hp, h[perm])


# ---------------------------------------------------------------- closed forms
def test_identity_regime_matches_matmul():
    """With a huge up bias every ReLU passes, so y = W_down_t^T (W_up x + b_up) + b_down."""
    rng = np.random.default_rng(13)
    d, F = 20, 50
    L = _rand_layer(rng, d, F, "relu")
    L["b_up"] = np.full(F, 1e4, np.float32)
    x = rng.standard_normal(d).astype(np.float32)
    y, _ = oracle.ffn(L, x)
    Wu, Wd = L["w_up"].astype(np.float64), L["w_down_t"].astype(np.float64)
    want = np.matmul(Wd.T, np.matmul(Wu, x.astype(np.float64)) + 1e4) + L["b_down"]
    assert np.allclose(y, want, rtol=1e-12, atol=1e-9)


@pytest.mark.parametrize("act", ["relu", "reglu", "drelu"])
def test_zero_token_gives_bias_terms(act):
    rng = np.random.default_rng(14)
    d, F = 12, 30
    L = _rand_layer(rng, d, F, act)
    mask = (rng.random(F) < 0.5).astype(np.uint8)
    y, _ = oracle.ffn(L, np.zeros(d, np.float32), mask)
    bu = L["b_up"].astype(np.float64)
    bg = None if L["b_gate"] is None else L["b_gate"].astype(np.float64)
    h = _act(act, bu, bg) * mask
    want = L["w_down_t"].astype(np.float64).T @ h + L["b_down"]
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)


def test_single_neuron_is_rank_one():
    rng = np.random.default_rng(15)
    d, F = 10, 25
    L = _rand_layer(rng, d, F, "reglu", bias_down=False)
    x = rng.standard_normal(d).astype(np.float32)
    for i in [0, 7, F - 1]:
        mask = np.zeros(F, np.uint8)
        mask[i] = 1
        y, h = oracle.ffn(L, x, mask)
        assert np.count_nonzero(h) <= 1
        assert np.allclose(y, h[i] * L["w_down_t"][i].astype(np.float64), rtol=0, atol=0)


def test_empty_mask_gives_bias():
    rng = np.random.default_rng(16)
    L = _rand_layer(rng, 8, 16, "relu")
    y, h = oracle.ffn(L, rng.standard_normal(8).astype(np.float32), np.zeros(16, np.uint8))
    assert not h.any()
    assert np.array_equal(y, L["b_down"].astype(np.float64))


# ---------------------------------------------------------------- predictor properties
def test_selector_predictor_is_exact():
    """A one-hot P1 makes z = x restricted to the selected coordinates, exactly."""
    rng = np.random.default_rng(17)
    d, r, F = 40, 8, 32
    sel = rng.choice(d, r, replace=False)
    p1 = np.zeros((r, d), np.float16)
    p1[np.arange(r), sel] = 1
    p2 = rng.standard_normal((F, r)).astype(np.float16)
    x = rng.standard_normal(d).astype(np.float16)
    res = oracle.predictor(p1, p2, None, None, x, 0.5)
    assert np.array_equal(res["z"], x[sel].astype(np.float64))


def test_threshold_monotone_and_extremes():
    rng = np.random.default_rng(18)
    d, r, F = 16, 4, 64
    p1 = rng.standard_normal((r, d)).astype(np.float32)
    p2 = rng.standard_normal((F, r)).astype(np.float32)
    x = rng.standard_normal(d).astype(np.float32)
    prev = None
    for tau in [1e-12, 0.1, 0.3, 0.5, 0.7, 0.9, 1.0]:
        a = oracle.predictor(p1, p2, None, None, x, tau)["active"].astype(bool)
        if prev is not None:
            assert not (a & ~prev).any()  # A(tau2) is a subset of A(tau1) for tau1 < tau2
        prev = a
        if tau == 1e-12:
            assert a.all()
        if tau == 1.0:
            assert not a.any()


# ---------------------------------------------------------------- int4 exactness
def _decode_i4_numpy(packed, scales):
    lo = (packed & 0xF).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    q = np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)
    q = np.where(q >= 8, q - 16, q)
    return q * np.repeat(scales.astype(np.float64), 32, axis=1)


def test_int4_oracle_equals_oracle_on_decoded_weights():
    """s*q is exact, so the FFN on int4 storage equals the FFN on the decoded fp32 weights,
    bit for bit (the decoding here is numpy's, independent of the oracle's)."""
    rng = np.random.default_rng(19)
    d, F = 64, 24
    L = {"act": "drelu"}
    F32 = {"act": "drelu"}
    for name in ["w_up", "w_gate", "w_down_t"]:
        packed = rng.integers(0, 256, size=(F, d // 2), dtype=np.uint8)
        scales = (rng.random((F, d // 32)) * 0.1).astype(np.float16)
        L[name], L["s" + name[1:]] = packed, scales
        dec = _decode_i4_numpy(packed, scales)
        assert np.array_equal(dec.astype(np.float32).astype(np.float64), dec)
        F32[name] = np.ascontiguousarray(dec.astype(np.float32))
    for k in ["b_up", "b_gate"]:
        L[k] = F32[k] = rng.standard_normal(F).astype(np.float32) * 0.1
    x = rng.standard_normal(d).astype(np.float16)
    mask = (rng.random(F) < 0.5).astype(np.uint8)
    y4, h4 = oracle.ffn(L, x, mask)
    y32, h32 = oracle.ffn(F32, x, mask)
    assert np.array_equal(y4, y32) and np.array_equal(h4, h32)


# ---------------------------------------------------------------- router / mixture
def test_router_weights_and_ties():
    rng = np.random.default_rng(20)
    E, d = 8, 32
    R = (rng.standard_normal((E, d)) * 0.1).astype(np.float16)
    for _ in range(10):
        x = rng.standard_normal(d).astype(np.float16)
        ids, w, logits = oracle.router(R, x, 2)
        assert abs(w.sum() - 1.0) < 1e-15 and w[0] >= w[1]
        order = sorted(range(E), key=lambda e: (-logits[e], e))
        assert ids.tolist() == order[:2]
        assert math.isclose(w[0], 1 / (1 + math.exp(logits[ids[1]] - logits[ids[0]])),
                            rel_tol=1e-14)
        assert np.allclose(logits, R.astype(np.float64) @ x.astype(np.float64), rtol=1e-12,
                           atol=1e-14)


def test_moe_identical_experts_reduce_to_one_ffn():
    rng = np.random.default_rng(21)
    d, F, r, E = 16, 32, 4, 4
    L = _rand_layer(rng, d, F, "drelu")
    L.update(p1=rng.standard_normal((r, d)).astype(np.float32),
             p2=rng.standard_normal((F, r)).astype(np.float32), c1=None, c2=None, tau=0.5)
    R = (rng.standard_normal((E, d)) * 0.3).astype(np.float16)
    x = rng.standard_normal(d).astype(np.float32).astype(np.float16)
    y, ids, w, _ = oracle.moe_token([L] * E, R, x.astype(np.float32), 2)
    y1, _ = oracle.sparse_token(L, x.astype(np.float32))
    assert np.allclose(y, y1, rtol=1e-13, atol=1e-13)


def test_moe_forced_pair_bruteforce():
    rng = np.random.default_rng(22)
    d, F, E = 8, 16, 4
    experts = []
    for e in range(E):
        L = _rand_layer(rng, d, F, "relu")
        L.update(p1=None, p2=None)
        experts.append(L)
    R = np.zeros((E, d), np.float16)
    R[1, 0] = 4
    R[3, 0] = 2
    x = np.zeros(d, np.float32)
    x[0] = 1
    x[1:] = rng.standard_normal(d - 1)
    masks = [np.ones(F, np.uint8)] * 2
    y, ids, w, _ = oracle.moe_token(experts, R, x, 2, masks=masks)
    assert ids.tolist() == [1, 3]
    w1 = 1 / (1 + math.exp(-2.0))
    want = w1 * _brute(experts[1], x, None)[0] + (1 - w1) * _brute(experts[3], x, None)[0]
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
