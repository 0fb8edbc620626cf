"""Pins of the least-squares predictor fit and its closed-form quality (no GPU needed).

The fit (``synth.fit``) is pinned against things other than its own formula: the Eckart-Young
residual from numpy's SVD, exact recovery of the true active sets by the CPU oracle at full rank,
and the closed-form recall / precision against the oracle's own sets on sampled tokens; the
bivariate normal orthant helper against scipy's multivariate normal CDF.
"""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import synth
from parity import oracle_layer
from synth import fit


def test_phi2_matches_scipy():
    rng = np.random.default_rng(3)
    h, k = rng.standard_normal(12) * 1.5, rng.standard_normal(12) * 1.5
    rho = rng.uniform(0.02, 0.98, 12)
    got = fit._phi2(h, k, rho)
    for i in range(12):
        ref = scipy.stats.multivariate_normal(mean=[0, 0], cov=[[1, rho[i]], [rho[i], 1]]).cdf(
            [h[i], k[i]])
        assert abs(got[i] - ref) < 1e-7


def _cfg(act, alpha=0.0, **kw):
    base = dict(d=64, ffn=256, rank=16, act=act, w_dtype="f32", x_dtype="f32", p_dtype="f32",
                density=0.1, bias_gate=act != "relu", bias_up=True)
    base.update(kw)
    return synth.with_(synth.small_config(**base), spectrum_alpha=alpha)


@pytest.mark.parametrize("rank", [4, 16, 40])
def test_eckart_young_residual(rank):
    L = synth.make_layer(_cfg("relu", alpha=0.7), layer=2)
    F = fit.fit_predictor(L, rank)
    W = L["w_up"].double().numpy()
    P1, P2 = F["p1"].double().numpy(), F["p2"].double().numpy()
    sv = np.linalg.svd(W, compute_uv=False)
    assert np.allclose(P1 @ P1.T, np.eye(rank), atol=1e-6)
    resid = np.linalg.norm(W - P2 @ P1) ** 2
    assert abs(resid - (sv[rank:] ** 2).sum()) <= 1e-5 * (sv ** 2).sum()


@pytest.mark.parametrize("act", ["relu", "reglu", "drelu"])
def test_full_rank_fit_recovers_the_true_sets(act):
    """Rank d, no margin: the scores are the source pre-activations, so the oracle's predicted
    set is the set of neurons whose h is nonzero (the pages' ideal predictor)."""
    cfg = _cfg(act)
    L = synth.make_layer(cfg, layer=1)
    F = fit.fit_predictor(L, cfg.d)
    OF = oracle_layer(F)
    x = synth.make_tokens(cfg, 20, layer=1).numpy()
    for t in range(20):
        pred = oracle.predictor(OF["p1"], OF["p2"], OF["c1"], OF["c2"], x[t], OF["tau"])
        _, h = oracle.ffn(OF, x[t])
        src = oracle.ffn(dict(OF, act="relu", w_up=OF["w_up" if act == "relu" else "w_gate"],
                              b_up=OF["b_up" if act == "relu" else "b_gate"]), x[t])[1]
        # the source pre-activation sign (its ReLU) decides the prediction; away from 0 the
        # predicted set equals it exactly
        firm = np.abs(pred["s"]) > 1e-4
        assert np.array_equal(pred["active"][firm] != 0, src[firm] > 0)
        if act != "drelu":
            assert np.array_equal((h != 0)[firm], src[firm] > 0)


@pytest.mark.parametrize("act,alpha,rank,margin", [("reglu", 0.0, 16, 0.0),
                                                   ("reglu", 1.0, 8, 0.5),
                                                   ("relu", 0.5, 24, 1.0),
                                                   ("drelu", 1.0, 16, 0.0)])
def test_closed_form_quality_matches_sampled_sets(act, alpha, rank, margin):
    """Expected recall / precision from the bivariate normal closed form against the oracle's
    predicted and true sets on 600 sampled tokens (about 15 000 active pairs)."""
    cfg = _cfg(act, alpha=alpha)
    L = synth.make_layer(cfg, layer=3)
    F = fit.fit_predictor(L, rank, margin=margin)
    rec, prec, dp, dt = fit.expected_quality(L, rank, margin)
    assert np.allclose(fit.expected_quality_of(F), (rec, prec, dp, dt), atol=2e-3)
    OF = oracle_layer(F)
    x = synth.make_tokens(cfg, 600, layer=3, salt=5).numpy()
    tp = npred = ntrue = 0
    for t in range(600):
        pred = oracle.predictor(OF["p1"], OF["p2"], OF["c1"], OF["c2"], x[t], OF["tau"])
        _, h = oracle.ffn(OF, x[t])
        a, b = pred["active"] != 0, h != 0
        tp += int((a & b).sum())
        npred += int(a.sum())
        ntrue += int(b.sum())
    assert abs(tp / ntrue - rec) < 0.03, (tp / ntrue, rec)
    assert abs(tp / npred - prec) < 0.03, (tp / npred, prec)
    assert abs(ntrue / (600 * cfg.ffn) - dt) < 0.01


def test_selector_predictor_quality_is_its_projection_share():
    """The generator's default predictor (a coordinate selector with a density-matched c2) is a
    projection predictor too; with iid weights its expected recall equals its precision."""
    cfg = synth.CONFIGS["llama2_7b_reglu_f16"]
    L = synth.make_layer(synth.with_(cfg, d=512, ffn=1024, rank=32), layer=0)
    rec, prec, dp, dt = fit.expected_quality_of(L)
    assert abs(dp - dt) < 2e-3 and abs(rec - prec) < 2e-3


def test_choose_rank_is_the_smallest_reaching_the_target():
    cfg = _cfg("reglu", alpha=0.8)
    L = synth.make_layer(cfg, layer=0)
    V = fit.spectrum(L)[0]
    for target in (0.5, 0.8, 0.95):
        r, q = fit.choose_rank(L, target, margin=0.5, step=8, basis=V)
        assert q[0] >= target or r == cfg.d
        if r > 8:
            assert fit.expected_quality(L, r - 8, 0.5, V)[0] < target
    r, q = fit.choose_rank(L, 1.0 - 1e-9, step=8, basis=V)
    assert r == cfg.d


def test_power_law_spectrum_keeps_row_norms():
    """spectrum_alpha reshapes the singular values of the predictor's source matrix only; its
    rows keep the generator's norm (so the bias calibration is unchanged)."""
    cfg = _cfg("reglu", alpha=1.0, d=128, ffn=512)
    L = synth.make_layer(cfg)
    W = L["w_gate"].double()
    sv = torch.linalg.svdvals(W)
    assert float(sv[0] / sv[-1]) > 20.0
    assert abs(float(W.square().sum(1).mean()) / (0.02 ** 2 * 128) - 1.0) < 0.1
    plain = synth.make_layer(synth.with_(cfg, spectrum_alpha=0.0))
    assert torch.equal(L["w_up"], plain["w_up"]) and torch.equal(L["w_down_t"], plain["w_down_t"])
