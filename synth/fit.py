"""Least-squares low-rank activation predictors for the synthetic layers, and the rank choice per
layer (PowerInfer, unite.ai, section "Adaptive sparse predictor": each layer gets its own small
predictor, sized from the layer's sparsity and skewness and trained offline; the naive,
oversized predictors can outweigh the model itself).

These functions make predictor *weights* (input bytes for the operator), as the rest of
``synth`` makes layer weights: nothing here predicts a set or evaluates the FFN.

Fit.  The predictor scores ``s = P2 (P1 x) + c2`` are fitted to the source pre-activation
``t = W_src x + b_src`` (W_src = W_up for ReLU, W_gate for ReGLU / dReLU) in least squares over
the tokens the generator draws, x ~ N(0, I).  For those tokens E|t - s|^2 = |W_src - P2 P1|_F^2 +
|b_src - c2|^2, so the fit is the rank-r truncated SVD of W_src (Eckart-Young) and the intercept
c2 = b_src.  With V_r the top r right singular vectors (eigenvectors of W_src^T W_src, largest
first): P1 = V_r^T, P2 = W_src V_r, c1 absent.  An optional recall margin m lowers the decision
boundary by m residual standard deviations per neuron: c2_i = b_i + m * sqrt(|w_i|^2 - |P2_i|^2).

Rank choice.  For x ~ N(0, I) a neuron's true pre-activation t_i and its fitted score s_i are
jointly normal: t_i ~ N(b_i, |w_i|^2), s_i ~ N(c2_i, |P2_i|^2), cov = |P2_i|^2 (P2_i is the
projection of w_i).  So the expected recall and precision of the predicted sets follow from
bivariate normal orthant probabilities, for every rank at once from the cumulative projections;
``choose_rank`` takes the smallest rank (in steps) whose expected recall reaches the target.
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch

from . import F16, F32, I4G32


def _decode_i4(packed: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """int4 group-32 rows -> float64 values s * q (the stored weights, exactly)."""
    lo = (packed & 0xF).to(torch.int16)
    hi = (packed >> 4).to(torch.int16)
    q = torch.stack([lo, hi], dim=2).reshape(packed.shape[0], -1)
    q = torch.where(q >= 8, q - 16, q).to(torch.float64)
    s = scales.to(torch.float64).repeat_interleave(32, dim=1)
    return q * s


def source(layer: dict):
    """(W_src float64 [ffn][d], b_src float64 [ffn]) of a layer dict, from its stored bytes."""
    key = "up" if layer["act"] == "relu" else "gate"
    w = layer["w_" + key]
    if layer.get("s_" + key) is not None:
        W = _decode_i4(w, layer["s_" + key])
    else:
        W = w.to(torch.float64)
    b = layer.get("b_" + key)
    b = torch.zeros(W.shape[0], dtype=torch.float64, device=W.device) if b is None else b.double()
    return W, b


def spectrum(layer: dict):
    """Right singular vectors V (columns, largest singular value first) and the singular values
    of the layer's W_src, from the symmetric eigendecomposition of W_src^T W_src (float64)."""
    W, _ = source(layer)
    evals, V = torch.linalg.eigh(W.T @ W)
    evals, V = evals.flip(0), V.flip(1)
    return V, evals.clamp(min=0).sqrt()


def fit_predictor(layer: dict, rank: int, margin: float = 0.0, p_dtype: str | None = None,
                  basis=None) -> dict:
    """The least-squares rank-``rank`` predictor of ``layer`` (module docstring).  Returns the
    layer dict with p1, p2, c1 (None), c2 replaced and ``fit`` = (rank, margin)."""
    W, b = source(layer)
    d = W.shape[1]
    assert 0 < rank <= d
    V = basis if basis is not None else spectrum(layer)[0]
    Vr = V[:, :rank]
    P2 = W @ Vr                                             # [ffn][rank]
    resid = (W.square().sum(1) - P2.square().sum(1)).clamp(min=0).sqrt()
    c2 = b + margin * resid
    pt = {F32: torch.float32, F16: torch.float16}[p_dtype or layer["cfg"].p_dtype]
    out = dict(layer)
    out.update(p1=Vr.T.contiguous().to(pt), p2=P2.to(pt).contiguous(), c1=None,
               c2=c2.float().contiguous(), fit=(rank, margin), selector=None)
    return out


def _phi2(h: np.ndarray, k: np.ndarray, rho: np.ndarray) -> np.ndarray:
    """P(X <= h, Y <= k) for standard normals with correlation rho (Owen's T form)."""
    h = np.where(h == 0.0, 1e-300, h)
    k = np.where(k == 0.0, 1e-300, k)
    r = np.sqrt(np.maximum(1.0 - rho * rho, 1e-300))
    ah = (k - rho * h) / (h * r)
    ak = (h - rho * k) / (k * r)
    beta = np.where(h * k > 0, 0.0, 0.5)
    return (0.5 * scipy.special.ndtr(h) + 0.5 * scipy.special.ndtr(k)
            - scipy.special.owens_t(h, ah) - scipy.special.owens_t(k, ak) - beta)


def _other(layer: dict, n: int) -> np.ndarray:
    """Probability that the rest of the activation lets h be nonzero once the source row fires:
    1, except dReLU, whose up row must fire too (independent rows)."""
    if layer["act"] != "drelu":
        return np.ones(n)
    Wu = _decode_i4(layer["w_up"], layer["s_up"]) if layer.get("s_up") is not None \
        else layer["w_up"].double()
    bu = layer.get("b_up")
    bu = np.zeros(n) if bu is None else bu.double().cpu().numpy()
    return scipy.special.ndtr(bu / np.sqrt(Wu.square().sum(1).cpu().numpy()))


def expected_quality(layer: dict, rank: int, margin: float = 0.0, basis=None):
    """Expected (recall, precision, predicted density, true density) of the rank-``rank``
    least-squares predictor over tokens x ~ N(0, I), from the closed form."""
    return expected_quality_curve(layer, [rank], margin, basis)[0]


def expected_quality_curve(layer: dict, ranks, margin: float = 0.0, basis=None):
    W, b = source(layer)
    V = spectrum(layer)[0] if basis is None else basis
    proj = (W @ V).square()                                 # [ffn][d] per-direction energy
    cum = proj.cumsum(dim=1).cpu().numpy()                  # |P2_i|^2 for every rank
    wn2 = W.square().sum(1).cpu().numpy()
    bb = b.cpu().numpy()
    other = _other(layer, len(bb))
    out = []
    for r in ranks:
        ps2 = np.maximum(cum[:, r - 1], 1e-300)
        ps = np.sqrt(ps2)
        pt = np.sqrt(wn2)
        res = np.sqrt(np.maximum(wn2 - ps2, 0.0))
        c2 = bb + margin * res
        p_true = scipy.special.ndtr(bb / pt) * other
        p_pred = scipy.special.ndtr(c2 / ps)
        rho = np.minimum(ps / pt, 1.0)
        p_both = _phi2(bb / pt, c2 / ps, rho) * other
        out.append((float(p_both.sum() / p_true.sum()), float(p_both.sum() / p_pred.sum()),
                    float(p_pred.mean()), float(p_true.mean())))
    return out


def expected_quality_of(layer: dict):
    """Expected (recall, precision, predicted density, true density) of the layer's own
    predictor, when it is a projection predictor: P1 with orthonormal rows and P2 = W_src P1^T
    (the least-squares fit above, and also the generator's default coordinate selector), c1
    absent, threshold 1/2."""
    W, b = source(layer)
    P1 = layer["p1"].double()
    P2 = layer["p2"].double()
    assert layer.get("c1") is None and layer["tau"] == 0.5
    ref = W @ P1.T
    assert float((P2 - ref).abs().max()) <= 1e-2 * float(ref.abs().max()), "not a projection"
    ps = P2.square().sum(1).clamp(min=1e-300).sqrt().cpu().numpy()
    pt = W.square().sum(1).sqrt().cpu().numpy()
    bb = b.cpu().numpy()
    c2 = np.zeros_like(bb) if layer.get("c2") is None else layer["c2"].double().cpu().numpy()
    other = _other(layer, len(bb))
    p_true = scipy.special.ndtr(bb / pt) * other
    p_pred = scipy.special.ndtr(c2 / ps)
    p_both = _phi2(bb / pt, c2 / ps, np.minimum(ps / pt, 1.0)) * other
    return (float(p_both.sum() / p_true.sum()), float(p_both.sum() / p_pred.sum()),
            float(p_pred.mean()), float(p_true.mean()))


def choose_rank(layer: dict, target_recall: float, margin: float = 0.0, step: int = 32,
                max_rank: int | None = None, basis=None):
    """Smallest rank (a multiple of ``step``, at most ``max_rank`` = d) whose expected recall
    reaches ``target_recall``; returns (rank, (recall, precision, predicted density, true
    density)).  The largest rank is returned when none reaches the target."""
    d = layer["w_up"].shape[1] * (2 if layer.get("s_up") is not None else 1)
    max_rank = max_rank or d
    ranks = list(range(step, max_rank + 1, step))
    V = spectrum(layer)[0] if basis is None else basis
    q = expected_quality_curve(layer, ranks, margin, V)
    for r, qq in zip(ranks, q):
        if qq[0] >= target_recall:
            return r, qq
    return ranks[-1], q[-1]
