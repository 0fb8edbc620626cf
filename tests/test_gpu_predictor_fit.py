"""GPU parity of least-squares fitted predictors (rank chosen per layer from the closed-form
recall) through the C ABI: the kernels' sets and outputs against the CPU oracle on the fitted
weights, and the measured recall / precision of the kernels' sets against the closed form."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, check_index_list, mask_from_idx, normwise, oracle_layer, to_device
from synth import fit

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ffn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_ffn_gemv_amd as m
    return m


@pytest.mark.parametrize("alpha,target,margin", [(1.0, 0.95, 0.0), (0.5, 0.85, 1.0)])
def test_fitted_predictor_parity_and_recall(ffn, alpha, target, margin):
    cfg = synth.with_(synth.small_config(d=1024, ffn=4128, rank=64, act="reglu", w_dtype="f16",
                                         x_dtype="f16", p_dtype="f16", density=0.1,
                                         bias_gate=True), spectrum_alpha=alpha)
    L = synth.make_layer(cfg, layer=0, device="cuda")
    V = fit.spectrum(L)[0]
    rank, (rec, prec, _, _) = fit.choose_rank(L, target, margin=margin, step=32, basis=V)
    assert rec >= target and rank < cfg.d
    F = to_device(fit.fit_predictor(L, rank, margin=margin, basis=V))
    OF = oracle_layer(F)
    n = 48
    x = synth.make_tokens(cfg, n, layer=0, salt=3).cuda()
    m = ffn.SparseFFN(F, max_batch=1)
    idx = torch.zeros(n, cfg.ffn, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")
    y = torch.zeros(n, cfg.d, dtype=torch.float32, device="cuda")
    for t in range(n):
        m.forward(x[t:t + 1], y=y[t:t + 1], idx=idx[t:t + 1], cnt=cnt[t:t + 1])
    torch.cuda.synchronize()
    m.close()
    xh, idx_h, cnt_h, y_h = x.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), y.cpu().numpy()
    tp = npred = ntrue = 0
    for t in range(n):
        lst = idx_h[t, :cnt_h[t]]
        pred = oracle.predictor(OF["p1"], OF["p2"], OF["c1"], OF["c2"], xh[t], OF["tau"])
        check_index_list(lst, pred, OF["tau"])
        mk = mask_from_idx(lst, cfg.ffn)
        y_ref, _ = oracle.ffn(OF, xh[t], mk)
        assert normwise(y_h[t], y_ref) <= TOL["f16"]
        _, h = oracle.ffn(OF, xh[t])                        # the true set: h != 0
        a, b = mk != 0, h != 0
        tp += int((a & b).sum())
        npred += int(a.sum())
        ntrue += int(b.sum())
    assert abs(tp / ntrue - rec) < 0.05, (tp / ntrue, rec)
    assert abs(tp / npred - prec) < 0.05, (tp / npred, prec)
