"""GPU parity of the hot head (neurons ordered hottest first, the first n_hot always active, the
rest predicted) against the CPU oracle's ``predictor_hot``, through the C ABI: batch-1 decode in
both variants, the batched union path, the dense / AUTO paths and the Llama-2-shaped layer."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, check_index_list, mask_from_idx, normwise, oracle_layer, to_device

pytestmark = pytest.mark.gpu

SENTINEL = -7.25


@pytest.fixture(scope="module")
def ffn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_ffn_gemv_amd as m
    return m


def _run(ffn, L, x, n_hot, variant=0, mask=None, path=None):
    B = x.shape[0]
    F = L["w_up"].shape[0]
    m = ffn.SparseFFN(L, max_batch=B)
    m.set_hot_head(n_hot)
    if variant:
        ffn.ffn_plan_set_decode_variant(m.plan, variant)
    y = torch.full((B, m.d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, F), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    scores = torch.full((B, F), SENTINEL, dtype=torch.float32, device="cuda")
    kw = {} if path is None else {"path": path}
    m.forward(x, y=y, mask=mask, idx=idx, cnt=cnt, scores=scores, **kw)
    torch.cuda.synchronize()
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    lists = [idx_h[b, :cnt_h[b]] for b in range(B)]
    m.close()
    return y.cpu().numpy(), lists, cnt_h, scores.cpu().numpy()


def _check(ffn, cfg, n_hot, n_tokens, variant=0, path=None, tokens=None, layer_no=0):
    H = synth.hot_first(synth.make_layer(cfg, layer=layer_no, device="cuda"))
    L, OL = to_device(H), oracle_layer(H)
    x = synth.make_tokens(cfg, n_tokens, layer=layer_no).cuda()
    y, lists, cnt, scores = _run(ffn, L, x, n_hot, variant=variant, path=path)
    xh = x.cpu().numpy()
    for t in (range(n_tokens) if tokens is None else tokens):
        pred = oracle.predictor_hot(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"], n_hot)
        check_index_list(lists[t], pred, OL["tau"])
        assert np.array_equal(lists[t][:n_hot], np.arange(n_hot)), "head not all active"
        assert cnt[t] == len(lists[t])
        if path is None:                     # batch-1 / batched sparse paths write the scores
            assert np.all(scores[t, :n_hot] == SENTINEL), "head scores were written"
            if n_hot < cfg.ffn:
                e = normwise(scores[t, n_hot:], pred["s"][n_hot:])
                assert e <= (1e-5 if cfg.p_dtype == "f32" else 2e-3), e
        y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lists[t], cfg.ffn))
        e = normwise(y[t], y_ref)
        assert e <= TOL[cfg.w_dtype], (t, e)
    return lists


SHAPES = [
    dict(d=512, ffn=2080, rank=64, act="relu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
         bias_up=True),
    dict(d=256, ffn=1056, rank=32, act="reglu", w_dtype="f32", x_dtype="f32", p_dtype="f32",
         bias_gate=True, bias_down=True),
    dict(d=256, ffn=1024, rank=32, act="drelu", w_dtype="i4g32", x_dtype="f16", p_dtype="f16",
         bias_gate=True, bias_up=True),
]


@pytest.mark.parametrize("n_hot", [32, 96, 1024])
@pytest.mark.parametrize("kw", SHAPES, ids=lambda k: "%s_%s" % (k["act"], k["w_dtype"]))
def test_hot_head_decode(ffn, kw, n_hot):
    cfg = synth.small_config(density=0.1, **kw)
    _check(ffn, cfg, n_hot, n_tokens=3)


@pytest.mark.parametrize("n_hot", [32, 64, 96])
def test_hot_head_fused_variant(ffn, n_hot):
    """Variant 1 scores 64 neurons per workgroup: n_hot = 32 and 96 split a workgroup between
    head and tail, 64 gives it wholly to the head."""
    cfg = synth.small_config(d=2048, ffn=2080, rank=64, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True)
    _check(ffn, cfg, n_hot, n_tokens=3, variant=1)


@pytest.mark.parametrize("B", [7, 33])
def test_hot_head_batched(ffn, B):
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True)
    _check(ffn, cfg, 64, n_tokens=B)


def test_hot_head_dense_and_auto(ffn):
    """From 64 tokens the dense GEMMs run; each token's h is still zeroed outside its set, which
    holds the head."""
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_up=True)
    _check(ffn, cfg, 128, n_tokens=70, path=ffn.FFN_PATH_DENSE, tokens=[0, 33, 69])
    _check(ffn, cfg, 128, n_tokens=70, path=ffn.FFN_PATH_AUTO, tokens=[0, 33, 69])
    # 128+ tokens: the head's words come from the score GEMM's epilogue
    _check(ffn, cfg, 128, n_tokens=130, path=ffn.FFN_PATH_AUTO, tokens=[0, 64, 129])
    _check(ffn, cfg, 128, n_tokens=130, tokens=[0, 64, 129])      # sparse: head scores untouched


def test_caller_mask_ignores_the_head(ffn):
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_up=True)
    H = synth.hot_first(synth.make_layer(cfg, device="cuda"))
    L, OL = to_device(H), oracle_layer(H)
    x = synth.make_tokens(cfg, 1).cuda()
    mask = np.zeros(cfg.ffn, np.uint8)
    mask[[3, 40, 700]] = 1
    y, lists, _, _ = _run(ffn, L, x, 64, mask=torch.from_numpy(mask).cuda().view(1, -1))
    assert lists[0].tolist() == [3, 40, 700]
    y_ref, _ = oracle.ffn(OL, x.cpu().numpy()[0], mask)
    assert normwise(y[0], y_ref) <= TOL["f16"]


def test_hot_head_rejects_bad_lengths(ffn):
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_up=True)
    m = ffn.SparseFFN(to_device(synth.make_layer(cfg, device="cuda")))
    for bad in (-32, 16, 1056):
        with pytest.raises(RuntimeError):
            m.set_hot_head(bad)
    m.set_hot_head(0)
    m.close()


def test_llama2_7b_shape_hot_head(ffn):
    """Llama-2-shaped ReGLU layer, head = the neurons at the firing cap (256 of 11008)."""
    cfg = synth.CONFIGS["llama2_7b_reglu_f16"]
    n_hot = synth.hot_head_size(synth.make_layer(cfg, device="cuda"))
    assert n_hot == 256
    _check(ffn, cfg, n_hot, n_tokens=2, layer_no=0)
