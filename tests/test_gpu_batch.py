"""GPU parity of the batched path (fp16 layers, several tokens per call: the union of the tokens'
active sets is read once per pass of up to 32 tokens, each token keeps its own set) against the
CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, check_index_list, mask_from_idx, normwise, oracle_layer, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ffn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_ffn_gemv_amd as m
    return m


def _run(ffn, L, x, mask=None):
    B = x.shape[0]
    F = L["w_up"].shape[0]
    m = ffn.SparseFFN(L, max_batch=B)
    y = torch.full((B, m.d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, F), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, F), dtype=torch.float32, device="cuda")
    m.forward(x, y=y, mask=mask, idx=idx, cnt=cnt, scores=scores)
    torch.cuda.synchronize()
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    lists = [idx_h[b, :cnt_h[b]] for b in range(B)]
    m.close()
    return y.cpu().numpy(), lists, cnt_h, scores.cpu().numpy()


def _check(ffn, cfg, B, tokens=None, layer_dev="cuda"):
    host = synth.make_layer(cfg, device=layer_dev)
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, B).cuda()
    y, lists, cnt, scores = _run(ffn, L, x)
    xh = x.cpu().numpy()
    union = set()
    for t in (range(B) if tokens is None else tokens):
        pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
        check_index_list(lists[t], pred, OL["tau"])
        assert cnt[t] == len(lists[t])
        assert normwise(scores[t], pred["s"]) <= 2e-3
        y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lists[t], cfg.ffn))
        e = normwise(y[t], y_ref)
        assert e <= TOL["f16"], (t, e)
    for t in range(B):
        union |= set(lists[t].tolist())
    return y, lists, len(union)


@pytest.mark.parametrize("kw,B", [
    (dict(d=1024, ffn=4128, rank=128, act="reglu", bias_gate=True), 128),
    (dict(d=512, ffn=2048, rank=64, act="relu", bias_up=True, bias_down=True), 300),
    (dict(d=1024, ffn=1120, rank=96, act="drelu", bias_gate=True, bias_up=True), 161),
], ids=["reglu_f4128_B128", "relu_B300", "drelu_f1120_B161"])
def test_large_call_scores_on_the_matrix_cores(ffn, kw, B):
    """Calls of 128+ tokens compute predictor stage 2 as one GEMM whose epilogue writes the
    bitmap and union words: sets, scores and y against the oracle, with a last 256-neuron tile
    cut short (ffn 4128, 1120) and a short last pass of 32 tokens (300, 161)."""
    cfg = synth.small_config(w_dtype="f16", x_dtype="f16", p_dtype="f16", density=0.1, **kw)
    _check(ffn, cfg, B, tokens=[0, 1, 31, 32, 100, B - 2, B - 1])


BATCH_SHAPES = [
    dict(d=512, ffn=2048, rank=64, act="relu", bias_up=True, bias_down=True),
    dict(d=1024, ffn=4128, rank=128, act="reglu", bias_gate=True),
    dict(d=520, ffn=1184, rank=40, act="drelu", bias_gate=True, bias_up=True, bias_down=True),
    dict(d=136, ffn=1056, rank=24, act="reglu", bias_gate=True),
    dict(d=264, ffn=1056, rank=24, act="relu", bias_up=True),      # odd number of 32-row tiles
    dict(d=1024, ffn=1120, rank=520, act="drelu", bias_gate=True, bias_up=True),  # ragged rank chunks
]


@pytest.mark.parametrize("B", [2, 7, 8, 31, 32, 33, 45])
@pytest.mark.parametrize("kw", BATCH_SHAPES, ids=lambda k: "%s_d%d_f%d" % (k["act"], k["d"],
                                                                          k["ffn"]))
def test_batched_predicted_path(ffn, kw, B):
    cfg = synth.small_config(w_dtype="f16", x_dtype="f16", p_dtype="f16", density=0.1, **kw)
    _check(ffn, cfg, B)


@pytest.mark.parametrize("kw", BATCH_SHAPES[:3], ids=lambda k: "%s_d%d_f%d" % (k["act"], k["d"],
                                                                              k["ffn"]))
def test_batched_predicted_path_512_tokens(ffn, kw):
    """512 tokens on the sparse path: sixteen passes of 32 tokens, each with its own union;
    sampled tokens at the pass edges and the last one are checked against the oracle."""
    cfg = synth.small_config(w_dtype="f16", x_dtype="f16", p_dtype="f16", density=0.1, **kw)
    _check(ffn, cfg, 512, tokens=[0, 31, 32, 33, 255, 256, 480, 511])


def test_batched_caller_masks(ffn):
    """Per-token caller masks: each token's result is the oracle over its own mask; the lists
    returned are exactly the masks."""
    cfg = synth.small_config(d=256, ffn=1024, rank=0, act="drelu", w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_gate=True, bias_up=True,
                             bias_down=True)
    host = synth.make_layer(cfg)
    L, OL = to_device(host), oracle_layer(host)
    B = 9
    x = synth.make_tokens(cfg, B).cuda()
    rng = np.random.default_rng(11)
    masks = (rng.random((B, cfg.ffn)) < rng.uniform(0.0, 0.4, size=(B, 1))).astype(np.uint8)
    masks[3] = 0                                   # one token with an empty set
    masks[5] = 1                                   # one with every neuron
    y, lists, cnt, _ = _run(ffn, L, x, mask=torch.from_numpy(masks).cuda())
    xh = x.cpu().numpy()
    for t in range(B):
        assert np.array_equal(lists[t], np.nonzero(masks[t])[0])
        y_ref, _ = oracle.ffn(OL, xh[t], masks[t])
        assert normwise(y[t], y_ref) <= TOL["f16"]
    assert np.array_equal(y[3], np.asarray(OL["b_down"], np.float32))


def test_batched_deterministic_and_close_to_single(ffn):
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, 12).cuda()
    yb, lb, _, _ = _run(ffn, L, x)
    yb2, _, _, _ = _run(ffn, L, x)
    assert np.array_equal(yb, yb2)
    for t in (0, 5, 11):
        y1, l1, _, _ = _run(ffn, L, x[t:t + 1])
        assert np.array_equal(l1[0], lb[t])
        assert normwise(yb[t], y1[0].astype(np.float64)) <= 1e-3


def test_llama2_7b_shape_batch8(ffn):
    _, lists, nu = _check(ffn, synth.CONFIGS["llama2_7b_reglu_f16"], 8, tokens=[0, 7])
    assert nu > max(len(a) for a in lists)


@pytest.mark.parametrize("B", [8, 32])
def test_falcon_40b_shape_batched(ffn, B):
    """The 8192 x 32768 ReLU layer at batch 8 and 32 (the union grows with the batch)."""
    cfg = synth.CONFIGS["falcon_40b_relu_f16"]
    _, lists, nu = _check(ffn, cfg, B, tokens=[0, B // 2, B - 1])
    assert nu / cfg.ffn > 0.3


# ---- dense fallback and path choice --------------------------------------------------------
@pytest.mark.parametrize("B", [1, 3, 40, 64, 130])
@pytest.mark.parametrize("wd,act,d", [("f16", "relu", 256), ("f16", "reglu", 264),
                                      ("f16", "drelu", 520), ("f32", "reglu", 256),
                                      ("i4g32", "drelu", 256)])
def test_dense_forward_is_the_dense_ffn(ffn, wd, act, d, B):
    """fp16 with 64 tokens or more runs the two MFMA GEMMs (ragged token, K and column tiles
    here), fewer tokens the batched kernels over every neuron; fp32 and int4 layers run every
    token through the batch-1 kernels over every neuron."""
    xd = "f32" if wd == "f32" else "f16"
    cfg = synth.small_config(d=d, ffn=1056, rank=32, act=act, w_dtype=wd, x_dtype=xd,
                             p_dtype=xd, density=0.1, bias_up=True, bias_gate=True,
                             bias_down=True)
    host = synth.make_layer(cfg)
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, B).cuda()
    m = ffn.SparseFFN(L, max_batch=B)
    y = m.dense(x)
    rng = np.random.default_rng(5)
    masks = (rng.random((B, cfg.ffn)) < 0.3).astype(np.uint8)
    ym = m.dense(x, mask=torch.from_numpy(masks).cuda())
    torch.cuda.synchronize()
    xh, yh, ymh = x.cpu().numpy(), y.cpu().numpy(), ym.cpu().numpy()
    for t in (range(B) if B <= 40 else [0, 1, 63, B - 1]):
        y_ref, _ = oracle.ffn(OL, xh[t], None)
        assert normwise(yh[t], y_ref) <= TOL[wd], (t, normwise(yh[t], y_ref))
        y_ref, _ = oracle.ffn(OL, xh[t], masks[t])
        assert normwise(ymh[t], y_ref) <= TOL[wd]
    m.close()


@pytest.mark.parametrize("B", [1, 6, 32, 70])
def test_dense_and_auto_paths_equal_sparse(ffn, B):
    """path=DENSE reads every neuron's rows but keeps each token's predicted set (h = 0 outside
    it), so DENSE, AUTO and SPARSE agree within rounding and report the same index lists."""
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="drelu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True,
                             bias_up=True)
    host = synth.make_layer(cfg)
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, B).cuda()
    m = ffn.SparseFFN(L, max_batch=B)
    out = {}
    for path in (ffn.FFN_PATH_SPARSE, ffn.FFN_PATH_DENSE, ffn.FFN_PATH_AUTO):
        idx = torch.full((B, cfg.ffn), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
        y = m.forward(x, idx=idx, cnt=cnt, path=path)
        torch.cuda.synchronize()
        out[path] = (y.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy())
    xh = x.cpu().numpy()
    ys, idxs, cnts = out[ffn.FFN_PATH_SPARSE]
    for path in (ffn.FFN_PATH_DENSE, ffn.FFN_PATH_AUTO):
        yp, idxp, cntp = out[path]
        for t in range(B):
            lt = idxp[t, :cntp[t]]
            pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
            check_index_list(lt, pred, OL["tau"])
            y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lt, cfg.ffn))
            assert normwise(yp[t], y_ref) <= TOL["f16"]
    m.close()


def test_falcon_40b_shape_prefill_dense(ffn):
    """Prefill-style dense GEMMs of the 8192 x 32768 layer over 64 tokens."""
    cfg = synth.CONFIGS["falcon_40b_relu_f16"]
    host = synth.make_layer(cfg, device="cuda")
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, 64).cuda()
    m = ffn.SparseFFN(L, max_batch=64)
    y = m.dense(x)
    torch.cuda.synchronize()
    xh, yh = x.cpu().numpy(), y.cpu().numpy()
    for t in (0, 63):
        y_ref, _ = oracle.ffn(OL, xh[t], None)
        assert normwise(yh[t], y_ref) <= TOL["f16"]
    m.close()


@pytest.mark.parametrize("B", [8, 96])
def test_auto_follows_the_device_choice(ffn, B):
    """AUTO with the crossover forced to 0 takes the dense rows (bit-identical to DENSE); with
    the crossover at 1 it keeps the sparse rows (bit-identical to SPARSE)."""
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, B).cuda()
    m = ffn.SparseFFN(L, max_batch=B)
    y_sp = m.forward(x, path=ffn.FFN_PATH_SPARSE).clone()
    y_de = m.forward(x, path=ffn.FFN_PATH_DENSE).clone()
    ffn.ffn_plan_set_crossover(m.plan, B, 0.0)
    y_a0 = m.forward(x, path=ffn.FFN_PATH_AUTO).clone()
    ffn.ffn_plan_set_crossover(m.plan, B, 1.0)
    y_a1 = m.forward(x, path=ffn.FFN_PATH_AUTO).clone()
    torch.cuda.synchronize()
    assert torch.equal(y_a0, y_de)
    assert torch.equal(y_a1, y_sp)
    assert normwise(y_de.cpu().numpy(), y_sp.cpu().numpy().astype(np.float64)) <= 1e-3
    m.close()


def test_calibrated_crossover(ffn):
    """calibrate=1 times the plan's own dense and sparse kernels and stores a crossover density
    per batch bucket; AUTO then follows it and still gives the oracle's result."""
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="relu", w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_up=True)
    host = synth.make_layer(cfg)
    L, OL = to_device(host), oracle_layer(host)
    m = ffn.SparseFFN(L, max_batch=128, calibrate=True)
    rho = {B: m.crossover(B) for B in (1, 2, 8, 32, 64, 128)}
    assert rho[1] == 1.0                          # batch 1 is never calibrated: sparse
    assert all(0.0 <= v <= 1.0 for v in rho.values()), rho
    B = 100
    x = synth.make_tokens(cfg, B).cuda()
    idx = torch.full((B, cfg.ffn), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    y = m.forward(x, idx=idx, cnt=cnt, path=ffn.FFN_PATH_AUTO)
    torch.cuda.synchronize()
    xh, yh, ih, ch = x.cpu().numpy(), y.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    for t in (0, 50, 99):
        lt = ih[t, :ch[t]]
        pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
        check_index_list(lt, pred, OL["tau"])
        y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lt, cfg.ffn))
        assert normwise(yh[t], y_ref) <= TOL["f16"]
    m.close()


def test_largest_batch_dense_and_auto(ffn):
    """max_batch = 4096 tokens of a small fp16 layer: the dense GEMMs at their largest M (and
    AUTO choosing them), sampled rows against the oracle on each token's own set."""
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="reglu", w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_gate=True, bias_down=True)
    host = synth.make_layer(cfg, device="cuda")
    L, OL = to_device(host), oracle_layer(host)
    B = 4096
    x = synth.make_tokens(cfg, B).cuda()
    m = ffn.SparseFFN(L, max_batch=B)
    ffn.ffn_plan_set_crossover(m.plan, B, 0.0)          # AUTO: always dense at this batch
    for path in (ffn.FFN_PATH_DENSE, ffn.FFN_PATH_AUTO):
        y = torch.full((B, cfg.d), float("nan"), device="cuda")
        idx = torch.full((B, cfg.ffn), -1, dtype=torch.int32, device="cuda")
        cnt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        m.forward(x, y=y, idx=idx, cnt=cnt, path=path)
        torch.cuda.synchronize()
        yh, ih, ch = y.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
        xh = x.cpu().numpy()
        for t in (0, 31, 32, 2047, 4064, 4095):
            pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
            check_index_list(ih[t, :ch[t]], pred, OL["tau"])
            y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(ih[t, :ch[t]], cfg.ffn))
            assert normwise(yh[t], y_ref) <= TOL["f16"], (path, t)
    m.close()


@pytest.mark.parametrize("act,B", [("drelu", 70), ("relu", 256)])
def test_dense_path_is_deterministic(ffn, act, B):
    """The dense GEMMs (every copy into LDS waited for before its stage is read) give
    bit-identical outputs call after call."""
    kw = dict(bias_gate=True, bias_up=True) if act == "drelu" else dict(bias_up=True)
    cfg = synth.small_config(d=1024, ffn=4096, rank=64, act=act, w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, **kw)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, B).cuda()
    m = ffn.SparseFFN(L, max_batch=B)
    y0 = m.dense(x).clone()
    torch.cuda.synchronize()
    for _ in range(12):
        y = m.dense(x)
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
    m.close()
