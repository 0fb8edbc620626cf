"""GPU parity of the sparse decode path (predictor -> compaction -> gathered rows -> down) against
the CPU oracle, through the C ABI, on seeded synthetic layers."""
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


def _run(ffn, L, x, mask=None, tau=None):
    """Forward through the library; returns y, idx list per token, cnt, scores (numpy)."""
    dev = x.device
    B = x.shape[0]
    F = L["w_up"].shape[0]
    layer = dict(L)
    if tau is not None:
        layer["tau"] = tau
    m = ffn.SparseFFN(layer, max_batch=B)
    y = torch.full((B, m.d), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((B, F), -1, dtype=torch.int32, device=dev)
    cnt = torch.full((B,), -1, dtype=torch.int32, device=dev)
    scores = torch.zeros((B, F), dtype=torch.float32, device=dev)
    m.forward(x, y=y, mask=mask, idx=idx, cnt=cnt, scores=scores)
    torch.cuda.synchronize()
    cnt_h = cnt.cpu().numpy()
    idx_h = idx.cpu().numpy()
    lists = [idx_h[b, :cnt_h[b]] for b in range(B)]
    m.close()
    return y.cpu().numpy(), lists, cnt_h, scores.cpu().numpy()


def _check_predicted(ffn, cfg, n_tokens, layer_no=0, tau=None):
    host = synth.make_layer(cfg, layer=layer_no, device="cuda")
    L = to_device(host)
    OL = oracle_layer(host)
    if tau is not None:
        OL["tau"] = tau
    x = synth.make_tokens(cfg, n_tokens, layer=layer_no).cuda()
    y, lists, cnt, scores = _run(ffn, L, x, tau=tau)
    xh = x.cpu().numpy()
    worst = 0.0
    for t in range(n_tokens):
        pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
        check_index_list(lists[t], pred, OL["tau"])
        assert cnt[t] == len(lists[t])
        # scores: fp32 sums of the predictor vs the fp64 oracle
        err_s = normwise(scores[t], pred["s"])
        assert err_s <= (1e-5 if cfg.p_dtype == "f32" else 2e-3), err_s
        y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lists[t], cfg.ffn))
        e = normwise(y[t], y_ref)
        worst = max(worst, e)
        assert e <= TOL[cfg.w_dtype], (t, e)
    return worst, lists


SMALL = [
    dict(d=64, ffn=256, rank=16, act="relu", w_dtype="f32", x_dtype="f32", p_dtype="f32"),
    dict(d=256, ffn=1056, rank=32, act="reglu", w_dtype="f32", x_dtype="f32", p_dtype="f32",
         bias_gate=True, bias_down=True),
    dict(d=136, ffn=608, rank=24, act="drelu", w_dtype="f32", x_dtype="f32", p_dtype="f32",
         bias_gate=True, bias_up=True),
    dict(d=512, ffn=2080, rank=64, act="relu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
         bias_up=True, bias_down=True),
    dict(d=1024, ffn=4128, rank=128, act="reglu", w_dtype="f16", x_dtype="f16",
         p_dtype="f16", bias_gate=True),
    dict(d=520, ffn=1184, rank=40, act="drelu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
         bias_gate=True, bias_up=True, bias_down=True),
    dict(d=256, ffn=1024, rank=32, act="drelu", w_dtype="i4g32", x_dtype="f16", p_dtype="f16",
         bias_gate=True, bias_up=True, bias_down=True),
    dict(d=288, ffn=1056, rank=24, act="relu", w_dtype="i4g32", x_dtype="f16", p_dtype="f16",
         bias_up=True),
    dict(d=544, ffn=2080, rank=48, act="reglu", w_dtype="i4g32", x_dtype="f16", p_dtype="f16",
         bias_gate=True),
]


@pytest.mark.parametrize("kw", SMALL, ids=lambda k: "%s_%s_d%d_f%d" % (k["act"], k["w_dtype"],
                                                                       k["d"], k["ffn"]))
def test_predicted_path_small(ffn, kw):
    cfg = synth.small_config(density=0.12, **kw)
    _check_predicted(ffn, cfg, n_tokens=6)


def test_opt125m_shape_all_tokens(ffn):
    cfg = synth.CONFIGS["opt125m_relu_f32"]
    worst, lists = _check_predicted(ffn, cfg, n_tokens=cfg.tokens)
    dens = np.mean([len(a) for a in lists]) / cfg.ffn
    assert 0.07 < dens < 0.13


def test_llama2_7b_shape_sampled_tokens(ffn):
    _check_predicted(ffn, synth.CONFIGS["llama2_7b_reglu_f16"], n_tokens=3)


def test_mistral_7b_shape_sampled_tokens(ffn):
    _check_predicted(ffn, synth.CONFIGS["turbosparse_mistral_7b_drelu_f16"], n_tokens=2)


@pytest.mark.parametrize("expert", [0, 7])
def test_mixtral_int4_expert_shape_sampled_tokens(ffn, expert):
    """One int4 group-32 dReLU expert of the mixture workload (d=4096, ffn=14336), the least and
    the most dense expert."""
    cfg = synth.CONFIGS["turbosparse_mixtral_47b_moe_int4"]
    host = synth.make_layer(cfg, layer=0, expert=expert, device="cuda")
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, 2, layer=0).cuda()
    y, lists, cnt, _ = _run(ffn, L, x)
    xh = x.cpu().numpy()
    for t in range(2):
        pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
        check_index_list(lists[t], pred, OL["tau"])
        y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lists[t], cfg.ffn))
        assert normwise(y[t], y_ref) <= TOL["i4g32"]
    dens = np.mean(cnt) / cfg.ffn
    assert abs(dens - cfg.expert_density[expert]) < 0.03


def test_falcon_40b_shape_sampled_token(ffn):
    """The widest layer (d=8192, ffn=32768, rank 1024): two column chunks per gather thread."""
    _check_predicted(ffn, synth.CONFIGS["falcon_40b_relu_f16"], n_tokens=1)


@pytest.mark.parametrize("act", ["relu", "reglu", "drelu"])
@pytest.mark.parametrize("wd", ["f32", "f16", "i4g32"])
def test_true_mask_equals_dense_on_gpu(ffn, act, wd):
    """With the mask set to the true positive set the sparse result equals the dense FFN
    (inactive neurons contribute exactly zero); with all ones it equals the dense FFN too."""
    xd = "f32" if wd == "f32" else "f16"
    cfg = synth.small_config(d=256, ffn=1024, rank=0, act=act, w_dtype=wd, x_dtype=xd,
                             p_dtype=xd, density=0.1, bias_up=True, bias_gate=True,
                             bias_down=True)
    host = synth.make_layer(cfg)
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, 3).cuda()
    xh = x.cpu().numpy()
    masks_true, masks_ones = [], []
    for t in range(3):
        _, h = oracle.ffn(OL, xh[t], None)
        masks_true.append((h != 0).astype(np.uint8))
        masks_ones.append(np.ones(cfg.ffn, np.uint8))
    for masks in (masks_true, masks_ones):
        mk = torch.from_numpy(np.stack(masks)).cuda()
        y, lists, cnt, _ = _run(ffn, L, x, mask=mk)
        for t in range(3):
            y_dense, _ = oracle.ffn(OL, xh[t], None)
            assert normwise(y[t], y_dense) <= TOL[wd]
            assert np.array_equal(lists[t], np.nonzero(masks[t])[0])


def test_empty_and_full_sets(ffn):
    cfg = synth.small_config(d=128, ffn=512, rank=16, act="relu", density=0.2, bias_down=True)
    host = synth.make_layer(cfg)
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, 2).cuda()
    # tau = 1: nothing is active -> y = b_down exactly, count 0
    y, lists, cnt, _ = _run(ffn, L, x, tau=1.0)
    assert (cnt == 0).all()
    assert np.array_equal(y, np.tile(OL["b_down"], (2, 1)))
    # tau tiny: everything is active -> the dense FFN
    y, lists, cnt, _ = _run(ffn, L, x, tau=1e-30)
    assert (cnt == cfg.ffn).all()
    for t in range(2):
        y_dense, _ = oracle.ffn(OL, x.cpu().numpy()[t], None)
        assert normwise(y[t], y_dense) <= TOL["f32"]
    # an all-zero caller mask
    mk = torch.zeros(2, cfg.ffn, dtype=torch.uint8, device="cuda")
    y, lists, cnt, _ = _run(ffn, L, x, mask=mk)
    assert (cnt == 0).all() and np.array_equal(y, np.tile(OL["b_down"], (2, 1)))


def test_fig8_split_additive_on_gpu(ffn):
    """Partial results over disjoint neuron sets add up to the result over their union."""
    cfg = synth.small_config(d=64, ffn=256, rank=0, act="relu", density=0.3, bias_up=True)
    host = synth.make_layer(cfg)
    L = to_device(host)
    x = synth.make_tokens(cfg, 1).cuda()
    rng = np.random.default_rng(3)
    a = (rng.random(cfg.ffn) < 0.3).astype(np.uint8)
    b = ((rng.random(cfg.ffn) < 0.3) & (a == 0)).astype(np.uint8)
    ys = []
    for m in (a, b, a | b):
        y, _, _, _ = _run(ffn, L, x, mask=torch.from_numpy(m[None]).cuda())
        ys.append(y[0].astype(np.float64))
    assert normwise(ys[0] + ys[1], ys[2]) <= 1e-5


@pytest.mark.parametrize("wd", ["f32", "i4g32"])
def test_batch_equals_single_tokens_and_is_deterministic(ffn, wd):
    """fp32 and int4 layers run a batch token by token: bit-identical to single-token calls."""
    xd = "f32" if wd == "f32" else "f16"
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="reglu", w_dtype=wd, x_dtype=xd,
                             p_dtype=xd, density=0.1, bias_gate=True)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, 5).cuda()
    yb, lb, _, _ = _run(ffn, L, x)
    yb2, _, _, _ = _run(ffn, L, x)
    assert np.array_equal(yb, yb2)              # no atomics: bit-reproducible
    for t in range(5):
        y1, l1, _, _ = _run(ffn, L, x[t:t + 1])
        assert np.array_equal(y1[0], yb[t]) and np.array_equal(l1[0], lb[t])


def test_stage_timing_events(ffn):
    """The instrumentation hook attaches events to each kernel's dispatch; the result of the
    forward is unchanged by it."""
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="relu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_up=True)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, 1).cuda()
    m = ffn.SparseFFN(L)
    y0 = m.forward(x).clone()
    for stage in range(4):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        ffn.ffn_plan_set_timing_events(m.plan, stage, a.cuda_event, b.cuda_event)
        y1 = m.forward(x)
        torch.cuda.synchronize()
        ffn.ffn_plan_set_timing_events(m.plan, stage, 0, 0)
        assert a.elapsed_time(b) > 0
        assert torch.equal(y0, y1)
    with pytest.raises(ffn.FFNError):
        ffn.ffn_plan_set_timing_events(m.plan, 9, 0, 0)
    m.close()


def test_index_and_count_outputs_are_independent(ffn):
    """idx without cnt, cnt without idx, and neither: each combination gives the same y and
    the requested outputs only (regression: the count-only call once wrote through the absent
    index pointer)."""
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.15, bias_up=True)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, 2).cuda()
    m = ffn.SparseFFN(L, max_batch=2)
    idx = torch.full((2, cfg.ffn), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    y_both = m.forward(x, idx=idx, cnt=cnt).clone()
    torch.cuda.synchronize()
    ref_idx, ref_cnt = idx.clone(), cnt.clone()
    cnt2 = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    y_cnt = m.forward(x, cnt=cnt2).clone()
    idx2 = torch.full((2, cfg.ffn), -1, dtype=torch.int32, device="cuda")
    y_idx = m.forward(x, idx=idx2).clone()
    y_none = m.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(cnt2, ref_cnt)
    for b in range(2):
        n = int(ref_cnt[b])
        assert torch.equal(idx2[b, :n], ref_idx[b, :n])
    for yy in (y_cnt, y_idx, y_none):
        assert torch.equal(yy, y_both)
    m.close()


@pytest.mark.parametrize("cfgname,tokens", [("llama2_7b_reglu_f16", 3),
                                            ("turbosparse_mistral_7b_drelu_f16", 2),
                                            ("falcon_40b_relu_f16", 1),
                                            ("opt125m_relu_f32", 8)])
def test_fused_decode_variant(ffn, cfgname, tokens):
    """The fused predictor + gather variant against the oracle (and the balanced variant)."""
    cfg = synth.CONFIGS[cfgname]
    host = synth.make_layer(cfg, device="cuda")
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, tokens).cuda()
    m = ffn.SparseFFN(L, max_batch=1)
    outs = []
    for variant in (0, 1):
        ffn.ffn_plan_set_decode_variant(m.plan, variant)
        y = torch.zeros(tokens, cfg.d, device="cuda")
        idx = torch.full((tokens, cfg.ffn), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(tokens, dtype=torch.int32, device="cuda")
        for t in range(tokens):
            m.forward(x[t:t + 1], y=y[t:t + 1], idx=idx[t:t + 1], cnt=cnt[t:t + 1])
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()))
    xh = x.cpu().numpy()
    (y0, i0, c0), (y1, i1, c1) = outs
    for t in range(tokens):
        lt = i1[t, :c1[t]]
        pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
        check_index_list(lt, pred, OL["tau"])
        assert np.array_equal(lt, i0[t, :c0[t]])          # same predictor arithmetic
        y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lt, cfg.ffn))
        assert normwise(y1[t], y_ref) <= TOL[cfg.w_dtype]
        assert normwise(y1[t], y0[t].astype(np.float64)) <= 1e-5
    with pytest.raises(ffn.FFNError):
        ffn.ffn_plan_set_decode_variant(m.plan, 2)
    m.close()


def test_fused_variant_small_and_edge_sets(ffn):
    """Fused variant with a ragged ffn (last workgroup owns 32 neurons), tau = 1 (nothing
    fires: y = b_down) and a tiny tau (everything fires: the dense FFN)."""
    cfg = synth.small_config(d=2048, ffn=1056, rank=32, act="drelu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.15, bias_gate=True,
                             bias_up=True, bias_down=True)
    host = synth.make_layer(cfg)
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, 2).cuda()
    xh = x.cpu().numpy()
    for tau in (0.5, 1.0, 1e-30):
        layer = dict(L)
        layer["tau"] = tau
        m = ffn.SparseFFN(layer, max_batch=1)
        ffn.ffn_plan_set_decode_variant(m.plan, 1)
        for t in range(2):
            idx = torch.full((1, cfg.ffn), -1, dtype=torch.int32, device="cuda")
            cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
            y = m.forward(x[t:t + 1], idx=idx, cnt=cnt)
            torch.cuda.synchronize()
            lt = idx[0, :int(cnt[0])].cpu().numpy()
            if tau == 1.0:
                assert lt.size == 0
                assert np.array_equal(y[0].cpu().numpy(), np.asarray(OL["b_down"], np.float32))
            else:
                if tau < 1e-10:
                    assert lt.size == cfg.ffn
                y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lt, cfg.ffn))
                assert normwise(y[0].cpu().numpy(), y_ref) <= TOL["f16"]
        m.close()


@pytest.mark.parametrize("kw", [
    dict(d=2048, ffn=1024, rank=2048, act="reglu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
         bias_gate=True),                                        # the largest fp16 rank
    dict(d=1024, ffn=512, rank=1024, act="relu", w_dtype="f32", x_dtype="f32", p_dtype="f32",
         bias_up=True),                                          # the largest fp32 rank
    dict(d=8192, ffn=1024, rank=64, act="drelu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
         bias_gate=True, bias_up=True),                          # the widest fp16 rows
    dict(d=4096, ffn=512, rank=64, act="relu", w_dtype="f32", x_dtype="f32", p_dtype="f32",
         bias_up=True),                                          # the widest fp32 rows
], ids=["f16_rank2048", "f32_rank1024", "f16_d8192", "f32_d4096"])
def test_shape_limits(ffn, kw):
    cfg = synth.small_config(density=0.1, **kw)
    _check_predicted(ffn, cfg, n_tokens=3)
