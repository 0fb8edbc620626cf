"""The allocation-free decode entry point, ffn_sparse_forward_static (no plan, no workspace: the
per-token scratch is a fixed device array inside the library), against the planned entry point
ffn_sparse_forward through the C ABI.

Two calls in a row share the GPU's one scratch array; the second has a smaller layer and fewer
tokens, so whatever the first left in the array must not leak into it.  Each call's outputs are
compared with ffn_sparse_forward run token by token on the same layer (the same kernels, so y,
the index lists and the counts are bit-identical), and with the oracle on the GPU's own sets.
"""
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


def _static_then_planned(ffn, cfg, B, with_mask):
    print("no-alloc case: %s d=%d ffn=%d rank=%d B=%d mask=%s" % (
        cfg.name, cfg.d, cfg.ffn, cfg.rank, B, with_mask), flush=True)
    host = synth.make_layer(cfg, device="cuda")
    L, OL = to_device(host), oracle_layer(host)
    x = synth.make_tokens(cfg, B, device="cuda")
    m = ffn.SparseFFN(L, max_batch=B)
    mask = None
    if with_mask:
        g = torch.Generator(device="cuda")
        g.manual_seed(7)
        mask = (torch.rand(B, cfg.ffn, generator=g, device="cuda") < 0.15).to(torch.uint8)
    out = {}
    for kind in ("static", "planned"):
        y = torch.full((B, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((B, cfg.ffn), -1, dtype=torch.int32, device="cuda")
        cnt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        if kind == "static":
            ffn.ffn_sparse_forward_static(m.desc, m.weights, x.data_ptr(), B, y.data_ptr(),
                                          0 if mask is None else mask.data_ptr(),
                                          idx.data_ptr(), cnt.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
        else:
            for t in range(B):                      # the batch-1 kernels, token by token
                m.forward(x[t:t + 1], y=y[t:t + 1], idx=idx[t:t + 1], cnt=cnt[t:t + 1],
                          mask=None if mask is None else mask[t:t + 1])
        torch.cuda.synchronize()
        out[kind] = (y.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy())
    m.close()
    ys, is_, cs = out["static"]
    yp, ip, cp = out["planned"]
    assert np.array_equal(cs, cp)
    assert np.array_equal(ys, yp), "static and planned y differ"
    xh = x.cpu().numpy()
    for t in range(B):
        n = int(cs[t])
        assert np.array_equal(is_[t, :n], ip[t, :n])
        lt = is_[t, :n]
        if mask is None:
            pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh[t], OL["tau"])
            check_index_list(lt, pred, OL["tau"])
        else:
            assert np.array_equal(lt, np.flatnonzero(mask[t].cpu().numpy()))
        y_ref, _ = oracle.ffn(OL, xh[t], mask_from_idx(lt, cfg.ffn))
        assert normwise(ys[t], y_ref) <= TOL[cfg.w_dtype], (t, normwise(ys[t], y_ref))


def test_static_entry_point_two_calls_second_smaller(ffn):
    big = synth.with_(synth.CONFIGS["llama2_7b_reglu_f16"], layers=1)
    small = synth.small_config(d=512, ffn=2048, rank=64, act="drelu", w_dtype="f16",
                               x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True,
                               bias_up=True, bias_down=True)
    _static_then_planned(ffn, big, 3, with_mask=False)
    _static_then_planned(ffn, small, 2, with_mask=False)


def test_static_entry_point_caller_mask_and_fp32(ffn):
    opt = synth.CONFIGS["opt125m_relu_f32"]
    _static_then_planned(ffn, opt, 2, with_mask=False)
    small = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16",
                               x_dtype="f16", p_dtype="f16", density=0.1, bias_up=True)
    _static_then_planned(ffn, small, 1, with_mask=True)


def test_static_entry_point_rejects_larger_layers_before_any_launch(ffn):
    cfg = synth.with_(synth.CONFIGS["falcon_40b_relu_f16"], layers=1)
    desc = ffn.ffn_layer_desc(d=cfg.d, ffn=cfg.ffn, rank=cfg.rank, act=ffn.FFN_ACT_RELU,
                              w_dtype=ffn.FFN_F16, x_dtype=ffn.FFN_F16, p_dtype=ffn.FFN_F16,
                              threshold=0.5, max_batch=1)
    w = ffn.ffn_layer_weights(w_up=0x1000, w_down_t=0x2000, p1=0x3000, p2=0x4000)
    with pytest.raises(ffn.FFNError) as e:
        ffn.ffn_sparse_forward_static(desc, w, 0x5000, 1, 0x6000)
    assert e.value.status == ffn.FFN_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in ffn.ffn_last_error()


def test_static_entry_point_in_a_graph(ffn):
    """Callers under graph capture are the ones this entry point is for: the call is captured
    once and replayed three times, with eager work and a static call on another layer (which
    leaves that layer's bytes in the shared scratch) between the replays; every replay equals
    the eager call bit for bit."""
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True,
                             bias_down=True)
    other = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16",
                               x_dtype="f16", p_dtype="f16", density=0.2, bias_up=True)
    print("no-alloc graph case: d=%d ffn=%d B=2, other layer d=%d ffn=%d" % (
        cfg.d, cfg.ffn, other.d, other.ffn), flush=True)
    m = ffn.SparseFFN(to_device(synth.make_layer(cfg, device="cuda")), max_batch=2)
    mo = ffn.SparseFFN(to_device(synth.make_layer(other, device="cuda")), max_batch=1)
    x = synth.make_tokens(cfg, 2, device="cuda")
    xo = synth.make_tokens(other, 1, device="cuda")
    y = torch.zeros(2, cfg.d, device="cuda")
    yo = torch.zeros(1, other.d, device="cuda")
    idx = torch.zeros(2, cfg.ffn, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int32, device="cuda")

    def run():
        ffn.ffn_sparse_forward_static(m.desc, m.weights, x.data_ptr(), 2, y.data_ptr(), 0,
                                      idx.data_ptr(), cnt.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
    torch.cuda.synchronize()
    ref = (y.clone(), idx.clone(), cnt.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        idx.fill_(-1)
        cnt.fill_(-1)
        junk = torch.randn(1 << 20, device="cuda").sum()
        ffn.ffn_sparse_forward_static(mo.desc, mo.weights, xo.data_ptr(), 1, yo.data_ptr(),
                                      stream=torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]), "replay %d: y differs" % rep
        assert torch.equal(cnt, ref[2]), "replay %d: counts differ" % rep
        for t in range(2):
            n = int(ref[2][t])
            assert torch.equal(idx[t, :n], ref[1][t, :n]), "replay %d: index list differs" % rep
        del junk
    del g
    m.close()
    mo.close()
