"""The forward calls only enqueue work (no allocation, no synchronisation, no memset nodes), so a
caller can capture them in a HIP graph: every path is captured once and replayed several times,
with eager work and synchronisations in between, and every replay must equal the eager result
bit for bit."""
import pytest
import torch

import synth
from parity import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ffn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_ffn_gemv_amd as m
    return m


def _replays_match(run, out, n=3):
    """run() enqueues on the current stream and writes `out`; compare graph replays to eager."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(n):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs" % rep
        del junk


@pytest.mark.parametrize("wd,B,path", [("f16", 1, "sparse"), ("f16", 5, "sparse"),
                                       ("f16", 70, "auto"), ("f16", 70, "dense"),
                                       ("i4g32", 1, "sparse"), ("f32", 2, "sparse")])
def test_forward_in_a_graph(ffn, wd, B, path):
    xd = "f32" if wd == "f32" else "f16"
    cfg = synth.small_config(d=512, ffn=2048, rank=64, act="reglu", w_dtype=wd, x_dtype=xd,
                             p_dtype=xd, density=0.1, bias_gate=True, bias_down=True)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, B).cuda()
    m = ffn.SparseFFN(L, max_batch=B)
    if path == "auto":
        ffn.ffn_plan_set_crossover(m.plan, B, 0.3)        # let the device choose the dense rows
    y = torch.zeros(B, cfg.d, device="cuda")
    idx = torch.zeros(B, cfg.ffn, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    p = {"sparse": ffn.FFN_PATH_SPARSE, "auto": ffn.FFN_PATH_AUTO,
         "dense": ffn.FFN_PATH_DENSE}[path]
    _replays_match(lambda: m.forward(x, y=y, idx=idx, cnt=cnt, path=p), y)
    m.close()


def test_mixture_in_a_graph(ffn):
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="drelu", w_dtype="i4g32",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True,
                             bias_up=True)
    experts = [to_device(synth.make_layer(cfg, expert=e)) for e in range(4)]
    R = synth.make_router(synth.with_(cfg, n_experts=4), device="cuda")
    x = synth.make_tokens(cfg, 3).cuda()
    moe = ffn.MoEFFN(experts, R, top_k=2, max_batch=3)
    y = torch.zeros(3, cfg.d, device="cuda")
    _replays_match(lambda: moe.forward(x, y=y), y)
    moe.close()


def test_dense_forward_in_a_graph(ffn):
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_up=True)
    L = to_device(synth.make_layer(cfg))
    x = synth.make_tokens(cfg, 96).cuda()
    m = ffn.SparseFFN(L, max_batch=96)
    y = torch.zeros(96, cfg.d, device="cuda")
    _replays_match(lambda: m.dense(x, y=y), y)
    m.close()


def test_auto_choice_in_a_graph_follows_the_data(ffn):
    """One captured AUTO call of 130 tokens (two passes in one launch per kernel) replayed with
    different caller sets in the same mask buffer: a dense set (union above the crossover) makes
    the device run the dense GEMMs, a sparse one the sparse passes, replay after replay, and each
    replay equals the eager call on the same sets bit for bit."""
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_up=True, bias_down=True)
    L = to_device(synth.make_layer(cfg))
    B = 130
    x = synth.make_tokens(cfg, B).cuda()
    m = ffn.SparseFFN(L, max_batch=B)
    ffn.ffn_plan_set_crossover(m.plan, B, 0.5)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    masks = {
        # every token's set: 90% of the neurons (union 100%: dense) or a shared 5% (sparse)
        "dense": (torch.rand(B, cfg.ffn, generator=g, device="cuda") < 0.9).to(torch.uint8),
        "sparse": (torch.rand(1, cfg.ffn, generator=g, device="cuda") < 0.05)
        .to(torch.uint8).expand(B, cfg.ffn).contiguous(),
    }
    mask = torch.zeros(B, cfg.ffn, dtype=torch.uint8, device="cuda")
    y = torch.zeros(B, cfg.d, device="cuda")

    def run():
        m.forward(x, y=y, mask=mask, path=ffn.FFN_PATH_AUTO)

    s = torch.cuda.Stream()
    ref = {}
    for kind, mk in masks.items():
        mask.copy_(mk)
        with torch.cuda.stream(s):
            run()
        torch.cuda.synchronize()
        assert m.last_auto_path() == kind, (kind, m.last_auto_path())
        ref[kind] = y.clone()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(gr, stream=s):
            run()
    torch.cuda.synchronize()
    for kind in ("dense", "sparse", "sparse", "dense", "dense", "sparse"):
        mask.copy_(masks[kind])
        y.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert m.last_auto_path() == kind
        assert torch.equal(y, ref[kind]), "replay with the %s sets differs" % kind
        del junk
    del gr
    m.close()


@pytest.mark.parametrize("predicted", [True, False])
def test_attention_in_a_graph(ffn, predicted):
    """The attention block's forward (predicted heads, or a caller mask) captured and replayed:
    y, the head list and the cache position it writes equal the eager call's on every replay."""
    cfg = synth.AttnConfig("graph", d=512, heads=8, kv_heads=2, head_dim=64, rank=32,
                           density=0.5, context=40)
    L = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
         for k, v in synth.make_attn_layer(cfg).items()}
    K, V = (t.cuda() for t in synth.make_kv_cache(cfg))
    x = synth.make_attn_tokens(cfg, 1)[0].cuda()
    m = ffn.SparseAttention(L, max_seq=cfg.seq)
    mask = None if predicted else (torch.arange(8, device="cuda") % 3 == 0).to(torch.uint8)
    y = torch.zeros(cfg.d, device="cuda")
    idx = torch.zeros(8, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run():
        m.forward(x, cfg.context, K, V, y=y, mask=mask, idx=idx, cnt=cnt)

    _replays_match(run, y)
    # the list and the cache position of the last replay equal a fresh eager call's
    idx0, cnt0, k0 = idx.clone(), cnt.clone(), K[:, cfg.context].clone()
    run()
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt0) and torch.equal(idx[:int(cnt0)], idx0[:int(cnt0)])
    assert torch.equal(K[:, cfg.context], k0)
    m.close()
