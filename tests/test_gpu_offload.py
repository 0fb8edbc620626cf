"""GPU parity of the neuron cache over host-resident rows, through the C ABI: every token's y,
index list and count bit-identical to the same layer held in device memory, and the pool's
tables and per-call counts identical to the CPU model of the LRU policy (oracle.NeuronCache) fed
with the same active sets."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, mask_from_idx, normwise, oracle_layer, to_device

pytestmark = pytest.mark.gpu

ROWS = ("w_up", "w_gate", "w_down_t")


@pytest.fixture(scope="module")
def ffn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_ffn_gemv_amd as m
    return m


def _host_rows(L):
    H = dict(L)
    for k in ROWS:
        if L.get(k) is not None:
            H[k] = L[k].cpu().contiguous().pin_memory()
    return H


def _run_pair(ffn, cfg, capacity, n_tokens, n_pinned=0, hot=False, layer_no=0):
    host = synth.make_layer(cfg, layer=layer_no, device="cuda")
    if hot:
        host = synth.hot_first(host)
        host["n_hot"] = n_pinned
    L = to_device(host)
    res = ffn.SparseFFN(L, max_batch=1)
    off = ffn.OffloadFFN(_host_rows(L), capacity, n_pinned=n_pinned)
    model = oracle.NeuronCache(cfg.ffn, capacity, n_pinned)
    x = synth.make_tokens(cfg, n_tokens, layer=layer_no, salt=7).cuda()
    F = cfg.ffn
    out = []
    tot = [0, 0, 0, 0]
    for t in range(n_tokens):
        ys = []
        lists = []
        for m in (res, off):
            y = torch.full((1, cfg.d), float("nan"), device="cuda")
            idx = torch.full((1, F), -1, dtype=torch.int32, device="cuda")
            cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            m.forward(x[t:t + 1], y=y, idx=idx, cnt=cnt)
            torch.cuda.synchronize()
            ys.append(y.clone())
            lists.append(idx[0, :int(cnt[0])].cpu().numpy())
        assert torch.equal(ys[0], ys[1]), "token %d: y differs from the resident layer" % t
        assert np.array_equal(lists[0], lists[1])
        src, victim = model.step(lists[1])
        slot_of, neuron_of, last_use, stats = off.tables()
        assert np.array_equal(slot_of.cpu().numpy(), model.slot_of), t
        assert np.array_equal(neuron_of.cpu().numpy(), model.neuron_of), t
        assert np.array_equal(last_use.cpu().numpy(), model.last_use), t
        hits = sum(s >= 0 for s in src)
        adm = sum(v >= 0 for v in victim)
        assert stats.cpu().tolist()[:4] == [hits, len(src) - hits, adm, len(src)], t
        tot = [tot[0] + hits, tot[1] + len(src) - hits, tot[2] + adm, tot[3] + len(src)]
        assert stats.cpu().tolist()[4:] == tot, t
        out.append((x[t].cpu().numpy(), lists[1], ys[1][0].cpu().numpy(), hits, adm))
    res.close()
    off.close()
    return host, out


@pytest.mark.parametrize("act,d,capacity", [("reglu", 512, 256), ("relu", 1024, 128),
                                            ("drelu", 4096, 512), ("reglu", 8192, 96)])
def test_offload_bit_identical_and_lru_exact(ffn, act, d, capacity):
    """Small pools against sets of ~10% of the neurons: hits, admissions, evictions and (for
    the smallest pools) misses read without admission, across 20 tokens."""
    ffn_n = 2048 if d <= 4096 else 1024
    cfg = synth.small_config(d=d, ffn=ffn_n, rank=64, act=act, w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_gate=act != "relu", bias_up=True,
                             bias_down=True)
    host, out = _run_pair(ffn, cfg, capacity, 20)
    assert sum(o[3] for o in out) > 0 and sum(o[4] for o in out) > 0   # the pool was used
    OL = oracle_layer(host)
    for xt, lst, y, _, _ in out[:3]:
        y_ref, _ = oracle.ffn(OL, xt, mask_from_idx(lst, cfg.ffn))
        assert normwise(y, y_ref) <= TOL["f16"]


def test_offload_pool_smaller_than_the_set(ffn):
    """A 32-slot pool against ~200 active neurons: most misses are read from host memory without
    admission, and y stays bit-identical."""
    cfg = synth.small_config(d=1024, ffn=2048, rank=64, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True)
    _, out = _run_pair(ffn, cfg, 32, 6)
    assert all(len(o[1]) > 32 for o in out)


def test_offload_pinned_hot_head(ffn):
    """Neurons ordered hottest first, the head always active (hot head) and pinned in the pool:
    its slots never change and every head neuron is a hit."""
    cfg = synth.small_config(d=1024, ffn=2048, rank=64, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True)
    _, out = _run_pair(ffn, cfg, 256, 12, n_pinned=64, hot=True)
    for _, lst, _, hits, _ in out:
        assert np.array_equal(lst[:64], np.arange(64)) and hits >= 64


def test_offload_graph_replay_matches_eager(ffn):
    """The pool's state advances inside a captured graph exactly as in eager calls."""
    cfg = synth.small_config(d=1024, ffn=2048, rank=64, act="relu", w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_up=True)
    L = to_device(synth.make_layer(cfg, device="cuda"))
    H = _host_rows(L)
    x = synth.make_tokens(cfg, 8, salt=9).cuda()
    eager = ffn.OffloadFFN(H, 128)
    ye = torch.zeros(8, cfg.d, device="cuda")
    for t in range(8):
        eager.forward(x[t:t + 1], y=ye[t:t + 1])
    torch.cuda.synchronize()
    te = eager.tables()
    graph = ffn.OffloadFFN(H, 128)
    yg = torch.zeros(8, cfg.d, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for t in range(8):
                graph.forward(x[t:t + 1], y=yg[t:t + 1])
        # capture enqueues nothing: the pool is still fresh; one replay runs the 8 tokens
        g.replay()
    torch.cuda.synchronize()
    tg = graph.tables()
    assert torch.equal(ye, yg)
    for a, b in zip(te, tg):
        assert torch.equal(a, b)
    eager.close()
    graph.close()


def test_offload_dense_and_caller_mask(ffn):
    """A caller mask goes through the pool like a predicted set; the dense FFN reads every row
    straight from host memory and leaves the pool as it was.  Both bit-identical to the
    resident layer, the pool following the model."""
    cfg = synth.small_config(d=1024, ffn=2048, rank=64, act="drelu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True,
                             bias_up=True, bias_down=True)
    L = to_device(synth.make_layer(cfg, device="cuda"))
    res = ffn.SparseFFN(L, max_batch=1)
    off = ffn.OffloadFFN(_host_rows(L), 256)
    model = oracle.NeuronCache(cfg.ffn, 256)
    x = synth.make_tokens(cfg, 3, salt=11).cuda()
    rng = np.random.default_rng(4)
    for t in range(3):
        y0 = res.dense(x[t:t + 1]).clone()
        y1 = off.dense(x[t:t + 1]).clone()
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)
        mask = (rng.random(cfg.ffn) < 0.2).astype(np.uint8)
        mt = torch.from_numpy(mask).cuda().view(1, -1)
        y0 = res.forward(x[t:t + 1], mask=mt).clone()
        y1 = off.forward(x[t:t + 1], mask=mt).clone()
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)
        model.step(np.flatnonzero(mask))
        slot_of, neuron_of, last_use, stats = off.tables()
        assert np.array_equal(neuron_of.cpu().numpy(), model.neuron_of)
        assert np.array_equal(last_use.cpu().numpy(), model.last_use)
    res.close()
    off.close()
