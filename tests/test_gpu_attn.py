"""GPU parity of the attention block with a head-level active set (head predictor -> query / key /
value rows -> scores, softmax and values over the cache -> output-projection rows of the active
heads) against the CPU oracle, through the C ABI, on seeded synthetic blocks.

Comparison rules: the head list is bit-exact outside the 1e-4 threshold band; the key and value
written at the token's position are within fp16 rounding of the oracle's exact ones; every other
cache position is untouched (bit-exact); y is within 2e-3 normwise of the oracle evaluated on the
GPU's own head set and the oracle's own cache (fp16 weights and cache, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_index_list, mask_from_idx, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-3
KEYS = ["w_q", "w_k", "w_v", "w_o_t", "p1", "p2", "c1", "c2"]


@pytest.fixture(scope="module")
def ffn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_ffn_gemv_amd as m
    return m


def _layers(cfg, layer=0):
    host = synth.make_attn_layer(cfg, layer=layer)
    dev = dict(host)
    for k in KEYS:
        if isinstance(host.get(k), torch.Tensor):
            dev[k] = host[k].cuda().contiguous()
    ol = {k: (None if host.get(k) is None else np.ascontiguousarray(host[k].numpy()))
          for k in KEYS}
    ol.update(tau=cfg.tau, head_dim=cfg.head_dim)
    return dev, ol


def _check_token(ffn, m, cfg, OL, x, pos, Kd, Vd, Kh, Vh, mask=None):
    """One forward on the device caches (Kd, Vd) and the oracle on its own (Kh, Vh); returns the
    oracle's updated caches."""
    H = cfg.heads
    y = torch.full((cfg.d,), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((H,), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    scores = torch.zeros(H, dtype=torch.float32, device="cuda")
    before_k, before_v = Kd.clone(), Vd.clone()
    mk = None if mask is None else torch.from_numpy(mask).cuda()
    m.forward(x, pos, Kd, Vd, y=y, mask=mk, idx=idx, cnt=cnt, scores=scores)
    torch.cuda.synchronize()
    xh = x.cpu().numpy()
    n = int(cnt.item())
    heads = idx.cpu().numpy()[:n]
    if mask is None:
        pred = oracle.predictor(OL["p1"], OL["p2"], OL["c1"], OL["c2"], xh, OL["tau"])
        check_index_list(heads, pred, OL["tau"])
        assert normwise(scores.cpu().numpy(), pred["s"]) <= TOL
    else:
        assert np.array_equal(heads, np.flatnonzero(mask))
    # the caches: position pos within fp16 rounding of the exact key / value, the rest untouched
    k, v = oracle.attn_kv(OL["w_k"], OL["w_v"], xh, cfg.head_dim)
    G, e = cfg.kv_heads, cfg.head_dim
    for got, exact in ((Kd[:, pos].cpu().numpy(), k), (Vd[:, pos].cpu().numpy(), v)):
        exact = exact.reshape(G, e)
        assert np.all(np.abs(got.astype(np.float64) - exact) <= 2.0 ** -10 * np.abs(exact) + 1e-6)
    keep = [j for j in range(Kd.shape[1]) if j != pos]
    assert torch.equal(Kd[:, keep], before_k[:, keep]) and torch.equal(Vd[:, keep], before_v[:, keep])
    # y on the GPU's head set, the oracle's own cache
    y_ref, _, Kn, Vn = oracle.attn_token(OL, Kh, Vh, xh, pos, mask_from_idx(heads, H))
    err = normwise(y.cpu().numpy(), y_ref)
    assert err <= TOL, (pos, n, err)
    return Kn, Vn, n


def _run_case(ffn, cfg, positions, masks=None, layer=0):
    dev, OL = _layers(cfg, layer)
    Kd, Vd = (t.cuda() for t in synth.make_kv_cache(cfg, layer))
    Kh, Vh = (t.numpy() for t in synth.make_kv_cache(cfg, layer))
    xs = synth.make_attn_tokens(cfg, len(positions), layer).cuda()
    m = ffn.SparseAttention(dev, max_seq=cfg.seq)
    counts = []
    try:
        for i, pos in enumerate(positions):
            print("attn case %s pos=%d" % (cfg.name, pos), flush=True)
            mask = None if masks is None else masks[i]
            Kh, Vh, n = _check_token(ffn, m, cfg, OL, xs[i], pos, Kd, Vd, Kh, Vh, mask)
            counts.append(n)
    finally:
        m.close()
    return counts


SMALL = [
    # name, d, H, G, e, rank, seq
    ("mha_e64", 256, 4, 4, 64, 16, 40),
    ("gqa_e128", 512, 8, 2, 128, 32, 70),
    ("opt125m_e64", 768, 12, 12, 64, 32, 100),
    ("ragged_d", 328, 6, 3, 64, 8, 33),
    ("h128_e64", 1024, 128, 8, 64, 64, 20),
    ("mqa_e128", 1024, 16, 1, 128, 128, 300),
    # a long context: 256 chunk records per head (the most the workspace holds)
    ("long_ctx", 256, 4, 2, 64, 16, 8192),
    # chunks of two load batches or more (the score kernel's double-buffered form), ragged ends
    ("pipe_e128", 512, 32, 8, 128, 32, 4096),
    ("pipe_e64", 256, 32, 4, 64, 16, 8192),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_attn_small_sequence(ffn, case):
    """A run of tokens at growing positions (the cache written by each is read by the next),
    starting at 0, through chunk tails, to the last position of the cache."""
    name, d, H, G, e, r, seq = case
    cfg = synth.AttnConfig(name, d=d, heads=H, kv_heads=G, head_dim=e, rank=r, density=0.5,
                           context=seq - 5, max_seq=seq)
    positions = [0, 1, seq // 2 + 1, seq - 5, seq - 4, seq - 1]
    counts = _run_case(ffn, cfg, positions)
    assert 0 < sum(counts) < H * len(positions)


@pytest.mark.parametrize("kind", ["all", "none", "one", "alternate"])
def test_attn_caller_masks(ffn, kind):
    cfg = synth.AttnConfig("masks", d=512, heads=8, kv_heads=4, head_dim=64, rank=16,
                           density=0.5, context=30, max_seq=48)
    H = cfg.heads
    mk = {"all": np.ones(H, np.uint8), "none": np.zeros(H, np.uint8),
          "one": np.eye(1, H, 5, dtype=np.uint8)[0],
          "alternate": (np.arange(H) % 2).astype(np.uint8)}[kind]
    counts = _run_case(ffn, cfg, [30, 31, 47], masks=[mk] * 3)
    assert counts == [int(mk.sum())] * 3


def test_attn_empty_set_gives_zero(ffn):
    cfg = synth.AttnConfig("empty", d=256, heads=4, kv_heads=2, head_dim=64, rank=8,
                           density=0.5, context=10, max_seq=16)
    dev, _ = _layers(cfg)
    Kd, Vd = (t.cuda() for t in synth.make_kv_cache(cfg))
    m = ffn.SparseAttention(dev, max_seq=cfg.seq)
    x = synth.make_attn_tokens(cfg, 1)[0].cuda()
    y = torch.full((cfg.d,), float("nan"), device="cuda")
    m.forward(x, 10, Kd, Vd, y=y, mask=torch.zeros(4, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    m.close()


def test_attn_is_bit_reproducible(ffn):
    cfg = synth.ATTN_CONFIGS["mistral_7b_attn_f16"]
    dev, _ = _layers(cfg)
    K0, V0 = (t.cuda() for t in synth.make_kv_cache(cfg))
    x = synth.make_attn_tokens(cfg, 1)[0].cuda()
    m = ffn.SparseAttention(dev, max_seq=cfg.seq)
    ys = []
    for _ in range(3):
        K, V = K0.clone(), V0.clone()
        ys.append(m.forward(x, cfg.context, K, V).clone())
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
    m.close()


@pytest.mark.parametrize("name", list(synth.ATTN_CONFIGS))
def test_attn_full_shape(ffn, name):
    """The benchmark's blocks at full size, at the benchmark's position and at position 0."""
    cfg = synth.ATTN_CONFIGS[name]
    counts = _run_case(ffn, cfg, [cfg.context, 0], layer=3)
    assert all(0 < c < cfg.heads for c in counts)


def test_attn_plan_without_predictor(ffn):
    """rank 0: no predictor weights at all (P1, P2 NULL); the caller's mask picks the heads."""
    cfg = synth.AttnConfig("nopred", d=256, heads=4, kv_heads=4, head_dim=64, rank=8,
                           density=0.5, context=12, max_seq=16)
    dev, OL = _layers(cfg)
    for k in ("p1", "p2", "c1", "c2"):
        dev[k] = None
    Kd, Vd = (t.cuda() for t in synth.make_kv_cache(cfg))
    Kh, Vh = (t.numpy() for t in synth.make_kv_cache(cfg))
    m = ffn.SparseAttention(dev, max_seq=cfg.seq)
    assert m.desc.rank == 0
    x = synth.make_attn_tokens(cfg, 1)[0].cuda()
    with pytest.raises(ffn.FFNError):                  # no predictor and no mask
        m.forward(x, 12, Kd, Vd)
    mk = np.array([0, 1, 1, 0], np.uint8)
    _check_token(ffn, m, cfg, OL, x, 12, Kd, Vd, Kh, Vh, mk)
    m.close()
