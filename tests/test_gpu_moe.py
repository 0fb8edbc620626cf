"""GPU parity of the mixture of experts (on-device top-k router + sparse experts) against the CPU
oracle, through the C ABI.

The routing decision is an integer decided by floating point: the chosen experts must equal the
oracle's (fp64 logits) unless the oracle's k-th and (k+1)-th logits are closer than ROUTE_BAND
(relative to the largest |logit|), where either choice is accepted.  Each chosen expert's active
set is taken from the same library's single-expert forward (its parity is covered by the decode
tests), and y is compared with the oracle's weighted sum evaluated on those sets."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, mask_from_idx, normwise, oracle_layer, to_device

pytestmark = pytest.mark.gpu

ROUTE_BAND = 1e-5


@pytest.fixture(scope="module")
def ffn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_ffn_gemv_amd as m
    return m


def _expert_sets(ffn, L, x):
    """Active lists of every token under one expert, from the single-expert forward (token by
    token, the kernels the mixture runs)."""
    m = ffn.SparseFFN(L, max_batch=1)
    F = L["w_up"].shape[0]
    idx = torch.zeros(x.shape[0], F, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(x.shape[0], dtype=torch.int32, device="cuda")
    for t in range(x.shape[0]):
        m.forward(x[t:t + 1], idx=idx[t:t + 1], cnt=cnt[t:t + 1])
    torch.cuda.synchronize()
    out = [idx[b, :int(cnt[b])].cpu().numpy() for b in range(x.shape[0])]
    m.close()
    return out


def _check_moe(ffn, cfg, n_experts, top_k, n_tokens, experts=None, R=None):
    if experts is None:
        experts = [to_device(synth.make_layer(cfg, layer=0, expert=e, device="cuda"))
                   for e in range(n_experts)]
    if R is None:
        R = synth.make_router(synth.with_(cfg, n_experts=n_experts), device="cuda")
        if cfg.x_dtype == "f32":
            R = R.float()
    x = synth.make_tokens(cfg, n_tokens).cuda()
    moe = ffn.MoEFFN(experts, R, top_k=top_k, max_batch=n_tokens)
    y = torch.full((n_tokens, cfg.d), float("nan"), device="cuda")
    ids = torch.full((n_tokens, top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros(n_tokens, top_k, dtype=torch.float32, device="cuda")
    cnt = torch.full((n_tokens, top_k), -1, dtype=torch.int32, device="cuda")
    moe.forward(x, y=y, expert_idx=ids, expert_w=w, expert_cnt=cnt)
    torch.cuda.synchronize()
    y_h, ids_h, w_h = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    cnt_h = cnt.cpu().numpy()
    moe.close()

    OLs = [oracle_layer(e) for e in experts]
    Rh = R.cpu().numpy()
    xh = x.cpu().numpy()
    sets = {}
    for t in range(n_tokens):
        ids_ref, w_ref, logits = oracle.router(Rh, xh[t], top_k)
        srt = np.sort(logits)[::-1]
        tie = top_k < n_experts and (srt[top_k - 1] - srt[top_k]) <= ROUTE_BAND * np.abs(srt).max()
        if not tie:
            assert np.array_equal(ids_h[t], ids_ref), (t, ids_h[t], ids_ref)
            assert np.allclose(w_h[t], w_ref, rtol=0, atol=2e-6), (w_h[t], w_ref)
        assert abs(w_h[t].sum() - 1.0) < 1e-6
        assert len(set(ids_h[t].tolist())) == top_k
        masks = []
        for j, e in enumerate(ids_h[t]):
            if e not in sets:
                sets[e] = _expert_sets(ffn, experts[e], x)
            masks.append(mask_from_idx(sets[e][t], cfg.ffn))
            assert cnt_h[t, j] == len(sets[e][t]), (t, j, cnt_h[t, j], len(sets[e][t]))
        # oracle on the GPU's routing decision and the GPU's active sets
        y_ref = np.zeros(cfg.d)
        for j, e in enumerate(ids_h[t]):
            ye, _ = oracle.ffn(OLs[e], xh[t], masks[j])
            y_ref += float(w_h[t, j]) * ye
        assert normwise(y_h[t], y_ref) <= TOL[cfg.w_dtype], (t, normwise(y_h[t], y_ref))
    return ids_h


@pytest.mark.parametrize("kw,E,K", [
    (dict(d=256, ffn=1024, rank=32, act="drelu", w_dtype="i4g32", x_dtype="f16", p_dtype="f16",
          bias_gate=True, bias_up=True, bias_down=True), 4, 2),
    (dict(d=128, ffn=512, rank=16, act="relu", w_dtype="f32", x_dtype="f32", p_dtype="f32",
          bias_up=True), 3, 1),
    (dict(d=512, ffn=2048, rank=64, act="reglu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
          bias_gate=True, bias_down=True), 8, 2),
    (dict(d=256, ffn=1056, rank=24, act="drelu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
          bias_gate=True, bias_up=True), 16, 4),
    # expert counts that leave some waves' logit slots past the last expert (they re-read the
    # last expert's row and must not be used): 6 experts at two per wave, 13 at four per wave
    (dict(d=256, ffn=512, rank=16, act="reglu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
          bias_gate=True), 6, 2),
    (dict(d=384, ffn=768, rank=16, act="relu", w_dtype="f32", x_dtype="f32", p_dtype="f32",
          bias_up=True), 13, 3),
], ids=["i4_e4k2", "f32_e3k1", "f16_e8k2", "f16_e16k4", "f16_e6k2", "f32_e13k3"])
def test_moe_small(ffn, kw, E, K):
    cfg = synth.small_config(density=0.1, **kw)
    _check_moe(ffn, cfg, E, K, n_tokens=5)


def test_identical_experts_reduce_to_one_ffn(ffn):
    """With every expert the same layer the weighted sum is that layer's FFN (weights sum to 1),
    whichever experts the router picks."""
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="reglu", w_dtype="f16",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True)
    L = to_device(synth.make_layer(cfg, device="cuda"))
    R = synth.make_router(synth.with_(cfg, n_experts=4), device="cuda")
    x = synth.make_tokens(cfg, 3).cuda()
    moe = ffn.MoEFFN([L] * 4, R, top_k=2, max_batch=3)
    y_moe = moe.forward(x).clone()
    single = ffn.SparseFFN(L, max_batch=1)             # token by token, as the mixture runs
    y_one = torch.cat([single.forward(x[t:t + 1]).clone() for t in range(3)])
    torch.cuda.synchronize()
    for t in range(3):
        assert normwise(y_moe[t].cpu().numpy(), y_one[t].cpu().numpy().astype(np.float64)) <= 1e-5
    moe.close()
    single.close()


def test_forced_router_choice_is_exact(ffn):
    """Router rows built so that a known pair of experts wins by a wide margin: the ids and the
    weights follow in closed form (w = softmax of the two logits)."""
    cfg = synth.small_config(d=128, ffn=512, rank=16, act="relu", w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_up=True)
    experts = [to_device(synth.make_layer(cfg, expert=e, device="cuda")) for e in range(4)]
    x = torch.zeros(1, cfg.d, dtype=torch.float16, device="cuda")
    x[0, 0] = 1.0
    R = torch.zeros(4, cfg.d, dtype=torch.float16, device="cuda")
    R[2, 0], R[0, 0], R[1, 0], R[3, 0] = 3.0, 2.0, -1.0, 0.5    # winners 2 then 0
    moe = ffn.MoEFFN(experts, R, top_k=2, max_batch=1)
    ids = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    w = torch.zeros(1, 2, device="cuda")
    moe.forward(x, expert_idx=ids, expert_w=w)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [[2, 0]]
    wa = 1.0 / (1.0 + np.exp(2.0 - 3.0))
    assert np.allclose(w.cpu().numpy()[0], [wa, 1 - wa], atol=1e-6)
    moe.close()


def test_mixtral_int4_shape(ffn):
    """Eight int4 group-32 dReLU experts (d=4096, ffn=14336, rank 256), top-2, 2 tokens."""
    cfg = synth.CONFIGS["turbosparse_mixtral_47b_moe_int4"]
    _check_moe(ffn, cfg, cfg.n_experts, cfg.top_k, n_tokens=2)


def test_moe_batch_equals_single_tokens(ffn):
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="drelu", w_dtype="i4g32",
                             x_dtype="f16", p_dtype="f16", density=0.1, bias_gate=True,
                             bias_up=True)
    experts = [to_device(synth.make_layer(cfg, expert=e, device="cuda")) for e in range(4)]
    R = synth.make_router(synth.with_(cfg, n_experts=4), device="cuda")
    x = synth.make_tokens(cfg, 4).cuda()
    moe = ffn.MoEFFN(experts, R, top_k=2, max_batch=4)
    yb = moe.forward(x).clone()
    for t in range(4):
        y1 = moe.forward(x[t:t + 1]).clone()
        torch.cuda.synchronize()
        assert torch.equal(y1[0], yb[t])
    moe.close()


def test_chosen_expert_with_an_empty_set(ffn):
    """The router's first choice is an expert whose predictor fires for no neuron (c2 far below
    the threshold): its slot reports |A| = 0, reads no row, and y is the other expert's weighted
    FFN plus the empty expert's weighted b_down (the oracle on the same sets)."""
    cfg = synth.small_config(d=256, ffn=1024, rank=32, act="relu", w_dtype="f16", x_dtype="f16",
                             p_dtype="f16", density=0.1, bias_up=True, bias_down=True)
    experts = [to_device(synth.make_layer(cfg, expert=e, device="cuda")) for e in range(4)]
    experts[2]["c2"] = torch.full_like(experts[2]["c2"], -1.0e4)   # expert 2 never fires
    x = synth.make_tokens(cfg, 1).cuda()
    R = torch.zeros(4, cfg.d, dtype=torch.float16, device="cuda")
    k = int(torch.argmax(x[0].abs()))
    s = 1.0 if float(x[0, k]) > 0 else -1.0
    R[2, k], R[0, k], R[1, k], R[3, k] = 3.0 * s, 2.0 * s, -1.0 * s, 0.5 * s   # winners 2, then 0
    moe = ffn.MoEFFN(experts, R, top_k=2, max_batch=1)
    y = torch.full((1, cfg.d), float("nan"), device="cuda")
    ids = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    w = torch.zeros(1, 2, device="cuda")
    cnt = torch.full((1, 2), -1, dtype=torch.int32, device="cuda")
    moe.forward(x, y=y, expert_idx=ids, expert_w=w, expert_cnt=cnt)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [[2, 0]]
    cnt_h, w_h = cnt.cpu().numpy()[0], w.cpu().numpy()[0]
    assert cnt_h[0] == 0
    set0 = _expert_sets(ffn, experts[0], x)[0]
    assert cnt_h[1] == len(set0)
    xh = x.cpu().numpy()[0]
    y2, _ = oracle.ffn(oracle_layer(experts[2]), xh, np.zeros(cfg.ffn, np.uint8))
    y0, _ = oracle.ffn(oracle_layer(experts[0]), xh, mask_from_idx(set0, cfg.ffn))
    y_ref = float(w_h[0]) * y2 + float(w_h[1]) * y0
    assert normwise(y.cpu().numpy()[0], y_ref) <= TOL["f16"]
    moe.close()
