"""The seeded input generator: determinism and the power-law density it is calibrated to."""
import numpy as np
import torch

import synth


def test_zipf_probs_mean_cap_and_determinism():
    for F, rho in [(3072, 0.10), (11008, 0.10), (32768, 0.15), (14336, 0.05)]:
        p = synth.zipf_probs(F, rho, 1.1, 0.99, seed=5)
        assert abs(p.mean() - rho) < 1e-9
        assert p.max() <= 0.99 and p.min() > 0
        assert np.array_equal(p, synth.zipf_probs(F, rho, 1.1, 0.99, seed=5))
        assert not np.array_equal(p, synth.zipf_probs(F, rho, 1.1, 0.99, seed=6))
        # power law: sorted probabilities fall as rank^-1.1 below the cap
        q = np.sort(p)[::-1]
        free = q < 0.99
        k = np.arange(1, F + 1)[free]
        slope = np.polyfit(np.log(k), np.log(q[free]), 1)[0]
        assert abs(slope + 1.1) < 0.02


def test_make_layer_deterministic_small():
    cfg = synth.small_config(act="drelu", w_dtype="f16", x_dtype="f16", p_dtype="f16",
                             bias_gate=True)
    a = synth.make_layer(cfg, layer=1)
    b = synth.make_layer(cfg, layer=1)
    c = synth.make_layer(cfg, layer=2)
    for k in ["w_up", "w_gate", "w_down_t", "p1", "p2", "c2", "b_gate", "b_up"]:
        assert torch.equal(a[k], b[k]), k
    assert not torch.equal(a["w_up"], c["w_up"])
    x1 = synth.make_tokens(cfg, 4, layer=1)
    assert torch.equal(x1, synth.make_tokens(cfg, 4, layer=1))
    assert x1.dtype == torch.float16 and x1.shape == (4, cfg.d)


def test_calibrated_firing_rate_opt125m_shape():
    """True ReLU firing rate over seeded N(0,1) tokens matches the 10% target and the hot head
    fires almost always; the selector predictor's density tracks it."""
    cfg = synth.CONFIGS["opt125m_relu_f32"]
    L = synth.make_layer(cfg)
    x = synth.make_tokens(cfg, 256).double()
    u = x @ L["w_up"].double().T + L["b_up"].double()
    fire = (u > 0).double()
    assert abs(fire.mean().item() - 0.10) < 0.01
    hot = torch.from_numpy(L["probs"]) >= 0.99
    assert hot.sum() > 10
    assert fire[:, hot].mean().item() > 0.95
    z = x @ L["p1"].double().T
    s = z @ L["p2"].double().T + L["c2"].double()
    pred = (s > 0).double()
    assert abs(pred.mean().item() - 0.10) < 0.015
    # the predicted set overlaps the true set far above chance
    inter = (pred * fire).sum() / fire.sum()
    assert inter.item() > 0.4


def test_int4_quantizer_error_bound():
    w = torch.randn(16, 128, generator=torch.Generator().manual_seed(3)) * 0.02
    packed, scales = synth.quantize_i4g32(w)
    assert packed.dtype == torch.uint8 and packed.shape == (16, 64)
    assert scales.dtype == torch.float16 and scales.shape == (16, 4)
    pk = packed.numpy()
    lo = (pk & 0xF).astype(np.int64)
    hi = (pk >> 4).astype(np.int64)
    q = np.stack([lo, hi], -1).reshape(16, 128)
    q = np.where(q >= 8, q - 16, q)
    s = np.repeat(scales.numpy().astype(np.float64), 32, axis=1)
    err = np.abs(q * s - w.double().numpy())
    # s = fp16(max|w|/7): every element rounds to the nearest step, at most half a step away
    # (up to the fp16 rounding of s itself)
    assert (err <= s * 0.5 * (1 + 2e-3) + 1e-12).all()
    assert (q >= -8).all() and (q <= 7).all()


def test_attention_inputs_deterministic_and_shaped():
    cfg = synth.AttnConfig("t", d=128, heads=8, kv_heads=2, head_dim=64, rank=16, density=0.5,
                           context=30, max_seq=40)
    a = synth.make_attn_layer(cfg, layer=1)
    b = synth.make_attn_layer(cfg, layer=1)
    c = synth.make_attn_layer(cfg, layer=2)
    for k in ["w_q", "w_k", "w_v", "w_o_t", "p1", "p2", "c2"]:
        assert torch.equal(a[k], b[k]), k
    assert not torch.equal(a["w_q"], c["w_q"])
    assert a["w_q"].shape == (8 * 64, 128) and a["w_k"].shape == (2 * 64, 128)
    assert a["w_o_t"].shape == (8 * 64, 128) and a["w_q"].dtype == torch.float16
    assert a["p1"].shape == (16, 128) and a["p2"].shape == (8, 16) and a["c2"].shape == (8,)
    # P1 is a selector of 16 distinct input coordinates
    assert torch.equal(a["p1"].float().sum(dim=1), torch.ones(16))
    assert int((a["p1"].float().sum(dim=0) > 0).sum()) == 16
    K, V = synth.make_kv_cache(cfg, layer=1)
    assert K.shape == (2, 40, 64) and K.dtype == torch.float16
    K2, _ = synth.make_kv_cache(cfg, layer=1)
    assert torch.equal(K, K2) and not torch.equal(K, V)
    # the cache's spread is that of W_k x for x ~ N(0, I): 0.02 sqrt(d)
    assert abs(float(K.float().std()) - 0.02 * np.sqrt(128)) < 0.03
    x = synth.make_attn_tokens(cfg, 3, layer=1)
    assert x.shape == (3, 128) and torch.equal(x, synth.make_attn_tokens(cfg, 3, layer=1))


def test_attention_head_density_calibration():
    """s_h = P2[h] . x_S + c2_h is N(c2_h, |P2[h]|^2) for x ~ N(0, I), so with
    c2_h = |P2[h]| Phi^-1(density) a head is active (s > 0) with probability `density`."""
    for dens in (0.25, 0.5, 0.8):
        cfg = synth.AttnConfig("t", d=256, heads=64, kv_heads=8, head_dim=64, rank=32,
                               density=dens, context=4, seed=7)
        L = synth.make_attn_layer(cfg)
        x = torch.randn(4000, 256, generator=torch.Generator().manual_seed(3))
        z = x @ L["p1"].float().T
        s = z @ L["p2"].float().T + L["c2"]
        assert abs(float((s > 0).float().mean()) - dens) < 0.03, dens
