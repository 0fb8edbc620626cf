"""Seeded synthetic inputs for the activation-sparse FFN (shared by the oracle side and the GPU side).

This module only *makes input bytes*: weights, biases, predictor weights, router weights and
tokens.  It holds none of the operator's arithmetic (no prediction, no activation, no
projection); both the oracle and the HIP library consume the tensors it returns.

Recipe (the pages measure real ReLU-family models on chat prompts; neither is available, so these
synthetic layers stand in for them with the same shapes and a power-law activation structure --
PowerInfer, unite.ai, introduction and "Architecture and methodology": a few hot neurons fire for
almost every input, most cold neurons only for some inputs; nearauto.com Fig. 8: the hot neurons
are scattered through the matrix):

* weights ~ N(0, 0.02^2) (optionally, for the predictor's source matrix, shaped to a power-law
  singular spectrum with the same row norms: ``spectrum_alpha``), rounded once to the storage dtype (fp32, fp16 round-to-nearest-even,
  or int4 with one fp16 scale per 32 consecutive elements of a row:
  s = fp16(max|w| / 7), q = clamp(rint(w / s), -8, 7), q = 0 where s = 0; for int4 the bias
  calibration and the predictor use the weights before quantisation);
* per neuron i a firing probability p_i = min(0.99, c * k_i^-1.1) where k_i is the neuron's rank
  in a seeded random permutation and c is found by bisection so that mean(p) = density;
* biases turn p_i into the actual firing rate for tokens x ~ N(0, I): a pre-activation
  w.x + b is N(b, |w|^2), so b = |w| * Phi^-1(p) makes P(w.x + b > 0) = p
  (ReLU: up bias; ReGLU: gate bias; dReLU: gate and up biases each at Phi^-1(sqrt p));
* predictor of rank r: a seeded r-subset S of the input coordinates, P1[k, S_k] = 1 (a selector),
  P2[i, k] = W_src[i, S_k] (W_src = up for ReLU, gate otherwise), c2_i = |P2[i]| * Phi^-1(p_i),
  c1 absent, threshold tau = 0.5 -- the predicted set has density ~ p_i and tracks the true set;
* router of a mixture of experts: R[e] ~ N(0, 0.02^2), fp16;
* tokens x ~ N(0, 1) drawn independently per (token, layer), stored in the activation dtype;
* attention block (``AttnConfig``): W_q, W_k, W_v, W_o_t ~ N(0, 0.02^2) in fp16; a head
  predictor of the same selector form (P1 picks r input coordinates, P2 [heads][r] ~ N(0, 1),
  c2_h = |P2[h]| * Phi^-1(density), so each head is predicted active with probability
  ``density`` for x ~ N(0, I)); the key/value cache of the context ~ N(0, (0.02 sqrt d)^2) in
  fp16, the spread of W_k x for such tokens.

All random draws use torch generators seeded from (base seed, layer, expert, tensor id), on the
device the tensors are made on.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import scipy.special
import torch

F32, F16, I4G32 = "f32", "f16", "i4g32"


@dataclass(frozen=True)
class LayerConfig:
    name: str
    d: int
    ffn: int
    act: str                 # 'relu' | 'reglu' | 'drelu'
    w_dtype: str             # 'f32' | 'f16' | 'i4g32'
    x_dtype: str             # 'f32' | 'f16'
    p_dtype: str             # 'f32' | 'f16'
    rank: int
    density: float
    layers: int = 1
    tokens: int = 1
    n_experts: int = 1
    top_k: int = 1
    bias_up: bool = False
    bias_gate: bool = False
    bias_down: bool = False
    tau: float = 0.5
    zipf_s: float = 1.1
    cap: float = 0.99
    spectrum_alpha: float = 0.0  # > 0: the predictor's source matrix gets singular values ~ k^-alpha
    batches: tuple = (1,)
    seed: int = 1000
    expert_density: tuple = field(default=())


# The five workloads (shapes from the models the pages run; densities from the pages' sparsity
# statements and the per-token activation share they report).
CONFIGS = {
    "opt125m_relu_f32": LayerConfig(
        "opt125m_relu_f32", d=768, ffn=3072, act="relu", w_dtype=F32, x_dtype=F32, p_dtype=F32,
        rank=64, density=0.10, layers=1, tokens=256, bias_up=True, seed=1001),
    "llama2_7b_reglu_f16": LayerConfig(
        "llama2_7b_reglu_f16", d=4096, ffn=11008, act="reglu", w_dtype=F16, x_dtype=F16,
        p_dtype=F16, rank=256, density=0.10, layers=32, tokens=512, bias_gate=True, seed=1002),
    "turbosparse_mistral_7b_drelu_f16": LayerConfig(
        "turbosparse_mistral_7b_drelu_f16", d=4096, ffn=14336, act="drelu", w_dtype=F16,
        x_dtype=F16, p_dtype=F16, rank=512, density=0.10, layers=32, tokens=1024,
        bias_gate=True, bias_up=True, seed=1003),
    "turbosparse_mixtral_47b_moe_int4": LayerConfig(
        "turbosparse_mixtral_47b_moe_int4", d=4096, ffn=14336, act="drelu", w_dtype=I4G32,
        x_dtype=F16, p_dtype=F16, rank=256, density=0.075, layers=32, tokens=512, n_experts=8,
        top_k=2, bias_gate=True, bias_up=True, seed=1004,
        expert_density=tuple(0.05 + 0.05 * e / 7 for e in range(8))),
    "falcon_40b_relu_f16": LayerConfig(
        "falcon_40b_relu_f16", d=8192, ffn=32768, act="relu", w_dtype=F16, x_dtype=F16,
        p_dtype=F16, rank=1024, density=0.15, layers=60, tokens=256, bias_up=True,
        batches=(1, 8, 32), seed=1005),
}
CONFIG_ORDER = list(CONFIGS)


@dataclass(frozen=True)
class AttnConfig:
    """A self-attention block: H query heads, G key/value heads of width e, a head predictor of
    rank r, and a token at position ``context`` (positions 0..context-1 already in the cache)."""
    name: str
    d: int
    heads: int
    kv_heads: int
    head_dim: int
    rank: int
    density: float            # probability that a head is predicted active
    context: int
    max_seq: int = 0          # cache positions per head (0: context + 1)
    p_dtype: str = F16
    layers: int = 1
    tau: float = 0.5
    seed: int = 2000

    @property
    def seq(self) -> int:
        return self.max_seq if self.max_seq else self.context + 1


# Attention blocks of the pages' models (Llama-2-7B: 32 heads of 128; Mistral-7B: 32 query heads
# sharing 8 key/value heads; Falcon-40B: 128 query heads of 64 sharing 8 key/value heads), at a
# 512-token context.  The pages print no head-level activity figure; half the heads active is
# the stand-in.
ATTN_CONFIGS = {
    "llama2_7b_attn_f16": AttnConfig("llama2_7b_attn_f16", d=4096, heads=32, kv_heads=32,
                                     head_dim=128, rank=128, density=0.5, context=511,
                                     layers=32, seed=2001),
    "mistral_7b_attn_f16": AttnConfig("mistral_7b_attn_f16", d=4096, heads=32, kv_heads=8,
                                      head_dim=128, rank=128, density=0.5, context=511,
                                      layers=32, seed=2002),
    "falcon_40b_attn_f16": AttnConfig("falcon_40b_attn_f16", d=8192, heads=128, kv_heads=8,
                                      head_dim=64, rank=128, density=0.5, context=511,
                                      layers=60, seed=2003),
}


def make_attn_layer(cfg: AttnConfig, layer: int = 0, device="cpu") -> dict:
    """All tensors of one attention block of ``cfg`` (weights, head predictor) on ``device``."""
    d, H, G, e, r = cfg.d, cfg.heads, cfg.kv_heads, cfg.head_dim, cfg.rank

    def w(rows, tid):
        t = torch.randn(rows, d, generator=_gen(device, _seed(cfg, layer, 0, tid)),
                        device=device, dtype=torch.float32) * 0.02
        return t.to(torch.float16).contiguous()

    out = {"cfg": cfg, "tau": cfg.tau, "head_dim": e, "layer": layer,
           "w_q": w(H * e, 11), "w_k": w(G * e, 12), "w_v": w(G * e, 13), "w_o_t": w(H * e, 14)}
    sel = np.random.Generator(np.random.PCG64(_seed(cfg, layer, 0, 15))).choice(
        d, size=r, replace=False)
    pt = _tdtype(cfg.p_dtype)
    p1 = torch.zeros(r, d, dtype=pt, device=device)
    p1[torch.arange(r, device=device), torch.from_numpy(sel.astype(np.int64)).to(device)] = 1
    p2 = torch.randn(H, r, generator=_gen(device, _seed(cfg, layer, 0, 16)), device=device,
                     dtype=torch.float32).to(pt).contiguous()
    c2 = (p2.double().norm(dim=1) * float(_ndtri(np.array([cfg.density]))[0])).float()
    out.update(p1=p1.contiguous(), p2=p2, c1=None, c2=c2.contiguous(), selector=sel)
    return out


def make_kv_cache(cfg: AttnConfig, layer: int = 0, device="cpu"):
    """Key and value caches [G][seq][e] fp16 of one block; every position holds a seeded value
    (positions from ``context`` on are overwritten by the tokens that run)."""
    shape = (cfg.kv_heads, cfg.seq, cfg.head_dim)
    sd = 0.02 * np.sqrt(cfg.d)
    K = torch.randn(*shape, generator=_gen(device, _seed(cfg, layer, 0, 17)), device=device) * sd
    V = torch.randn(*shape, generator=_gen(device, _seed(cfg, layer, 0, 18)), device=device) * sd
    return K.to(torch.float16).contiguous(), V.to(torch.float16).contiguous()


def make_attn_tokens(cfg: AttnConfig, n: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """n tokens x ~ N(0, 1) [n][d] fp16 for one attention block."""
    g = _gen(device, _seed(cfg, layer, 0, 1019))
    return torch.randn(n, cfg.d, generator=g, device=device).to(torch.float16).contiguous()


def small_config(**kw) -> LayerConfig:
    base = dict(name="small", d=64, ffn=256, act="relu", w_dtype=F32, x_dtype=F32, p_dtype=F32,
                rank=16, density=0.2, bias_up=True)
    base.update(kw)
    return LayerConfig(**base)


def _seed(cfg: LayerConfig, layer: int, expert: int, tensor: int) -> int:
    return (cfg.seed * 1_000_003 + layer * 10_007 + expert * 101 + tensor) & 0x7FFFFFFFFFFF


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _ndtri(p: np.ndarray) -> np.ndarray:
    """Inverse standard normal CDF (float64, host)."""
    return scipy.special.ndtri(np.asarray(p, np.float64))


def zipf_probs(ffn: int, density: float, s: float, cap: float, seed: int) -> np.ndarray:
    """p_i = min(cap, c * rank_i^-s) with a seeded random permutation for the ranks and c chosen
    by bisection so that mean(p) = density."""
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(ffn)
    k = (perm + 1).astype(np.float64)
    base = k ** (-s)
    lo, hi = 0.0, 1.0
    while np.minimum(cap, hi * base).mean() < density:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(cap, mid * base).mean() < density:
            lo = mid
        else:
            hi = mid
    return np.minimum(cap, 0.5 * (lo + hi) * base)


def _tdtype(name: str):
    return {F32: torch.float32, F16: torch.float16}[name]


def quantize_i4g32(w: torch.Tensor):
    """fp32 [rows][d] -> (packed uint8 [rows][d/2], fp16 scales [rows][d/32]).  Element 2k sits in
    the low nibble of byte k; q is signed two's complement in [-8, 7]."""
    rows, d = w.shape
    assert d % 32 == 0
    g = w.reshape(rows, d // 32, 32)
    s16 = (g.abs().amax(dim=2) / 7.0).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(2)
    q = torch.where(s > 0, torch.round(g / torch.where(s > 0, s, torch.ones_like(s))),
                    torch.zeros_like(g))
    q = q.clamp(-8, 7).to(torch.int16).reshape(rows, d)
    nib = (q & 0xF).to(torch.uint8)
    packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return packed.contiguous(), s16.contiguous()


def _weight(cfg, rows, cols, device, seed, shaped=False):
    w = torch.randn(rows, cols, generator=_gen(device, seed), device=device,
                    dtype=torch.float32) * 0.02
    if shaped and cfg.spectrum_alpha > 0:
        # a trained-looking spectrum: w = A diag(sv) Q^T with a seeded orthonormal Q and
        # sv_k ~ (k+1)^-alpha, scaled so that rows keep E|w_row|^2 = 0.02^2 cols
        q, _ = torch.linalg.qr(torch.randn(cols, cols, generator=_gen(device, seed + 17),
                                           device=device, dtype=torch.float64))
        sv = torch.arange(1, cols + 1, device=device, dtype=torch.float64) ** (-cfg.spectrum_alpha)
        sv = sv * (0.02 * np.sqrt(cols) / sv.square().sum().sqrt())
        w = ((w.double() / 0.02) @ (sv[:, None] * q.T)).float()
    if cfg.w_dtype == I4G32:
        packed, scales = quantize_i4g32(w)
        return packed, scales, w          # norms taken before quantisation
    t = w.to(_tdtype(cfg.w_dtype)).contiguous()
    return t, None, t.to(torch.float32)


def make_layer(cfg: LayerConfig, layer: int = 0, expert: int = 0, device="cpu") -> dict:
    """All tensors of one FFN layer (one expert) of ``cfg`` on ``device``."""
    d, F, r = cfg.d, cfg.ffn, cfg.rank
    density = cfg.expert_density[expert] if cfg.expert_density else cfg.density
    probs = zipf_probs(F, density, cfg.zipf_s, cfg.cap, _seed(cfg, layer, expert, 0))
    out = {"cfg": cfg, "act": cfg.act, "probs": probs, "tau": cfg.tau, "layer": layer,
           "expert": expert}
    w_up, s_up, f_up = _weight(cfg, F, d, device, _seed(cfg, layer, expert, 1),
                               shaped=cfg.act == "relu")
    out["w_up"], out["s_up"] = w_up, s_up
    f_gate = None
    if cfg.act != "relu":
        w_gate, s_gate, f_gate = _weight(cfg, F, d, device, _seed(cfg, layer, expert, 2),
                                         shaped=True)
        out["w_gate"], out["s_gate"] = w_gate, s_gate
    else:
        out["w_gate"], out["s_gate"] = None, None
    w_dn, s_dn, _ = _weight(cfg, F, d, device, _seed(cfg, layer, expert, 3))
    out["w_down_t"], out["s_down_t"] = w_dn, s_dn

    # bias calibration: P(w.x + b > 0) = target for x ~ N(0, I)
    if cfg.act == "drelu":
        t = _ndtri(np.sqrt(probs))
    else:
        t = _ndtri(probs)
    tt = torch.from_numpy(t).to(device=device, dtype=torch.float64)
    out["b_up"] = out["b_gate"] = out["b_down"] = None
    if cfg.act == "relu" and cfg.bias_up:
        out["b_up"] = (f_up.float().norm(dim=1).double() * tt).float().contiguous()
    if cfg.act in ("reglu", "drelu") and cfg.bias_gate:
        out["b_gate"] = (f_gate.float().norm(dim=1).double() * tt).float().contiguous()
    if cfg.act == "drelu" and cfg.bias_up:
        out["b_up"] = (f_up.float().norm(dim=1).double() * tt).float().contiguous()
    if cfg.bias_down:
        out["b_down"] = (torch.randn(d, generator=_gen(device, _seed(cfg, layer, expert, 4)),
                                     device=device) * 0.02).float().contiguous()

    # predictor: selector P1, P2 = columns S of the source matrix, calibrated c2
    if r > 0:
        sel = np.random.Generator(np.random.PCG64(_seed(cfg, layer, expert, 5))).choice(
            d, size=r, replace=False)
        sel_t = torch.from_numpy(sel.astype(np.int64)).to(device)
        pt = _tdtype(cfg.p_dtype)
        p1 = torch.zeros(r, d, dtype=pt, device=device)
        p1[torch.arange(r, device=device), sel_t] = 1
        src = f_up if cfg.act == "relu" else f_gate
        p2 = src[:, sel_t].to(pt).contiguous()
        tp = torch.from_numpy(_ndtri(probs)).to(device=device, dtype=torch.float64)
        c2 = (p2.double().norm(dim=1) * tp).float().contiguous()
        out.update(p1=p1.contiguous(), p2=p2, c1=None, c2=c2, selector=sel)
    else:
        out.update(p1=None, p2=None, c1=None, c2=None, selector=None)
    return out


# Per-neuron arrays of a layer dict (rows for matrices, entries for vectors).
NEURON_KEYS = ("w_up", "s_up", "w_gate", "s_gate", "w_down_t", "s_down_t", "b_up", "b_gate",
               "p2", "c2", "probs")


def hot_first(layer: dict) -> dict:
    """The same layer with its neurons ordered by firing probability, hottest first (stable
    order among equals): the offline profile and placement step, with the generator's own
    probabilities standing in for a profiler.  Every per-neuron array is permuted alike, so the
    dense FFN and each neuron's predictor score are unchanged; ``order[j]`` is the original
    index of neuron j."""
    order = np.argsort(-np.asarray(layer["probs"]), kind="stable")
    out = dict(layer)
    for k in NEURON_KEYS:
        v = layer.get(k)
        if v is None:
            continue
        if isinstance(v, torch.Tensor):
            out[k] = v[torch.from_numpy(order).to(v.device)].contiguous()
        else:
            out[k] = np.ascontiguousarray(np.asarray(v)[order])
    out["order"] = order
    return out


def hot_head_size(layer: dict) -> int:
    """Neurons whose firing probability sits at the generator's cap (the always-firing head),
    rounded down to a multiple of 32."""
    cap = layer["cfg"].cap
    n = int(np.count_nonzero(np.asarray(layer["probs"]) >= cap * (1.0 - 1e-12)))
    return n - n % 32


def make_tokens(cfg: LayerConfig, n: int, layer: int = 0, device="cpu", offset: int = 0,
                salt: int = 0) -> torch.Tensor:
    """n tokens x ~ N(0, 1) [n][d] in the activation dtype, for one layer."""
    g = _gen(device, _seed(cfg, layer, 0, 1000 + salt) + 7919 * offset)
    x = torch.randn(n, cfg.d, generator=g, device=device, dtype=torch.float32)
    return x.to(_tdtype(cfg.x_dtype)).contiguous()


def make_router(cfg: LayerConfig, layer: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(device, _seed(cfg, layer, 0, 900))
    R = torch.randn(cfg.n_experts, cfg.d, generator=g, device=device) * 0.02
    return R.to(torch.float16).contiguous()


def to_numpy_layer(layer: dict) -> dict:
    """Host numpy copy of a layer dict (for the oracle)."""
    out = {}
    for k, v in layer.items():
        if isinstance(v, torch.Tensor):
            out[k] = v.detach().cpu().numpy().copy()
        else:
            out[k] = v
    return out


def with_(cfg: LayerConfig, **kw) -> LayerConfig:
    return replace(cfg, **kw)
