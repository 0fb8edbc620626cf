"""CPU oracle for the activation-sparse FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product path (the HIP library and its binding) never imports it, and the two
share no code.

The arithmetic lives in ``ffn_oracle.c`` (plain C, double accumulation, one thread); this module
only compiles it with gcc, marshals numpy arrays and composes per-token calls:

* ``predictor``   -- low-rank activation predictor + strict sigmoid threshold
  (PowerInfer, unite.ai, section "Adaptive sparse predictor").
* ``predictor_hot`` -- the same with an always-active hot head of profiled neurons placed first
  (unite.ai, sections "Offline stage" and "Neuron placement and management").
* ``ffn``         -- neuron-aware FFN over a mask (unite.ai, "Neuron-aware operator";
  citnews, "Dynamic neuron cache": inactive neurons do not change the output).
* ``router``/``moe`` -- top-k softmax router and the weighted sum of the chosen experts
  (TurboSparse-Mixtral, nubint.ai review and citnews).
* ``attn_kv``/``attn``/``attn_token`` -- the self-attention block of one token over a key/value
  cache with a head-level active set (unite.ai, "Adaptive sparse predictor": a second predictor
  per layer for the self-attention block; the unit it predicts is read as a head).
* ``NeuronCache`` -- the LRU neuron cache of host-resident FFN rows (citnews, "Dynamic neuron
  cache": an LRU pool of neurons, segmented by weight type).

Every function works on one token; batches are independent tokens, each with its own mask.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ffn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16, I4G32 = 0, 1, 2
RELU, REGLU, DRELU = 0, 1, 2
ACT_NAMES = {"relu": RELU, "reglu": REGLU, "drelu": DRELU}

_lib = None


def build(force: bool = False) -> str:
    """Compile ffn_oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-std=c99", "-Wall", "-Wextra",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, L_, I, D = ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_double
        L.oracle_half_to_double.restype = D
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_elem.restype = D
        L.oracle_elem.argtypes = [I, P, P, L_, L_, L_]
        L.oracle_predictor.restype = L_
        L.oracle_predictor.argtypes = [L_, L_, L_, I, P, P, P, P, I, P, D, P, P, P, P]
        L.oracle_active_list.restype = L_
        L.oracle_active_list.argtypes = [L_, P, P]
        L.oracle_ffn.restype = None
        L.oracle_ffn.argtypes = [L_, L_, I, I, P, P, P, P, P, P, P, P, P, I, P, P, P, P]
        L.oracle_router.restype = None
        L.oracle_router.argtypes = [L_, L_, L_, I, P, I, P, P, P, P]
        L.oracle_attn_kv.restype = None
        L.oracle_attn_kv.argtypes = [L_, L_, L_, I, P, P, I, P, P, P]
        L.oracle_attn.restype = None
        L.oracle_attn.argtypes = [L_, L_, L_, L_, L_, L_, I, P, P, I, P, P, I, P, P, P, P]
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle wants C-contiguous numpy"
    return a.ctypes.data


def _dtype_code(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise TypeError("unsupported dtype %s" % a.dtype)


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(bits)


def decode_matrix(w, scales=None, ncols=None) -> np.ndarray:
    """Decode a stored weight matrix element by element (f32 / f16 / int4-g32) into float64."""
    L = lib()
    if scales is None:
        code = _dtype_code(w)
        rows, cols = w.shape
    else:
        code = I4G32
        rows = w.shape[0]
        cols = ncols if ncols is not None else w.shape[1] * 2
    out = np.empty((rows, cols), np.float64)
    for r in range(rows):
        for c in range(cols):
            out[r, c] = L.oracle_elem(code, _ptr(w), _ptr(scales), r, c, cols)
    return out


def predictor(p1, p2, c1, c2, x, tau: float):
    """One token.  Returns dict(z, s, p, active(uint8), idx(int32 ascending), count)."""
    L = lib()
    rank, d = p1.shape
    ffn = p2.shape[0]
    assert p2.shape == (ffn, rank) and p1.dtype == p2.dtype and x.shape == (d,)
    z = np.empty(rank, np.float64)
    s = np.empty(ffn, np.float64)
    p = np.empty(ffn, np.float64)
    active = np.empty(ffn, np.uint8)
    n = L.oracle_predictor(d, ffn, rank, _dtype_code(p1), _ptr(p1), _ptr(p2), _ptr(c1), _ptr(c2),
                           _dtype_code(x), _ptr(x), float(tau), _ptr(z), _ptr(s), _ptr(p),
                           _ptr(active))
    idx = np.empty(ffn, np.int32)
    m = L.oracle_active_list(ffn, _ptr(active), _ptr(idx))
    assert m == n
    return {"z": z, "s": s, "p": p, "active": active, "idx": idx[:n].copy(), "count": int(n)}


def predictor_hot(p1, p2, c1, c2, x, tau: float, n_hot: int):
    """One token with an always-active hot head (unite.ai PowerInfer, "Offline stage" and "Neuron
    placement and management": profiled hot neurons are told apart from the rest and placed
    first).  Neurons [0, n_hot) are active whatever the predictor says; neurons [n_hot, ffn) are
    decided by ``predictor`` on rows n_hot.. of P2 and c2.  The head's scores are NaN (never
    computed).  Returns the same dict as ``predictor``."""
    ffn_n = p2.shape[0]
    assert 0 <= n_hot <= ffn_n
    active = np.zeros(ffn_n, np.uint8)
    active[:n_hot] = 1
    s = np.full(ffn_n, np.nan)
    p = np.full(ffn_n, np.nan)
    z = None
    if n_hot < ffn_n:
        tail = predictor(p1, np.ascontiguousarray(p2[n_hot:]), c1,
                         None if c2 is None else np.ascontiguousarray(c2[n_hot:]), x, tau)
        active[n_hot:] = tail["active"]
        s[n_hot:] = tail["s"]
        p[n_hot:] = tail["p"]
        z = tail["z"]
    idx = np.flatnonzero(active).astype(np.int32)
    return {"z": z, "s": s, "p": p, "active": active, "idx": idx, "count": int(idx.size)}


def ffn(layer: dict, x, mask=None):
    """One token through the neuron-aware FFN.  ``layer`` holds numpy arrays:
    act ('relu'|'reglu'|'drelu'), w_up, w_gate, w_down_t ([ffn][d] f32/f16, or uint8 [ffn][d/2]
    for int4 with s_up/s_gate/s_down_t fp16 [ffn][d/32]), b_up, b_gate, b_down (f32 or None).
    ``mask`` is a uint8 [ffn] array (None = all neurons).  Returns (y float64[d], h float64[ffn]).
    """
    L = lib()
    act = ACT_NAMES[layer["act"]] if isinstance(layer["act"], str) else int(layer["act"])
    w_up = layer["w_up"]
    ffn_n = w_up.shape[0]
    if layer.get("s_up") is not None:
        code = I4G32
        d = w_up.shape[1] * 2
    else:
        code = _dtype_code(w_up)
        d = w_up.shape[1]
    assert x.shape == (d,)
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.uint8)
        assert mask.shape == (ffn_n,)
    h = np.empty(ffn_n, np.float64)
    y = np.empty(d, np.float64)
    gate = layer.get("w_gate") if act != RELU else None
    L.oracle_ffn(d, ffn_n, act, code, _ptr(w_up), _ptr(gate), _ptr(layer["w_down_t"]),
                 _ptr(layer.get("s_up")), _ptr(layer.get("s_gate") if act != RELU else None),
                 _ptr(layer.get("s_down_t")), _ptr(layer.get("b_up")),
                 _ptr(layer.get("b_gate") if act != RELU else None), _ptr(layer.get("b_down")),
                 _dtype_code(x), _ptr(x), _ptr(mask), _ptr(h), _ptr(y))
    return y, h


def router(R, x, k: int = 2):
    """Top-k router for one token.  Returns (ids int32[k], w float64[k], logits float64[E])."""
    L = lib()
    n_exp, d = R.shape
    logits = np.empty(n_exp, np.float64)
    ids = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    L.oracle_router(d, n_exp, k, _dtype_code(R), _ptr(R), _dtype_code(x), _ptr(x),
                    _ptr(logits), _ptr(ids), _ptr(w))
    return ids, w, logits


def sparse_token(layer: dict, x, mask=None, n_hot: int = 0):
    """Predictor (unless a mask is given) followed by the FFN over the active set, one token.
    ``layer`` additionally holds p1, p2, c1, c2 and tau; n_hot > 0 takes ``predictor_hot``.
    Returns (y float64[d], pred dict|None)."""
    pred = None
    if mask is None:
        if n_hot:
            pred = predictor_hot(layer["p1"], layer["p2"], layer.get("c1"), layer.get("c2"), x,
                                 layer["tau"], n_hot)
        else:
            pred = predictor(layer["p1"], layer["p2"], layer.get("c1"), layer.get("c2"), x,
                             layer["tau"])
        mask = pred["active"]
    y, _ = ffn(layer, x, mask)
    return y, pred


def moe_token(experts, R, x, k: int = 2, masks=None):
    """Mixture of experts, one token: y = sum_t w_t * FFN_{e_t}(x), each chosen expert with its own
    predictor (or the caller's mask for that expert).  Returns (y, ids, w, preds)."""
    ids, w, _ = router(R, x, k)
    y = np.zeros(x.shape[0], np.float64)
    preds = []
    for t in range(k):
        e = int(ids[t])
        ye, pred = sparse_token(experts[e], x, None if masks is None else masks[t])
        preds.append(pred)
        y += w[t] * ye
    return y, ids, w, preds


def attn_kv(w_k, w_v, x, e: int):
    """Key and value of one token for every key/value head: (k, v) float64 [G*e] each."""
    L = lib()
    rows, d = w_k.shape
    assert w_v.shape == (rows, d) and w_v.dtype == w_k.dtype and x.shape == (d,) and rows % e == 0
    k = np.empty(rows, np.float64)
    v = np.empty(rows, np.float64)
    L.oracle_attn_kv(d, rows // e, e, _dtype_code(w_k), _ptr(w_k), _ptr(w_v), _dtype_code(x),
                     _ptr(x), _ptr(k), _ptr(v))
    return k, v


def attn(w_q, w_o_t, Kc, Vc, x, t: int, mask=None):
    """Output of the attention block for the token at position t over the cache Kc, Vc
    ([G][S][e], positions 0..t filled, t being the token's own).  mask uint8 [H] or None (every
    head).  Returns (y float64[d], o float64[H][e])."""
    L = lib()
    G, S, e = Kc.shape
    He, d = w_q.shape
    H = He // e
    assert He == H * e and w_o_t.shape == (He, d) and Vc.shape == Kc.shape and Vc.dtype == Kc.dtype
    assert H % G == 0 and 0 <= t < S and x.shape == (d,) and e <= 512
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.uint8)
        assert mask.shape == (H,)
    o = np.empty(He, np.float64)
    y = np.empty(d, np.float64)
    L.oracle_attn(d, H, G, e, S, t, _dtype_code(w_q), _ptr(w_q), _ptr(w_o_t), _dtype_code(Kc),
                  _ptr(Kc), _ptr(Vc), _dtype_code(x), _ptr(x), _ptr(mask), _ptr(o), _ptr(y))
    return y, o.reshape(H, e)


def attn_token(layer: dict, Kc, Vc, x, t: int, mask=None):
    """One token through the attention block at position t: the head predictor (unless a mask is
    given), this token's key and value for every key/value head, stored at position t of copies
    of the caches in the caches' dtype (numpy's round-to-nearest-even conversion), then ``attn``
    over the active heads.  ``layer`` holds numpy w_q, w_k, w_v, w_o_t, p1, p2, c1, c2, tau and
    head_dim.  Returns (y, pred dict|None, Kc', Vc')."""
    e = int(layer["head_dim"])
    pred = None
    if mask is None:
        pred = predictor(layer["p1"], layer["p2"], layer.get("c1"), layer.get("c2"), x,
                         layer["tau"])
        mask = pred["active"]
    k, v = attn_kv(layer["w_k"], layer["w_v"], x, e)
    G = Kc.shape[0]
    Kn, Vn = Kc.copy(), Vc.copy()
    Kn[:, t, :] = k.reshape(G, e).astype(Kc.dtype)
    Vn[:, t, :] = v.reshape(G, e).astype(Vc.dtype)
    y, _ = attn(layer["w_q"], layer["w_o_t"], Kn, Vn, x, t, mask)
    return y, pred, Kn, Vn


PINNED = 0xFFFFFFFF


class NeuronCache:
    """LRU cache of FFN neurons in device memory, one token at a time (citnews.com.cn PowerInfer-2
    article, section "Dynamic neuron cache": an in-memory pool of neurons managed by LRU, the
    cache segmented by weight type -- here the predictor segment is always resident and only the
    FFN rows of neurons are cached).

    ``capacity`` slots; slots [0, n_pinned) hold neurons [0, n_pinned) for good (the hot head).
    ``step(active)`` takes one token's active neurons in ascending order and returns, per rank,
    the slot the neuron is read from (-1: read from host memory) and the slot it is admitted to
    (-1: none):
      * the token's stamp is the previous one plus 1 (the first token has stamp 1);
      * a resident neuron is a hit; its slot's last use becomes the stamp (pinned slots keep
        theirs);
      * the misses, in rank order, take the free or least recently used slots -- the slots not
        used by this token and not pinned, in ascending (last use, slot) order (free slots have
        last use 0); a miss beyond those slots is read from host memory and not admitted;
      * an admitted neuron evicts the slot's previous neuron, and the slot's last use becomes the
        stamp.
    """

    def __init__(self, ffn: int, capacity: int, n_pinned: int = 0):
        assert 0 <= n_pinned <= capacity and n_pinned <= ffn
        self.slot_of = np.full(ffn, -1, np.int64)
        self.neuron_of = np.full(capacity, -1, np.int64)
        self.last_use = np.zeros(capacity, np.int64)
        self.slot_of[:n_pinned] = np.arange(n_pinned)
        self.neuron_of[:n_pinned] = np.arange(n_pinned)
        self.last_use[:n_pinned] = PINNED
        self.stamp = 0

    def step(self, active):
        self.stamp += 1
        active = [int(n) for n in active]
        src = [int(self.slot_of[n]) for n in active]
        for s in src:
            if s >= 0 and self.last_use[s] != PINNED:
                self.last_use[s] = self.stamp
        free = sorted((int(self.last_use[s]), s) for s in range(len(self.last_use))
                      if self.last_use[s] < self.stamp)
        victim = [-1] * len(active)
        k = 0
        for j, n in enumerate(active):
            if src[j] >= 0 or k >= len(free):
                continue
            v = free[k][1]
            k += 1
            old = int(self.neuron_of[v])
            if old >= 0:
                self.slot_of[old] = -1
            self.neuron_of[v] = n
            self.slot_of[n] = v
            self.last_use[v] = self.stamp
            victim[j] = v
        return src, victim
