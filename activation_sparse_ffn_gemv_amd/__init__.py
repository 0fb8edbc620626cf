"""Python binding of libffn_sparse (the MI355X activation-sparse FFN), argument marshalling only.

The functions below carry the names of the C ABI in ``include/ffn_sparse.h`` and pass plain
pointers through ctypes; every step of the operator runs in the library's HIP kernels.  PyTorch
is used for device memory and streams only.  There is no fallback: if the library is not built,
importing this package raises.

``SparseFFN`` is a thin convenience holder: it keeps the weight tensors and the workspace alive
and fills the descriptor structs from torch tensors.
"""
from __future__ import annotations

import ctypes
import os

import torch  # load torch's HIP runtime first so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libffn_sparse.so")

FFN_OK, FFN_ERR_INVALID_ARGUMENT, FFN_ERR_UNSUPPORTED = 0, 1, 2
FFN_ERR_WORKSPACE_TOO_SMALL, FFN_ERR_HIP, FFN_ERR_INTERNAL = 3, 4, 5
FFN_ACT_RELU, FFN_ACT_REGLU, FFN_ACT_DRELU = 0, 1, 2
FFN_F32, FFN_F16, FFN_I4G32 = 0, 1, 2
FFN_PATH_AUTO, FFN_PATH_SPARSE, FFN_PATH_DENSE = 0, 1, 2
FFN_STAGE_PRED_Z, FFN_STAGE_PRED_S, FFN_STAGE_GATHER, FFN_STAGE_REDUCE = 0, 1, 2, 3
FFN_STAGE_BATCH_UPGATE, FFN_STAGE_BATCH_DOWN = 4, 5
FFN_STAGE_DENSE_UP, FFN_STAGE_DENSE_DOWN, FFN_STAGE_DENSE_REDUCE = 6, 7, 8
FFN_STAGE_ATTN_PROJ, FFN_STAGE_ATTN_SCORES = 9, 10
FFN_STAGE_ATTN_OUT, FFN_STAGE_ATTN_REDUCE = 11, 12
STAGES = ("pred_z", "pred_s", "gather", "reduce")          # the batch-1 decode kernels
BATCH_STAGES = ("batch_upgate", "batch_down")
DENSE_STAGES = ("dense_up", "dense_down", "dense_reduce")
ATTN_STAGES = ("pred_z", "attn_proj", "attn_scores", "attn_out", "attn_reduce")

ACT = {"relu": FFN_ACT_RELU, "reglu": FFN_ACT_REGLU, "drelu": FFN_ACT_DRELU}
DTYPE = {"f32": FFN_F32, "f16": FFN_F16, "i4g32": FFN_I4G32}

# Every symbol the header declares (checked by the tests).
EXPORTS = [
    "ffn_workspace_size", "ffn_sparse_plan", "ffn_sparse_forward", "ffn_sparse_forward_static",
    "ffn_dense_forward",
    "ffn_plan_crossover", "ffn_plan_set_crossover", "ffn_plan_path_flag",
    "ffn_plan_set_decode_variant",
    "ffn_plan_set_hot_head", "ffn_offload_workspace_size", "ffn_offload_plan",
    "ffn_offload_tables", "ffn_plan_destroy", "ffn_plan_set_timing_events", "ffn_status_string",
    "ffn_last_error",
    "ffn_moe_workspace_size",
    "ffn_moe_plan", "ffn_moe_forward", "ffn_moe_destroy",
    "ffn_attn_workspace_size", "ffn_attn_plan", "ffn_attn_forward", "ffn_attn_set_timing_events",
    "ffn_attn_destroy",
]


class FFNError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("ffn status %d: %s" % (status, msg))
        self.status = status


class ffn_layer_desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("ffn", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("act", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("x_dtype", ctypes.c_int32), ("p_dtype", ctypes.c_int32),
                ("threshold", ctypes.c_float), ("max_batch", ctypes.c_int32)]


class ffn_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ["w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down_t", "b_up", "b_gate",
                 "b_down", "p1", "p2", "c1", "c2"]]


class ffn_attn_desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("threshold", ctypes.c_float)]


class ffn_attn_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ["w_q", "w_k", "w_v", "w_o_t", "p1", "p2", "c1", "c2"]]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libffn_sparse.so is not built; run "
                              "`python activation_sparse_ffn_gemv_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        st = ctypes.c_int
        L.ffn_last_error.restype = ctypes.c_char_p
        L.ffn_last_error.argtypes = []
        L.ffn_status_string.restype = ctypes.c_char_p
        L.ffn_status_string.argtypes = [ctypes.c_int]
        L.ffn_workspace_size.restype = st
        L.ffn_workspace_size.argtypes = [ctypes.POINTER(ffn_layer_desc), ctypes.POINTER(S)]
        L.ffn_sparse_plan.restype = st
        L.ffn_sparse_plan.argtypes = [ctypes.POINTER(ffn_layer_desc),
                                      ctypes.POINTER(ffn_layer_weights), P, S, P, I,
                                      ctypes.POINTER(P)]
        L.ffn_sparse_forward.restype = st
        L.ffn_sparse_forward.argtypes = [P, P, I, P, P, P, P, P, I, P]
        L.ffn_sparse_forward_static.restype = st
        L.ffn_sparse_forward_static.argtypes = [ctypes.POINTER(ffn_layer_desc),
                                                ctypes.POINTER(ffn_layer_weights), P, I, P, P,
                                                P, P, P]
        L.ffn_dense_forward.restype = st
        L.ffn_dense_forward.argtypes = [P, P, I, P, P, P]
        L.ffn_plan_crossover.restype = st
        L.ffn_plan_crossover.argtypes = [P, I, ctypes.POINTER(ctypes.c_float)]
        L.ffn_plan_set_crossover.restype = st
        L.ffn_plan_set_crossover.argtypes = [P, I, ctypes.c_float]
        L.ffn_plan_path_flag.restype = st
        L.ffn_plan_path_flag.argtypes = [P, ctypes.POINTER(P)]
        L.ffn_plan_set_decode_variant.restype = st
        L.ffn_plan_set_decode_variant.argtypes = [P, I]
        L.ffn_plan_set_hot_head.restype = st
        L.ffn_plan_set_hot_head.argtypes = [P, I]
        L.ffn_offload_workspace_size.restype = st
        L.ffn_offload_workspace_size.argtypes = [ctypes.POINTER(ffn_layer_desc), I,
                                                 ctypes.POINTER(S)]
        L.ffn_offload_plan.restype = st
        L.ffn_offload_plan.argtypes = [ctypes.POINTER(ffn_layer_desc),
                                       ctypes.POINTER(ffn_layer_weights), I, I, P, S, P,
                                       ctypes.POINTER(P)]
        L.ffn_offload_tables.restype = st
        L.ffn_offload_tables.argtypes = [P] + [ctypes.POINTER(P)] * 4
        L.ffn_plan_destroy.restype = st
        L.ffn_plan_destroy.argtypes = [P]
        L.ffn_plan_set_timing_events.restype = st
        L.ffn_plan_set_timing_events.argtypes = [P, I, P, P]
        L.ffn_moe_workspace_size.restype = st
        L.ffn_moe_workspace_size.argtypes = [I, I, P, ctypes.POINTER(S)]
        L.ffn_moe_plan.restype = st
        L.ffn_moe_plan.argtypes = [I, I, P, ctypes.POINTER(P), P, S, ctypes.POINTER(P)]
        L.ffn_moe_forward.restype = st
        L.ffn_moe_forward.argtypes = [P, P, I, P, P, P, P, P]
        L.ffn_moe_destroy.restype = st
        L.ffn_moe_destroy.argtypes = [P]
        L.ffn_attn_workspace_size.restype = st
        L.ffn_attn_workspace_size.argtypes = [ctypes.POINTER(ffn_attn_desc), ctypes.POINTER(S)]
        L.ffn_attn_plan.restype = st
        L.ffn_attn_plan.argtypes = [ctypes.POINTER(ffn_attn_desc),
                                    ctypes.POINTER(ffn_attn_weights), P, S, ctypes.POINTER(P)]
        L.ffn_attn_forward.restype = st
        L.ffn_attn_forward.argtypes = [P, P, I, P, P, P, P, P, P, P, P]
        L.ffn_attn_set_timing_events.restype = st
        L.ffn_attn_set_timing_events.argtypes = [P, I, P, P]
        L.ffn_attn_destroy.restype = st
        L.ffn_attn_destroy.argtypes = [P]
        _lib = L
    return _lib


def _check(status: int):
    if status != FFN_OK:
        raise FFNError(status, "%s: %s" % (ffn_status_string(status), ffn_last_error()))


def ffn_status_string(status: int) -> str:
    return lib().ffn_status_string(status).decode()


def ffn_last_error() -> str:
    return lib().ffn_last_error().decode()


def ffn_workspace_size(desc: ffn_layer_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ffn_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ffn_sparse_plan(desc, weights, workspace: int, workspace_bytes: int, stream: int = 0,
                    calibrate: int = 0) -> int:
    out = ctypes.c_void_p(0)
    _check(lib().ffn_sparse_plan(ctypes.byref(desc), ctypes.byref(weights), workspace,
                                 workspace_bytes, stream or None, calibrate, ctypes.byref(out)))
    return out.value


def ffn_sparse_forward(plan: int, x: int, B: int, y: int, mask: int = 0, idx: int = 0,
                       cnt: int = 0, scores: int = 0, path: int = FFN_PATH_SPARSE,
                       stream: int = 0):
    _check(lib().ffn_sparse_forward(plan, x, B, y, mask or None, idx or None, cnt or None,
                                    scores or None, path, stream or None))


def ffn_sparse_forward_static(desc, weights, x: int, B: int, y: int, mask: int = 0,
                              idx: int = 0, cnt: int = 0, stream: int = 0):
    _check(lib().ffn_sparse_forward_static(ctypes.byref(desc), ctypes.byref(weights), x, B, y,
                                           mask or None, idx or None, cnt or None,
                                           stream or None))


def ffn_dense_forward(plan: int, x: int, B: int, y: int, mask: int = 0, stream: int = 0):
    _check(lib().ffn_dense_forward(plan, x, B, y, mask or None, stream or None))


def ffn_plan_crossover(plan: int, B: int) -> float:
    v = ctypes.c_float(0)
    _check(lib().ffn_plan_crossover(plan, B, ctypes.byref(v)))
    return v.value


def ffn_plan_set_crossover(plan: int, B: int, density: float):
    _check(lib().ffn_plan_set_crossover(plan, B, density))


def ffn_plan_path_flag(plan: int) -> int:
    """Device address of the int32 recording the path of the last AUTO call of >= 64 tokens."""
    v = ctypes.c_void_p(0)
    _check(lib().ffn_plan_path_flag(plan, ctypes.byref(v)))
    return v.value


def ffn_plan_set_decode_variant(plan: int, variant: int):
    _check(lib().ffn_plan_set_decode_variant(plan, variant))


def ffn_plan_set_hot_head(plan: int, n_hot: int):
    _check(lib().ffn_plan_set_hot_head(plan, n_hot))


def ffn_offload_workspace_size(desc: ffn_layer_desc, capacity: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ffn_offload_workspace_size(ctypes.byref(desc), capacity, ctypes.byref(n)))
    return n.value


def ffn_offload_plan(desc, weights, capacity: int, n_pinned: int, workspace: int,
                     workspace_bytes: int, stream: int = 0) -> int:
    out = ctypes.c_void_p(0)
    _check(lib().ffn_offload_plan(ctypes.byref(desc), ctypes.byref(weights), capacity, n_pinned,
                                  workspace, workspace_bytes, stream or None, ctypes.byref(out)))
    return out.value


def ffn_offload_tables(plan: int):
    """Device addresses of (slot_of, neuron_of, last_use, stats) inside the plan's workspace."""
    ptrs = [ctypes.c_void_p(0) for _ in range(4)]
    _check(lib().ffn_offload_tables(plan, *[ctypes.byref(q) for q in ptrs]))
    return tuple(q.value for q in ptrs)


def ffn_plan_destroy(plan: int):
    _check(lib().ffn_plan_destroy(plan))


def ffn_plan_set_timing_events(plan: int, stage: int, start: int = 0, stop: int = 0):
    """start / stop: hipEvent_t handles (torch.cuda.Event(enable_timing=True).cuda_event)."""
    _check(lib().ffn_plan_set_timing_events(plan, stage, start or None, stop or None))


def ffn_moe_workspace_size(n_experts: int, top_k: int, expert0: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ffn_moe_workspace_size(n_experts, top_k, expert0, ctypes.byref(n)))
    return n.value


def ffn_moe_plan(n_experts: int, top_k: int, w_router: int, experts, workspace: int,
                 workspace_bytes: int) -> int:
    arr = (ctypes.c_void_p * len(experts))(*experts)
    out = ctypes.c_void_p(0)
    _check(lib().ffn_moe_plan(n_experts, top_k, w_router, arr, workspace, workspace_bytes,
                              ctypes.byref(out)))
    return out.value


def ffn_moe_forward(moe: int, x: int, B: int, y: int, expert_idx: int = 0, expert_w: int = 0,
                    expert_cnt: int = 0, stream: int = 0):
    _check(lib().ffn_moe_forward(moe, x, B, y, expert_idx or None, expert_w or None,
                                 expert_cnt or None, stream or None))


def ffn_moe_destroy(moe: int):
    _check(lib().ffn_moe_destroy(moe))


def ffn_attn_workspace_size(desc: ffn_attn_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ffn_attn_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ffn_attn_plan(desc, weights, workspace: int, workspace_bytes: int) -> int:
    out = ctypes.c_void_p(0)
    _check(lib().ffn_attn_plan(ctypes.byref(desc), ctypes.byref(weights), workspace,
                               workspace_bytes, ctypes.byref(out)))
    return out.value


def ffn_attn_forward(plan: int, x: int, pos: int, k_cache: int, v_cache: int, y: int,
                     mask: int = 0, idx: int = 0, cnt: int = 0, scores: int = 0,
                     stream: int = 0):
    _check(lib().ffn_attn_forward(plan, x, pos, k_cache, v_cache, y, mask or None, idx or None,
                                  cnt or None, scores or None, stream or None))


def ffn_attn_set_timing_events(plan: int, stage: int, start: int = 0, stop: int = 0):
    _check(lib().ffn_attn_set_timing_events(plan, stage, start or None, stop or None))


def ffn_attn_destroy(plan: int):
    _check(lib().ffn_attn_destroy(plan))


# ---------------------------------------------------------------------------------------------
def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


class SparseFFN:
    """Holds one layer's device tensors, its workspace and its plan.

    ``layer`` maps the names of ``ffn_layer_weights`` to device tensors (missing or None = NULL)
    and carries ``act``; the storage dtypes are read from the tensors (uint8 up rows = int4).
    An optional ``n_hot`` sets the always-active head (``ffn_plan_set_hot_head``).
    """

    def __init__(self, layer: dict, max_batch: int = 1, threshold: float = 0.5,
                 workspace: torch.Tensor | None = None, calibrate: bool = False):
        w_up = layer["w_up"]
        dev = w_up.device
        if w_up.dtype == torch.uint8:
            w_dtype, d = FFN_I4G32, w_up.shape[1] * 2
        else:
            w_dtype, d = (FFN_F32 if w_up.dtype == torch.float32 else FFN_F16), w_up.shape[1]
        p1 = layer.get("p1")
        rank = 0 if p1 is None else p1.shape[0]
        x_dtype = FFN_F32 if w_dtype == FFN_F32 else FFN_F16
        p_dtype = x_dtype if p1 is None else (FFN_F32 if p1.dtype == torch.float32 else FFN_F16)
        act = layer["act"]
        self.desc = ffn_layer_desc(d=d, ffn=w_up.shape[0], rank=rank,
                                   act=ACT[act] if isinstance(act, str) else int(act),
                                   w_dtype=w_dtype, x_dtype=x_dtype, p_dtype=p_dtype,
                                   threshold=float(layer.get("tau", threshold)),
                                   max_batch=max_batch)
        self.tensors = {k: layer.get(k) for k, _ in ffn_layer_weights._fields_}
        self.weights = ffn_layer_weights(**{k: (_ptr(v) or None) for k, v in self.tensors.items()})
        self.ws_bytes = ffn_workspace_size(self.desc)
        if workspace is None:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        assert workspace.numel() >= self.ws_bytes
        self.workspace = workspace
        self.d, self.ffn, self.x_dtype = d, self.desc.ffn, x_dtype
        self.plan = ffn_sparse_plan(self.desc, self.weights, workspace.data_ptr(),
                                    workspace.numel(), _stream(), int(calibrate))
        if layer.get("n_hot"):
            self.set_hot_head(int(layer["n_hot"]))

    def set_hot_head(self, n_hot: int):
        """Neurons [0, n_hot) always active (the layer's neurons ordered hottest first)."""
        ffn_plan_set_hot_head(self.plan, n_hot)

    def forward(self, x, y=None, mask=None, idx=None, cnt=None, scores=None,
                path=FFN_PATH_SPARSE):
        B = x.shape[0]
        if y is None:
            y = torch.empty(B, self.d, dtype=torch.float32, device=x.device)
        ffn_sparse_forward(self.plan, x.data_ptr(), B, y.data_ptr(), _ptr(mask), _ptr(idx),
                           _ptr(cnt), _ptr(scores), path, _stream())
        return y

    def dense(self, x, y=None, mask=None):
        B = x.shape[0]
        if y is None:
            y = torch.empty(B, self.d, dtype=torch.float32, device=x.device)
        ffn_dense_forward(self.plan, x.data_ptr(), B, y.data_ptr(), _ptr(mask), _stream())
        return y

    def crossover(self, B: int) -> float:
        return ffn_plan_crossover(self.plan, B)

    def last_auto_path(self) -> str:
        """The path the device chose on the last AUTO call of 64 tokens or more (a copy of the
        plan's flag: 'dense' or 'sparse')."""
        base = self.workspace.data_ptr()
        off = ffn_plan_path_flag(self.plan) - base
        return "dense" if int(self.workspace[off:off + 4].view(torch.int32)[0]) == 1 else "sparse"

    def close(self):
        if self.plan:
            ffn_plan_destroy(self.plan)
            self.plan = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class OffloadFFN(SparseFFN):
    """A layer whose up / gate / down rows stay in pinned host memory behind a pool of
    ``capacity`` neuron slots in device memory (``ffn_offload_plan``).  ``layer`` holds the rows
    as pinned CPU tensors (``pin_memory=True``) and the predictor and biases as device tensors;
    neurons [0, n_pinned) are kept in the pool for good.  One token per call."""

    def __init__(self, layer: dict, capacity: int, n_pinned: int = 0, threshold: float = 0.5,
                 device=None):
        w_up = layer["w_up"]
        assert w_up.dtype == torch.float16 and w_up.is_pinned(), "rows: pinned fp16 CPU tensors"
        dev = device or layer["p1"].device
        p1 = layer["p1"]
        act = layer["act"]
        self.desc = ffn_layer_desc(d=w_up.shape[1], ffn=w_up.shape[0], rank=p1.shape[0],
                                   act=ACT[act] if isinstance(act, str) else int(act),
                                   w_dtype=FFN_F16, x_dtype=FFN_F16,
                                   p_dtype=FFN_F32 if p1.dtype == torch.float32 else FFN_F16,
                                   threshold=float(layer.get("tau", threshold)), max_batch=1)
        self.tensors = {k: layer.get(k) for k, _ in ffn_layer_weights._fields_}
        self.weights = ffn_layer_weights(**{k: (_ptr(v) or None) for k, v in self.tensors.items()})
        self.ws_bytes = ffn_offload_workspace_size(self.desc, capacity)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.d, self.ffn, self.x_dtype = self.desc.d, self.desc.ffn, FFN_F16
        self.capacity = capacity
        self.plan = ffn_offload_plan(self.desc, self.weights, capacity, n_pinned,
                                     self.workspace.data_ptr(), self.ws_bytes, _stream())
        if layer.get("n_hot"):
            self.set_hot_head(int(layer["n_hot"]))

    def tables(self):
        """(slot_of [ffn], neuron_of [capacity], last_use [capacity] (as int64), stats [8]) --
        copies of the pool's device tables (stats: the last call's hits, misses, admissions, |A|,
        then their running totals)."""
        base = self.workspace.data_ptr()
        so, no, lu, st = ffn_offload_tables(self.plan)

        def view(addr, n):
            return self.workspace[addr - base: addr - base + 4 * n].view(torch.int32)
        last = view(lu, self.capacity).clone().to(torch.int64) & 0xFFFFFFFF
        return (view(so, self.ffn).clone(), view(no, self.capacity).clone(), last,
                view(st, 8).clone())


class MoEFFN:
    """A mixture of sparse-FFN experts with an on-device top-k router.

    ``experts`` is a list of layer dicts (as for ``SparseFFN``); ``router`` is the [E][d] router
    matrix in the experts' activation dtype.  The expert plans share one workspace (they are
    only used for their weights and shapes); the mixture has its own.
    """

    def __init__(self, experts, router: torch.Tensor, top_k: int = 2, max_batch: int = 1):
        self.experts = [SparseFFN(e, max_batch=max_batch) for e in experts]
        self.router = router
        self.top_k = top_k
        self.d = self.experts[0].d
        plans = [e.plan for e in self.experts]
        n = ffn_moe_workspace_size(len(plans), top_k, plans[0])
        self.workspace = torch.empty(n, dtype=torch.uint8, device=router.device)
        self.moe = ffn_moe_plan(len(plans), top_k, router.data_ptr(), plans,
                                self.workspace.data_ptr(), n)

    def forward(self, x, y=None, expert_idx=None, expert_w=None, expert_cnt=None):
        B = x.shape[0]
        if y is None:
            y = torch.empty(B, self.d, dtype=torch.float32, device=x.device)
        ffn_moe_forward(self.moe, x.data_ptr(), B, y.data_ptr(), _ptr(expert_idx), _ptr(expert_w),
                        _ptr(expert_cnt), _stream())
        return y

    def close(self):
        if self.moe:
            ffn_moe_destroy(self.moe)
            self.moe = 0
        for e in self.experts:
            e.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class SparseAttention:
    """Holds one attention block's device tensors, its workspace and its plan.

    ``layer`` maps the names of ``ffn_attn_weights`` to device fp16 tensors (c1 / c2 fp32, any
    may be None where the header allows NULL) and carries ``head_dim``, ``tau`` and the head
    counts through the tensors' shapes: w_q [H e][d], w_k [G e][d].  The caches are the
    caller's [G][max_seq][e] fp16 tensors, passed per call."""

    def __init__(self, layer: dict, max_seq: int, threshold: float = 0.5):
        w_q, w_k = layer["w_q"], layer["w_k"]
        e = int(layer["head_dim"])
        p1 = layer.get("p1")
        self.desc = ffn_attn_desc(d=w_q.shape[1], heads=w_q.shape[0] // e,
                                  kv_heads=w_k.shape[0] // e, head_dim=e,
                                  rank=0 if p1 is None else p1.shape[0], max_seq=max_seq,
                                  threshold=float(layer.get("tau", threshold)))
        self.tensors = {k: layer.get(k) for k, _ in ffn_attn_weights._fields_}
        self.weights = ffn_attn_weights(**{k: (_ptr(v) or None) for k, v in self.tensors.items()})
        self.ws_bytes = ffn_attn_workspace_size(self.desc)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=w_q.device)
        self.d, self.heads = self.desc.d, self.desc.heads
        self.plan = ffn_attn_plan(self.desc, self.weights, self.workspace.data_ptr(),
                                  self.ws_bytes)

    def forward(self, x, pos: int, k_cache, v_cache, y=None, mask=None, idx=None, cnt=None,
                scores=None):
        if y is None:
            y = torch.empty(self.d, dtype=torch.float32, device=x.device)
        ffn_attn_forward(self.plan, x.data_ptr(), pos, k_cache.data_ptr(), v_cache.data_ptr(),
                         y.data_ptr(), _ptr(mask), _ptr(idx), _ptr(cnt), _ptr(scores), _stream())
        return y

    def close(self):
        if self.plan:
            ffn_attn_destroy(self.plan)
            self.plan = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
