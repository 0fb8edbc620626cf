"""The C-ABI library: it loads, exports every symbol include/ffn_sparse.h declares, and its host
validation rejects bad arguments with the documented status codes (no GPU work is issued)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffn_sparse.h")

ffn = pytest.importorskip("activation_sparse_ffn_gemv_amd")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ffn_[a-z0-9_]+)\s*\(", src)))


def test_header_lists_match_binding():
    assert _declared() == sorted(ffn.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ffn.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ffn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in _declared():
        assert name in syms, name


def test_status_strings_cover_every_status():
    names = ["FFN_OK", "FFN_ERR_INVALID_ARGUMENT", "FFN_ERR_UNSUPPORTED",
             "FFN_ERR_WORKSPACE_TOO_SMALL", "FFN_ERR_HIP", "FFN_ERR_INTERNAL"]
    # the enum in the header and the binding's constants agree with the names
    src = open(HEADER).read()
    for v, n in enumerate(names):
        assert getattr(ffn, n) == v
        assert re.search(r"\b%s\s*=\s*%d\b" % (n, v), src), n
        assert ffn.ffn_status_string(v) == n
    for v in (-1, 6, 1 << 30):
        assert ffn.ffn_status_string(v) == "FFN_STATUS_UNKNOWN"
    # the same static string on every call (no allocation)
    L = ffn.lib()
    L.ffn_status_string.restype = ctypes.c_void_p
    try:
        assert L.ffn_status_string(3) == L.ffn_status_string(3)
    finally:
        L.ffn_status_string.restype = ctypes.c_char_p
    # an error raised by the binding names its status
    with pytest.raises(ffn.FFNError) as e:
        ffn.ffn_workspace_size(_desc(d=0))
    assert "FFN_ERR_INVALID_ARGUMENT" in str(e.value)


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", "-"],
                       input='#include "%s"\nint main(void){return 0;}\n' % HEADER,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _desc(**kw):
    base = dict(d=4096, ffn=11008, rank=256, act=ffn.FFN_ACT_REGLU, w_dtype=ffn.FFN_F16,
                x_dtype=ffn.FFN_F16, p_dtype=ffn.FFN_F16, threshold=0.5, max_batch=1)
    base.update(kw)
    return ffn.ffn_layer_desc(**base)


def test_workspace_size_valid_and_monotone_in_batch():
    a = ffn.ffn_workspace_size(_desc())
    b = ffn.ffn_workspace_size(_desc(max_batch=32))
    assert a > 0 and b >= a and a % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d=0), ffn.FFN_ERR_INVALID_ARGUMENT),
    (dict(act=7), ffn.FFN_ERR_INVALID_ARGUMENT),
    (dict(threshold=0.0), ffn.FFN_ERR_INVALID_ARGUMENT),
    (dict(threshold=1.5), ffn.FFN_ERR_INVALID_ARGUMENT),
    (dict(d=4100), ffn.FFN_ERR_UNSUPPORTED),
    (dict(ffn=11000), ffn.FFN_ERR_UNSUPPORTED),
    (dict(rank=100), ffn.FFN_ERR_UNSUPPORTED),
    (dict(x_dtype=ffn.FFN_F32), ffn.FFN_ERR_UNSUPPORTED),
    (dict(w_dtype=ffn.FFN_I4G32, d=4104), ffn.FFN_ERR_UNSUPPORTED),
    (dict(d=16384), ffn.FFN_ERR_UNSUPPORTED),
    (dict(ffn=32800), ffn.FFN_ERR_UNSUPPORTED),
    (dict(rank=4096), ffn.FFN_ERR_UNSUPPORTED),
    (dict(max_batch=0), ffn.FFN_ERR_INVALID_ARGUMENT),
    (dict(d=8192, w_dtype=ffn.FFN_F32, x_dtype=ffn.FFN_F32, p_dtype=ffn.FFN_F32, rank=64),
     ffn.FFN_ERR_UNSUPPORTED),
])
def test_bad_descriptors_are_rejected(kw, status):
    with pytest.raises(ffn.FFNError) as e:
        ffn.ffn_workspace_size(_desc(**kw))
    assert e.value.status == status
    assert ffn.ffn_last_error()


def test_plan_validation_before_any_gpu_call():
    d = _desc()
    w = ffn.ffn_layer_weights()
    with pytest.raises(ffn.FFNError) as e:          # missing weights
        ffn.ffn_sparse_plan(d, w, 0x1000, 1 << 30)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    w = ffn.ffn_layer_weights(w_up=0x1000, w_gate=0x2000, w_down_t=0x3000, p1=0x4000,
                              p2=0x5000)
    with pytest.raises(ffn.FFNError) as e:          # workspace too small
        ffn.ffn_sparse_plan(d, w, 0x10000, 16)
    assert e.value.status == ffn.FFN_ERR_WORKSPACE_TOO_SMALL
    w.b_up = 0x1004                                 # misaligned pointer
    with pytest.raises(ffn.FFNError) as e:
        ffn.ffn_sparse_plan(d, w, 0x10000, 1 << 30)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    w.b_up = None
    plan = ffn.ffn_sparse_plan(d, w, 0x10000, 1 << 30)   # host-only: nothing is launched
    try:
        with pytest.raises(ffn.FFNError) as e:      # B out of range
            ffn.ffn_sparse_forward(plan, 0x1000, 2, 0x2000)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        with pytest.raises(ffn.FFNError) as e:      # bad path
            ffn.ffn_sparse_forward(plan, 0x1000, 1, 0x2000, path=9)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        with pytest.raises(ffn.FFNError):           # NULL y
            ffn.ffn_sparse_forward(plan, 0x1000, 1, 0)
        with pytest.raises(ffn.FFNError) as e:      # dense: B out of range, misaligned mask
            ffn.ffn_dense_forward(plan, 0x1000, 2, 0x2000)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        with pytest.raises(ffn.FFNError) as e:
            ffn.ffn_dense_forward(plan, 0x1000, 1, 0x2000, mask=0x3001)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        assert ffn.ffn_plan_crossover(plan, 1) <= 1.0
        with pytest.raises(ffn.FFNError) as e:              # max_batch 1: no dense GEMMs
            ffn.ffn_plan_path_flag(plan)
        assert e.value.status == ffn.FFN_ERR_UNSUPPORTED
        ffn.ffn_plan_set_crossover(plan, 8, 0.25)           # bucket 8..15
        assert ffn.ffn_plan_crossover(plan, 8) == 0.25
        assert ffn.ffn_plan_crossover(plan, 15) == 0.25
        assert ffn.ffn_plan_crossover(plan, 16) == 1.0
        with pytest.raises(ffn.FFNError) as e:
            ffn.ffn_plan_set_crossover(plan, 8, 1.5)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        for bad in (-32, 16, d.ffn + 32):                  # hot head: multiple of 32 in [0, ffn]
            with pytest.raises(ffn.FFNError) as e:
                ffn.ffn_plan_set_hot_head(plan, bad)
            assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        ffn.ffn_plan_set_hot_head(plan, d.ffn)
        ffn.ffn_plan_set_hot_head(plan, 0)
    finally:
        ffn.ffn_plan_destroy(plan)


def test_builtin_crossover_table():
    """Uncalibrated plans: never dense below 64 tokens; from 64 on, dense above the union density
    at which ceil(B / 32) sparse passes read as many row bytes as one dense read."""
    plan = _fake_plan(max_batch=4096)
    try:
        for B in (1, 2, 5, 32, 63):
            assert ffn.ffn_plan_crossover(plan, B) == 1.0
        for B, rho in ((64, 0.5), (100, 0.5), (128, 0.25), (256, 0.125), (512, 1 / 16),
                       (4096, 1 / 128)):
            assert abs(ffn.ffn_plan_crossover(plan, B) - rho) < 1e-7, B
        flag = ffn.ffn_plan_path_flag(plan)                 # inside the workspace
        assert 0x10000 <= flag < 0x10000 + ffn.ffn_workspace_size(_desc(max_batch=4096))
        assert flag % 4 == 0
    finally:
        ffn.ffn_plan_destroy(plan)


def test_static_entry_point_validation_before_any_gpu_call():
    """The allocation-free entry point checks its descriptor, weights and sizes on every call
    and returns before anything touches the GPU."""
    w = ffn.ffn_layer_weights(w_up=0x1000, w_gate=0x2000, w_down_t=0x3000, p1=0x4000,
                              p2=0x5000)
    with pytest.raises(ffn.FFNError) as e:                     # bad descriptor
        ffn.ffn_sparse_forward_static(_desc(d=0), w, 0x6000, 1, 0x7000)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # missing gate rows
        ffn.ffn_sparse_forward_static(_desc(), ffn.ffn_layer_weights(w_up=0x1000, w_down_t=0x3000,
                                                                     p1=0x4000, p2=0x5000),
                                      0x6000, 1, 0x7000)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # B beyond max_batch
        ffn.ffn_sparse_forward_static(_desc(max_batch=2), w, 0x6000, 3, 0x7000)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # misaligned y
        ffn.ffn_sparse_forward_static(_desc(), w, 0x6000, 1, 0x7004)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # no predictor and no mask
        ffn.ffn_sparse_forward_static(_desc(rank=0), w, 0x6000, 1, 0x7000)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # beyond the static scratch
        ffn.ffn_sparse_forward_static(_desc(d=8192, ffn=32768, rank=1024, act=ffn.FFN_ACT_RELU),
                                      w, 0x6000, 1, 0x7000)
    assert e.value.status == ffn.FFN_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in ffn.ffn_last_error()


def test_no_predictor_requires_mask():
    d = _desc(rank=0)
    w = ffn.ffn_layer_weights(w_up=0x1000, w_gate=0x2000, w_down_t=0x3000)
    plan = ffn.ffn_sparse_plan(d, w, 0x10000, 1 << 30)
    try:
        with pytest.raises(ffn.FFNError) as e:
            ffn.ffn_sparse_forward(plan, 0x1000, 1, 0x2000)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    finally:
        ffn.ffn_plan_destroy(plan)


def test_binding_loads_only_the_in_tree_library():
    assert os.path.dirname(ffn.LIB_PATH) == os.path.join(ROOT, "activation_sparse_ffn_gemv_amd")
    assert isinstance(ffn.lib(), ctypes.CDLL)


def _fake_plan(**kw):
    d = _desc(**kw)
    w = ffn.ffn_layer_weights(w_up=0x1000, w_gate=0x2000, w_down_t=0x3000, p1=0x4000,
                              p2=0x5000)
    return ffn.ffn_sparse_plan(d, w, 0x10000, 1 << 30)


def test_moe_validation_before_any_gpu_call():
    e = [_fake_plan() for _ in range(3)]
    odd = _fake_plan(rank=128)
    try:
        n = ffn.ffn_moe_workspace_size(3, 2, e[0])
        assert n > 0 and n % 256 == 0
        assert ffn.ffn_moe_workspace_size(3, 1, e[0]) < n      # one decode scratch per slot
        for E, K in [(0, 1), (17, 2), (3, 0), (3, 4), (8, 5)]:
            with pytest.raises(ffn.FFNError) as ex:
                ffn.ffn_moe_workspace_size(E, K, e[0])
            assert ex.value.status == ffn.FFN_ERR_UNSUPPORTED
        with pytest.raises(ffn.FFNError) as ex:           # descriptors differ
            ffn.ffn_moe_plan(2, 1, 0x8000, [e[0], odd], 0x20000, n)
        assert ex.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        with pytest.raises(ffn.FFNError) as ex:           # workspace too small
            ffn.ffn_moe_plan(3, 2, 0x8000, e, 0x20000, 64)
        assert ex.value.status == ffn.FFN_ERR_WORKSPACE_TOO_SMALL
        m = ffn.ffn_moe_plan(3, 2, 0x8000, e, 0x20000, n)
        try:
            with pytest.raises(ffn.FFNError) as ex:       # B out of range
                ffn.ffn_moe_forward(m, 0x1000, 2, 0x2000)
            assert ex.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
            with pytest.raises(ffn.FFNError):             # NULL y
                ffn.ffn_moe_forward(m, 0x1000, 1, 0)
        finally:
            ffn.ffn_moe_destroy(m)
    finally:
        for p in e + [odd]:
            ffn.ffn_plan_destroy(p)


def test_offload_validation_before_any_gpu_call():
    d = _desc()
    d.w_dtype, d.x_dtype, d.p_dtype = ffn.FFN_F16, ffn.FFN_F16, ffn.FFN_F16
    assert ffn.ffn_offload_workspace_size(d, 64) > ffn.ffn_workspace_size(d) // 2
    for cap in (0, 16, 48, d.ffn + 32, 8192 + 32):              # multiple of 32 in [32, min]
        with pytest.raises(ffn.FFNError) as e:
            ffn.ffn_offload_workspace_size(d, cap)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    f32 = _desc()
    f32.w_dtype = ffn.FFN_F32
    with pytest.raises(ffn.FFNError) as e:                     # fp16 rows only
        ffn.ffn_offload_workspace_size(f32, 64)
    assert e.value.status == ffn.FFN_ERR_UNSUPPORTED
    w = ffn.ffn_layer_weights(w_up=0x1000, w_gate=0x2000, w_down_t=0x3000, p1=0x4000,
                              p2=0x5000)
    with pytest.raises(ffn.FFNError) as e:                     # rows not pinned host memory
        ffn.ffn_offload_plan(d, w, 64, 0, 0x10000, 1 << 30)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # n_pinned beyond the pool
        ffn.ffn_offload_plan(d, w, 64, 96, 0x10000, 1 << 30)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # not a pool plan
        ffn.ffn_offload_tables(0)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT


def _adesc(**kw):
    base = dict(d=4096, heads=32, kv_heads=8, head_dim=128, rank=128, max_seq=512,
                threshold=0.5)
    base.update(kw)
    return ffn.ffn_attn_desc(**base)


def test_attn_validation_before_any_gpu_call():
    n = ffn.ffn_attn_workspace_size(_adesc())
    assert n > 256 * 4096 * 4 and n % 256 == 0
    for kw, status in [(dict(d=4100), ffn.FFN_ERR_UNSUPPORTED),
                       (dict(d=16384), ffn.FFN_ERR_UNSUPPORTED),
                       (dict(heads=0), ffn.FFN_ERR_UNSUPPORTED),
                       (dict(heads=129), ffn.FFN_ERR_UNSUPPORTED),
                       (dict(kv_heads=5), ffn.FFN_ERR_UNSUPPORTED),      # does not divide H
                       (dict(head_dim=96), ffn.FFN_ERR_UNSUPPORTED),
                       (dict(rank=12), ffn.FFN_ERR_UNSUPPORTED),
                       (dict(rank=2048), ffn.FFN_ERR_UNSUPPORTED),
                       (dict(max_seq=0), ffn.FFN_ERR_INVALID_ARGUMENT),
                       (dict(threshold=0.0), ffn.FFN_ERR_INVALID_ARGUMENT),
                       (dict(threshold=1.5), ffn.FFN_ERR_INVALID_ARGUMENT)]:
        with pytest.raises(ffn.FFNError) as e:
            ffn.ffn_attn_workspace_size(_adesc(**kw))
        assert e.value.status == status, kw
    w = ffn.ffn_attn_weights(w_q=0x1000, w_k=0x2000, w_v=0x3000, w_o_t=0x4000, p1=0x5000,
                             p2=0x6000)
    with pytest.raises(ffn.FFNError) as e:
        ffn.ffn_attn_plan(_adesc(), w, 0x10000, n - 1)
    assert e.value.status == ffn.FFN_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(ffn.FFNError) as e:                     # predictor without P2
        ffn.ffn_attn_plan(_adesc(), ffn.ffn_attn_weights(w_q=0x1000, w_k=0x2000, w_v=0x3000,
                                                         w_o_t=0x4000, p1=0x5000), 0x10000, n)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    with pytest.raises(ffn.FFNError) as e:                     # misaligned weight
        ffn.ffn_attn_plan(_adesc(), ffn.ffn_attn_weights(w_q=0x1008, w_k=0x2000, w_v=0x3000,
                                                         w_o_t=0x4000, p1=0x5000, p2=0x6000),
                          0x10000, n)
    assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    p = ffn.ffn_attn_plan(_adesc(), w, 0x10000, n)
    try:
        for pos in (-1, 512):                                  # outside [0, max_seq)
            with pytest.raises(ffn.FFNError) as e:
                ffn.ffn_attn_forward(p, 0x1000, pos, 0x2000, 0x3000, 0x4000)
            assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        with pytest.raises(ffn.FFNError) as e:                 # NULL cache
            ffn.ffn_attn_forward(p, 0x1000, 0, 0, 0x3000, 0x4000)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
        with pytest.raises(ffn.FFNError) as e:                 # not an attention stage
            ffn.ffn_attn_set_timing_events(p, ffn.FFN_STAGE_GATHER)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    finally:
        ffn.ffn_attn_destroy(p)
    p0 = ffn.ffn_attn_plan(_adesc(rank=0), ffn.ffn_attn_weights(w_q=0x1000, w_k=0x2000,
                                                                w_v=0x3000, w_o_t=0x4000),
                           0x10000, n)
    try:
        with pytest.raises(ffn.FFNError) as e:                 # no predictor, no mask
            ffn.ffn_attn_forward(p0, 0x1000, 0, 0x2000, 0x3000, 0x4000)
        assert e.value.status == ffn.FFN_ERR_INVALID_ARGUMENT
    finally:
        ffn.ffn_attn_destroy(p0)
