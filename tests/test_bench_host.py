"""Host-side logic of bench.py (no GPU): the single-GPU contract, the byte accounting helpers and
the lookup of profiled traffic."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_row_bytes_and_predictor_bytes():
    c2 = synth.CONFIGS["llama2_7b_reglu_f16"]
    assert bench.row_bytes(c2) == 2 * 4096
    assert bench.n_rows(c2) == 3 and bench.n_bias(c2) == 1
    pz, ps = bench.pred_bytes(c2)
    assert pz == 256 * 4096 * 2 and ps == 11008 * 256 * 2 + 4 * 11008
    c4 = synth.CONFIGS["turbosparse_mixtral_47b_moe_int4"]
    assert bench.row_bytes(c4) == 4096 // 2 + (4096 // 32) * 2       # packed nibbles + fp16 scales
    assert bench.n_bias(c4) == 2
    c1 = synth.CONFIGS["opt125m_relu_f32"]
    assert bench.row_bytes(c1) == 4 * 768 and bench.n_rows(c1) == 2


def test_profiled_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source v1\n")
    h = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k_x_w.md").write_text(
        "# summary\n\n- mean duration (kernel trace): 10.89 us\n\n"
        "    traffic kernel=k_x workload=w bytes_per_launch=1234 source=k.hip "
        "sha256=%s\n" % h)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("k_x", "w") == 1234
    assert bench.profiled_traffic("k_x", "w", with_trace=True) == (1234, 10.89)
    assert bench.profiled_traffic("k_x", "other") is None
    assert bench.profiled_traffic("k_y", "w", with_trace=True) == (None, None)
    src.write_text("kernel source v2\n")                 # kernel changed since the counters
    assert bench.profiled_traffic("k_x", "w") is None
    assert bench.profiled_traffic("k_x", "w", with_trace=True) == (None, None)


def test_profiled_mfma_busy_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("gemm v1\n")
    h = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k_g_w.md").write_text(
        "# summary\n\n- MFMA utilisation (busy cycles / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)): "
        "**45.9%%**\n\n    traffic kernel=k_g workload=w bytes_per_launch=1 source=k.hip "
        "sha256=%s\n" % h)
    (prof / "k_n_w.md").write_text(
        "    traffic kernel=k_n workload=w bytes_per_launch=1 source=k.hip sha256=%s\n" % h)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_mfma_busy("k_g", "w") == 0.459
    assert bench.profiled_mfma_busy("k_n", "w") is None       # no counter pass in the summary
    assert bench.profiled_mfma_busy("k_g", "other") is None
    src.write_text("gemm v2\n")
    assert bench.profiled_mfma_busy("k_g", "w") is None


def test_committed_prefill_summaries_carry_mfma_busy():
    for k in ("k_dupq", "k_ddq"):
        u = bench.profiled_mfma_busy(k, "falcon_40b_relu_f16:prefill512")
        assert u is not None and 0.0 < u < 1.0, (k, u)


def test_committed_profiles_name_existing_sources():
    pdir = os.path.join(ROOT, "profiles")
    n = 0
    for f in os.listdir(pdir):
        for line in open(os.path.join(pdir, f)):
            t = line.split()
            if t and t[0] == "traffic":
                kv = dict(x.split("=", 1) for x in t[1:])
                assert os.path.exists(os.path.join(ROOT, kv["source"])), kv["source"]
                assert int(kv["bytes_per_launch"]) > 0
                n += 1
    assert n >= 1


def test_bench_refuses_more_than_one_gpu():
    """More than one GPU is refused with a message before anything touches a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
