"""The library's host code (argument checks, workspace layout, plan objects, status strings) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The HIP sources are compiled with the sanitizers on their host side only (the device code is the
same as in the product build) into a separate library, and tests/abi_sanitize.c -- built with the
same compiler and sanitizer runtime -- drives every host-side path that returns before anything is
enqueued: valid and rejected descriptors of every storage type, plans over fake device pointers
and every call on them, forward calls with bad arguments, a mixture, the neuron-cache plan and the
allocation-free entry point's checks.  Each struct lives in a heap block of exactly its size and
every plan is destroyed, so an out-of-bounds access, a use after free, a double free or an
undefined operation in the host code is reported.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_sparse_ffn_gemv_amd", "csrc")
ROCM_LLVM = "/opt/rocm/lib/llvm"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = os.path.join(ROCM_LLVM, "bin", "clang")

# sanitizers on the host side of each translation unit only (each -fsanitize= right after
# -Xarch_host), the rest as in the product build
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _runtime_dir():
    hits = glob.glob(os.path.join(ROCM_LLVM, "lib", "clang", "*", "lib", "linux",
                                  "libclang_rt.asan-x86_64.so"))
    return os.path.dirname(hits[0]) if hits else None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _runtime_dir()),
                    reason="needs hipcc and clang's sanitizer runtimes")
def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *FLAGS, *SAN, "-c", src, "-o", obj], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libffn_sparse_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_sanitize")
    r = subprocess.run([CLANG, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-shared-libsan", os.path.join(ROOT, "tests", "abi_sanitize.c"),
                        "-L" + str(tmp_path), "-lffn_sparse_san",
                        "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + _runtime_dir(),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ,
               # the HIP runtime the library loads is not instrumented: its own allocations at
               # exit are not this code's leaks; memory errors and undefined behaviour still abort
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1",
               LD_LIBRARY_PATH=":".join([str(tmp_path), _runtime_dir(),
                                         os.environ.get("LD_LIBRARY_PATH", "")]))
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "abi sanitizer run: OK" in run.stdout
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr, \
        run.stderr[-3000:]
    # the instrumentation is live in the library: a descriptor one field short is reported as a
    # heap-buffer-overflow inside the library's own check
    bad = subprocess.run([exe, "planted"], capture_output=True, text=True, env=env, timeout=300)
    assert bad.returncode != 0 and "heap-buffer-overflow" in bad.stderr, bad.stdout + bad.stderr
    assert "check_desc" in bad.stderr or "ffn_workspace_size" in bad.stderr, bad.stderr[-3000:]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and _runtime_dir()),
                    reason="needs hipcc and clang's sanitizer runtimes")
def test_kernel_index_arithmetic_in_a_cpu_build(tmp_path):
    """The kernels' index functions (csrc/index.h) compiled for the CPU with ASan and UBSan and
    walked over every workgroup and thread of the library's launch shapes (tests/index_check.cpp:
    partial-sum writes and reads, rank and segment splits, the XCD-ordered (block, pass) map, the
    per-pass buffer offsets of calls that run all their passes in one launch, and the dense down
    projection's and the stage-1 GEMM's tile maps, K slices and partial-sum stores)."""
    lib_dir = os.path.join(ROOT, "activation_sparse_ffn_gemv_amd")
    if not os.path.exists(os.path.join(lib_dir, "libffn_sparse.so")):
        pytest.skip("library not built")
    exe = str(tmp_path / "index_check")
    r = subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", "-g",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan",
                        os.path.join(ROOT, "tests", "index_check.cpp"),
                        "-L" + lib_dir, "-l:libffn_sparse.so", "-Wl,-rpath," + lib_dir,
                        "-Wl,-rpath," + _runtime_dir(), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               LD_LIBRARY_PATH=":".join([_runtime_dir(), os.environ.get("LD_LIBRARY_PATH", "")]))
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "index check: OK" in run.stdout, run.stdout[-2000:]
    assert "runtime error" not in run.stderr, run.stderr[-3000:]
