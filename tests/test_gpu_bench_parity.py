"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

Each case runs bench.py's main() in this process on one of the workloads (all layers,
HIP-graph replay of whole steps), then checks the JSON line it prints: the outputs the timed run
wrote, at layer 0 and at seeded random (layer, token) pairs over the whole stack, must match the
oracle evaluated on the GPU's own active sets within the tolerance (1e-5 for fp32 weights, 2e-3
for fp16 / int4), and the line must carry the roofline and CPU-baseline fields.
"""
import json
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (case id, bench arguments, smallest number of (layer, token) pairs checked)
CASES = [
    ("opt125m", ["--config", "opt125m_relu_f32", "--steps", "8", "--cpu-tokens", "4"], 4),
    # the 7B-shaped stacks: the first two tokens at every one of the 32 layers, plus random pairs
    ("llama2", ["--config", "llama2_7b_reglu_f16", "--steps", "4", "--parity-pairs", "6",
                "--parity-stack-tokens", "2"], 64),
    ("mistral", ["--config", "turbosparse_mistral_7b_drelu_f16", "--steps", "4",
                 "--parity-pairs", "6", "--parity-stack-tokens", "2"], 64),
    ("mixtral_int4", ["--config", "turbosparse_mixtral_47b_moe_int4", "--steps", "4",
                      "--parity-pairs", "6", "--parity-stack-tokens", "2"], 64),
    ("falcon_b1", ["--config", "falcon_40b_relu_f16", "--steps", "2", "--parity-pairs", "3"], 4),
    ("falcon_b8", ["--config", "falcon_40b_relu_f16", "--batch", "8", "--steps", "2",
                   "--parity-pairs", "3"], 4),
    ("falcon_b32", ["--config", "falcon_40b_relu_f16", "--batch", "32", "--steps", "1",
                    "--parity-pairs", "3"], 4),
    ("falcon_prefill512", ["--config", "falcon_40b_relu_f16", "--prefill", "512", "--steps", "1",
                           "--parity-pairs", "2"], 3),
    # attention blocks (32 blocks, a token at position 511 of each block's cache)
    ("llama2_attn", ["--config", "llama2_7b_attn_f16", "--steps", "4", "--parity-pairs", "8"], 6),
    ("mistral_attn", ["--config", "mistral_7b_attn_f16", "--steps", "4", "--parity-pairs", "8"],
     6),
    ("falcon_attn", ["--config", "falcon_40b_attn_f16", "--steps", "2", "--parity-pairs", "3"],
     3),
]


@pytest.fixture(scope="module")
def bench_main():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    return bench.main


@pytest.mark.parametrize("argv,min_pairs", [c[1:] for c in CASES], ids=[c[0] for c in CASES])
def test_full_size_parity_in_bench_configuration(bench_main, capsys, argv, min_pairs):
    common = ["--warmup", "1", "--kernel-sample", "1", "--cpu-budget", "0.1"]
    if "--cpu-tokens" not in argv:
        common += ["--cpu-tokens", "1"]
    try:
        bench_main(argv + common)
    finally:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    out = capsys.readouterr().out.strip().splitlines()
    line = json.loads(out[-1])
    par = line["parity_sample"]
    assert par is not None and par["pairs"] >= min_pairs, par
    assert par["within_tolerance"], par
    assert par["max_normwise_err"] <= par["tolerance"]
    if "opt125m" not in argv[1]:
        assert len(par["layers"]) > 1, par              # beyond layer 0
    if "--parity-stack-tokens" in argv:
        assert len(par["layers"]) == line["config"]["layers"], par     # every layer
    assert line["value"] > 0 and line["n_gpus"] == 1
    roof = line["roofline"]
    assert roof["achieved"] > 0 and 0 < roof["frac"] < 1, roof
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] == 1
    if "--prefill" in argv:
        # the bench's prefill goes through AUTO on an uncalibrated plan: the device took the
        # dense GEMMs at every layer (the 512-token union is far above the built-in crossover)
        pp = line["prefill_path"]
        assert line["config"]["path"] == "auto" and pp["path"] == "dense", pp
        assert pp["dense_layers"] == line["config"]["layers"], pp
