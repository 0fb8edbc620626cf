#!/usr/bin/env python3
"""Decode benchmark of the activation-sparse FFN on one MI355X.

A step is one decode token (batch 1) through every layer of the workload: per layer the
predictor picks the token's active neurons and only their rows are read (PowerInfer, unite.ai,
"Adaptive sparse predictor" / "Neuron-aware operator").  Layers run one after another on one
stream, as in a real decode.  Inputs are seeded synthetic tensors already resident in HBM; the
timed region replays HIP graphs of the library's launches.

Printed (one JSON line on stdout): decode tokens/s, the effective HBM bandwidth over the bytes
the method touches, the roofline of the dominant kernel (the gathered-row main kernel, timed with
HIP events attached to its own dispatches), and the CPU oracle timed on the host as a baseline.
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def row_bytes(cfg) -> float:
    return {"f32": 4 * cfg.d, "f16": 2 * cfg.d, "i4g32": cfg.d // 2 + (cfg.d // 32) * 2}[cfg.w_dtype]


def stage_bytes(cfg):
    """Algorithmic bytes of each kernel as (fixed bytes per launch, bytes per active neuron):
    the weights the method must read.  x, y, z, the bitmap and the (index, h) list are overhead
    and not counted."""
    pb = 4 if cfg.p_dtype == "f32" else 2
    rows = 2 if cfg.act == "relu" else 3
    nbias = (1 if cfg.bias_up else 0) + (1 if (cfg.act != "relu" and cfg.bias_gate) else 0)
    return {
        "pred_z": (cfg.rank * cfg.d * pb, 0),                      # P1 (c1 absent)
        "pred_s": (cfg.ffn * cfg.rank * pb + 4 * cfg.ffn, 0),      # P2 + c2
        # the active neurons' up (+ gate) and transposed-down rows and their biases
        "gather": (0, rows * row_bytes(cfg) + 4 * nbias),
        "reduce": (0, 0),                                          # partials only (overhead)
    }


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from a committed rocprofv3 summary under
    profiles/ (FETCH_SIZE + WRITE_SIZE, scaled against a copy of known size), or None when there
    is none or the kernel source has changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            f = line.split()
            if not f or f[0] != "traffic":
                continue
            kv = dict(t.split("=", 1) for t in f[1:] if "=" in t)
            if kv.get("kernel") != kernel or kv.get("workload") != workload:
                continue
            src = os.path.join(ROOT, kv["source"])
            if not os.path.exists(src):
                return None
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("sha256"):
                return None
            return int(kv["bytes_per_launch"])
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode tokens (default: all)")
    ap.add_argument("--warmup", type=int, default=16, help="untimed tokens replayed first")
    ap.add_argument("--config", default="llama2_7b_reglu_f16")
    ap.add_argument("--kernel-sample", type=int, default=32,
                    help="tokens whose kernel launches are timed with dispatch events")
    ap.add_argument("--cpu-tokens", type=int, default=3,
                    help="tokens (x all layers) the CPU oracle baseline runs; 0 = skip")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB five times (a known "
                         "size against which a profiler's HBM byte counters are scaled)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the operator "
              "would shard by neurons, see the design notes); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_sparse_ffn_gemv_amd as ffn
    import synth

    cfg = synth.CONFIGS[args.config]
    if cfg.n_experts > 1:
        raise SystemExit("the mixture-of-experts workload has its own bench mode (not built yet)")
    L, T = cfg.layers, cfg.tokens
    K = args.steps if args.steps else T
    W = min(args.warmup, K)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log("config %s: d=%d ffn=%d rank=%d act=%s w=%s layers=%d tokens=%d" % (
        cfg.name, cfg.d, cfg.ffn, cfg.rank, cfg.act, cfg.w_dtype, L, K))

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 5 x %d MiB device-to-device" % args.copy_mib)
        del src, dst

    t0 = time.time()
    layers, plans = [], []
    for l in range(L):
        layers.append(synth.make_layer(cfg, layer=l, device=dev))
    x = torch.stack([synth.make_tokens(cfg, K, layer=l, device=dev) for l in range(L)])  # [L][K][d]
    y = torch.empty(L, K, cfg.d, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("inputs generated on the GPU in %.1f s" % (time.time() - t0))

    stream = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream
    probe = ffn.SparseFFN(layers[0], max_batch=1)
    ws = torch.empty(probe.ws_bytes, dtype=torch.uint8, device=dev)   # one workspace, shared
    probe.close()
    mods = [ffn.SparseFFN(layers[l], max_batch=1, workspace=ws) for l in range(L)]
    plans = [m.plan for m in mods]
    xb = x.element_size() * cfg.d
    xp = [[x[l].data_ptr() + t * xb for t in range(K)] for l in range(L)]
    yp = [[y[l].data_ptr() + t * cfg.d * 4 for t in range(K)] for l in range(L)]

    def token(t):
        for l in range(L):
            ffn.ffn_sparse_forward(plans[l], xp[l][t], 1, yp[l][t], path=ffn.FFN_PATH_SPARSE,
                                   stream=sp)

    # ---- active-set sizes of every timed (token, layer): a separate, untimed counting pass
    cnt = torch.zeros(L, K, dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for t in range(K):
            for l in range(L):
                ffn.ffn_sparse_forward(plans[l], xp[l][t], 1, yp[l][t],
                                       cnt=cnt[l].data_ptr() + 4 * t, stream=sp)
    torch.cuda.synchronize()
    cnt_h = cnt.cpu().numpy().astype(np.int64)
    density = float(cnt_h.mean() / cfg.ffn)
    log("measured density %.4f (mean |A| = %.1f of %d)" % (density, cnt_h.mean(), cfg.ffn))

    # ---- HIP graphs of whole tokens (all layers), G tokens per graph
    G = max(1, 256 // L)
    graphs = []
    with torch.cuda.stream(stream):
        for g0 in range(0, K, G):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(g0, min(K, g0 + G)):
                    token(t)
            graphs.append(g)
    torch.cuda.synchronize()
    log("captured %d graphs of %d tokens" % (len(graphs), G))

    with torch.cuda.stream(stream):
        for g in graphs[:max(1, (W + G - 1) // G)]:
            g.replay()
    torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for g in graphs:
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    tok_s = K / (ms / 1e3)
    SB = stage_bytes(cfg)
    touched = sum(f * L * K + a * cnt_h.sum() for f, a in SB.values())
    eff_gbps = touched / (ms / 1e3) / 1e9
    log("timed %d tokens: %.3f ms/token, %.1f tok/s, %.1f GB/s effective over touched bytes" % (
        K, ms / K, tok_s, eff_gbps))

    # ---- per-kernel durations: HIP events attached to each kernel's own dispatch (plain
    # launches of the same tokens); the dominant kernel gives the roofline
    S = min(args.kernel_sample, K)
    stages = {}
    for si, sname in enumerate(ffn.STAGES):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(S * L)]
        with torch.cuda.stream(stream):
            for a, b in evs:            # materialise the events
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        i = 0
        with torch.cuda.stream(stream):
            for t in range(S):
                for l in range(L):
                    a, b = evs[i]
                    ffn.ffn_plan_set_timing_events(plans[l], si, a.cuda_event, b.cuda_event)
                    ffn.ffn_sparse_forward(plans[l], xp[l][t], 1, yp[l][t], stream=sp)
                    i += 1
        torch.cuda.synchronize()
        for p in plans:
            ffn.ffn_plan_set_timing_events(p, si, 0, 0)
        dur_ms = np.array([a.elapsed_time(b) for a, b in evs])
        fixed, per_a = SB[sname]
        nbytes = fixed * S * L + per_a * cnt_h[:, :S].sum()
        stages[sname] = {"avg_us": round(float(dur_ms.mean()) * 1e3, 3),
                         "bytes_per_launch": int(nbytes / (S * L)),
                         "gbps": round(nbytes / (dur_ms.sum() / 1e3) / 1e9, 1)}
        log("kernel %-7s %8.2f us avg over %d launches, %7.1f GB/s algorithmic" % (
            sname, dur_ms.mean() * 1e3, S * L, stages[sname]["gbps"]))
    dom = max(stages, key=lambda k: stages[k]["avg_us"])
    achieved = stages[dom]["gbps"]

    # ---- CPU oracle baseline on a bounded sample (first tokens x all layers), one thread, plus a
    # parity spot check of the GPU outputs of the timed run on the same sample
    cpu, parity = None, None
    nt = min(args.cpu_tokens, K)
    if nt > 0:
        import oracle
        oracle.build()
        idx = torch.zeros(L, nt, cfg.ffn, dtype=torch.int32, device=dev)
        cn = torch.zeros(L, nt, dtype=torch.int32, device=dev)
        ychk = torch.empty(L, nt, cfg.d, dtype=torch.float32, device=dev)
        with torch.cuda.stream(stream):
            for t in range(nt):
                for l in range(L):
                    ffn.ffn_sparse_forward(plans[l], xp[l][t], 1, ychk[l, t].data_ptr(),
                                           idx=idx[l, t].data_ptr(), cnt=cn[l, t].data_ptr(),
                                           stream=sp)
        torch.cuda.synchronize()
        same = bool(torch.equal(ychk, y[:, :nt]))
        t_cpu, worst, flips = 0.0, 0.0, 0
        keys = ["w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down_t", "b_up", "b_gate",
                "b_down", "p1", "p2", "c1", "c2"]
        for l in range(L):
            OL = {k: (None if layers[l].get(k) is None else
                      np.ascontiguousarray(layers[l][k].cpu().numpy())) for k in keys}
            OL["act"], OL["tau"] = cfg.act, cfg.tau
            xh = x[l, :nt].cpu().numpy()
            for t in range(nt):
                c0 = time.perf_counter()
                yref, pred = oracle.sparse_token(OL, xh[t])
                t_cpu += time.perf_counter() - c0
                got = idx[l, t, :int(cn[l, t])].cpu().numpy()
                if not np.array_equal(got, pred["idx"]):
                    flips += 1
                    band = np.abs(pred["p"] - cfg.tau) <= 1e-4
                    assert np.array_equal(got[~band[got]], pred["idx"][~band[pred["idx"]]])
                    mask = np.zeros(cfg.ffn, np.uint8)
                    mask[got] = 1
                    yref, _ = oracle.ffn(OL, xh[t], mask)
                yg = y[l, t].cpu().numpy().astype(np.float64)
                worst = max(worst, float(np.max(np.abs(yg - yref)) / np.max(np.abs(yref))))
            del OL
        cpu = {"value": round(nt / t_cpu, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": "first %d token(s) x %d layers, predictor + FFN, single-threaded C, "
                         "fp64 accumulation (%.1f s)" % (nt, L, t_cpu)}
        parity = {"tokens": nt, "layers": L, "max_normwise_err": worst,
                  "band_flips": flips, "timed_outputs_reproduced": same}
        log("oracle: %.2f s for %d token(s); GPU parity max normwise error %.2e" % (
            t_cpu, nt, worst))

    result = {
        "metric": "sparse-FFN decode tokens/s at 1 GPU; effective HBM GB/s of touched weights",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16xf16->f32", "i4g32": "i4g32xf16->f32"}[cfg.w_dtype],
        "data": "synthetic (seeded; power-law hot set)",
        "config": {"workload": cfg.name, "d": cfg.d, "ffn": cfg.ffn, "rank": cfg.rank,
                   "act": cfg.act, "layers": L, "tokens": K, "batch": 1,
                   "target_density": cfg.density, "measured_density": round(density, 5)},
        "effective_gbps": round(eff_gbps, 1),
        "touched_bytes_per_token": int(touched / K),
        "roofline": {"bound": "hbm", "kernel": "k_" + dom,
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": profiled_traffic("k_" + dom, cfg.name),
                     "avg_us": stages[dom]["avg_us"],
                     "bytes_per_launch": stages[dom]["bytes_per_launch"]},
        "kernels": stages,
        "cpu_baseline": cpu,
        "parity_sample": parity,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
