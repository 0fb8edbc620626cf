#!/usr/bin/env python3
"""Benchmark of the activation-sparse FFN on one MI355X.

Default: decode of the Llama-2-7B-shaped ReGLU layer stack (d=4096, ffn=11008, predictor rank
256, fp16 weights, 32 layers, 512 tokens, batch 1), followed by short runs of every other workload
(each in a child process), summarised under "all_configs" in the one JSON line.  A step is one decode token through every
layer: per layer the predictor picks the token's active neurons and only their rows are read
(PowerInfer, unite.ai, "自适应稀疏预测器" / "神经元感知运算符").  Layers run one after another on one
stream, as in a real decode.  Other workloads: --config (the OPT-125m, Mistral-7B dReLU,
Mixtral-47B int4 mixture and Falcon-40B shaped ones), --batch N (decode steps of N tokens whose
active sets are united), --prefill N (N tokens per layer with the path chosen on the device:
the predictor's sets, their union density against the plan's crossover, and the dense MFMA GEMMs
above it).

Inputs are seeded synthetic tensors already resident in HBM; the timed region replays HIP graphs
of the library's launches.  Printed (one JSON line on stdout): tokens/s, the effective HBM
bandwidth over the bytes the method touches, the roofline of the dominant kernel (timed with
HIP events attached to its own dispatches), and the CPU oracle timed on the host as a baseline.
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published
CPU_BUDGET_S = 25.0            # CPU oracle sample: stop adding layers past this much CPU time


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def row_bytes(cfg) -> float:
    return {"f32": 4 * cfg.d, "f16": 2 * cfg.d, "i4g32": cfg.d // 2 + (cfg.d // 32) * 2}[cfg.w_dtype]


def n_rows(cfg) -> int:
    return 2 if cfg.act == "relu" else 3


def n_bias(cfg) -> int:
    return (1 if cfg.bias_up else 0) + (1 if (cfg.act != "relu" and cfg.bias_gate) else 0)


def pred_bytes(cfg, n_hot=0):
    """Predictor bytes per token-layer (per step-layer in a batch): stage 1 (P1), stage 2 (P2 and
    c2 of the predicted neurons: all but an always-active head of n_hot)."""
    pb = 4 if cfg.p_dtype == "f32" else 2
    nf = cfg.ffn - n_hot
    return cfg.rank * cfg.d * pb, nf * cfg.rank * pb + 4 * nf


def profiled_traffic(kernel: str, workload: str, with_trace: bool = False):
    """HBM bytes per launch of `kernel` on `workload` from a committed rocprofv3 summary under
    profiles/ (FETCH_SIZE + WRITE_SIZE, scaled against a copy of known size), or None when there
    is none or the kernel source has changed since the counters were taken.  with_trace: also
    the summary's kernel-trace mean duration in microseconds (or None), as a pair."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        lines = open(path).read().splitlines()
        for line in lines:
            f = line.split()
            if not f or f[0] != "traffic":
                continue
            kv = dict(t.split("=", 1) for t in f[1:] if "=" in t)
            if kv.get("kernel") != kernel or kv.get("workload") != workload:
                continue
            src = os.path.join(ROOT, kv["source"])
            if (not os.path.exists(src) or
                    hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("sha256")):
                return (None, None) if with_trace else None
            trace_us = None
            for ln in lines:
                if ln.startswith("- mean duration (kernel trace):"):
                    trace_us = float(ln.split(":", 1)[1].split()[0])
            nb = int(kv["bytes_per_launch"])
            return (nb, trace_us) if with_trace else nb
    return (None, None) if with_trace else None


def profiled_mfma_busy(kernel: str, workload: str):
    """MFMA utilisation (a fraction) of `kernel` on `workload` from the busy-cycle counter pass
    in its committed rocprofv3 summary (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCD x
    1024 SIMDs), or None when the summary has no such pass or its kernel source has changed."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        lines = open(path).read().splitlines()
        tl = [ln.split() for ln in lines if ln.split()[:1] == ["traffic"]]
        kv = next((dict(t.split("=", 1) for t in f[1:] if "=" in t) for f in tl), None)
        if kv is None or kv.get("kernel") != kernel or kv.get("workload") != workload:
            continue
        src = os.path.join(ROOT, kv["source"])
        if (not os.path.exists(src) or
                hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("sha256")):
            return None
        for ln in lines:
            m = re.match(r"- MFMA utilisation .*\*\*([0-9.]+)%\*\*", ln)
            if m:
                return round(float(m.group(1)) / 100.0, 4)
        return None
    return None


HEADLINE = "llama2_7b_reglu_f16"

# The other workloads of the default run: (workload, extra arguments).  Short step counts keep
# the whole default run within a few minutes; each checks its timed outputs against the oracle
# on a few (layer, token) pairs.
OTHERS = [
    # the OPT-125m-shaped layer is launch-bound: the fused variant's three launches beat the
    # balanced four there (measured 95.3 k against 88.7 k tokens/s)
    ("opt125m_relu_f32", ["--steps", "256", "--parity-pairs", "0", "--decode-variant", "1"]),
    ("turbosparse_mistral_7b_drelu_f16", ["--steps", "64"]),
    ("turbosparse_mixtral_47b_moe_int4", ["--steps", "64"]),
    ("falcon_40b_relu_f16", ["--steps", "32"]),
    ("falcon_40b_relu_f16", ["--batch", "8", "--steps", "8"]),
    ("falcon_40b_relu_f16", ["--batch", "32", "--steps", "4"]),
    ("falcon_40b_relu_f16", ["--prefill", "512", "--steps", "2"]),
    ("falcon_40b_relu_f16", ["--prefill", "512", "--steps", "2", "--prefill-path", "dense"]),
    # attention blocks with a head-level active set (a token at position 511 of a 512 context)
    ("llama2_7b_attn_f16", ["--steps", "64"]),
    ("mistral_7b_attn_f16", ["--steps", "64"]),
    ("llama2_7b_attn_f16", ["--steps", "32", "--context", "8191"]),
    ("falcon_40b_attn_f16", ["--steps", "16"]),
]


def summarise(r: dict) -> dict:
    """The fields of one workload's JSON line kept in the default run's summary."""
    roof, par, c = r.get("roofline") or {}, r.get("parity_sample") or {}, r["config"]
    out = {"workload": c["workload"], "mode": c["mode"], "tokens_per_call": c["tokens_per_call"],
           "path": c.get("path"), "layers": c["layers"], "tokens_per_s": r["value"],
           "ms_per_step": r["ms_per_step"], "effective_gbps": r.get("effective_gbps"),
           "measured_density": c.get("measured_density"),
           "dominant_kernel": roof.get("kernel"), "bound": roof.get("bound"),
           "achieved": roof.get("achieved"), "unit": roof.get("unit"), "frac": roof.get("frac"),
           "traffic": roof.get("traffic"), "mfma_busy": roof.get("mfma_busy"),
           "parity": {k: par.get(k) for k in ("pairs", "max_normwise_err", "tolerance",
                                              "within_tolerance")} if par else None}
    if r.get("prefill_path"):
        out["prefill_path"] = r["prefill_path"]
    return out


def run_others() -> list:
    """Short runs of the other workloads, one child process each (so that each starts with the
    GPU memory of its own inputs only); a failed run is recorded with its error."""
    import subprocess
    out = []
    for name, extra in OTHERS:
        cmd = [sys.executable, os.path.abspath(__file__), "--config", name, "--warmup", "2",
               "--kernel-sample", "8", "--cpu-tokens", "1", "--cpu-budget", "2",
               "--parity-pairs", "2"] + extra
        log("other workload: %s %s" % (name, " ".join(extra)))
        t0 = time.time()
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=400)
            lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
            if r.returncode != 0 or not lines:
                raise RuntimeError("exit %d: %s" % (r.returncode, r.stderr.strip()[-400:]))
            rec = summarise(json.loads(lines[-1]))
        except Exception as e:  # recorded, the default line is still printed
            rec = {"workload": name, "args": extra, "error": str(e)[-500:]}
        rec["wall_s"] = round(time.time() - t0, 1)
        log("  -> %s" % json.dumps(rec)[:300])
        out.append(rec)
    return out


def copy_calibration(mib: int, dev):
    """Five device-to-device copies of `mib` MiB: the known-size kernel that the HBM byte
    counters of a profiled run are scaled against."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 5 x %d MiB device-to-device" % mib)
    del src, dst


def run_attn(args):
    """Decode of a stack of attention blocks with a head-level active set: a step is one token
    at the context's last position through every block (predictor, key / value rows of every
    head into the cache, the active heads' query rows, scores over the cache and output rows).
    Prints the same JSON line as the FFN workloads."""
    import numpy as np
    import torch

    import activation_sparse_ffn_gemv_amd as ffn
    import synth

    cfg = synth.ATTN_CONFIGS[args.config]
    if args.batch != 1 or args.prefill or args.offload or args.hot_head or args.fit_recall:
        raise SystemExit("attention blocks are measured at batch-1 decode (no batch, prefill, "
                         "offload, hot head or predictor fit)")
    if args.context:
        import dataclasses
        cfg = dataclasses.replace(cfg, context=args.context, max_seq=0)
    wl = cfg.name if not args.context else "%s:ctx%d" % (cfg.name, cfg.context)
    L = args.layers or cfg.layers
    K = args.steps if args.steps else 64
    W = min(args.warmup, K)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d, H, G, e, r, pos = cfg.d, cfg.heads, cfg.kv_heads, cfg.head_dim, cfg.rank, cfg.context
    log("attention %s: d=%d heads=%d kv_heads=%d head_dim=%d rank=%d position=%d layers=%d "
        "steps=%d" % (cfg.name, d, H, G, e, r, pos, L, K))
    if args.copy_mib:
        copy_calibration(args.copy_mib, dev)
    t0 = time.time()
    layers = [synth.make_attn_layer(cfg, layer=l, device=dev) for l in range(L)]
    caches = [synth.make_kv_cache(cfg, layer=l, device=dev) for l in range(L)]
    x = torch.stack([synth.make_attn_tokens(cfg, K, layer=l, device=dev) for l in range(L)])
    y = torch.empty(L, K, d, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("inputs generated on the GPU in %.1f s" % (time.time() - t0))
    stream = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream
    mods = [ffn.SparseAttention(layers[l], max_seq=cfg.seq) for l in range(L)]
    xb = 2 * d

    def call(l, t, **kw):
        ffn.ffn_attn_forward(mods[l].plan, x[l].data_ptr() + t * xb, pos, caches[l][0].data_ptr(),
                             caches[l][1].data_ptr(), y[l, t].data_ptr(), stream=sp, **kw)

    # bytes the method touches per (layer, step), from each call's |A| (untimed counting pass)
    cnt = torch.zeros(L, K, dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for t in range(K):
            for l in range(L):
                call(l, t, cnt=cnt[l].data_ptr() + 4 * t)
    torch.cuda.synchronize()
    n_act = cnt.cpu().numpy().astype(np.float64)
    b_pz = r * d * 2 + d * 2
    b_proj_fixed = H * r * 2 + H * 4 + 2 * G * e * d * 2 + 2 * G * e * 2  # P2, c2, K/V rows+writes
    b_q = e * d * 2                                                     # per active head
    b_cache = (pos + 1) * e * 2 * 2                                     # per active head
    b_o = e * d * 2                                                     # per active head
    touched = b_pz + b_proj_fixed + n_act * (b_q + b_cache + b_o)
    density = float(n_act.mean() / H)
    log("measured head density %.4f (mean |A| = %.2f of %d)" % (density, n_act.mean(), H))

    gsteps = max(1, min(K, 256 // L))
    graphs = []
    with torch.cuda.stream(stream):
        for g0 in range(0, K, gsteps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(g0, min(K, g0 + gsteps)):
                    for l in range(L):
                        call(l, t)
            graphs.append(g)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for g in graphs[:max(1, (W + gsteps - 1) // gsteps)]:
            g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for g in graphs:
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    tok_s = K / (ms / 1e3)
    eff_gbps = touched.sum() / (ms / 1e3) / 1e9
    log("timed %d step(s): %.3f ms/step, %.1f tokens/s, %.1f GB/s effective over touched bytes"
        % (K, ms / K, tok_s, eff_gbps))

    # per-kernel durations: plain launches of the sampled steps with HIP events on one stage's
    # dispatches (on the stream they run on)
    S = min(args.kernel_sample, K)
    per_call = touched[:, :S].sum() / (L * S)
    na = float(n_act[:, :S].mean())
    kinds = [("pred_z", ffn.FFN_STAGE_PRED_Z, b_pz),
             ("attn_proj", ffn.FFN_STAGE_ATTN_PROJ, b_proj_fixed + na * b_q),
             ("attn_scores", ffn.FFN_STAGE_ATTN_SCORES, na * b_cache),
             ("attn_out", ffn.FFN_STAGE_ATTN_OUT, na * b_o),
             ("attn_reduce", ffn.FFN_STAGE_ATTN_REDUCE, 0.0)]
    assert abs(sum(k[2] for k in kinds) - per_call) < 1e-6 * per_call
    stages = {}
    for sname, sid, nb in kinds:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(S * L)]
        with torch.cuda.stream(stream):
            for a, b in evs:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i, (a, b) in enumerate(evs):
                l, t = i % L, i // L
                ffn.ffn_attn_set_timing_events(mods[l].plan, sid, a.cuda_event, b.cuda_event)
                call(l, t)
        torch.cuda.synchronize()
        for m in mods:
            ffn.ffn_attn_set_timing_events(m.plan, sid, 0, 0)
        dur = np.array([a.elapsed_time(b) for a, b in evs])
        stages[sname] = {"avg_us": round(float(dur.mean()) * 1e3, 3), "bytes_per_launch": int(nb),
                         "gbps": round(nb / (dur.mean() / 1e3) / 1e9, 1)}
        log("kernel %-13s %9.2f us avg over %d launches  %.1f GB/s algorithmic" % (
            sname, dur.mean() * 1e3, len(dur), stages[sname]["gbps"]))
    knames = {"pred_z": "k_pred_z", "attn_proj": "k_attn_proj", "attn_scores": "k_attn_part",
              "attn_out": "k_attn_out", "attn_reduce": "k_attn_reduce"}
    movers = [k for k in stages if stages[k]["bytes_per_launch"] > 0]
    dom = max(movers, key=lambda k: stages[k]["avg_us"])
    prof = profiled_traffic(knames[dom], wl, with_trace=True)
    roof = {"bound": "hbm", "kernel": knames[dom], "achieved": stages[dom]["gbps"],
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(stages[dom]["gbps"] / HBM_PEAK_GBPS, 4), "traffic": prof[0],
            "trace_avg_us": prof[1], "avg_us": stages[dom]["avg_us"],
            "bytes_per_launch": stages[dom]["bytes_per_launch"]}

    # CPU oracle on a bounded sample, and parity of the timed outputs on (layer, token) pairs:
    # the oracle's cache is the generator's with position `pos` holding the token's own key and
    # value, which is the state every timed step saw
    cpu, parity = None, None
    nt = min(args.cpu_tokens, K)
    if nt > 0:
        import oracle
        oracle.build()
        keys = ["w_q", "w_k", "w_v", "w_o_t", "p1", "p2", "c1", "c2"]

        def host(l):
            OL = {k: (None if layers[l].get(k) is None else
                      np.ascontiguousarray(layers[l][k].cpu().numpy())) for k in keys}
            OL.update(tau=cfg.tau, head_dim=e)
            # the device caches: positions below pos are the generator's, untouched by the run
            Kh, Vh = (np.ascontiguousarray(c.cpu().numpy()) for c in caches[l])
            return OL, Kh, Vh

        t_cpu, L_cpu = 0.0, 0
        for l in range(L):
            OL, Kh, Vh = host(l)
            xh = x[l, :nt].cpu().numpy()
            for t in range(nt):
                c0 = time.perf_counter()
                oracle.attn_token(OL, Kh, Vh, xh[t], pos)
                t_cpu += time.perf_counter() - c0
            L_cpu = l + 1
            if t_cpu > args.cpu_budget:
                break
        rate = nt * L_cpu / t_cpu / L
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                                  if ln.startswith("model name")), "")
        except OSError:
            pass
        cpu = {"value": round(rate, 5), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": "first %d token(s) x %d of %d blocks, head predictor + attention block, "
                         "single-threaded C with fp64 accumulation (%.1f s of CPU), scaled to all "
                         "blocks" % (nt, L_cpu, L, t_cpu),
               "s_per_token": round(1.0 / rate, 3),
               "host": {"cpu_model": cpu_model, "logical_cpus": os.cpu_count()}}
        rng = np.random.default_rng(cfg.seed)
        pairs = sorted({(0, t) for t in range(nt)} |
                       {(int(l), int(t)) for l, t in zip(rng.integers(0, L, args.parity_pairs),
                                                         rng.integers(0, K, args.parity_pairs))})
        worst = 0.0
        ie = torch.zeros(H, dtype=torch.int32, device=dev)
        ce = torch.zeros(1, dtype=torch.int32, device=dev)
        yy = torch.zeros(d, dtype=torch.float32, device=dev)
        for l, t in pairs:
            OL, Kh, Vh = host(l)
            yg = y[l, t].cpu().numpy().astype(np.float64)          # from the timed run
            ffn.ffn_attn_forward(mods[l].plan, x[l].data_ptr() + t * xb, pos,
                                 caches[l][0].data_ptr(), caches[l][1].data_ptr(),
                                 yy.data_ptr(), idx=ie.data_ptr(), cnt=ce.data_ptr(), stream=sp)
            torch.cuda.synchronize()
            mk = np.zeros(H, np.uint8)
            mk[ie[:int(ce[0])].cpu().numpy()] = 1
            yref, _, _, _ = oracle.attn_token(OL, Kh, Vh, x[l, t].cpu().numpy(), pos, mk)
            worst = max(worst, float(np.max(np.abs(yg - yref)) / np.max(np.abs(yref))))
        parity = {"pairs": len(pairs), "layers": sorted({l for l, _ in pairs}),
                  "max_normwise_err": worst, "tolerance": 2e-3, "within_tolerance": worst <= 2e-3}
        log("oracle: %.2f s for %d token(s) x %d block(s); GPU parity over %d pairs: max "
            "normwise error %.2e" % (t_cpu, nt, L_cpu, len(pairs), worst))

    result = {
        "metric": "sparse-attention decode tokens/s at 1 GPU (head-level active set); effective "
                  "HBM GB/s of touched bytes",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms / K, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16xf16->f32",
        "data": "synthetic (seeded; cache of the context drawn at the projections' spread)",
        "config": {"workload": wl, "mode": "decode", "tokens_per_call": 1, "d": d,
                   "path": "sparse", "heads": H, "kv_heads": G, "head_dim": e, "rank": r,
                   "position": pos, "layers": L, "target_density": cfg.density,
                   "measured_density": round(density, 5)},
        "effective_gbps": round(eff_gbps, 1),
        "touched_bytes_per_step": int(touched.sum() / K),
        "roofline": roof, "kernels": stages, "cpu_baseline": cpu, "parity_sample": parity,
    }
    print(json.dumps(result), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's token count / batch)")
    ap.add_argument("--warmup", type=int, default=16, help="untimed steps replayed first")
    ap.add_argument("--config", default=None,
                    help="one workload (default: the Llama-2-shaped stack, then short runs of "
                         "the others); the *_attn_* names run attention blocks")
    ap.add_argument("--no-others", action="store_true",
                    help="default workload only: skip the short runs of the other workloads")
    ap.add_argument("--batch", type=int, default=1, help="tokens per decode step (union path)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="tokens per layer in one call (prefill) instead of decode")
    ap.add_argument("--prefill-path", choices=("auto", "dense"), default="auto",
                    help="prefill calls: 'auto' = ffn_sparse_forward with FFN_PATH_AUTO (the "
                         "predictor's sets, the device's choice by union density, per-token "
                         "masks); 'dense' = ffn_dense_forward (the dense FFN, no predictor)")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0: all)")
    ap.add_argument("--context", type=int, default=0,
                    help="attention blocks: the token's position (its context length; 0: 511)")
    ap.add_argument("--kernel-sample", type=int, default=32,
                    help="steps whose kernel launches are timed with dispatch events")
    ap.add_argument("--parity-pairs", type=int, default=8,
                    help="seeded random (layer, token) pairs beyond layer 0 whose timed-run "
                         "outputs are checked against the oracle (prefill: at most 2)")
    ap.add_argument("--parity-stack-tokens", type=int, default=0,
                    help="also check the first N tokens at every layer of the stack")
    ap.add_argument("--cpu-tokens", type=int, default=3,
                    help="tokens the CPU oracle baseline runs per layer; 0 = skip")
    ap.add_argument("--decode-variant", type=int, default=None,
                    help="batch-1 decode variant for every plan (0 balanced, 1 fused); "
                         "default: the library's")
    ap.add_argument("--hot-head", action="store_true",
                    help="order each layer's neurons hottest first (the generator's firing "
                         "probabilities stand in for a profile) and keep the capped head always "
                         "active; only the rest is predicted")
    ap.add_argument("--spectrum-alpha", type=float, default=0.0,
                    help="shape the predictor's source matrix to singular values ~ k^-alpha")
    ap.add_argument("--fit-recall", type=float, default=0.0,
                    help="replace each layer's predictor by a least-squares fit whose rank is the "
                         "smallest (step 32) with this expected recall")
    ap.add_argument("--fit-margin", type=float, default=0.0,
                    help="recall margin of the fitted predictors (residual standard deviations)")
    ap.add_argument("--offload", type=int, default=0,
                    help="keep each layer's up/gate/down rows in pinned host memory behind a "
                         "neuron cache of this many slots per layer (fp16 decode workloads)")
    ap.add_argument("--pin", type=int, default=0,
                    help="with --offload: neurons [0, N) stay in the cache for good (use with "
                         "--hot-head and N = the head)")
    ap.add_argument("--calibrate", type=int, default=0,
                    help="also calibrate layer 0's plan for batches up to this size and report "
                         "its measured crossover densities (fp16 layers)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB five times (a known "
                         "size against which a profiler's HBM byte counters are scaled)")
    ap.add_argument("--cpu-budget", type=float, default=CPU_BUDGET_S,
                    help="seconds of CPU time after which the oracle baseline stops adding layers")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the operator "
              "would shard by neurons, see the design notes); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_sparse_ffn_gemv_amd as ffn
    import synth

    if args.config in synth.ATTN_CONFIGS:
        return run_attn(args)
    others = args.config is None and not args.no_others
    cfg = synth.CONFIGS[args.config or HEADLINE]
    if args.spectrum_alpha > 0:
        cfg = synth.with_(cfg, spectrum_alpha=args.spectrum_alpha)
    L = args.layers or cfg.layers
    moe = cfg.n_experts > 1
    prefill = args.prefill > 0
    Bt = args.prefill if prefill else args.batch      # tokens per layer call
    if moe and (Bt != 1 or prefill):
        raise SystemExit("the mixture workload is measured at batch-1 decode")
    if args.hot_head and (moe or prefill):
        raise SystemExit("--hot-head applies to the single-layer decode workloads")
    if args.offload and (moe or prefill or Bt != 1 or cfg.w_dtype != "f16"):
        raise SystemExit("--offload applies to the fp16 single-layer workloads at batch 1")
    # batch-1 decode with the fused predictor-stage-2 + gather kernel (the plans' variant 1)
    fused = args.decode_variant == 1 and Bt == 1 and not (moe or prefill or args.offload)
    K = args.steps if args.steps else (4 if prefill else max(1, cfg.tokens // Bt))
    W = min(args.warmup, K)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    mode = "prefill" if prefill else "decode"
    log("config %s (%s, %d token(s) per call): d=%d ffn=%d rank=%d act=%s w=%s layers=%d "
        "steps=%d" % (cfg.name, mode, Bt, cfg.d, cfg.ffn, cfg.rank, cfg.act, cfg.w_dtype, L, K))

    if args.copy_mib:
        copy_calibration(args.copy_mib, dev)

    # ---- inputs, resident in HBM
    t0 = time.time()
    E = cfg.n_experts
    layers = [[synth.make_layer(cfg, layer=l, expert=e, device=dev) for e in range(E)]
              for l in range(L)]
    fitq = None
    if args.fit_recall > 0:
        if moe or prefill:
            raise SystemExit("--fit-recall applies to the single-layer decode workloads")
        from synth import fit
        t1 = time.time()
        fitq = []
        for row in layers:
            V = fit.spectrum(row[0])[0]
            r, q = fit.choose_rank(row[0], args.fit_recall, margin=args.fit_margin, step=32,
                                   basis=V)
            row[0] = fit.fit_predictor(row[0], r, margin=args.fit_margin, basis=V)
            fitq.append((r,) + tuple(q))
            del V
        fitq = np.array(fitq)
        log("fitted predictors in %.1f s: rank per layer %s; expected recall %.3f precision %.3f"
            % (time.time() - t1, fitq[:, 0].astype(int).tolist(), fitq[:, 1].mean(),
               fitq[:, 2].mean()))
    ranks = np.array([row[0]["p1"].shape[0] for row in layers], np.float64)[:, None]
    n_hot = 0
    if args.hot_head:
        layers = [[synth.hot_first(le) for le in row] for row in layers]
        n_hot = synth.hot_head_size(layers[0][0])
        for row in layers:
            for le in row:
                le["n_hot"] = n_hot
    routers = [synth.make_router(cfg, layer=l, device=dev) for l in range(L)] if moe else None
    x = torch.stack([synth.make_tokens(cfg, K * Bt, layer=l, device=dev) for l in range(L)])
    y = torch.empty(L, K * Bt, cfg.d, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("inputs generated on the GPU in %.1f s" % (time.time() - t0))

    stream = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream
    with torch.cuda.stream(stream):
        if args.offload:
            # rows to pinned host memory; each layer's cache (and its state) in its own workspace
            t1 = time.time()
            for row in layers:
                for k in ("w_up", "w_gate", "w_down_t"):
                    if row[0].get(k) is not None:
                        row[0][k] = row[0][k].cpu().pin_memory()
            torch.cuda.empty_cache()
            mods = [[ffn.OffloadFFN(layers[l][0], args.offload, n_pinned=args.pin)]
                    for l in range(L)]
            log("rows of %d layers in pinned host memory (%.1f s); %d-slot cache per layer, %d "
                "pinned" % (L, time.time() - t1, args.offload, args.pin))
        else:
            probe = ffn.SparseFFN(layers[0][0], max_batch=Bt)
            ws = torch.empty(probe.ws_bytes, dtype=torch.uint8, device=dev)   # one, shared
            probe.close()
            mods = [[ffn.SparseFFN(layers[l][e], max_batch=Bt, workspace=ws) for e in range(E)]
                    for l in range(L)]
        moes = None
        if moe:
            n = ffn.ffn_moe_workspace_size(E, cfg.top_k, mods[0][0].plan)
            mws = torch.empty(n, dtype=torch.uint8, device=dev)
            moes = [ffn.ffn_moe_plan(E, cfg.top_k, routers[l].data_ptr(),
                                     [m.plan for m in mods[l]], mws.data_ptr(), n)
                    for l in range(L)]
    plans = [m.plan for row in mods for m in row]
    if args.decode_variant is not None:
        for q in plans:
            ffn.ffn_plan_set_decode_variant(q, args.decode_variant)
    xb = x.element_size() * cfg.d
    xp = [[x[l].data_ptr() + t * Bt * xb for t in range(K)] for l in range(L)]
    yp = [[y[l].data_ptr() + t * Bt * cfg.d * 4 for t in range(K)] for l in range(L)]

    auto_prefill = prefill and args.prefill_path == "auto"

    def call(l, t, **kw):
        if prefill and not auto_prefill:
            ffn.ffn_dense_forward(mods[l][0].plan, xp[l][t], Bt, yp[l][t], stream=sp)
        elif prefill:
            ffn.ffn_sparse_forward(mods[l][0].plan, xp[l][t], Bt, yp[l][t],
                                   path=ffn.FFN_PATH_AUTO, stream=sp, **kw)
        elif moe:
            ffn.ffn_moe_forward(moes[l], xp[l][t], 1, yp[l][t], stream=sp, **kw)
        else:
            ffn.ffn_sparse_forward(mods[l][0].plan, xp[l][t], Bt, yp[l][t],
                                   path=ffn.FFN_PATH_SPARSE, stream=sp, **kw)

    def step(t):
        for l in range(L):
            call(l, t)

    # ---- bytes the method touches per (layer, step): an untimed counting pass
    pz, ps = pred_bytes(cfg, n_hot)
    pz, ps = pz * ranks / cfg.rank, ps * ranks / cfg.rank       # [L][1]: each layer's own rank
    rowb = n_rows(cfg) * row_bytes(cfg) + 4 * n_bias(cfg)
    router_b = cfg.n_experts * cfg.d * 2 if moe else 0
    path_chosen = None
    if prefill:
        # every row once per call (plus, on the AUTO path, the predictor once per call)
        touched = np.full((L, K), float(cfg.ffn * rowb)) + ((pz + ps) if auto_prefill else 0.0)
        density = 1.0
        if auto_prefill:
            # the device's choice at every layer (each layer's call, then its plan's flag)
            ch = []
            with torch.cuda.stream(stream):
                for l in range(L):
                    call(l, 0)
                    stream.synchronize()
                    ch.append(mods[l][0].last_auto_path())
            n_dense = ch.count("dense")
            path_chosen = {"dense_layers": n_dense, "layers": L,
                           "crossover_density": round(mods[0][0].crossover(Bt), 4),
                           "path": "dense" if n_dense == L else "sparse" if n_dense == 0
                           else "mixed"}
            log("AUTO prefill: the device chose the dense GEMMs at %d of %d layers (crossover "
                "density %.4f for %d tokens)" % (n_dense, L, path_chosen["crossover_density"], Bt))
    elif moe:
        # the mixture's own calls report each chosen expert's |A| (the launches the bench times)
        ids = torch.zeros(L, K, cfg.top_k, dtype=torch.int32, device=dev)
        cnt = torch.zeros(L, K, cfg.top_k, dtype=torch.int32, device=dev)
        with torch.cuda.stream(stream):
            for t in range(K):
                for l in range(L):
                    call(l, t, expert_idx=ids[l, t].data_ptr(), expert_cnt=cnt[l, t].data_ptr())
        torch.cuda.synchronize()
        cnt_h = cnt.cpu().numpy().astype(np.float64)
        touched = router_b + cfg.top_k * (pz + ps) + cnt_h.sum(axis=2) * rowb
        density = float(cnt_h.mean() / cfg.ffn)
        log("measured density %.4f over the chosen experts" % density)
    elif Bt == 1:
        cnt = torch.zeros(L, K, dtype=torch.int32, device=dev)
        with torch.cuda.stream(stream):
            for t in range(K):
                for l in range(L):
                    call(l, t, cnt=cnt[l].data_ptr() + 4 * t)
        torch.cuda.synchronize()
        cnt_h = cnt.cpu().numpy().astype(np.float64)
        touched = pz + ps + cnt_h * rowb
        density = float(cnt_h.mean() / cfg.ffn)
        log("measured density %.4f (mean |A| = %.1f of %d)" % (density, cnt_h.mean(), cfg.ffn))
    else:
        F = cfg.ffn
        union = np.zeros((L, K))
        idx = torch.zeros(Bt, F, dtype=torch.int32, device=dev)
        cnt = torch.zeros(Bt, dtype=torch.int32, device=dev)
        ar = torch.arange(F, device=dev)
        per_tok = []
        for t in range(K):
            for l in range(L):
                with torch.cuda.stream(stream):
                    call(l, t, idx=idx.data_ptr(), cnt=cnt.data_ptr())
                stream.synchronize()
                valid = ar[None, :] < cnt[:, None].long()
                m = torch.zeros(Bt, F, dtype=torch.bool, device=dev)
                m.scatter_(1, torch.where(valid, idx.long(), 0), valid)
                union[l, t] = float(m.any(dim=0).sum())
                per_tok.append(float(cnt.float().mean()))
        touched = pz + ps + union * rowb
        density = float(np.mean(per_tok) / F)
        log("measured per-token density %.4f, union density %.4f" % (
            density, union.mean() / F))
    torch.cuda.synchronize()

    # ---- predictor quality on a few tokens of every layer: the kernels' sets against the true
    # sets (h != 0, from the source pre-activations computed here in float64 for measurement)
    quality = None
    if not prefill and not moe and Bt == 1:
        from synth import fit as sfit
        ns = min(K, 8)
        qi = torch.zeros(ns, cfg.ffn, dtype=torch.int32, device=dev)
        qc = torch.zeros(ns, dtype=torch.int32, device=dev)
        ar = torch.arange(cfg.ffn, device=dev)
        tp = npred = ntrue = 0
        for l in range(L):
            with torch.cuda.stream(stream):
                for t in range(ns):
                    call(l, t, idx=qi[t].data_ptr(), cnt=qc[t].data_ptr())
            torch.cuda.synchronize()
            valid = ar[None, :] < qc[:, None].long()
            pm = torch.zeros(ns, cfg.ffn, dtype=torch.bool, device=dev)
            pm.scatter_(1, torch.where(valid, qi.long(), 0), valid)
            xs = x[l, :ns].double()
            w_src, b_src = sfit.source(layers[l][0])
            tm = (xs @ w_src.to(dev).T + b_src.to(dev)) > 0
            if cfg.act == "drelu":
                w_u, b_u = sfit.source(dict(layers[l][0], act="relu"))
                tm &= (xs @ w_u.to(dev).T + b_u.to(dev)) > 0
            del w_src
            tp += int((pm & tm).sum())
            npred += int(pm.sum())
            ntrue += int(tm.sum())
        quality = {"tokens": ns, "measured_recall": round(tp / max(ntrue, 1), 4),
                   "measured_precision": round(tp / max(npred, 1), 4),
                   "rank_per_layer": ranks[:, 0].astype(int).tolist()}
        if fitq is not None:
            quality.update(expected_recall=round(float(fitq[:, 1].mean()), 4),
                           expected_precision=round(float(fitq[:, 2].mean()), 4),
                           fit_target_recall=args.fit_recall, fit_margin=args.fit_margin)
        log("predictor on %d token(s) x %d layers: recall %.3f, precision %.3f" % (
            ns, L, quality["measured_recall"], quality["measured_precision"]))

    # ---- HIP graphs of whole steps (all layers)
    G = 1 if prefill else max(1, min(K, 256 // L))
    graphs = []
    with torch.cuda.stream(stream):
        for g0 in range(0, K, G):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(g0, min(K, g0 + G)):
                    step(t)
            graphs.append(g)
    torch.cuda.synchronize()
    log("captured %d graph(s) of %d step(s)" % (len(graphs), G))
    with torch.cuda.stream(stream):
        for g in graphs[:max(1, (W + G - 1) // G)]:
            g.replay()
    torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    tot0 = [m[0].tables()[3][4:].double() for m in mods] if args.offload else None
    with torch.cuda.stream(stream):
        e0.record(stream)
        for g in graphs:
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    offload = None
    if args.offload:
        # cache counters over the timed steps (running totals, modulo 2^32)
        dt = sum((m[0].tables()[3][4:].double() - t0v) % 2.0 ** 32 for m, t0v in zip(mods, tot0))
        hits, misses, adm, act = [float(v) for v in dt]
        pcie = misses * (n_rows(cfg) * row_bytes(cfg))
        offload = {"capacity": args.offload, "pinned": args.pin,
                   "hit_rate": round(hits / max(act, 1.0), 4),
                   "admitted_per_token_layer": round(adm / (K * L), 2),
                   "pcie_bytes_per_token": int(pcie / K),
                   "pcie_gbps": round(pcie / (ms / 1e3) / 1e9, 2)}
        log("cache: hit rate %.4f, %.1f MB per token over PCIe (%.1f GB/s)" % (
            offload["hit_rate"], pcie / K / 1e6, offload["pcie_gbps"]))
    tok_s = K * Bt / (ms / 1e3)
    eff_gbps = touched.sum() / (ms / 1e3) / 1e9
    log("timed %d step(s): %.3f ms/step, %.1f tokens/s, %.1f GB/s effective over touched bytes"
        % (K, ms / K, tok_s, eff_gbps))

    # ---- per-kernel durations: plain launches of the sampled steps with HIP events attached to
    # the dispatches of one stage's kernel (on the stream they run on)
    S = min(args.kernel_sample, K)
    passes = 1 if (prefill or Bt == 1) else (Bt + 31) // 32
    if prefill:
        kinds = [("dense_up", ffn.FFN_STAGE_DENSE_UP,
                  2.0 * Bt * cfg.d * cfg.ffn * (1 if cfg.act == "relu" else 2)),
                 ("dense_down", ffn.FFN_STAGE_DENSE_DOWN, 2.0 * Bt * cfg.d * cfg.ffn)]
    elif Bt > 1:
        kinds = [("batch_upgate", ffn.FFN_STAGE_BATCH_UPGATE, None),
                 ("batch_down", ffn.FFN_STAGE_BATCH_DOWN, None)]
    elif fused:
        # the fused variant: predictor stage 2 and the gather are one kernel (timed as the gather
        # stage), so there is no stage-2 launch to time
        kinds = [("pred_z", ffn.FFN_STAGE_PRED_Z, None), ("fused", ffn.FFN_STAGE_GATHER, None),
                 ("reduce", ffn.FFN_STAGE_REDUCE, None)]
    else:
        kinds = [(n, i, None) for i, n in enumerate(ffn.STAGES)]
    stages = {}
    for sname, sid, flops in kinds:
        n_launch = S * L
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_launch)]
        with torch.cuda.stream(stream):
            for a, b in evs:              # materialise the events
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(n_launch):
                l, t = i % L, i // L
                a, b = evs[i]
                for m in mods[l]:
                    ffn.ffn_plan_set_timing_events(m.plan, sid, a.cuda_event, b.cuda_event)
                call(l, t)
        torch.cuda.synchronize()
        for q in plans:
            ffn.ffn_plan_set_timing_events(q, sid, 0, 0)
        dur = np.array([a.elapsed_time(b) for a, b in evs])      # ms, last launch of each call
        rec = {"avg_us": round(float(dur.mean()) * 1e3, 3)}
        if flops is not None:
            rec["tflops"] = round(flops / (dur.mean() / 1e3) / 1e12, 1)
            rec["flops_per_launch"] = flops
        else:
            per_call = touched[:, :S].sum() / (L * S)
            k = cfg.top_k if moe else 1
            pzm, psm = float(pz.mean()), float(ps.mean())
            if sname == "pred_z":
                # the slots run side by side; a mixture's stage 1 runs in the router's launch
                # (the algorithmic bytes: the router and the chosen experts' P1)
                nb = pzm * k + router_b
            elif sname == "pred_s":
                nb = psm * k
            elif sname == "gather":
                nb = per_call - router_b - k * (pzm + psm)           # all expert slots' rows
            elif sname == "fused":
                nb = per_call - pzm                                  # P2 and c2, and the rows
            elif sname == "reduce":
                nb = 0.0
            else:
                rows_u = (per_call - pzm - psm) / rowb / passes       # union rows per pass
                nb = rows_u * (n_rows(cfg) - 1 if sname == "batch_upgate" else 1) * row_bytes(cfg)
            rec["bytes_per_launch"] = int(nb)
            rec["gbps"] = round(nb / (dur.mean() / 1e3) / 1e9, 1)
        stages[sname] = rec
        log("kernel %-13s %9.2f us avg over %d launches  %s" % (
            sname, dur.mean() * 1e3, len(dur),
            ("%.1f TFLOP/s" % rec["tflops"]) if "tflops" in rec else
            ("%.1f GB/s algorithmic" % rec["gbps"])))
    # the dominant kernel: the longest of those that move the method's bytes (or flops); a
    # reduction of partial sums moves none, so it is never the roofline's kernel
    movers = [k for k in stages if stages[k].get("bytes_per_launch", 1) > 0]
    dom = max(movers or list(stages), key=lambda k: stages[k]["avg_us"])
    knames = {"pred_z": "k_pred_z", "pred_s": "k_pred_s", "gather": "k_gather", "fused": "k_fused",
              "reduce": "k_reduce", "batch_upgate": "k_bug", "batch_down": "k_bdown",
              # rows in whole 32-wide K stages take the LDS-copy up projection
              "dense_up": "k_dupq" if cfg.d % 32 == 0 else "k_dup",
              # 256-token tiles where they pad the tokens no more than 128-token ones
              "dense_down": ("k_ddq" if (Bt + 255) // 256 * 256 == (Bt + 127) // 128 * 128
                             else "k_ddown")}
    if prefill:
        prof = profiled_traffic(knames[dom], cfg.name + ":prefill%d" % Bt, with_trace=True)
        roof = {"bound": "mfma", "kernel": knames[dom], "achieved": stages[dom]["tflops"],
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(stages[dom]["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": prof[0], "trace_avg_us": prof[1],
                "mfma_busy": profiled_mfma_busy(knames[dom], cfg.name + ":prefill%d" % Bt),
                "avg_us": stages[dom]["avg_us"],
                "flops_per_launch": stages[dom]["flops_per_launch"]}
    else:
        wl = ((cfg.name if Bt == 1 else cfg.name + ":batch%d" % Bt) + (":hot" if n_hot else "")
              + (":fit" if fitq is not None or cfg.spectrum_alpha else "")
              + (":offload" if args.offload else ""))
        prof = profiled_traffic(knames[dom], wl, with_trace=True)
        roof = {"bound": "hbm", "kernel": knames[dom], "achieved": stages[dom]["gbps"],
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(stages[dom]["gbps"] / HBM_PEAK_GBPS, 4),
                "traffic": prof[0], "trace_avg_us": prof[1],
                "avg_us": stages[dom]["avg_us"],
                "bytes_per_launch": stages[dom]["bytes_per_launch"]}

    # ---- CPU oracle baseline on a bounded sample (the first tokens, layer after layer until the
    # CPU budget is spent; single thread), and a parity spot check of the GPU on layer 0
    cpu, parity = None, None
    nt = min(args.cpu_tokens, K * Bt)
    if nt > 0:
        import oracle
        oracle.build()
        keys = ["w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down_t", "b_up", "b_gate",
                "b_down", "p1", "p2", "c1", "c2"]

        def host(layer):
            OL = {k: (None if layer.get(k) is None else
                      np.ascontiguousarray(layer[k].cpu().numpy())) for k in keys}
            OL["act"], OL["tau"] = cfg.act, cfg.tau
            return OL

        t_cpu, L_cpu = 0.0, 0
        for l in range(L):
            xh = x[l, :nt].cpu().numpy()
            if moe:
                OLs = [host(e) for e in layers[l]]
                Rh = routers[l].cpu().numpy()
            else:
                OL = host(layers[l][0])
            for t in range(nt):
                c0 = time.perf_counter()
                if prefill and not auto_prefill:
                    oracle.ffn(OL, xh[t], None)
                elif moe:
                    oracle.moe_token(OLs, Rh, xh[t], cfg.top_k)
                else:
                    oracle.sparse_token(OL, xh[t], n_hot=n_hot)
                t_cpu += time.perf_counter() - c0
            L_cpu = l + 1
            if t_cpu > args.cpu_budget:
                break
        rate = nt * L_cpu / t_cpu / L          # tokens through all L layers per second
        what = ("dense FFN" if prefill and not auto_prefill else
                "router + the chosen experts' predictor and sparse FFN" if moe else
                "predictor + sparse FFN")
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                                  if ln.startswith("model name")), "")
        except OSError:
            pass
        tok_bytes = touched.sum() / (K * Bt)              # touched bytes per token, all layers
        cpu = {"value": round(rate, 5), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": "first %d token(s) x %d of %d layers, %s, single-threaded C with fp64 "
                         "accumulation (%.1f s of CPU), scaled to all layers" % (
                             nt, L_cpu, L, what, t_cpu),
               "s_per_token": round(1.0 / rate, 3),
               "gbps_over_touched_bytes": round(rate * tok_bytes / 1e9, 4),
               "host": {"cpu_model": cpu_model, "logical_cpus": os.cpu_count()}}

        # parity spot check against the oracle evaluated on the GPU's own sets: the sampled
        # tokens of layer 0, then seeded random (layer, token) pairs over the whole stack; every
        # GPU output is the one the timed run wrote
        rng = np.random.default_rng(cfg.seed)
        n_pairs = min(args.parity_pairs, 2) if prefill else args.parity_pairs
        pairs = [(0, t) for t in range(nt)]
        if L > 1 and n_pairs > 0:
            pairs += [(int(l), int(t)) for l, t in zip(rng.integers(1, L, size=n_pairs),
                                                       rng.integers(0, K * Bt, size=n_pairs))]
        pairs += [(l, t) for l in range(L) for t in range(min(args.parity_stack_tokens, K * Bt))]
        pairs = sorted(set(pairs))
        worst = 0.0
        torch.cuda.synchronize()

        def gpu_set(plan, t_ptr):
            ie = torch.zeros(1, cfg.ffn, dtype=torch.int32, device=dev)
            ce = torch.zeros(1, dtype=torch.int32, device=dev)
            yy = torch.zeros(1, cfg.d, dtype=torch.float32, device=dev)
            ffn.ffn_sparse_forward(plan, t_ptr, 1, yy.data_ptr(), idx=ie.data_ptr(),
                                   cnt=ce.data_ptr(), stream=sp)
            torch.cuda.synchronize()
            mk = np.zeros(cfg.ffn, np.uint8)
            mk[ie[0, :int(ce[0])].cpu().numpy()] = 1
            return mk

        t_par = time.time()
        l_host, OLs = -1, None
        for l, t in pairs:
            if l != l_host:                                  # one layer on the host at a time
                OLs, l_host = None, l
                OLs = [host(e) for e in layers[l]]
            t_ptr = x[l].data_ptr() + t * xb
            xh_t = x[l, t].cpu().numpy()
            yg = y[l, t].cpu().numpy().astype(np.float64)          # from the timed run
            if prefill and not auto_prefill:
                yref, _ = oracle.ffn(OLs[0], xh_t, None)
            elif moe:
                idsc = torch.zeros(1, cfg.top_k, dtype=torch.int32, device=dev)
                wc = torch.zeros(1, cfg.top_k, dtype=torch.float32, device=dev)
                yy = torch.zeros(1, cfg.d, dtype=torch.float32, device=dev)
                ffn.ffn_moe_forward(moes[l], t_ptr, 1, yy.data_ptr(), idsc.data_ptr(),
                                    wc.data_ptr(), stream=sp)
                torch.cuda.synchronize()
                yref = np.zeros(cfg.d)
                for j in range(cfg.top_k):
                    e = int(idsc[0, j])
                    ye, _ = oracle.ffn(OLs[e], xh_t, gpu_set(mods[l][e].plan, t_ptr))
                    yref += float(wc[0, j]) * ye
            elif Bt == 1:
                yref, _ = oracle.ffn(OLs[0], xh_t, gpu_set(mods[l][0].plan, t_ptr))
            else:
                # the token's set from its own step's batched call
                st, j = divmod(t, Bt)
                idx = torch.zeros(Bt, cfg.ffn, dtype=torch.int32, device=dev)
                cn = torch.zeros(Bt, dtype=torch.int32, device=dev)
                yb = torch.zeros(Bt, cfg.d, dtype=torch.float32, device=dev)
                ffn.ffn_sparse_forward(mods[l][0].plan, xp[l][st], Bt, yb.data_ptr(),
                                       idx=idx.data_ptr(), cnt=cn.data_ptr(),
                                       path=ffn.FFN_PATH_AUTO if auto_prefill
                                       else ffn.FFN_PATH_SPARSE, stream=sp)
                torch.cuda.synchronize()
                mk = np.zeros(cfg.ffn, np.uint8)
                mk[idx[j, :int(cn[j])].cpu().numpy()] = 1
                yref, _ = oracle.ffn(OLs[0], xh_t, mk)
            worst = max(worst, float(np.max(np.abs(yg - yref)) / np.max(np.abs(yref))))
        OLs = None
        tol = 1e-5 if cfg.w_dtype == "f32" else 2e-3
        parity = {"pairs": len(pairs), "layers": sorted({l for l, _ in pairs}),
                  "max_normwise_err": worst, "tolerance": tol, "within_tolerance": worst <= tol}
        log("oracle: %.2f s for %d token(s) x %d layer(s); GPU parity over %d (layer, token) "
            "pairs of %d layer(s) (%.1f s): max normwise error %.2e" % (
                t_cpu, nt, L_cpu, len(pairs), len(parity["layers"]), time.time() - t_par, worst))

    crossover = None
    if args.calibrate and cfg.w_dtype == "f16":
        t_cal = time.time()
        with torch.cuda.stream(stream):
            cal = ffn.SparseFFN(layers[0][0], max_batch=args.calibrate, calibrate=True)
        crossover = {str(1 << k): round(cal.crossover(1 << k), 4)
                     for k in range(13) if (1 << k) <= args.calibrate}
        cal.close()
        log("calibrated crossover densities (%.1f s): %s" % (time.time() - t_cal, crossover))

    dtype = {"f32": "f32", "f16": "f16xf16->f32", "i4g32": "i4g32xf16->f32"}[cfg.w_dtype]
    result = {
        "metric": ("sparse-FFN decode tokens/s at 1 GPU; effective HBM GB/s of touched weights"
                   if not prefill else
                   "prefill tokens/s at 1 GPU (path chosen on the device by union density)"
                   if auto_prefill else "dense-FFN prefill tokens/s at 1 GPU (MFMA fallback)"),
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; power-law hot set)",
        "config": {"workload": cfg.name, "mode": mode, "tokens_per_call": Bt, "d": cfg.d,
                   "path": ("auto" if auto_prefill else "dense") if prefill else "sparse",
                   "decode_variant": args.decode_variant, "hot_head": n_hot or None,
                   "spectrum_alpha": cfg.spectrum_alpha or None,
                   "ffn": cfg.ffn, "rank": cfg.rank, "act": cfg.act, "layers": L,
                   "experts": cfg.n_experts, "top_k": cfg.top_k if moe else None,
                   "target_density": cfg.density, "measured_density": round(density, 5)},
        "predictor": quality,
        "prefill_path": path_chosen,
        "offload": offload,
        "effective_gbps": round(eff_gbps, 1),
        "touched_bytes_per_step": int(touched.sum() / K),
        "roofline": roof,
        "kernels": stages,
        "cpu_baseline": cpu,
        "parity_sample": parity,
    }
    if crossover is not None:
        result["crossover_density"] = crossover
    if others:
        del layers, mods, graphs, x, y
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["all_configs"] = run_others()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
