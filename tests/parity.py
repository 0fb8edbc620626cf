"""Helpers shared by the GPU parity tests: move seeded layers to the device, run the oracle on the
same bytes, and apply the comparison rules.

Rules (the operator's outputs and how they are compared):
* active index list: bit-exact, except neurons whose oracle probability lies within 1e-4 of the
  threshold (the "band"), which may fall either way;
* y: normwise relative error max_j |y_gpu - y_ref| / max_j |y_ref| per token, with y_ref the
  oracle evaluated on the GPU's own active set (so a band flip does not count twice);
  tolerance 1e-5 for fp32 weights, 2e-3 for fp16 / int4 weights (fp32 accumulation).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

BAND = 1e-4
TOL = {"f32": 1e-5, "f16": 2e-3, "i4g32": 2e-3}

LAYER_KEYS = ["w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down_t", "b_up", "b_gate",
              "b_down", "p1", "p2", "c1", "c2"]


def to_device(layer: dict, device="cuda") -> dict:
    out = dict(layer)
    for k in LAYER_KEYS:
        if isinstance(layer.get(k), torch.Tensor):
            out[k] = layer[k].to(device).contiguous()
    return out


def oracle_layer(layer: dict) -> dict:
    """numpy copies of a layer (from host or device tensors) in the form oracle.ffn wants."""
    out = {"act": layer["act"], "tau": layer["tau"]}
    for k in LAYER_KEYS:
        v = layer.get(k)
        out[k] = None if v is None else np.ascontiguousarray(v.detach().cpu().numpy())
    return out


def normwise(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    den = np.max(np.abs(y_ref))
    num = np.max(np.abs(np.asarray(y_gpu, np.float64) - y_ref))
    return float(num / den) if den > 0 else float(num)


def check_index_list(idx_gpu, pred_ref, tau: float):
    """A_gpu minus the band == A_ref minus the band (ordered), and A_gpu ascending/unique."""
    idx_gpu = np.asarray(idx_gpu)
    assert np.all(np.diff(idx_gpu) > 0), "index list not strictly ascending"
    band = np.abs(pred_ref["p"] - tau) <= BAND
    a = idx_gpu[~band[idx_gpu]] if idx_gpu.size else idx_gpu
    r = pred_ref["idx"][~band[pred_ref["idx"]]] if pred_ref["count"] else pred_ref["idx"]
    assert np.array_equal(a, r), "active lists differ outside the threshold band: %s vs %s" % (
        np.setdiff1d(a, r)[:10], np.setdiff1d(r, a)[:10])
    return int(band.sum())


def mask_from_idx(idx, ffn: int) -> np.ndarray:
    m = np.zeros(ffn, np.uint8)
    m[np.asarray(idx, np.int64)] = 1
    return m
