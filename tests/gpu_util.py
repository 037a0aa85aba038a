"""Helpers for the GPU parity tests: moving stored bits to the device and back,
and the parity bars.

Bars (float32 accumulation, bf16 or float32 storage):
  norms            max_i |n_gpu - n_ref| / n_ref <= 1e-3
  outputs / grads  max |gpu - ref| <= 2e-2 * max |ref|  and  cosine(gpu, ref) >= 0.9999
                   (a reference that is identically zero must come back exactly zero)
"""
from __future__ import annotations

import numpy as np
import torch

import synth

NORM_RTOL = 1e-3
OUT_ATOL_FRAC = 2e-2
OUT_COS = 0.9999


def upload(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def download(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_to_f64(bits)
    return t.float().cpu().numpy().astype(np.float64)


def layer_to_device(layer: dict, dtype: str, device="cuda") -> dict:
    return {k: upload(v, dtype, device) for k, v in layer.items()}


def rel_norm_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-30))) if ref.size else 0.0


def check_norm(gpu, ref, what="norm", rtol=NORM_RTOL):
    err = rel_norm_err(gpu, ref)
    assert err <= rtol, f"{what}: max relative error {err:.3e} > {rtol:g}"
    return err


def out_stats(gpu, ref):
    gpu = np.asarray(gpu, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    den = float(np.linalg.norm(gpu) * np.linalg.norm(ref))
    cos = float(np.dot(gpu, ref) / den) if den > 0 else (1.0 if err == 0 else 0.0)
    return err, scale, cos


def check_out(gpu, ref, what, atol_frac=OUT_ATOL_FRAC, min_cos=OUT_COS):
    err, scale, cos = out_stats(gpu, ref)
    if scale == 0.0:
        assert err == 0.0, f"{what}: reference is zero but max|gpu| = {err:.3e}"
        return err, cos
    assert err <= atol_frac * scale, f"{what}: max|diff| {err:.3e} > {atol_frac:g} * {scale:.3e}"
    assert cos >= min_cos, f"{what}: cosine {cos:.6f} < {min_cos}"
    return err, cos
