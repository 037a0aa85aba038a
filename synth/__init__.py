"""Seeded synthetic DoRA layers.

This module is the one place both sides of every parity check get their inputs
from: the float64 oracle and the HIP library receive the identical stored bits.
It holds input recipes only (random draws, rounding the draws to the storage
format, decoding stored bits to float64) and no step of the DoRA computation.

Workloads stand in for the projection layers of the 8-32B vision-language
models the Scaling DoRA paper measures at rank 384 in bf16 (Scaling DoRA
summary page, abstract); no model weights or datasets are involved.

Distributions (all dense, iid, per layer):
  W0 ~ N(0, 0.02^2)            frozen base weight      [d_out, d_in]
  A  ~ U(-1/sqrt(d_in), +1/sqrt(d_in))   LoRA down     [r, d_in]
       (fan-in scaled Kaiming-uniform; DoRA reading notes, Sec. 1.3 and
        Algorithm 1 name Kaiming-uniform without a bound)
  B  ~ N(0, 0.01^2)            LoRA up                 [d_out, r]
  m_i = ||W0_i|| * (1 + U(-0.05, 0.05))   magnitude    [d_out]
       (||W0_i|| from the already-rounded W0; m then rounded itself)
  x  ~ N(0, 1)                 input tokens            [tokens, d_in]
  gy ~ N(0, 1)                 upstream gradient       [tokens, d_out]
Draw order per layer: W0, A, B, m-noise, x, gy, each in float32 from
numpy's PCG64 seeded with the given seed, then rounded to bf16 with
round-to-nearest-even once (skipped for float32 layers).
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "LayerShape", "CONFIGS", "config", "make_layer", "bf16_bits", "bf16_to_f64",
    "to_f64", "storage_dtype",
]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d_out: int
    d_in: int
    r: int
    tokens: int
    s: float = 2.0
    dtype: str = "bf16"          # "bf16" or "f32": storage type of every tensor
    name: str = ""

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny float32 layer, the crossover size below which the
# paper says launch latency dominates, the paper's d_in=8192 / r=384 headline
# layer, a wide MLP up-projection, and the backward of the headline layer.
CONFIGS = {
    "tiny_f32": LayerShape(256, 512, 16, 64, 2.0, "f32", "tiny_f32"),
    "crossover_bf16": LayerShape(2048, 6144, 64, 2048, 2.0, "bf16", "crossover_bf16"),
    "highrank_bf16": LayerShape(8192, 8192, 384, 4096, 2.0, "bf16", "highrank_bf16"),
    "widemlp_bf16": LayerShape(27648, 5120, 256, 8192, 2.0, "bf16", "widemlp_bf16"),
    "highrank_bwd_bf16": LayerShape(8192, 8192, 384, 4096, 2.0, "bf16", "highrank_bwd_bf16"),
}
CONFIG_SEED = {name: i for i, name in enumerate(CONFIGS)}


def config(name: str) -> LayerShape:
    return CONFIGS[name]


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # no overflow: |a| <= FLT_MAX keeps u + 0x8000 < 2^32
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (bf16 bits or float32) -> float64, exactly."""
    if dtype == "bf16":
        return bf16_to_f64(stored)
    return np.asarray(stored, dtype=np.float32).astype(np.float64)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def make_layer(shape: LayerShape, seed: int | None = None, *, grad: bool = False,
               b_std: float = 0.01, w_std: float = 0.02, zero_b: bool = False) -> dict:
    """Draw one synthetic layer in storage form.

    Returns a dict of contiguous numpy arrays: W0, A, B, m, x and (grad=True) gy,
    each uint16 bf16 bits or float32 per ``shape.dtype``.  ``b_std`` selects the
    "large-B" stress distribution (e.g. 0.1) and ``zero_b`` the B = 0 start of
    training (DoRA reading notes, Algorithm 1).
    """
    if seed is None:
        seed = CONFIG_SEED.get(shape.name, 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    d_out, d_in, r, T, dt = shape.d_out, shape.d_in, shape.r, shape.tokens, shape.dtype
    f32 = np.float32
    W0 = _store(rng.standard_normal((d_out, d_in), dtype=f32) * f32(w_std), dt)
    bound = f32(1.0 / np.sqrt(d_in))
    A = _store(rng.uniform(-1.0, 1.0, size=(r, d_in)).astype(f32) * bound, dt)
    B32 = rng.standard_normal((d_out, r), dtype=f32) * f32(b_std)
    if zero_b:
        B32[...] = 0
    B = _store(B32, dt)
    noise = rng.uniform(-0.05, 0.05, size=d_out)
    w0 = to_f64(W0, dt)
    row_len = np.sqrt(np.einsum("ij,ij->i", w0, w0))
    m = _store((row_len * (1.0 + noise)).astype(f32), dt)
    x = _store(rng.standard_normal((T, d_in), dtype=f32), dt)
    out = dict(W0=W0, A=A, B=B, m=m, x=x)
    if grad:
        out["gy"] = _store(rng.standard_normal((T, d_out), dtype=f32), dt)
    return out


def layer_f64(layer: dict, dtype: str) -> dict:
    """Decode every stored tensor of a layer to float64."""
    return {k: to_f64(v, dtype) for k, v in layer.items()}
