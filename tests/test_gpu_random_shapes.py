"""A seeded sweep of layer shapes against the float64 oracle, compared in full.

The shapes are drawn once, from a fixed generator, over the ranges where the
library changes plan: dimensions that are multiples of 8 but rarely of 64 (K
tails in every segment, ragged row and column tiles), ranks from 0 to beyond
d_in / 2, token counts from 0 up to the 256 x 256 tile's range, both storage
dtypes and every flag combination (undetached norm gradient, separate
compose).  Each case runs dora_forward + dora_backward through the C ABI and
checks every output at the parity bars of tests/gpu_util.py.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import LayerShape
from tests.gpu_util import check_norm, check_out, download, layer_to_device


def _draw_cases():
    rng = np.random.Generator(np.random.PCG64(20261204))
    cases = []

    def mult8(lo, hi):
        return int(rng.integers(lo // 8, hi // 8 + 1)) * 8

    for i in range(20):   # small and mid-size layers: split-K tiles, the float32 small path
        dtype = "bf16" if i % 4 else "f32"
        d_out, d_in = mult8(8, 1200), mult8(8, 1600)
        r = 0 if i % 7 == 3 else mult8(8, min(520, 2 * d_in))
        T = 0 if i % 9 == 5 else int(rng.integers(1, 700))
        flags = int(rng.integers(0, 4))
        cases.append((f"s{i}_{dtype}", LayerShape(d_out, d_in, r, T, 2.0, dtype), 100 + i, flags))
    for i in range(3):    # large outputs: the 256 x 256 tile with ragged last tiles
        d_out, d_in = 4096 + mult8(8, 504), mult8(520, 1560)
        r = mult8(8, 392)
        T = 4096 + int(rng.integers(1, 512))
        cases.append((f"l{i}_bf16", LayerShape(d_out, d_in, r, T, 2.0, "bf16"), 200 + i, i % 4))
    return cases


CASES = _draw_cases()


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from parameter_efficient_fine_dora_amd import ops as _ops, _lib
    _lib.lib()  # raises if the library is missing: there is no fallback
    return _ops


@pytest.mark.gpu
@pytest.mark.parametrize("name,shape,seed,flags", CASES, ids=[c[0] for c in CASES])
def test_random_shape_parity(ops, name, shape, seed, flags):
    print(f"random shape {name} {shape} flags={flags}", flush=True)
    sys.stdout.flush()
    layer = synth.make_layer(shape, seed, grad=True)
    dev = layer_to_device(layer, shape.dtype)
    y, norm, xs = ops.dora_forward(dev["x"], dev["W0"], dev["A"], dev["B"], dev["m"], shape.s,
                                   flags=flags)
    gx, gA, gB, gm = ops.dora_backward(dev["gy"], dev["x"], dev["W0"], dev["A"], dev["B"],
                                       dev["m"], norm, xs, y, shape.s, flags=flags)
    torch.cuda.synchronize()
    L = synth.layer_f64(layer, shape.dtype)
    y_ref, n_ref = oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_norm(download(norm), n_ref, "norm")
    g = oracle.dora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s,
                             exact=bool(flags & 1))
    if shape.tokens:
        check_out(download(y), y_ref, "y")
        if shape.r:
            check_out(download(xs), oracle.scaled_down_projection(L["x"], L["A"], shape.s), "xs")
    for k, t in (("dx", gx), ("dA", gA), ("dB", gB), ("dm", gm)):
        if t is not None and g[k].size:
            check_out(download(t), g[k], k)


def test_cases_cover_the_plans():
    """The draw reaches every regime it is meant to (checked on the host too)."""
    shapes = [c[1] for c in CASES]
    assert any(s.r == 0 for s in shapes) and any(s.tokens == 0 for s in shapes)
    assert any(s.dtype == "f32" for s in shapes) and any(s.r > s.d_in // 2 for s in shapes)
    assert any(s.d_in % 64 for s in shapes) and any(s.d_out % 256 for s in shapes)
    assert {c[3] for c in CASES} == {0, 1, 2, 3}
    assert any(s.tokens > 4096 and s.d_out > 4096 for s in shapes)
