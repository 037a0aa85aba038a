"""Metamorphic checks on the GPU path: input transformations whose effect on every
output is exact in floating point, so the HIP path must reproduce it bit for bit
(plus one stress input whose error is recorded, not gated).

* Scaling (W0, B, m) by 2 scales every intermediate by a power of two: g and
  g - 1 are unchanged, the norm, y, ts, dx and dA double, xs, gz, dB and dm do
  not change (DoRA's magnitude/direction decoupling, DoRA reading notes Sec. 4.1).
* Permuting the tokens permutes y, xs and dx (each token row is computed
  independently, with the K sum in a fixed order) and leaves the norm alone.
* The same power-of-two scaling, repeated on one reused workspace, pins the
  norm projection's cross-workgroup finish (the last workgroup of a tile row
  reads the other workgroups' partial sums); A scaled by c with B by 1/c leaves
  every norm unchanged while G scales, which pins the Gram matrix each call
  forms afresh in the same workspace.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import LayerShape
from tests.gpu_util import check_out, download, layer_to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from parameter_efficient_fine_dora_amd import ops as _ops, _lib
    _lib.lib()  # raises if the library is missing: there is no fallback
    return _ops


def step(ops, dev, s, flags=0):
    y, norm, xs = ops.dora_forward(dev["x"], dev["W0"], dev["A"], dev["B"], dev["m"], s, flags=flags)
    gx, gA, gB, gm = ops.dora_backward(dev["gy"], dev["x"], dev["W0"], dev["A"], dev["B"], dev["m"],
                                       norm, xs, y, s, flags=flags)
    torch.cuda.synchronize()
    return dict(y=y, norm=norm, xs=xs, dx=gx, dA=gA, dB=gB, dm=gm)


SHAPES = [
    ("multitile_bf16", LayerShape(520, 1032, 136, 300, 2.0, "bf16")),
    ("ragged_f32", LayerShape(264, 520, 24, 37, 2.0, "f32")),
]


@pytest.mark.parametrize("flags", [0, 2], ids=["fused", "separate"])
@pytest.mark.parametrize("name,shape", SHAPES, ids=[c[0] for c in SHAPES])
def test_power_of_two_scaling_is_exact(ops, name, shape, flags):
    say(f"scaling by 2: {name} flags={flags}")
    layer = synth.make_layer(shape, 51, grad=True)
    dev = layer_to_device(layer, shape.dtype)
    base = step(ops, dev, shape.s, flags)
    dev2 = dict(dev)
    for k in ("W0", "B", "m"):
        dev2[k] = dev[k] * 2   # exact in bf16 and fp32
    scaled = step(ops, dev2, shape.s, flags)
    for k in ("norm", "y", "dx", "dA"):
        assert torch.equal(scaled[k], base[k] * 2), k
    for k in ("xs", "dB", "dm"):
        assert torch.equal(scaled[k], base[k]), k


@pytest.mark.parametrize("name,shape", SHAPES, ids=[c[0] for c in SHAPES])
def test_token_permutation_is_exact(ops, name, shape):
    say(f"token permutation: {name}")
    layer = synth.make_layer(shape, 52, grad=True)
    dev = layer_to_device(layer, shape.dtype)
    base = step(ops, dev, shape.s)
    perm = torch.from_numpy(np.random.Generator(np.random.PCG64(53)).permutation(shape.tokens)).cuda()
    dev2 = dict(dev)
    dev2["x"] = dev["x"][perm].contiguous()
    dev2["gy"] = dev["gy"][perm].contiguous()
    moved = step(ops, dev2, shape.s)
    assert torch.equal(moved["norm"], base["norm"])
    for k in ("y", "xs", "dx"):
        assert torch.equal(moved[k], base[k][perm]), k
    # sums over tokens: another order of the same terms
    for k in ("dA", "dB", "dm"):
        check_out(download(moved[k]), download(base[k]), f"{k} (tokens permuted)")


def test_near_cancelling_rows_recorded(ops):
    """Rows whose adapted weight nearly cancels (W0_i = c A_j, B_ij = -(c/s)(1 + eps)):
    the factored n^2 is a difference of terms ~c^2 |A_j|^2, so its relative error grows
    like fp32 rounding / eps^2.  The error is printed, not gated; the norm must stay
    finite and non-negative."""
    shape = LayerShape(64, 512, 16, 8, 2.0, "bf16")
    layer = synth.make_layer(shape, 54, grad=True)
    W0 = synth.to_f64(layer["W0"], "bf16")
    A = synth.to_f64(layer["A"], "bf16")
    B = synth.to_f64(layer["B"], "bf16")
    c = 0.5
    eps = [2.0 ** -k for k in (2, 4, 6, 7)]
    for i, e in enumerate(eps):
        W0[i] = c * A[i]
        B[i] = 0.0
        B[i, i] = -(c / shape.s) * (1.0 + e)
    layer["W0"] = synth.bf16_bits(W0.astype(np.float32))
    layer["B"] = synth.bf16_bits(B.astype(np.float32))
    dev = layer_to_device(layer, "bf16")
    n = download(ops.dora_norm(dev["W0"], dev["A"], dev["B"], shape.s))
    L = synth.layer_f64(layer, "bf16")
    n_ref = oracle.dora_norm(L["W0"], L["A"], L["B"], shape.s)
    assert np.all(np.isfinite(n)) and np.all(n >= 0)
    for i, e in enumerate(eps):
        rel = abs(n[i] - n_ref[i]) / n_ref[i]
        say(f"near-cancelling row eps=2^{int(np.log2(e))}: n_ref {n_ref[i]:.4e}, relative error {rel:.2e}")
    # the other rows are ordinary
    rest = slice(len(eps), None)
    assert np.max(np.abs(n[rest] - n_ref[rest]) / n_ref[rest]) <= 1e-3


REUSE = [
    # r in 257..384: one 128 x 384 tile per row block, K split nine ways
    ("rank320_bf16", LayerShape(2048, 4096, 320, 1, 2.0, "bf16")),
    # two column tiles of the generic 128 x 128 plan
    ("rank200_bf16", LayerShape(1032, 2056, 200, 1, 2.0, "bf16")),
    # 64 tile rows
    ("rank64_bf16", LayerShape(8192, 1024, 64, 1, 2.0, "bf16")),
]


@pytest.mark.parametrize("name,shape", REUSE, ids=[c[0] for c in REUSE])
def test_norm_calls_on_one_workspace(ops, name, shape):
    """dora_norm called over and over on ONE workspace, W0 and B scaled by a
    different power of two each time: the norms scale by exactly that factor
    (every term of n^2 scales by its square), so a row norm formed from any
    partial sum left in the workspace by the previous call, or read before
    another workgroup's partial landed, shows up as a bit difference.  The
    first call is checked against the oracle."""
    from parameter_efficient_fine_dora_amd import _lib
    say(f"repeated dora_norm on one workspace: {name} {shape}")
    layer = synth.make_layer(shape, 71)
    dev = layer_to_device(layer, "bf16")
    sh = _lib.shape(shape.d_out, shape.d_in, shape.r, 0, _lib.BF16, shape.s)
    ws = torch.empty(_lib.workspace_bytes(sh, _lib.OP_NORM), dtype=torch.uint8, device="cuda")
    base = ops.dora_norm(dev["W0"], dev["A"], dev["B"], shape.s, workspace=ws).clone()
    torch.cuda.synchronize()
    L = synth.layer_f64(layer, "bf16")
    n_ref = oracle.dora_norm(L["W0"], L["A"], L["B"], shape.s)
    assert np.max(np.abs(download(base) - n_ref) / n_ref) <= 1e-3
    for c in (2.0, 0.5, 4.0, 1.0, 0.25, 8.0, 1.0, 2.0):
        n = ops.dora_norm(dev["W0"] * c, dev["A"], dev["B"] * c, shape.s, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(n, base * c), f"scale {c}"
    # A scaled by c and B by 1/c: BA, and so every norm, is bitwise unchanged, while
    # G = A A^T (formed again by each call) scales by c^2, so a Gram term built
    # from the previous call's G or its partial sums shows up as a bit difference.
    for c in (2.0, 0.5, 4.0, 0.25, 1.0, 8.0):
        n = ops.dora_norm(dev["W0"], dev["A"] * c, dev["B"] / c, shape.s, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(n, base), f"A scaled by {c}"
