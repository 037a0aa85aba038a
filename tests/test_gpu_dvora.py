"""DVoRA (DoRA with VeRA's direction update diag(b) B_sh diag(d) A_sh) on the GPU
vs the float64 oracle: the effective-B scaling, the b / d gradient reductions,
and whole forward + backward passes composed from the C entry points, with the
norm detached and undetached."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import LayerShape
from tests.gpu_util import check_norm, check_out, download, layer_to_device, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from parameter_efficient_fine_dora_amd import ops as _ops, _lib
    _lib.lib()
    return _ops


def vera_layer(shape, seed):
    """A DoRA layer whose B serves as B_shared, plus the two VeRA vectors."""
    layer = synth.make_layer(shape, seed, grad=True, b_std=0.3)
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    store = synth.bf16_bits if shape.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    layer["b"] = store(rng.normal(0.0, 0.2, shape.d_out).astype(np.float32))
    layer["d"] = store(rng.normal(0.0, 0.2, shape.r).astype(np.float32))
    return layer


CASES = [
    ("ragged_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 31),
    ("ragged_f32", LayerShape(264, 520, 24, 37, 2.0, "f32"), 32),
    ("multitile_bf16", LayerShape(520, 1032, 136, 300, 1.0, "bf16"), 33),
    ("minimal_bf16", LayerShape(8, 8, 8, 1, 1.0, "bf16"), 34),
]


@pytest.mark.parametrize("name,shape,seed", CASES, ids=[c[0] for c in CASES])
def test_vera_scale_and_grads(ops, name, shape, seed):
    print(f"vera kernels {name}", flush=True)
    layer = vera_layer(shape, seed)
    dev = layer_to_device(layer, shape.dtype)
    L = synth.layer_f64(layer, shape.dtype)
    Be = download(ops.dora_vera_scale(dev["B"], dev["b"], dev["d"]))
    check_out(Be, L["b"][:, None] * L["B"] * L["d"][None, :], "B_eff")
    rng = np.random.Generator(np.random.PCG64(seed + 2000))
    gBe_stored = (synth.bf16_bits if shape.dtype == "bf16" else (lambda a: a))(
        rng.standard_normal((shape.d_out, shape.r)).astype(np.float32))
    gBe = synth.to_f64(gBe_stored, shape.dtype)
    gb, gd = ops.dora_vera_grads(upload(gBe_stored, shape.dtype), dev["B"], dev["b"], dev["d"])
    check_out(download(gb), np.sum(gBe * L["B"] * L["d"][None, :], axis=1), "grad_b")
    check_out(download(gd), np.sum(gBe * L["B"] * L["b"][:, None], axis=0), "grad_d")
    gb2, gd2 = ops.dora_vera_grads(upload(gBe_stored, shape.dtype), dev["B"], dev["b"], dev["d"])
    assert torch.equal(gb, gb2) and torch.equal(gd, gd2), "fixed-order reductions are deterministic"


@pytest.mark.parametrize("flags", [0, 1], ids=["detached", "exact"])
@pytest.mark.parametrize("name,shape,seed", CASES, ids=[c[0] for c in CASES])
def test_dvora_forward_backward(ops, name, shape, seed, flags):
    print(f"dvora {name} flags={flags}", flush=True)
    layer = vera_layer(shape, seed)
    dev = layer_to_device(layer, shape.dtype)
    Be = ops.dora_vera_scale(dev["B"], dev["b"], dev["d"])
    y, norm, xs = ops.dora_forward(dev["x"], dev["W0"], dev["A"], Be, dev["m"], shape.s, flags=flags)
    gx, _, gBe, gm = ops.dora_backward(dev["gy"], dev["x"], dev["W0"], dev["A"], Be, dev["m"], norm,
                                       xs, y, shape.s, need=("x", "B", "m"), flags=flags)
    gb, gd = ops.dora_vera_grads(gBe, dev["B"], dev["b"], dev["d"])
    torch.cuda.synchronize()
    L = synth.layer_f64(layer, shape.dtype)
    # the oracle forms V' from the VeRA product of the stored vectors (the GPU
    # rounds B_eff to the layer dtype once; the tolerance covers it)
    y_ref, n_ref = oracle.dvora_forward(L["x"], L["W0"], L["A"], L["B"], L["b"], L["d"], L["m"], shape.s)
    check_norm(download(norm), n_ref, "norm")
    check_out(download(y), y_ref, "y")
    g = oracle.dvora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["b"], L["d"], L["m"],
                              shape.s, exact=bool(flags & 1))
    check_out(download(gx), g["dx"], "dx")
    check_out(download(gm), g["dm"], "dm")
    check_out(download(gb), g["db"], "db")
    check_out(download(gd), g["dd"], "dd")


def test_dvora_linear_module(ops):
    from parameter_efficient_fine_dora_amd.module import DVoRALinear
    shape = LayerShape(136, 200, 16, 24, 1.0, "f32")
    layer = vera_layer(shape, 41)
    dev = layer_to_device(layer, shape.dtype)
    mod = DVoRALinear(dev["W0"], dev["A"], dev["B"], s=shape.s, d_init=0.1)
    with torch.no_grad():
        mod.b.copy_(dev["b"])
        mod.d.copy_(dev["d"])
    x = dev["x"].clone().requires_grad_(True)
    y = mod(x)
    (y * dev["gy"]).sum().backward()
    L = synth.layer_f64(layer, shape.dtype)
    m0 = download(mod.m.detach())
    y_ref, _ = oracle.dvora_forward(L["x"], L["W0"], L["A"], L["B"], L["b"], L["d"], m0, shape.s)
    check_out(download(y.detach()), y_ref, "module y")
    g = oracle.dvora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["b"], L["d"], m0, shape.s)
    check_out(download(x.grad), g["dx"], "module dx")
    check_out(download(mod.b.grad), g["db"], "module db")
    check_out(download(mod.d.grad), g["dd"], "module dd")
    check_out(download(mod.m.grad), g["dm"], "module dm")
