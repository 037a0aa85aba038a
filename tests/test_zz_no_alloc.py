"""dora_forward_noalloc (the allocation-free forward) against dora_forward, through
the C ABI: two calls in a row on the library's static workspace, the second on a
smaller layer, each bit-identical to dora_forward with a caller workspace; the
size limit; and no device memory taken by the call."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import synth
from synth import LayerShape
from tests.gpu_util import layer_to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from parameter_efficient_fine_dora_amd import _lib
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _outputs(shape, dev_dt):
    T, d_out, r = shape.tokens, shape.d_out, shape.r
    y = torch.full((T, d_out), float("nan"), dtype=dev_dt, device="cuda")
    norm = torch.full((d_out,), float("nan"), dtype=torch.float32, device="cuda")
    xs = torch.full((T, r), float("nan"), dtype=dev_dt, device="cuda")
    return y, norm, xs


def _forward(lib, shape, d, noalloc):
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    code = lib.BF16 if shape.dtype == "bf16" else lib.F32
    sh = lib.shape(shape.d_out, shape.d_in, shape.r, shape.tokens, code, shape.s)
    y, norm, xs = _outputs(shape, dt)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = lib.lib()
    if noalloc:
        rc = L.dora_forward_noalloc(ctypes.byref(sh), _p(d["x"]), _p(d["W0"]), _p(d["A"]),
                                    _p(d["B"]), _p(d["m"]), _p(y), _p(norm), _p(xs), st)
    else:
        nb = lib.workspace_bytes(sh, lib.OP_FORWARD)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        rc = L.dora_forward(ctypes.byref(sh), _p(d["x"]), _p(d["W0"]), _p(d["A"]), _p(d["B"]),
                            _p(d["m"]), _p(y), _p(norm), _p(xs), _p(ws), nb, st)
    assert rc == 0, lib.strerror(rc)
    torch.cuda.synchronize()
    return y, norm, xs


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


CASES = [
    ("crossover_bf16", synth.CONFIGS["crossover_bf16"], 1),      # 7.0 MiB of workspace
    ("ragged_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 2),
    ("tiny_f32", synth.CONFIGS["tiny_f32"], 3),
]


def test_noalloc_matches_dora_forward_twice_in_a_row(lib):
    """Two consecutive calls on the shared static workspace, the second smaller (it
    sees the first call's leftovers), each equal to dora_forward bit for bit."""
    for name, shape, seed in CASES:
        say(f"noalloc vs dora_forward: {name} {shape}")
        layer = synth.make_layer(shape, seed)
        d = layer_to_device(layer, shape.dtype)
        ref = _forward(lib, shape, d, noalloc=False)
        got = _forward(lib, shape, d, noalloc=True)
        for k, a, b in zip(("y", "norm", "xs"), got, ref):
            assert np.array_equal(_bits(a), _bits(b)), f"{name}: {k} differs"


def test_noalloc_takes_no_device_memory(lib):
    shape = LayerShape(520, 1032, 136, 300, 2.0, "bf16")
    layer = synth.make_layer(shape, 4)
    d = layer_to_device(layer, shape.dtype)
    dt = torch.bfloat16
    sh = lib.shape(shape.d_out, shape.d_in, shape.r, shape.tokens, lib.BF16, shape.s)
    y, norm, xs = _outputs(shape, dt)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = lib.lib()
    args = (ctypes.byref(sh), _p(d["x"]), _p(d["W0"]), _p(d["A"]), _p(d["B"]), _p(d["m"]), _p(y),
            _p(norm), _p(xs), st)
    assert L.dora_forward_noalloc(*args) == 0
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        assert L.dora_forward_noalloc(*args) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0, (free0, free1)


def test_noalloc_rejects_shapes_beyond_its_workspace(lib):
    sh = lib.shape(8192, 8192, 384, 131072, lib.BF16, 2.0)
    assert lib.workspace_bytes(sh, lib.OP_FORWARD) > lib.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: the call returns before any launch
    rc = lib.lib().dora_forward_noalloc(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, fake,
                                        fake, None)
    assert rc == lib.ERR_CODE["DORA_ERR_WORKSPACE"]
    fits = lib.shape(8192, 8192, 384, 65536, lib.BF16, 2.0)
    assert lib.workspace_bytes(fits, lib.OP_FORWARD) <= lib.NOALLOC_SCRATCH_BYTES
