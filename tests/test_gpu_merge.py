"""dora_merge (the deploy-time merged weight) on the GPU vs the float64 oracle.

W_out_i = g_i (W0_i + s (BA)_i) with g_i = m_i / max(n_i, eps): compared element
by element with oracle.merged_weight on small and ragged layers, on sampled rows
of the full-size layer, on a hand-worked row (exact), and through its purpose:
x W_out^T reproduces the layer output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import LayerShape
from tests.gpu_util import check_out, download, layer_to_device, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from parameter_efficient_fine_dora_amd import ops as _ops, _lib
    _lib.lib()
    return _ops


CASES = [
    ("tiny_f32", synth.CONFIGS["tiny_f32"], 0, {}),
    ("tiny_as_bf16", synth.CONFIGS["tiny_f32"].replace(dtype="bf16"), 0, {}),
    ("ragged_bf16", LayerShape(264, 520, 24, 0, 2.0, "bf16"), 1, {}),
    ("ragged_f32", LayerShape(264, 520, 24, 0, 2.0, "f32"), 1, {}),
    ("multitile_bf16", LayerShape(520, 1032, 136, 0, 2.0, "bf16"), 2, {}),
    ("minimal_bf16", LayerShape(8, 8, 8, 0, 2.0, "bf16"), 4, {}),
    ("rank0_bf16", LayerShape(136, 200, 0, 0, 2.0, "bf16"), 5, {}),
    ("sneg_f32", LayerShape(136, 200, 16, 0, -0.75, "f32"), 8, {}),
    ("largeB_bf16", LayerShape(264, 520, 24, 0, 2.0, "bf16"), 9, dict(b_std=0.1)),
]


@pytest.mark.parametrize("given_norm", [False, True], ids=["norm_computed", "norm_given"])
@pytest.mark.parametrize("name,shape,seed,kw", CASES, ids=[c[0] for c in CASES])
def test_merge_parity(ops, name, shape, seed, kw, given_norm):
    print(f"merge {name} seed={seed} norm_given={given_norm}", flush=True)
    layer = synth.make_layer(shape, seed, **kw)
    dev = layer_to_device(layer, shape.dtype)
    norm = ops.dora_norm(dev["W0"], dev["A"], dev["B"], shape.s) if given_norm else None
    got = download(ops.dora_merge(dev["W0"], dev["A"], dev["B"], dev["m"], shape.s, norm=norm))
    torch.cuda.synchronize()
    L = synth.layer_f64(layer, shape.dtype)
    ref = oracle.merged_weight(L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_out(got, ref, "merged weight")
    # every row keeps its magnitude: ||W_out_i|| = m_i up to one rounding per element
    rel = np.abs(np.linalg.norm(got, axis=1) - L["m"]) / L["m"]
    assert rel.max() <= (4e-3 if shape.dtype == "bf16" else 1e-5), rel.max()


def test_merge_worked_row_exact(ops):
    """V'_0 = (3,4,12), n = 13, m = 26: the merged row is (6, 8, 24), exact in bf16 and f32."""
    for dtype in ("bf16", "f32"):
        d = 8
        W0 = np.zeros((d, d)); A = np.zeros((d, d)); B = np.zeros((d, d)); m = np.ones(d)
        W0[0, :3] = (3, 4, 0); A[0, 2] = 1; B[0, 0] = 6; m[0] = 26
        W0[1:, d - 1] = 1   # unit rows: n = m = 1, merged row = W0 row
        t = {k: upload(synth.bf16_bits(v.astype(np.float32)) if dtype == "bf16" else v.astype(np.float32), dtype)
             for k, v in dict(W0=W0, A=A, B=B, m=m).items()}
        got = download(ops.dora_merge(t["W0"], t["A"], t["B"], t["m"], 2.0))
        exp = W0.copy(); exp[0, :3] = (6, 8, 24)
        assert np.array_equal(got, exp), (dtype, got[:2])


def test_merge_reproduces_layer_output(ops):
    shape = LayerShape(264, 520, 24, 37, 2.0, "bf16")
    layer = synth.make_layer(shape, 21)
    dev = layer_to_device(layer, shape.dtype)
    Wm = download(ops.dora_merge(dev["W0"], dev["A"], dev["B"], dev["m"], shape.s))
    L = synth.layer_f64(layer, shape.dtype)
    y_ref, _ = oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_out(L["x"] @ Wm.T, y_ref, "x W_merged^T")


def test_merge_fullsize_sampled(ops):
    shape = synth.CONFIGS["highrank_bf16"]
    print(f"merge full size {shape}", flush=True)
    layer = synth.make_layer(shape, synth.CONFIG_SEED["highrank_bf16"])
    dev = layer_to_device({k: layer[k] for k in ("W0", "A", "B", "m")}, shape.dtype)
    out = ops.dora_merge(dev["W0"], dev["A"], dev["B"], dev["m"], shape.s)
    norm = ops.dora_norm(dev["W0"], dev["A"], dev["B"], shape.s)
    torch.cuda.synchronize()
    for given in (None, norm):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            ops.dora_merge(dev["W0"], dev["A"], dev["B"], dev["m"], shape.s, norm=given, out=out)
        e1.record()
        torch.cuda.synchronize()
        print(f"merge {shape.d_out}x{shape.d_in} r={shape.r} ({'norm given' if given is not None else 'with norm'}):"
              f" {e0.elapsed_time(e1) / 5 * 1e3:.1f} us", flush=True)
    rows = np.random.default_rng(0).choice(shape.d_out, 48, replace=False)
    got = download(out[torch.from_numpy(rows).to(out.device)])
    L = synth.layer_f64({k: layer[k] for k in ("W0", "A", "B", "m")}, shape.dtype)
    ref = oracle.merged_weight(L["W0"][rows], L["A"], L["B"][rows], L["m"][rows], shape.s)
    check_out(got, ref, "merged rows")


def test_merge_ragged_rows_on_the_eight_wave_tile(ops):
    """d_out = 4104 on the merge's 256 x 256 tile: the last tile-row holds 8 rows of B."""
    shape = LayerShape(4104, 4096, 16, 0, 2.0, "bf16")
    print(f"merge ragged eight-wave tile {shape}", flush=True)
    layer = synth.make_layer(shape, 35)
    dev = layer_to_device(layer, shape.dtype)
    got = download(ops.dora_merge(dev["W0"], dev["A"], dev["B"], dev["m"], shape.s))
    L = synth.layer_f64(layer, shape.dtype)
    check_out(got, oracle.merged_weight(L["W0"], L["A"], L["B"], L["m"], shape.s), "merged weight")
