"""HIP path vs the float64 oracle, element by element, through the C ABI.

Every case draws its inputs from synth (identical bits on both sides), runs
dora_norm / dora_forward / dora_backward on the GPU through the torch binding
(marshalling only) and compares with the oracle at the parity bars stated in
tests/gpu_util.py.  Full-size layers are compared on sampled outputs (and
on every row norm).
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import LayerShape
from tests.gpu_util import (check_norm, check_out, download, layer_to_device, out_stats, upload)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_rows.json")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from parameter_efficient_fine_dora_amd import ops as _ops, _lib
    _lib.lib()  # raises if the library is missing: there is no fallback
    return _ops


def run_layer(ops, shape: LayerShape, layer: dict, flags=0, backward=True, need=("x", "A", "B", "m")):
    dev = layer_to_device(layer, shape.dtype)
    y, norm, xs = ops.dora_forward(dev["x"], dev["W0"], dev["A"], dev["B"], dev["m"], shape.s,
                                   flags=flags)
    out = dict(y=y, norm=norm, xs=xs)
    if backward:
        gx, gA, gB, gm = ops.dora_backward(dev["gy"], dev["x"], dev["W0"], dev["A"], dev["B"],
                                           dev["m"], norm, xs, y, shape.s, need=need, flags=flags)
        out.update(dx=gx, dA=gA, dB=gB, dm=gm)
    torch.cuda.synchronize()
    return {k: (download(v) if v is not None else None) for k, v in out.items()}


def compare_full(shape, layer, got, backward=True):
    L = synth.layer_f64(layer, shape.dtype)
    y_ref, n_ref = oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_norm(got["norm"], n_ref, "norm")
    if shape.tokens:
        check_out(got["y"], y_ref, "y")
        if shape.r:
            check_out(got["xs"], oracle.scaled_down_projection(L["x"], L["A"], shape.s), "xs")
    if backward:
        g = oracle.dora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
        for k in ("dx", "dA", "dB", "dm"):
            if got.get(k) is not None and g[k].size:
                check_out(got[k], g[k], k)


# ---- hand-worked integer rows: bit-exact ---------------------------------------

def golden_layer(e, dtype):
    """Embed one worked example in a layer padded to multiples of 8.

    Rows past the example's are unit rows W0_i = e_{d_in-1}, B_i = 0, m_i = 1
    (n_i = 1), with x and gy zero in the padded columns, so they add nothing to
    the example's outputs.
    """
    W0e, Ae, Be = (np.array(e[k], dtype=np.float64) for k in ("W0", "A", "B"))
    d_oe, d_ie = W0e.shape
    r_e = Ae.shape[0]
    d_out, d_in, r = 8, 8, 8
    W0 = np.zeros((d_out, d_in)); W0[:d_oe, :d_ie] = W0e
    for i in range(d_oe, d_out):
        W0[i, d_in - 1] = 1.0
    A = np.zeros((r, d_in)); A[:r_e, :d_ie] = Ae
    B = np.zeros((d_out, r)); B[:d_oe, :r_e] = Be
    m = np.ones(d_out); m[:d_oe] = e.get("m", np.ones(d_oe))
    xe = np.array(e.get("x", [[1.0] * d_ie]), dtype=np.float64)
    T = xe.shape[0]
    x = np.zeros((T, d_in)); x[:, :d_ie] = xe
    gy = np.zeros((T, d_out)); gy[:, :d_oe] = np.array(e.get("gy", np.zeros((T, d_oe))))
    store = (lambda a: synth.bf16_bits(a.astype(np.float32))) if dtype == "bf16" else (
        lambda a: a.astype(np.float32))
    layer = {k: store(v) for k, v in dict(W0=W0, A=A, B=B, m=m, x=x, gy=gy).items()}
    return LayerShape(d_out, d_in, r, T, e["s"], dtype), layer, d_oe, d_ie, r_e


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, 2])
def test_worked_rows_exact(ops, dtype, flags):
    for e in json.load(open(GOLDEN))["examples"]:
        say(f"worked row {e['name']} {dtype} flags={flags}")
        shape, layer, d_oe, d_ie, r_e = golden_layer(e, dtype)
        got = run_layer(ops, shape, layer, flags=flags)
        n = got["norm"][:d_oe]
        n_exp = np.array(e["norm"], float)
        if all(float(v).is_integer() for v in n_exp):
            assert np.array_equal(n, n_exp), (e["name"], n)
        else:   # n^2 is exact; the float32 square root is correctly rounded
            np.testing.assert_allclose(n, n_exp, rtol=2e-7, atol=0)
        if "y" in e:
            y_exp = np.array(e["y"], float)
            if all(float(v).is_integer() for v in y_exp.ravel()):
                assert np.array_equal(got["y"][:, :d_oe], y_exp), got["y"]
            else:
                np.testing.assert_allclose(got["y"][:, :d_oe], y_exp, rtol=2 ** -8)
        if "gy" in e:
            assert np.array_equal(got["dx"][:, :d_ie], np.array(e["dx"], float)), got["dx"]
            assert np.array_equal(got["dA"][:r_e, :d_ie], np.array(e["dA"], float)), got["dA"]
            assert np.array_equal(got["dB"][:d_oe, :r_e], np.array(e["dB"], float)), got["dB"]
            np.testing.assert_allclose(got["dm"][:d_oe], e["dm"], rtol=1e-6)
            assert not got["dx"][:, d_ie:].any() and not got["dB"][d_oe:].any()



# ---- small and ragged layers: full comparison ------------------------------------

SMALL = [
    ("tiny_f32", synth.CONFIGS["tiny_f32"], 0, {}),
    ("tiny_f32_seed100", synth.CONFIGS["tiny_f32"], 100, {}),
    ("tiny_f32_seed200", synth.CONFIGS["tiny_f32"], 200, {}),
    ("tiny_as_bf16", synth.CONFIGS["tiny_f32"].replace(dtype="bf16"), 0, {}),
    ("ragged_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 1, {}),
    ("ragged_f32", LayerShape(264, 520, 24, 37, 2.0, "f32"), 1, {}),
    ("multitile_bf16", LayerShape(520, 1032, 136, 300, 2.0, "bf16"), 2, {}),
    ("bigtile_ragged_bf16", LayerShape(776, 584, 72, 1031, 2.0, "bf16"), 3, {}),
    ("minimal_bf16", LayerShape(8, 8, 8, 1, 2.0, "bf16"), 4, {}),
    ("rank0_bf16", LayerShape(136, 200, 0, 19, 2.0, "bf16"), 5, {}),
    ("rank0_f32", LayerShape(136, 200, 0, 19, 2.0, "f32"), 5, {}),
    ("tokens0_bf16", LayerShape(136, 200, 16, 0, 2.0, "bf16"), 6, {}),
    ("s0_bf16", LayerShape(136, 200, 16, 9, 0.0, "bf16"), 7, {}),
    ("sneg_f32", LayerShape(136, 200, 16, 9, -0.75, "f32"), 8, {}),
    ("largeB_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 9, dict(b_std=0.1)),
    ("zeroB_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 10, dict(zero_b=True)),
    # r > d_in / 2 and K tails in every segment (d_in, r, d_out not multiples of 64)
    ("widerank_bf16", LayerShape(1032, 2056, 1016, 260, 2.0, "bf16"), 11, {}),
    ("widerank_f32", LayerShape(520, 776, 392, 70, 2.0, "f32"), 12, {}),
    # float32 layers at the edge of the two-kernel small forward (64 tokens,
    # rank 32, d_out and d_in just under their limits), and one token past it
    ("smallmax_f32", LayerShape(4088, 1016, 32, 64, 2.0, "f32"), 14, {}),
    ("small_t65_f32", LayerShape(136, 200, 16, 65, 2.0, "f32"), 15, {}),
    # one token, the smallest nonzero rank, one K chunk and one row block
    ("small_t1_r8_f32", LayerShape(16, 64, 8, 1, 2.0, "f32"), 16, {}),
    # rank 32 with B = 0 (the start of training): the norm is ||W0_i|| and y = m-scaled base
    ("small_zeroB_f32", LayerShape(72, 136, 32, 5, 2.0, "f32"), 17, dict(zero_b=True)),
]


@pytest.mark.parametrize("flags", [0, 2], ids=["fused", "separate"])
@pytest.mark.parametrize("name,shape,seed,kw", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(ops, name, shape, seed, kw, flags):
    say(f"small parity {name} flags={flags} shape={shape}")
    layer = synth.make_layer(shape, seed, grad=True, **kw)
    got = run_layer(ops, shape, layer, flags=flags)
    compare_full(shape, layer, got)
    if kw.get("zero_b"):
        assert not got["dA"].any(), "B = 0 gives dA = 0 exactly"


def test_fullrank_large_tile_transposed_products(ops):
    """r close to d: the dB (d_out x r) and dA (r x d_in) products have 272 output
    tiles each, enough for the 256 x 256 tile with both operands transposed; every
    dimension is ragged against it and K = T = 333 ends on a partial step."""
    shape = LayerShape(4104, 4104, 4040, 333, 2.0, "bf16")
    say(f"full-rank large-tile parity shape={shape}")
    layer = synth.make_layer(shape, 13, grad=True)
    got = run_layer(ops, shape, layer)
    compare_full(shape, layer, got)


TAIL = [
    # fused forward on 4 x 65 tiles of 256 x 256 over K = 2080: the last round (4 tiles) is
    # the last tile column, which runs as a second launch on 256 x 128 tiles
    ("fwd_tail", LayerShape(16640, 2056, 24, 1024, 2.0, "bf16"), 41),
    # dx (W0 read transposed) on 4 x 65 tiles over K = 2080, ragged d_out
    ("dx_tail", LayerShape(2040, 16640, 40, 1024, 2.0, "bf16"), 42),
]


@pytest.mark.parametrize("name,shape,seed", TAIL, ids=[c[0] for c in TAIL])
def test_tail_columns_on_narrower_tiles(ops, name, shape, seed):
    """A large-tile GEMM whose last round of workgroups is at most half full runs
    that round's tile columns on 256 x 128 tiles; every output matches the oracle
    in full (and the merged weight of the same layer does too)."""
    say(f"tail columns {name} shape={shape}")
    layer = synth.make_layer(shape, seed, grad=True)
    got = run_layer(ops, shape, layer)
    compare_full(shape, layer, got)
    # the split is taken: the GEMM runs as two launches (timing hook, serial order)
    ops.timing_enable(True)
    try:
        run_layer(ops, shape, layer)
        rec = ops.timing_collect()
    finally:
        ops.timing_enable(False)
    label = "fused_fwd_gemm" if name == "fwd_tail" else "dx_gemm"
    assert rec[label][0] == 2, rec
    dev = layer_to_device(layer, "bf16")
    W = download(ops.dora_merge(dev["W0"], dev["A"], dev["B"], dev["m"], shape.s))
    L = synth.layer_f64(layer, "bf16")
    check_out(W, oracle.merged_weight(L["W0"], L["A"], L["B"], L["m"], shape.s), "merged weight")


def test_skip_outputs_and_recompute_xs(ops):
    shape = LayerShape(264, 520, 24, 37, 2.0, "bf16")
    layer = synth.make_layer(shape, 11, grad=True)
    dev = layer_to_device(layer, "bf16")
    y, norm, _ = ops.dora_forward(dev["x"], dev["W0"], dev["A"], dev["B"], dev["m"], shape.s,
                                  keep_xs=False)
    gx, gA, gB, gm = ops.dora_backward(dev["gy"], dev["x"], dev["W0"], dev["A"], dev["B"],
                                       dev["m"], norm, None, y, shape.s, need=("B", "m"))
    assert gx is None and gA is None
    L = synth.layer_f64(layer, "bf16")
    g = oracle.dora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_out(download(gB), g["dB"], "dB with xs recomputed")
    check_out(download(gm), g["dm"], "dm")


# ---- the crossover layer (2048 x 6144, r 64): full comparison ----------------------

def test_crossover_parity(ops):
    shape = synth.CONFIGS["crossover_bf16"]
    for seed in (synth.CONFIG_SEED["crossover_bf16"], 100, 200):
        say(f"crossover parity seed={seed}")
        layer = synth.make_layer(shape, seed, grad=True)
        for flags in (0, 2):
            got = run_layer(ops, shape, layer, flags=flags, backward=(seed == 1))
            compare_full(shape, layer, got, backward=(seed == 1))


# ---- full-size layers: every norm, sampled outputs ----------------------------------

def _sample(rng, n, k):
    return rng.integers(0, n, size=k)


@pytest.mark.parametrize("name", ["highrank_bf16", "widemlp_bf16"])
def test_fullsize_forward_sampled(ops, name):
    shape = synth.CONFIGS[name]
    say(f"full-size forward {name}")
    layer = synth.make_layer(shape, synth.CONFIG_SEED[name])
    for flags in (0, 2):
        got = run_layer(ops, shape, layer, flags=flags, backward=False)
        L = layer
        W0 = synth.to_f64(L["W0"], "bf16")
        A = synth.to_f64(L["A"], "bf16")
        B = synth.to_f64(L["B"], "bf16")
        n_ref = oracle.dora_norm(W0, A, B, shape.s)
        check_norm(got["norm"], n_ref, f"{name} norm (all rows)")
        rng = np.random.Generator(np.random.PCG64(7))
        tok = _sample(rng, shape.tokens, 4096)
        rows = _sample(rng, shape.d_out, 4096)
        tok[:8] = shape.tokens - 1
        rows[:8] = np.arange(shape.d_out - 8, shape.d_out)
        x = synth.to_f64(L["x"][np.unique(tok)], "bf16")
        remap = {t: i for i, t in enumerate(np.unique(tok))}
        m = synth.to_f64(L["m"], "bf16")
        y_ref = oracle.dora_forward_entries(x, W0, A, B, m, shape.s,
                                            np.array([remap[t] for t in tok]), rows)
        check_out(got["y"][tok, rows], y_ref, f"{name} y (sampled)")
        xs_ref = oracle.scaled_down_projection(x, A, shape.s)
        check_out(got["xs"][np.unique(tok)], xs_ref, f"{name} xs (sampled tokens)")
        del got


@pytest.mark.parametrize("name", ["highrank_bwd_bf16", "widemlp_bf16"])
def test_fullsize_backward_sampled(ops, name):
    """The backward at full size on sampled tokens, rows and columns: the 8192 x 8192
    (r 384) layer of the headline step and the 27648 x 5120 (r 256, T 8192) one,
    whose d_out != d_in and long K = d_out + r in dx."""
    shape = synth.CONFIGS[name]
    say(f"full-size backward {name}")
    layer = synth.make_layer(shape, synth.CONFIG_SEED[name], grad=True)
    got = run_layer(ops, shape, layer)
    L = synth.layer_f64(layer, "bf16")
    y_ref, n_ref = oracle.dora_forward(L["x"][:64], L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_norm(got["norm"], n_ref, "norm")
    check_out(got["y"][:64], y_ref, "y (first 64 tokens)")
    rng = np.random.Generator(np.random.PCG64(8))
    tok = np.unique(_sample(rng, shape.tokens, 48))
    rows = np.unique(_sample(rng, shape.d_out, 96))
    cols = np.unique(_sample(rng, shape.d_in, 96))
    tok[-1], rows[-1], cols[-1] = shape.tokens - 1, shape.d_out - 1, shape.d_in - 1
    ref = oracle.dora_backward_sampled(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s,
                                       tok, rows, cols)
    check_out(got["dx"][tok], ref["dx"], "dx (sampled tokens)")
    check_out(got["dB"][rows], ref["dB"], "dB (sampled rows)")
    check_out(got["dA"][:, cols], ref["dA"], "dA (sampled columns)")
    check_out(got["dm"][rows], ref["dm"], "dm (sampled rows)")


def test_long_batch_rebased_copies(ops):
    """A long token batch, T * d_out > 2^29: gz and x, the transposed operands of the
    dB and dA products, each span more than 1 GiB.  A buffer copy carries 32-bit
    offsets, so the copiers move their descriptor forward inside a launch (here at
    step 8192 of 10241, in the splits that reach it); ragged T checks the last step."""
    shape = LayerShape(1024, 1024, 64, 655397, 2.0, "bf16")
    assert shape.tokens * shape.d_out * 2 > 1 << 30
    say(f"long batch T={shape.tokens}")
    layer = synth.make_layer(shape, 71, grad=True)
    dev = layer_to_device(layer, "bf16")
    y, norm, xs = ops.dora_forward(dev["x"], dev["W0"], dev["A"], dev["B"], dev["m"], shape.s)
    gx, gA, gB, gm = ops.dora_backward(dev["gy"], dev["x"], dev["W0"], dev["A"], dev["B"], dev["m"],
                                       norm, xs, y, shape.s)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(72))
    tok = np.unique(np.concatenate([_sample(rng, shape.tokens, 48), [shape.tokens - 1]]))
    rows = np.unique(np.concatenate([_sample(rng, shape.d_out, 64), [shape.d_out - 1]]))
    cols = np.unique(np.concatenate([_sample(rng, shape.d_in, 64), [shape.d_in - 1]]))
    got_dx = download(gx[torch.from_numpy(tok).cuda()])
    got_dB, got_dA, got_dm = download(gB), download(gA), download(gm)
    del dev, y, xs, gx, gA, gB, gm
    torch.cuda.empty_cache()
    L = {k: synth.to_f64(v, "bf16") for k, v in layer.items()}
    del layer
    ref = oracle.dora_backward_sampled(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s,
                                       tok, rows, cols)
    check_out(got_dx, ref["dx"], "dx (sampled tokens)")
    check_out(got_dB[rows], ref["dB"], "dB (sampled rows)")
    check_out(got_dA[:, cols], ref["dA"], "dA (sampled columns)")
    check_out(got_dm[rows], ref["dm"], "dm (sampled rows)")


# ---- the three norm terms, separated by flipping B ------------------------------------

def test_norm_terms_separately(ops):
    """n^2(B) - n^2(-B) = 2 cross and n^2(B) + n^2(-B) = 2 (base + Gram), with the
    LoRA terms made comparable to the base term (B ~ N(0, 0.1^2))."""
    shape = LayerShape(1024, 2048, 64, 1, 2.0, "bf16")
    layer = synth.make_layer(shape, 12, b_std=0.1)
    dev = layer_to_device(layer, "bf16")
    n_p = download(ops.dora_norm(dev["W0"], dev["A"], dev["B"], shape.s))
    n_m = download(ops.dora_norm(dev["W0"], dev["A"], (-dev["B"].float()).to(torch.bfloat16), shape.s))
    L = synth.layer_f64(layer, "bf16")
    base, cross, gram = oracle.norm_terms(L["W0"], L["A"], L["B"], shape.s)
    say(f"cross/base ratio {np.abs(cross).mean() / base.mean():.3f}, gram/base {gram.mean() / base.mean():.3f}")
    check_out((n_p ** 2 - n_m ** 2) / 2, cross, "cross term", atol_frac=1e-3, min_cos=0.99999)
    check_out((n_p ** 2 + n_m ** 2) / 2, base + gram, "base + Gram", atol_frac=1e-4, min_cos=0.999999)
    # B = 0 leaves the base term alone: n = ||W0_i||
    n0 = download(ops.dora_norm(dev["W0"], dev["A"], torch.zeros_like(dev["B"]), shape.s))
    check_norm(n0, np.sqrt(base), "B = 0 norm", rtol=1e-5)


# ---- ||W0_i||^2 summed inside the cross/Gram projection -----------------------------

PROJ = [
    # 128 x 128 tiles, two K splits, the second of which sees no W0 step
    ("split_without_W0", LayerShape(1024, 64, 512, 0, 2.0, "bf16"), 21),
    # a partial 64-deep W0 step (d_in = 72) and a ragged last row tile
    ("ragged_W0_tail", LayerShape(1000, 72, 520, 0, 2.0, "bf16"), 22),
    # 256 x 128 tiles with four wave rows
    ("tiles_256x128", LayerShape(8192, 256, 1024, 0, 2.0, "bf16"), 23),
    # 256 x 256 tiles
    ("tiles_256x256", LayerShape(16384, 128, 4096, 0, 2.0, "bf16"), 24),
]


@pytest.mark.parametrize("name,shape,seed", PROJ, ids=[c[0] for c in PROJ])
def test_norm_projection_row_squares(ops, name, shape, seed):
    """Row norms when the base term comes from the projection's pass over W0,
    over the tile shapes and K splits the projection can take."""
    say(f"norm via projection row squares {name} shape={shape}")
    layer = synth.make_layer(shape, seed, b_std=0.05)
    dev = layer_to_device(layer, "bf16")
    n = download(ops.dora_norm(dev["W0"], dev["A"], dev["B"], shape.s))
    L = synth.layer_f64(layer, "bf16")
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = np.unique(np.concatenate([_sample(rng, shape.d_out, 512),
                                     np.arange(shape.d_out - 8, shape.d_out)]))
    n_ref = oracle.dora_norm(L["W0"][rows], L["A"], L["B"][rows], shape.s)
    check_norm(n[rows], n_ref, f"{name} norm (sampled rows)")
    # B = 0: the norm is ||W0_i|| alone
    n0 = download(ops.dora_norm(dev["W0"], dev["A"], torch.zeros_like(dev["B"]), shape.s))
    check_norm(n0[rows], np.linalg.norm(L["W0"][rows], axis=1), f"{name} B = 0 norm", rtol=1e-5)


# ---- near-unity rescaling (float32 storage, so the output can show it) ---------------

def test_near_unity_compose_f32(ops):
    """m = n (1 + 1e-4): y - x W'^T must be far below the 1e-4 rescaling itself.

    A compose that rounded g to a 16-bit float before subtracting 1 would be
    off by ~2e-3 |y|; the near-unity form keeps the error at float32 level.
    """
    shape = LayerShape(512, 1024, 32, 64, 2.0, "f32")
    layer = synth.make_layer(shape, 13)
    L = synth.layer_f64(layer, "f32")
    delta = 1e-4
    n_ref = oracle.dora_norm(L["W0"], L["A"], L["B"], shape.s)
    layer["m"] = (n_ref * (1 + delta)).astype(np.float32)
    L["m"] = layer["m"].astype(np.float64)
    y_ref, _ = oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    for flags in (0, 2):
        got = run_layer(ops, shape, layer, flags=flags, backward=False)
        err = np.max(np.abs(got["y"] - y_ref))
        say(f"near-unity flags={flags}: max err {err:.3e} vs delta*max|y| {delta * np.max(np.abs(y_ref)):.3e}")
        assert err <= 0.05 * delta * np.max(np.abs(y_ref))


# ---- determinism, memory, timing hook, argument errors ---------------------------------

def test_bitwise_deterministic(ops):
    shape = LayerShape(1032, 2056, 72, 515, 2.0, "bf16")
    layer = synth.make_layer(shape, 14, grad=True)
    a = run_layer(ops, shape, layer)
    b = run_layer(ops, shape, layer)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


def test_fused_and_separate_compose_agree(ops):
    shape = LayerShape(1032, 2056, 72, 515, 2.0, "bf16")
    layer = synth.make_layer(shape, 15)
    f = run_layer(ops, shape, layer, flags=0, backward=False)
    s = run_layer(ops, shape, layer, flags=2, backward=False)
    assert np.array_equal(f["norm"], s["norm"])
    err, scale, cos = out_stats(f["y"], s["y"])
    assert err <= 2 ** -6 * scale and cos > 0.99999, (err, scale, cos)


def test_no_dense_transient_memory(ops):
    """Peak device memory of a headline-size forward + backward is inputs, outputs and
    the declared workspace: no d_out x d_in buffer appears."""
    shape = synth.CONFIGS["highrank_bf16"]
    d_out, d_in, r, T = shape.d_out, shape.d_in, shape.r, shape.tokens
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(0)
    W0 = (torch.randn(d_out, d_in, device="cuda", generator=g) * 0.02).to(bf)
    A = ((torch.rand(r, d_in, device="cuda", generator=g) * 2 - 1) / d_in ** 0.5).to(bf)
    B = (torch.randn(d_out, r, device="cuda", generator=g) * 0.01).to(bf)
    m = torch.linalg.vector_norm(W0.float(), dim=1).to(bf)
    x = torch.randn(T, d_in, device="cuda", generator=g).to(bf)
    gy = torch.randn(T, d_out, device="cuda", generator=g).to(bf)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    y, norm, xs = ops.dora_forward(x, W0, A, B, m, shape.s)
    gx, gA, gB, gm = ops.dora_backward(gy, x, W0, A, B, m, norm, xs, y, shape.s)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    outputs = 2 * (T * d_out + T * r + T * d_in + r * d_in + d_out * r) + 8 * d_out
    ws = sum(ops.workspace_bytes(d_out, d_in, r, T, bf, op) for op in (1, 2))
    say(f"peak extra {peak / 1e6:.1f} MB; outputs {outputs / 1e6:.1f} MB; ws {ws / 1e6:.1f} MB; "
        f"dense d_out x d_in bf16 would be {d_out * d_in * 2 / 1e6:.0f} MB")
    assert peak <= outputs + ws + (32 << 20)
    # the only non-activation workspace (norm + forward) is far below one d_out x d_in matrix
    assert ops.workspace_bytes(d_out, d_in, r, T, bf, 1) < d_out * d_in * 2 / 2


def test_timing_hook(ops):
    shape = LayerShape(264, 520, 24, 37, 2.0, "bf16")
    layer = synth.make_layer(shape, 16, grad=True)
    ops.timing_enable(True)
    try:
        run_layer(ops, shape, layer)
        rec = ops.timing_collect()
    finally:
        ops.timing_enable(False)
    for k in ("gram_AAt", "gram_finalize", "cross_gram_proj", "fused_fwd_gemm", "compose_bwd", "dx_gemm"):
        assert k in rec and rec[k][0] >= 1 and rec[k][1] > 0, (k, rec)
    assert ops.timing_collect() == {}


@pytest.mark.parametrize("shape", [LayerShape(520, 1032, 136, 300, 2.0, "bf16"),
                                   LayerShape(4096, 4104, 136, 4096, 2.0, "bf16")],
                         ids=["small", "large"])
def test_side_stream_overlap_matches_serial(ops, shape):
    """On the large shape (forward GEMM and dx of at least 128 GFLOP) the
    down-projection (forward) and ts, dm (backward) run on a side stream beside
    the norm and the compose backward; with the timing hook on, and on the
    small shape, everything runs on the caller's stream.  Both orders must give
    the same bits (no shared buffer)."""
    layer = synth.make_layer(shape, 17, grad=True)
    outs = []
    for timing in (False, True, False):
        ops.timing_enable(timing)
        try:
            outs.append(run_layer(ops, shape, layer))
        finally:
            ops.timing_enable(False)
            ops.timing_collect()
    for k in outs[0]:
        for o in outs[1:]:
            assert np.array_equal(outs[0][k], o[k]), k


def test_measurement_probes(ops):
    """The bench's peak probes: the stream probe computes c = a + b exactly; the
    MFMA probe's checksum is finite and the same on every launch."""
    g = torch.Generator(device="cuda").manual_seed(5)
    n = (1 << 20) + 12   # a grid-stride tail
    a = torch.randn(n, device="cuda", generator=g)
    b = torch.randn(n, device="cuda", generator=g)
    c = torch.empty_like(a)
    ops.probe_stream(a, b, c)
    assert torch.equal(c, a + b)
    out1, flops = ops.probe_mfma(64, 8)
    first = out1.clone()
    ops.probe_mfma(64, 8, out=out1)
    torch.cuda.synchronize()
    assert torch.isfinite(first).all() and torch.equal(first, out1) and flops == 8 * 4 * 64 * 4 * 32768


def test_bad_arguments_raise_before_launch(ops):
    from parameter_efficient_fine_dora_amd._lib import DoraError, ERR_CODE
    W0 = torch.zeros(16, 17, dtype=torch.bfloat16, device="cuda")[:, 1:]
    A = torch.zeros(8, 16, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(16, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ops.dora_norm(W0, A, B, 2.0)          # not contiguous (caught by the binding)
    flat = torch.zeros(16 * 16 + 1, dtype=torch.bfloat16, device="cuda")
    W0m = flat[1:].view(16, 16)               # contiguous but 2-byte misaligned
    with pytest.raises(DoraError) as ei:
        ops.dora_norm(W0m, A, B, 2.0)
    assert ei.value.code == ERR_CODE["DORA_ERR_ALIGN"]
    W0o = torch.zeros(16, 12, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(DoraError) as ei:
        ops.dora_norm(W0o, torch.zeros(8, 12, dtype=torch.bfloat16, device="cuda"), B, 2.0)
    assert ei.value.code == ERR_CODE["DORA_ERR_SHAPE"]


def test_dora_linear_module(ops):
    from parameter_efficient_fine_dora_amd.module import DoRALinear
    shape = LayerShape(264, 520, 24, 37, 2.0, "bf16")
    layer = synth.make_layer(shape, 17, grad=True)
    dev = layer_to_device(layer, "bf16")
    mod = DoRALinear(dev["W0"], shape.r, shape.s)
    with torch.no_grad():
        mod.A.copy_(dev["A"]); mod.B.copy_(dev["B"]); mod.m.copy_(dev["m"])
    x = dev["x"].clone().requires_grad_(True)
    y = mod(x.view(1, shape.tokens, shape.d_in)).view(shape.tokens, shape.d_out)
    y.backward(dev["gy"])
    L = synth.layer_f64(layer, "bf16")
    y_ref, _ = oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    g = oracle.dora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_out(download(y), y_ref, "module y")
    check_out(download(x.grad), g["dx"], "module dx")
    check_out(download(mod.A.grad), g["dA"], "module dA")
    check_out(download(mod.B.grad), g["dB"], "module dB")
    check_out(download(mod.m.grad), g["dm"], "module dm")
    # a fresh module starts at the pretrained point: B = 0, m = ||W0_i||, so y = x W0^T
    fresh = DoRALinear(dev["W0"], shape.r, shape.s)
    y0 = download(fresh(dev["x"]))
    check_out(y0, L["x"] @ L["W0"].T, "fresh module y = x W0^T")


# ---- undetached norm gradient (DoRA reading notes, Appendix A.1) --------------------

EXACT = [
    ("ragged_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 21, {}),
    ("tiny_f32", synth.CONFIGS["tiny_f32"], 22, {}),
    ("multitile_bf16", LayerShape(520, 1032, 136, 300, 2.0, "bf16"), 23, {}),
    ("bigtile_ragged_bf16", LayerShape(776, 584, 72, 1031, 2.0, "bf16"), 24, {}),
    ("largeB_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 25, dict(b_std=0.1)),
    ("sneg_f32", LayerShape(136, 200, 16, 9, -0.75, "f32"), 26, {}),
    ("tokens0_bf16", LayerShape(136, 200, 16, 0, 2.0, "bf16"), 27, {}),
]


def aligned_grad_layer(shape, seed, kw):
    """Layer whose upstream gradient leans on y, so the projection of eq. (A.1) matters."""
    layer = synth.make_layer(shape, seed, grad=True, **kw)
    if shape.tokens:
        L = synth.layer_f64(layer, shape.dtype)
        y, _ = oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
        gy = L["gy"] + y / max(y.std(), 1e-30)
        layer["gy"] = (synth.bf16_bits(gy.astype(np.float32)) if shape.dtype == "bf16"
                       else gy.astype(np.float32))
    return layer


@pytest.mark.parametrize("flags", [1, 3], ids=["fused", "separate"])
@pytest.mark.parametrize("name,shape,seed,kw", EXACT, ids=[c[0] for c in EXACT])
def test_exact_norm_gradient(ops, name, shape, seed, kw, flags):
    say(f"exact gradient {name} flags={flags}")
    layer = aligned_grad_layer(shape, seed, kw)
    got = run_layer(ops, shape, layer, flags=flags)
    L = synth.layer_f64(layer, shape.dtype)
    g = oracle.dora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s, exact=True)
    for k in ("dx", "dA", "dB", "dm"):
        if g[k].size:
            check_out(got[k], g[k], "exact " + k)
    if shape.tokens and shape.r:
        # the detached result is measurably different here, so the flag is doing work
        det = run_layer(ops, shape, layer, flags=flags & ~1)
        err, scale, _ = out_stats(det["dB"], g["dB"])
        assert err > 0.05 * scale, "detached and exact gradients should differ on this layer"


def test_exact_norm_gradient_fullsize_sampled(ops):
    name = "highrank_bwd_bf16"
    shape = synth.CONFIGS[name]
    say(f"full-size exact backward {name}")
    layer = synth.make_layer(shape, synth.CONFIG_SEED[name], grad=True)
    got = run_layer(ops, shape, layer, flags=1)
    L = synth.layer_f64(layer, "bf16")
    rng = np.random.Generator(np.random.PCG64(9))
    tok = np.unique(_sample(rng, shape.tokens, 32))
    rows = np.unique(_sample(rng, shape.d_out, 96))
    cols = np.unique(_sample(rng, shape.d_in, 96))
    ref = oracle.dora_backward_sampled(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s,
                                       tok, rows, cols, exact=True)
    check_out(got["dx"][tok], ref["dx"], "exact dx (sampled tokens)")
    check_out(got["dB"][rows], ref["dB"], "exact dB (sampled rows)")
    check_out(got["dA"][:, cols], ref["dA"], "exact dA (sampled columns)")
    check_out(got["dm"][rows], ref["dm"], "exact dm (sampled rows)")


# ---- zero magnitudes: dm from the definition where y / m = z / n fails -------------

ZERO_M = [
    ("ragged_bf16", LayerShape(264, 520, 24, 37, 2.0, "bf16"), 31),
    ("ragged_f32", LayerShape(264, 520, 24, 37, 2.0, "f32"), 32),
    ("multitile_bf16", LayerShape(520, 1032, 136, 300, 2.0, "bf16"), 33),
]


@pytest.mark.parametrize("flags", [0, 1, 2, 3], ids=["fused", "fused_exact", "separate",
                                                     "separate_exact"])
@pytest.mark.parametrize("name,shape,seed", ZERO_M, ids=[c[0] for c in ZERO_M])
def test_zero_magnitude_rows(ops, name, shape, seed, flags):
    """Rows with m_i = 0 (a pruned magnitude): y_i = 0 exactly, every gradient finite
    and at the oracle's value, including dm_i (which the saved y cannot give)."""
    say(f"zero magnitudes {name} flags={flags}")
    layer = synth.make_layer(shape, seed, grad=True)
    zero = np.array([0, 5, shape.d_out // 2, shape.d_out - 1])
    layer["m"] = layer["m"].copy()
    layer["m"][zero] = 0
    got = run_layer(ops, shape, layer, flags=flags)
    for k, v in got.items():
        if v is not None:
            assert np.all(np.isfinite(v)), k
    assert not got["y"][:, zero].any(), "a zero magnitude gives a zero output column"
    L = synth.layer_f64(layer, shape.dtype)
    y_ref, n_ref = oracle.dora_forward(L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s)
    check_norm(got["norm"], n_ref, "norm")
    check_out(got["y"], y_ref, "y")
    g = oracle.dora_backward(L["gy"], L["x"], L["W0"], L["A"], L["B"], L["m"], shape.s,
                             exact=bool(flags & 1))
    for k in ("dx", "dA", "dB", "dm"):
        check_out(got[k], g[k], k)
    check_out(got["dm"][zero], g["dm"][zero], "dm of the zero-magnitude rows")


# ---- ragged token tile on the 256 x 256 (eight-wave) tile --------------------------

def test_ragged_rows_on_the_eight_wave_tile(ops):
    """T = 4100 on the 256 x 256 tile of the forward GEMM: its last tile-row holds 4
    tokens, so the copies of x must range-check every row they load."""
    shape = LayerShape(4096, 512, 16, 4100, 2.0, "bf16")
    say(f"ragged eight-wave tile {shape}")
    layer = synth.make_layer(shape, 34, grad=True)
    got = run_layer(ops, shape, layer)
    compare_full(shape, layer, got)
