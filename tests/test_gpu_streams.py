"""Streams, graphs and host threads.

The library runs on the caller's stream and forks independent work to a side
stream of its own (one per host thread and device), joining back through
events.  These tests check that the pattern survives HIP graph capture (the
captured forward + backward replays to the eager bits, with eager work and
synchronisations between replays) and concurrent calls from two host threads on
two streams (each reproduces the serial bits).
"""
from __future__ import annotations

import sys
import threading

import pytest
import torch

import synth
from synth import LayerShape
from tests.gpu_util import layer_to_device


# The forward forks its down-projection to the side stream only when its GEMM
# holds at least 128 GFLOP, the backward its ts chain only when dx does; the
# second shape is above that, the first below.
SHAPES = [LayerShape(520, 1032, 136, 300, 2.0, "bf16"),
          LayerShape(4096, 4104, 136, 4096, 2.0, "bf16")]
FORK_FLOP = 128e9


def test_shapes_cover_both_stream_arrangements():
    fwd = [2.0 * s.tokens * s.d_out * (s.d_in + s.r) for s in SHAPES]
    dx = [2.0 * s.tokens * s.d_in * (s.d_out + s.r) for s in SHAPES]
    assert fwd[0] < FORK_FLOP <= fwd[1] and dx[0] < FORK_FLOP <= dx[1]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from parameter_efficient_fine_dora_amd import ops as _ops, _lib
    _lib.lib()  # raises if the library is missing: there is no fallback
    return _ops


def buffers(ops, shape, dev):
    """Every output and workspace of one forward + backward, preallocated."""
    T, d_out, d_in, r = shape.tokens, shape.d_out, shape.d_in, shape.r
    bf = torch.bfloat16
    return dict(
        y=torch.empty(T, d_out, dtype=bf, device=dev), norm=torch.empty(d_out, device=dev),
        xs=torch.empty(T, r, dtype=bf, device=dev), gx=torch.empty(T, d_in, dtype=bf, device=dev),
        gA=torch.empty(r, d_in, dtype=bf, device=dev), gB=torch.empty(d_out, r, dtype=bf, device=dev),
        gm=torch.empty(d_out, device=dev),
        ws_f=torch.empty(ops.workspace_bytes(d_out, d_in, r, T, bf, 1), dtype=torch.uint8, device=dev),
        ws_b=torch.empty(ops.workspace_bytes(d_out, d_in, r, T, bf, 2), dtype=torch.uint8, device=dev))


def step(ops, d, o, s):
    ops.dora_forward(d["x"], d["W0"], d["A"], d["B"], d["m"], s, y=o["y"], norm_out=o["norm"],
                     xs_out=o["xs"], workspace=o["ws_f"])
    ops.dora_backward(d["gy"], d["x"], d["W0"], d["A"], d["B"], d["m"], o["norm"], o["xs"], o["y"],
                      s, grad_x=o["gx"], grad_A=o["gA"], grad_B=o["gB"], grad_m=o["gm"],
                      workspace=o["ws_b"])


OUTS = ("y", "norm", "xs", "gx", "gA", "gB", "gm")


@pytest.mark.parametrize("SHAPE", SHAPES, ids=["small", "large"])
@pytest.mark.gpu
def test_graph_capture_replays_to_eager_bits(ops, SHAPE):
    say(f"graph capture of forward + backward {SHAPE}")
    layer = synth.make_layer(SHAPE, 61, grad=True)
    d = layer_to_device(layer, "bf16")
    eager = buffers(ops, SHAPE, "cuda")
    step(ops, d, eager, SHAPE.s)
    torch.cuda.synchronize()
    ref = {k: eager[k].clone() for k in OUTS}

    o = buffers(ops, SHAPE, "cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture thread (creates the side stream)
        step(ops, d, o, SHAPE.s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(ops, d, o, SHAPE.s)
    for rep in range(3):
        for k in OUTS:
            o[k].fill_(0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(o[k], ref[k]), (rep, k)
        step(ops, d, eager, SHAPE.s)   # and the eager path still agrees in between
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(eager[k], ref[k]), (rep, k, "eager")


@pytest.mark.parametrize("SHAPE", SHAPES, ids=["small", "large"])
@pytest.mark.gpu
def test_two_host_threads_two_streams(ops, SHAPE):
    say(f"two host threads, two streams {SHAPE}")
    layer = synth.make_layer(SHAPE, 62, grad=True)
    d = layer_to_device(layer, "bf16")
    serial = buffers(ops, SHAPE, "cuda")
    step(ops, d, serial, SHAPE.s)
    torch.cuda.synchronize()
    outs = [buffers(ops, SHAPE, "cuda") for _ in range(2)]
    errors = []

    def worker(o):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(4):
                    step(ops, d, o, SHAPE.s)
            st.synchronize()
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(o,)) for o in outs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert not any(t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for o in outs:
        for k in OUTS:
            assert torch.equal(o[k], serial[k]), k
