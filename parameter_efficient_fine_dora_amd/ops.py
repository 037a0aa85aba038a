"""Thin torch binding of libdora.so: same names as the C ABI.

Only argument marshalling happens here: tensors are checked for device,
dtype, shape and contiguity, output and workspace buffers are allocated by
torch's caching allocator (the library allocates nothing), and the raw device
pointers plus torch's current HIP stream are passed to the library.  Every
step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
import json

import torch

from . import _lib
from ._lib import DoraError, FLAG_EXACT_NORM_GRAD, FLAG_SEPARATE_COMPOSE  # noqa: F401

_DT = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype=None, shape=None, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _layer_dtype(W0):
    if W0.dtype not in _DT:
        raise ValueError(f"unsupported dtype {W0.dtype}; use float32 or bfloat16")
    return _DT[W0.dtype]


def _ws(sh, op, dev, workspace):
    nbytes = _lib.workspace_bytes(sh, op)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def _check(rc, what):
    if rc != 0:
        raise DoraError(rc, what)


def workspace_bytes(d_out, d_in, r, tokens, dtype, op, flags=0) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return _lib.workspace_bytes(_lib.shape(d_out, d_in, r, tokens, dt, 1.0, flags), op)


def dora_norm(W0, A, B, s, *, out=None, workspace=None, flags=0):
    """Row norms ||W0_i + s (BA)_i|| (float32 [d_out]) by the factored method."""
    dev = W0.device
    dt = W0.dtype
    d_out, d_in = W0.shape
    r = A.shape[0]
    _need(W0, "W0", dt, (d_out, d_in))
    _need(A, "A", dt, (r, d_in), dev)
    _need(B, "B", dt, (d_out, r), dev)
    sh = _lib.shape(d_out, d_in, r, 0, _layer_dtype(W0), s, flags)
    if out is None:
        out = torch.empty(d_out, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (d_out,), dev)
    ws, nb = _ws(sh, _lib.OP_NORM, dev, workspace)
    _check(_lib.lib().dora_norm(ctypes.byref(sh), _ptr(W0), _ptr(A), _ptr(B), _ptr(out), _ptr(ws),
                                nb, _stream(dev)), "dora_norm")
    return out


def dora_forward(x, W0, A, B, m, s, *, y=None, norm_out=None, xs_out=None, keep_xs=True,
                 workspace=None, flags=0):
    """DoRA linear forward.  Returns (y [T, d_out], norm [d_out] f32, xs [T, r] or None)."""
    dev = W0.device
    dt = W0.dtype
    d_out, d_in = W0.shape
    r = A.shape[0]
    T = x.shape[0]
    _need(W0, "W0", dt)
    _need(x, "x", dt, (T, d_in), dev)
    _need(A, "A", dt, (r, d_in), dev)
    _need(B, "B", dt, (d_out, r), dev)
    _need(m, "m", dt, (d_out,), dev)
    sh = _lib.shape(d_out, d_in, r, T, _layer_dtype(W0), s, flags)
    if y is None:
        y = torch.empty(T, d_out, dtype=dt, device=dev)
    if norm_out is None:
        norm_out = torch.empty(d_out, dtype=torch.float32, device=dev)
    if xs_out is None and keep_xs:
        xs_out = torch.empty(T, r, dtype=dt, device=dev)
    _need(y, "y", dt, (T, d_out), dev)
    _need(norm_out, "norm_out", torch.float32, (d_out,), dev)
    if xs_out is not None:
        _need(xs_out, "xs_out", dt, (T, r), dev)
    ws, nb = _ws(sh, _lib.OP_FORWARD, dev, workspace)
    _check(_lib.lib().dora_forward(ctypes.byref(sh), _ptr(x), _ptr(W0), _ptr(A), _ptr(B), _ptr(m),
                                   _ptr(y), _ptr(norm_out), _ptr(xs_out), _ptr(ws), nb,
                                   _stream(dev)), "dora_forward")
    return y, norm_out, xs_out


def dora_forward_noalloc(x, W0, A, B, m, s, *, y=None, norm_out=None, xs_out=None, flags=0):
    """dora_forward on the library's static workspace (no workspace argument; the
    library allocates nothing).  Outputs not given are allocated here by torch,
    before the call.  Returns (y, norm, xs or None)."""
    dev = W0.device
    dt = W0.dtype
    d_out, d_in = W0.shape
    r = A.shape[0]
    T = x.shape[0]
    _need(W0, "W0", dt)
    _need(x, "x", dt, (T, d_in), dev)
    _need(A, "A", dt, (r, d_in), dev)
    _need(B, "B", dt, (d_out, r), dev)
    _need(m, "m", dt, (d_out,), dev)
    sh = _lib.shape(d_out, d_in, r, T, _layer_dtype(W0), s, flags)
    if y is None:
        y = torch.empty(T, d_out, dtype=dt, device=dev)
    if norm_out is None:
        norm_out = torch.empty(d_out, dtype=torch.float32, device=dev)
    _need(y, "y", dt, (T, d_out), dev)
    _need(norm_out, "norm_out", torch.float32, (d_out,), dev)
    if xs_out is not None:
        _need(xs_out, "xs_out", dt, (T, r), dev)
    _check(_lib.lib().dora_forward_noalloc(ctypes.byref(sh), _ptr(x), _ptr(W0), _ptr(A), _ptr(B),
                                           _ptr(m), _ptr(y), _ptr(norm_out), _ptr(xs_out),
                                           _stream(dev)), "dora_forward_noalloc")
    return y, norm_out, xs_out


def dora_backward(grad_y, x, W0, A, B, m, norm, xs, y, s, *, need=("x", "A", "B", "m"),
                  grad_x=None, grad_A=None, grad_B=None, grad_m=None, workspace=None, flags=0):
    """DoRA linear backward with the norm detached.

    Returns (grad_x, grad_A, grad_B, grad_m); entries not in ``need`` are None.
    grad_m is float32.
    """
    dev = W0.device
    dt = W0.dtype
    d_out, d_in = W0.shape
    r = A.shape[0]
    T = x.shape[0]
    _need(grad_y, "grad_y", dt, (T, d_out), dev)
    _need(x, "x", dt, (T, d_in), dev)
    _need(W0, "W0", dt)
    _need(A, "A", dt, (r, d_in), dev)
    _need(B, "B", dt, (d_out, r), dev)
    _need(m, "m", dt, (d_out,), dev)
    _need(norm, "norm", torch.float32, (d_out,), dev)
    _need(y, "y", dt, (T, d_out), dev)
    if xs is not None:
        _need(xs, "xs", dt, (T, r), dev)
    sh = _lib.shape(d_out, d_in, r, T, _layer_dtype(W0), s, flags)
    if "x" in need and grad_x is None:
        grad_x = torch.empty(T, d_in, dtype=dt, device=dev)
    if "A" in need and grad_A is None:
        grad_A = torch.empty(r, d_in, dtype=dt, device=dev)
    if "B" in need and grad_B is None:
        grad_B = torch.empty(d_out, r, dtype=dt, device=dev)
    if "m" in need and grad_m is None:
        grad_m = torch.empty(d_out, dtype=torch.float32, device=dev)
    for t, nm, shp, tdt in ((grad_x, "grad_x", (T, d_in), dt), (grad_A, "grad_A", (r, d_in), dt),
                            (grad_B, "grad_B", (d_out, r), dt),
                            (grad_m, "grad_m", (d_out,), torch.float32)):
        if t is not None:
            _need(t, nm, tdt, shp, dev)
    ws, nb = _ws(sh, _lib.OP_BACKWARD, dev, workspace)
    _check(_lib.lib().dora_backward(ctypes.byref(sh), _ptr(grad_y), _ptr(x), _ptr(W0), _ptr(A),
                                    _ptr(B), _ptr(m), _ptr(norm), _ptr(xs), _ptr(y), _ptr(grad_x),
                                    _ptr(grad_A), _ptr(grad_B), _ptr(grad_m), _ptr(ws), nb,
                                    _stream(dev)), "dora_backward")
    return grad_x, grad_A, grad_B, grad_m


def dora_merge(W0, A, B, m, s, *, norm=None, out=None, workspace=None):
    """Merged weight g_i (W0_i + s (BA)_i) for deployment ([d_out, d_in], layer dtype).

    ``norm`` (float32 [d_out], as from dora_norm / dora_forward) is computed when None.
    """
    dev = W0.device
    dt = W0.dtype
    d_out, d_in = W0.shape
    r = A.shape[0]
    _need(W0, "W0", dt)
    _need(A, "A", dt, (r, d_in), dev)
    _need(B, "B", dt, (d_out, r), dev)
    _need(m, "m", dt, (d_out,), dev)
    if norm is not None:
        _need(norm, "norm", torch.float32, (d_out,), dev)
    sh = _lib.shape(d_out, d_in, r, 0, _layer_dtype(W0), s)
    if out is None:
        out = torch.empty(d_out, d_in, dtype=dt, device=dev)
    _need(out, "out", dt, (d_out, d_in), dev)
    ws, nb = _ws(sh, _lib.OP_MERGE, dev, workspace)
    _check(_lib.lib().dora_merge(ctypes.byref(sh), _ptr(W0), _ptr(A), _ptr(B), _ptr(m),
                                 _ptr(norm), _ptr(out), _ptr(ws), nb, _stream(dev)), "dora_merge")
    return out


def dora_vera_scale(B_shared, b, d, *, out=None):
    """DVoRA's effective B = diag(b) B_shared diag(d) ([d_out, r], layer dtype)."""
    dev = B_shared.device
    dt = B_shared.dtype
    d_out, r = B_shared.shape
    _need(b, "b", dt, (d_out,), dev)
    _need(d, "d", dt, (r,), dev)
    sh = _lib.shape(d_out, 8, r, 0, _layer_dtype(B_shared), 1.0)
    if out is None:
        out = torch.empty(d_out, r, dtype=dt, device=dev)
    _need(out, "out", dt, (d_out, r), dev)
    _check(_lib.lib().dora_vera_scale(ctypes.byref(sh), _ptr(B_shared), _ptr(b), _ptr(d), _ptr(out),
                                      _stream(dev)), "dora_vera_scale")
    return out


def dora_vera_grads(grad_B_eff, B_shared, b, d, *, need=("b", "d"), workspace=None):
    """DVoRA's vector gradients from grad_B_eff: returns (grad_b [d_out], grad_d [r])."""
    dev = B_shared.device
    dt = B_shared.dtype
    d_out, r = B_shared.shape
    _need(grad_B_eff, "grad_B_eff", dt, (d_out, r), dev)
    _need(b, "b", dt, (d_out,), dev)
    _need(d, "d", dt, (r,), dev)
    sh = _lib.shape(d_out, 8, r, 0, _layer_dtype(B_shared), 1.0)
    gb = torch.empty(d_out, dtype=dt, device=dev) if "b" in need else None
    gd = torch.empty(r, dtype=dt, device=dev) if "d" in need else None
    ws, nb = _ws(sh, _lib.OP_VERA_GRADS, dev, workspace)
    _check(_lib.lib().dora_vera_grads(ctypes.byref(sh), _ptr(grad_B_eff), _ptr(B_shared), _ptr(b),
                                      _ptr(d), _ptr(gb), _ptr(gd), _ptr(ws), nb, _stream(dev)),
           "dora_vera_grads")
    return gb, gd


def timing_enable(on: bool = True):
    _lib.lib().dora_timing_enable(1 if on else 0)


def timing_collect() -> dict:
    """{kernel label: (launch count, total ms)} since the last collect."""
    buf = ctypes.create_string_buffer(1 << 16)
    rc = _lib.lib().dora_timing_collect(buf, len(buf))
    if rc < 0:
        raise DoraError(rc, "dora_timing_collect")
    return {k: (int(v[0]), float(v[1])) for k, v in json.loads(buf.value.decode()).items()}


def probe_mfma(iters: int, blocks: int, *, out=None):
    """Launch the sustained-MFMA probe on the current stream; returns (out, flops)."""
    import torch
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    L = _lib.lib()
    rc = L.dora_probe_mfma(int(iters), int(blocks), out.data_ptr(), st)
    if rc != 0:
        raise DoraError(rc, "dora_probe_mfma")
    return out, L.dora_probe_mfma_flops(int(iters), int(blocks))


def probe_stream(a, b, c):
    """c = a + b over float32 tensors on the current stream (HBM streaming probe)."""
    import torch
    for t in (a, b, c):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != a.numel():
            raise ValueError("probe_stream takes three contiguous float32 tensors of one size")
    st = torch.cuda.current_stream().cuda_stream
    rc = _lib.lib().dora_probe_stream(a.data_ptr(), b.data_ptr(), c.data_ptr(), a.numel() * 4, st)
    if rc != 0:
        raise DoraError(rc, "dora_probe_stream")
    return c

