"""DoRA and DVoRA linear layers on top of the C ABI (autograd glue only).

Forward saves norm, xs = s (x A^T) and y for the backward; the norm is
detached there (DoRA reading notes, Sec. 3.4).  DVoRA (Sec. 3.5) runs the same
entry points with B = diag(b) B_shared diag(d).
"""
from __future__ import annotations

import math

import torch

from . import ops


class DoRAFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, W0, A, B, m, s, flags):
        y, norm, xs = ops.dora_forward(x, W0, A, B, m, s, flags=flags)
        ctx.s = s
        ctx.flags = flags
        ctx.save_for_backward(x, W0, A, B, m, norm, xs, y)
        ctx.mark_non_differentiable(norm)
        return y, norm

    @staticmethod
    def backward(ctx, gy, _gnorm):
        x, W0, A, B, m, norm, xs, y = ctx.saved_tensors
        need = tuple(n for n, k in (("x", 0), ("A", 2), ("B", 3), ("m", 4))
                     if ctx.needs_input_grad[k])
        gx, gA, gB, gm = ops.dora_backward(gy.contiguous(), x, W0, A, B, m, norm, xs, y, ctx.s,
                                           need=need, flags=ctx.flags)
        if gm is not None:
            gm = gm.to(m.dtype)
        return gx, None, gA, gB, gm, None, None


class DoRALinear(torch.nn.Module):
    """y = (m / ||W0 + s B A||_row) * (x W0^T + s (x A^T) B^T), W0 frozen.

    Initialised as DoRA starts training (DoRA reading notes, Algorithm 1):
    m = row norms of W0, A Kaiming-uniform, B = 0.
    """

    def __init__(self, weight: torch.Tensor, r: int, s: float = 2.0, flags: int = 0):
        super().__init__()
        d_out, d_in = weight.shape
        dev, dt = weight.device, weight.dtype
        self.register_buffer("W0", weight.detach().contiguous())
        self.A = torch.nn.Parameter(torch.empty(r, d_in, device=dev, dtype=dt))
        torch.nn.init.kaiming_uniform_(self.A, a=math.sqrt(5))
        self.B = torch.nn.Parameter(torch.zeros(d_out, r, device=dev, dtype=dt))
        self.m = torch.nn.Parameter(torch.empty(d_out, device=dev, dtype=dt))
        with torch.no_grad():
            self.m.copy_(ops.dora_norm(self.W0, self.A, self.B, s).to(dt))
        self.s = float(s)
        self.flags = int(flags)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        y, _ = DoRAFunction.apply(x2, self.W0, self.A, self.B, self.m, self.s, self.flags)
        return y.reshape(*lead, y.shape[-1])


class DVoRAFunction(torch.autograd.Function):
    """DoRA with VeRA's direction update: A_shared, B_shared frozen; b, d, m trained."""

    @staticmethod
    def forward(ctx, x, W0, A_sh, B_sh, b, d, m, s, flags):
        Be = ops.dora_vera_scale(B_sh, b, d)
        y, norm, xs = ops.dora_forward(x, W0, A_sh, Be, m, s, flags=flags)
        ctx.s = s
        ctx.flags = flags
        ctx.save_for_backward(x, W0, A_sh, B_sh, b, d, Be, m, norm, xs, y)
        return y

    @staticmethod
    def backward(ctx, gy):
        x, W0, A_sh, B_sh, b, d, Be, m, norm, xs, y = ctx.saved_tensors
        want_vec = ctx.needs_input_grad[4] or ctx.needs_input_grad[5]
        need = tuple(n for n, ok in (("x", ctx.needs_input_grad[0]), ("B", want_vec),
                                      ("m", ctx.needs_input_grad[6])) if ok)
        gx, _, gBe, gm = ops.dora_backward(gy.contiguous(), x, W0, A_sh, Be, m, norm, xs, y, ctx.s,
                                           need=need, flags=ctx.flags)
        gb = gd = None
        if want_vec:
            gb, gd = ops.dora_vera_grads(gBe, B_sh, b, d)
        if gm is not None:
            gm = gm.to(m.dtype)
        return gx, None, None, None, gb, gd, gm, None, None


class DVoRALinear(torch.nn.Module):
    """DVoRA layer: y = (m / ||V'||_row) x V'^T, V' = W0 + s diag(b) B_sh diag(d) A_sh.

    A_shared [r, d_in] and B_shared [d_out, r] are frozen (shared by every layer
    of a model); the trainable vectors start at b = 0 (the update starts at zero,
    as DoRA's B = 0 does) and d = d_init, with m = ||W0_i||.
    """

    def __init__(self, weight, A_shared, B_shared, s: float = 1.0, d_init: float = 0.1,
                 flags: int = 0):
        super().__init__()
        d_out, d_in = weight.shape
        r = A_shared.shape[0]
        dev, dt = weight.device, weight.dtype
        self.register_buffer("W0", weight.detach().contiguous())
        self.register_buffer("A_shared", A_shared.detach().contiguous())
        self.register_buffer("B_shared", B_shared.detach().contiguous())
        self.b = torch.nn.Parameter(torch.zeros(d_out, device=dev, dtype=dt))
        self.d = torch.nn.Parameter(torch.full((r,), float(d_init), device=dev, dtype=dt))
        self.m = torch.nn.Parameter(torch.empty(d_out, device=dev, dtype=dt))
        with torch.no_grad():
            Be = ops.dora_vera_scale(self.B_shared, self.b, self.d)
            self.m.copy_(ops.dora_norm(self.W0, self.A_shared, Be, s).to(dt))
        self.s = float(s)
        self.flags = int(flags)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        y = DVoRAFunction.apply(x2, self.W0, self.A_shared, self.B_shared, self.b, self.d, self.m,
                                self.s, self.flags)
        return y.reshape(*lead, y.shape[-1])
