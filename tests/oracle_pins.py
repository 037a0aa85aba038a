"""Pins for the float64 oracle: checks that tie it to something other than itself.

Each ``pin_*`` takes an oracle module and raises AssertionError (or any
exception) if the oracle disagrees with
  * the hand-worked integer rows in tests/golden/worked_rows.json,
  * pure-Python brute-force loops on tiny layers,
  * the factored-norm identity (Scaling DoRA abstract: base + cross + Gram),
  * special cases with textbook answers (B = 0 is weight normalisation,
    DoRA reading notes eq. (2)-(3); m = n reduces to LoRA, eq. (1); s = 0),
  * invariances (joint scaling of W0 and B, token permutation),
  * central finite differences of the forward for the detached (Sec. 3.4,
    eq. (7)-(8)) and exact (Appendix A.1) gradients, and eq. (8)'s
    norm-times-cosine closed form.
tests/test_oracle_pins.py runs them on the real oracle;
tests/test_oracle_mutants.py plants mistakes in copies of the oracle and
checks that some pin catches each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_rows.json")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _layer(seed, d_out=6, d_in=9, r=3, T=5, b_std=0.3):
    """Small float64 layer with O(1) LoRA terms (non-square on every axis)."""
    g = _rng(seed)
    W0 = g.standard_normal((d_out, d_in))
    A = g.uniform(-1, 1, (r, d_in))
    B = g.standard_normal((d_out, r)) * b_std
    m = np.linalg.norm(W0, axis=1) * (1 + g.uniform(-0.3, 0.3, d_out))
    x = g.standard_normal((T, d_in))
    gy = g.standard_normal((T, d_out))
    return W0, A, B, m, x, gy


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max|diff| {err:.3e} > {rtol:g} * {scale:.3e}"


# ---------------------------------------------------------------------------

def pin_worked_rows(orc):
    with open(GOLDEN) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        W0, A, B = (np.array(e[k], dtype=np.float64) for k in ("W0", "A", "B"))
        s = e["s"]
        n = orc.dora_norm(W0, A, B, s)
        _close(n, e["norm"], 1e-15, e["name"] + " norm")
        _close(n * n, e["norm_sq"], 1e-14, e["name"] + " norm^2")
        base, cross, gram = orc.norm_terms(W0, A, B, s)
        _close(base, e["base"], 0, e["name"] + " base")
        assert np.array_equal(cross, np.array(e["cross"], dtype=float)), e["name"] + " cross"
        assert np.array_equal(gram, np.array(e["gram"], dtype=float)), e["name"] + " gram"
        if "y" in e:
            y, _ = orc.dora_forward(np.array(e["x"], float), W0, A, B, np.array(e["m"], float), s)
            _close(y, e["y"], 1e-15, e["name"] + " y")
        if "merged" in e:
            Wm = orc.merged_weight(W0, A, B, np.array(e["m"], float), s)
            _close(Wm, e["merged"], 1e-15, e["name"] + " merged")
        if "gy" in e:
            gr = orc.dora_backward(np.array(e["gy"], float), np.array(e["x"], float), W0, A, B,
                                   np.array(e["m"], float), s)
            for k in ("dm", "dB", "dA", "dx"):
                _close(gr[k], e[k], 1e-15, e["name"] + " " + k)


def brute_norm_forward(x, W0, A, B, m, s):
    """Pure-Python loops: V'_ik = W0_ik + s*sum_j B_ij A_jk; n_i; y_ti = sum_k x_tk*(m_i/n_i)*V'_ik."""
    d_out, d_in = len(W0), len(W0[0])
    r = len(A)
    V = [[W0[i][k] + s * sum(B[i][j] * A[j][k] for j in range(r)) for k in range(d_in)]
         for i in range(d_out)]
    n = [math.sqrt(sum(v * v for v in V[i])) for i in range(d_out)]
    y = [[sum(x[t][k] * (m[i] / n[i]) * V[i][k] for k in range(d_in)) for i in range(d_out)]
         for t in range(len(x))]
    return n, y


def pin_bruteforce(orc):
    for seed, (d_out, d_in, r, T) in enumerate([(4, 6, 3, 2), (3, 5, 1, 3), (2, 6, 2, 1)]):
        W0, A, B, m, x, _ = _layer(100 + seed, d_out, d_in, r, T)
        s = 1.5
        n_ref, y_ref = brute_norm_forward(x.tolist(), W0.tolist(), A.tolist(), B.tolist(), m.tolist(), s)
        _close(orc.dora_norm(W0, A, B, s), n_ref, 1e-13, "brute norm")
        y, n = orc.dora_forward(x, W0, A, B, m, s)
        _close(n, n_ref, 1e-13, "brute forward norm")
        _close(y, y_ref, 1e-13, "brute y")
        xs_ref = [[s * sum(x[t][k] * A[j][k] for k in range(d_in)) for j in range(r)]
                  for t in range(T)]
        _close(orc.scaled_down_projection(x, A, s), xs_ref, 1e-13, "brute xs")


def pin_factored_identity(orc):
    for seed, b_std in [(1, 0.3), (2, 3.0), (3, 0.01)]:
        W0, A, B, m, x, _ = _layer(seed, 7, 11, 4, 3, b_std)
        for s in (2.0, -0.7):
            n = orc.dora_norm(W0, A, B, s)
            base, cross, gram = orc.norm_terms(W0, A, B, s)
            _close(n * n, base + cross + gram, 1e-12, f"factored identity b_std={b_std} s={s}")
            # cross flips sign with B, Gram does not
            base2, cross2, gram2 = orc.norm_terms(W0, A, -B, s)
            _close(cross2, -cross, 1e-15, "cross odd in B")
            _close(gram2, gram, 1e-15, "gram even in B")
            # Gram term equals ||s (BA)_i||^2 computed with the library's row norm
            _close(gram, np.linalg.norm(s * (B @ A), axis=1) ** 2, 1e-12, "gram = ||sBA||^2")
            _close(base, np.linalg.norm(W0, axis=1) ** 2, 1e-14, "base = ||W0||^2")


def pin_b_zero(orc):
    W0, A, B, m, x, _ = _layer(4)
    B = np.zeros_like(B)
    n = orc.dora_norm(W0, A, B, 2.0)
    _close(n, np.linalg.norm(W0, axis=1), 1e-15, "B=0 norm is ||W0_i||")
    y, _ = orc.dora_forward(x, W0, A, B, np.linalg.norm(W0, axis=1), 2.0)
    _close(y, x @ W0.T, 1e-14, "B=0, m=||W0_i|| gives y = x W0^T")


def pin_g_one_is_lora(orc):
    W0, A, B, _, x, _ = _layer(5)
    s = 1.25
    m = orc.dora_norm(W0, A, B, s)
    y, _ = orc.dora_forward(x, W0, A, B, m, s)
    _close(y, x @ W0.T + s * ((x @ A.T) @ B.T), 1e-13, "m = n reduces to LoRA output")


def pin_scale_invariance(orc):
    W0, A, B, m, x, _ = _layer(6)
    s, c = 2.0, 3.5
    n = orc.dora_norm(W0, A, B, s)
    _close(orc.dora_norm(c * W0, A, c * B, s), c * n, 1e-14, "norm scales with (W0, B)")
    y, _ = orc.dora_forward(x, W0, A, B, m, s)
    y2, _ = orc.dora_forward(x, c * W0, A, c * B, m, s)
    _close(y2, y, 1e-13, "y invariant to joint scaling of (W0, B)")
    y3, _ = orc.dora_forward(x, W0, A, B, 2.0 * m, s)
    _close(y3, 2.0 * y, 1e-14, "y linear in m")


def pin_s_zero_weightnorm(orc):
    W0, A, B, m, x, _ = _layer(7)
    y, n = orc.dora_forward(x, W0, A, B, m, 0.0)
    wn = np.linalg.norm(W0, axis=1)
    _close(n, wn, 1e-15, "s=0 norm")
    _close(y, x @ ((m / wn)[:, None] * W0).T, 1e-13, "s=0 is weight normalisation")


def pin_token_permutation(orc):
    W0, A, B, m, x, _ = _layer(8, T=7)
    perm = _rng(9).permutation(7)
    y, _ = orc.dora_forward(x, W0, A, B, m, 2.0)
    yp, _ = orc.dora_forward(x[perm], W0, A, B, m, 2.0)
    _close(yp, y[perm], 1e-15, "token permutation equivariance")


def _fd_grads(orc, params, s, gy, frozen_norm):
    """Central differences of L = sum(gy * y) w.r.t. x, A, B, m."""
    def loss(p):
        if frozen_norm is not None:
            y, _ = orc.dora_forward(p["x"], p["W0"], p["A"], p["B"], p["m"], s, norm=frozen_norm)
        else:
            y, _ = orc.dora_forward(p["x"], p["W0"], p["A"], p["B"], p["m"], s)
        return float(np.sum(gy * y))

    out = {}
    for name in ("x", "A", "B", "m"):
        base = params[name]
        grad = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            h = 1e-6 * max(1.0, abs(base[idx]))
            p = dict(params)
            plus = base.copy(); plus[idx] += h
            minus = base.copy(); minus[idx] -= h
            p[name] = plus; lp = loss(p)
            p[name] = minus; lm = loss(p)
            grad[idx] = (lp - lm) / (2 * h)
        out["d" + name] = grad
    return out


def pin_fd_detached(orc):
    W0, A, B, m, x, gy = _layer(10, 4, 5, 2, 3)
    s = 1.7
    n0 = orc.dora_norm(W0, A, B, s)
    fd = _fd_grads(orc, dict(W0=W0, A=A, B=B, m=m, x=x), s, gy, frozen_norm=n0)
    an = orc.dora_backward(gy, x, W0, A, B, m, s)
    for k in ("dx", "dA", "dB", "dm"):
        _close(an[k], fd[k], 1e-6, "detached FD " + k)


def pin_fd_exact(orc):
    W0, A, B, m, x, gy = _layer(11, 4, 5, 2, 3)
    s = 1.7
    fd = _fd_grads(orc, dict(W0=W0, A=A, B=B, m=m, x=x), s, gy, frozen_norm=None)
    an = orc.dora_backward(gy, x, W0, A, B, m, s, exact=True)
    for k in ("dx", "dA", "dB", "dm"):
        _close(an[k], fd[k], 1e-6, "exact FD " + k)


def pin_fd_zero_magnitude(orc):
    """Rows whose magnitude is zero (pruned, or trained to 0): y_i is then 0, but
    L still depends on m_i, so dm_i is the finite difference, not 0 or NaN;
    detached (n frozen) and exact."""
    W0, A, B, m, x, gy = _layer(15, 4, 5, 2, 3)
    m = m.copy()
    m[[1, 3]] = 0.0
    s = 1.3
    n0 = orc.dora_norm(W0, A, B, s)
    for frozen, exact in ((n0, False), (None, True)):
        fd = _fd_grads(orc, dict(W0=W0, A=A, B=B, m=m, x=x), s, gy, frozen_norm=frozen)
        an = orc.dora_backward(gy, x, W0, A, B, m, s, exact=exact)
        for k in ("dx", "dA", "dB", "dm"):
            assert np.all(np.isfinite(an[k])), k
            _close(an[k], fd[k], 1e-6, f"m_i = 0 FD {k} (exact={exact})")
        assert np.all(np.abs(an["dm"][[1, 3]]) > 1e-3), "a zero magnitude still has a gradient"


def pin_eq8_closed_form(orc):
    W0, A, B, m, x, gy = _layer(12)
    s = 2.0
    dWp = gy.T @ x
    V = W0 + s * (B @ A)
    cos = np.sum(dWp * V, axis=1) / (np.linalg.norm(dWp, axis=1) * np.linalg.norm(V, axis=1))
    dm = orc.dora_backward(gy, x, W0, A, B, m, s)["dm"]
    _close(dm, np.linalg.norm(dWp, axis=1) * cos, 1e-13, "eq. 8: dm = ||dW'|| cos(dW', V')")


def pin_b_zero_backward(orc):
    W0, A, B, m, x, gy = _layer(13)
    B = np.zeros_like(B)
    s = 2.0
    gr = orc.dora_backward(gy, x, W0, A, B, m, s)
    assert np.all(gr["dA"] == 0.0), "B=0 gives dA = 0 exactly"
    g = m / np.linalg.norm(W0, axis=1)
    _close(gr["dx"], (gy * g[None, :]) @ W0, 1e-13, "B=0 dx = (gy*g) W0")


def pin_sampled_forms(orc):
    W0, A, B, m, x, gy = _layer(14, 9, 10, 3, 6)
    s = 2.0
    rows = np.array([0, 4, 8, 4])
    tok = np.array([5, 0, 2, 2])
    cols = np.array([1, 9, 3])
    _close(orc.dora_norm_rows(W0, A, B, s, rows), orc.dora_norm(W0, A, B, s)[rows], 1e-15, "norm rows")
    y, _ = orc.dora_forward(x, W0, A, B, m, s)
    _close(orc.dora_forward_entries(x, W0, A, B, m, s, tok, rows), y[tok, rows], 1e-14, "y entries")
    for exact in (False, True):
        full = orc.dora_backward(gy, x, W0, A, B, m, s, exact=exact)
        smp = orc.dora_backward_sampled(gy, x, W0, A, B, m, s, tok, rows, cols, exact=exact)
        _close(smp["dx"], full["dx"][tok], 1e-14, "dx rows")
        _close(smp["dm"], full["dm"][rows], 1e-14, "dm rows")
        _close(smp["dB"], full["dB"][rows], 1e-14, "dB rows")
        _close(smp["dA"], full["dA"][:, cols], 1e-14, "dA cols")


def pin_merged_weight(orc):
    """The deploy-time merge (Alg. 1): every row of W'_merged has norm m_i and
    direction V'_i; with B = 0 and m = ||W0_i|| it is W0 itself; x W'_merged^T is the
    layer output."""
    W0, A, B, m, x, _ = _layer(11)
    s = 1.5
    Wm = orc.merged_weight(W0, A, B, m, s)
    _close(np.linalg.norm(Wm, axis=1), m, 1e-14, "merged rows have norm m")
    V = W0 + s * (B @ A)
    cosines = np.sum(Wm * V, axis=1) / (np.linalg.norm(Wm, axis=1) * np.linalg.norm(V, axis=1))
    _close(cosines, np.ones_like(m), 1e-14, "merged rows point along V'")
    Wb = orc.merged_weight(W0, A, np.zeros_like(B), np.linalg.norm(W0, axis=1), s)
    _close(Wb, W0, 1e-14, "B=0, m=||W0_i|| merges to W0")
    y, _ = orc.dora_forward(x, W0, A, B, m, s)
    _close(x @ Wm.T, y, 1e-13, "x W'_merged^T is the layer output")


def _vera(seed, d_out=6, d_in=9, r=3, T=5):
    rng = _rng(seed)
    W0, A, B, m, x, gy = _layer(seed, d_out, d_in, r, T)
    b = rng.normal(0.0, 1.0, d_out)
    d = rng.normal(0.0, 1.0, r)
    return W0, A, B, b, d, m, x, gy


def pin_dvora_reduces_to_dora(orc):
    """DVoRA is DoRA with B = diag(b) B_sh diag(d) ([DN] Sec. 3.5): the forward, and the
    b, d gradients as the chain rule of DoRA's dB through that product."""
    W0, A, B, b, d, m, x, gy = _vera(12)
    s = 1.75
    Be = b[:, None] * B * d[None, :]
    y, n = orc.dvora_forward(x, W0, A, B, b, d, m, s)
    y2, n2 = orc.dora_forward(x, W0, A, Be, m, s)
    _close(n, n2, 1e-14, "DVoRA norm = DoRA norm with the effective B")
    _close(y, y2, 1e-13, "DVoRA y = DoRA y with the effective B")
    for exact in (False, True):
        gv = orc.dvora_backward(gy, x, W0, A, B, b, d, m, s, exact=exact)
        gd = orc.dora_backward(gy, x, W0, A, Be, m, s, exact=exact)
        _close(gv["db"], np.sum(gd["dB"] * B * d[None, :], axis=1), 1e-13, "db from dB")
        _close(gv["dd"], np.sum(gd["dB"] * B * b[:, None], axis=0), 1e-13, "dd from dB")
        _close(gv["dx"], gd["dx"], 1e-13, "DVoRA dx")
        _close(gv["dm"], gd["dm"], 1e-13, "DVoRA dm")
    # b = 1, d = 1: plain DoRA with B = B_sh
    y3, _ = orc.dvora_forward(x, W0, A, B, np.ones_like(b), np.ones_like(d), m, s)
    y4, _ = orc.dora_forward(x, W0, A, B, m, s)
    _close(y3, y4, 1e-13, "b = d = 1 is DoRA")


def pin_dvora_vera_loops(orc):
    """The VeRA product entry by entry: (Delta W)_ik = b_i sum_j B_ij d_j A_jk."""
    _, A, B, b, d, _, _, _ = _vera(13)
    dW = orc.vera_update(A, B, b, d)
    for i in range(B.shape[0]):
        for k in range(A.shape[1]):
            v = b[i] * sum(B[i, j] * d[j] * A[j, k] for j in range(B.shape[1]))
            assert abs(dW[i, k] - v) <= 1e-14 * max(1.0, abs(v)), (i, k)


def pin_dvora_fd(orc):
    """Central finite differences of L = sum(gy * y) in b and d, norm detached and exact."""
    W0, A, B, b, d, m, x, gy = _vera(14, d_out=4, d_in=5, r=2, T=3)
    s = 0.9
    for exact in (False, True):
        gr = orc.dvora_backward(gy, x, W0, A, B, b, d, m, s, exact=exact)
        for name, vec in (("db", b), ("dd", d)):
            num = np.zeros_like(vec)
            for k in range(vec.size):
                h = 1e-6
                vp, vm = vec.copy(), vec.copy()
                vp[k] += h
                vm[k] -= h
                args_p = (vp, d) if name == "db" else (b, vp)
                args_m = (vm, d) if name == "db" else (b, vm)
                if exact:
                    Lp = np.sum(gy * orc.dvora_forward(x, W0, A, B, *args_p, m, s)[0])
                    Lm = np.sum(gy * orc.dvora_forward(x, W0, A, B, *args_m, m, s)[0])
                else:   # detached: the norm is held at its value at the base point
                    n0 = orc.dvora_forward(x, W0, A, B, b, d, m, s)[1]
                    def y_frozen(bb, dd):
                        V = W0 + s * orc.vera_update(A, B, bb, dd)
                        return x @ ((m / np.maximum(n0, 1e-8))[:, None] * V).T
                    Lp = np.sum(gy * y_frozen(*args_p))
                    Lm = np.sum(gy * y_frozen(*args_m))
                num[k] = (Lp - Lm) / (2 * h)
            _close(gr[name], num, 1e-6, f"FD {name} exact={exact}")


ALL_PINS = [
    pin_worked_rows, pin_bruteforce, pin_factored_identity, pin_b_zero, pin_g_one_is_lora,
    pin_scale_invariance, pin_s_zero_weightnorm, pin_token_permutation, pin_fd_detached,
    pin_fd_exact, pin_fd_zero_magnitude, pin_eq8_closed_form, pin_b_zero_backward, pin_sampled_forms, pin_merged_weight,
    pin_dvora_reduces_to_dora, pin_dvora_vera_loops, pin_dvora_fd,
]
