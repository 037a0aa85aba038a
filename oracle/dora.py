"""Plain, dense, float64 oracle of DoRA's norm, forward and backward.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU-baseline leg, never by the library.  It is deliberately the slow dense
definition: it forms the adapted direction V' = W0 + s*B@A as a full
[d_out, d_in] matrix, takes its row norms, rescales and multiplies.  It uses
neither the factored norm nor the near-unity compose form of the fast path, so
agreement with the fast path is evidence, not tautology.

Sources (cited by page title and section):
  [SD]  Scaling DoRA summary page (gptget.net, arXiv 2603.22276), English
        abstract: row-wise norm of W + sBA over a dense [d_out, d_in] product;
        the factored base / cross / Gram terms.
  [DN]  DoRA reading notes (zhongzhuzhou.org): Sec. 3.1 eq. (6); Sec. 3.2
        Algorithm 1; Sec. 3.3 eq. (7), (8); Sec. 3.4 (detach);
        Sec. 3.5 (DVoRA: the direction update of VeRA); Appendix A.1 eq. (A.1).

Conventions (readings where the pages disagree or are silent):
  * nn.Linear layout: W0 [d_out, d_in], A [r, d_in], B [d_out, r], x [T, d_in],
    y [T, d_out].  The norm is taken per OUTPUT ROW ([SD]'s row-wise norm); the
    notes' eq. (3)/(6) write the same thing per column of a [d, k] matrix that
    multiplies x from the left, so m has one entry per output feature.
  * The LoRA scale s multiplies BA ([SD]: W + sBA); the notes use s = 1.
  * The norm is detached in the backward (treated as a constant), the notes'
    default implementation (Sec. 3.4); ``exact=True`` gives the undetached
    gradient of Appendix A.1 instead.
  * g = m / max(n, 1e-8): the notes clamp norms at 1e-8 in their analysis code
    (Sec. 7.3, weight-decomposition analysis code); unreached by non-degenerate rows.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
against closed forms, hand-worked integer rows, brute-force loops, special
cases and finite differences.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "NORM_EPS", "lora_update", "adapted_direction", "row_norms", "magnitude_scale",
    "dora_norm", "dora_forward", "dora_backward", "merged_weight", "norm_terms",
    "dora_norm_rows", "dora_forward_entries", "dora_backward_sampled",
    "scaled_down_projection", "vera_update", "dvora_forward", "dvora_backward",
]

NORM_EPS = 1e-8


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def lora_update(A, B):
    """Delta V = B @ A, the low-rank direction update ([DN] Alg. 1)."""
    return _f64(B) @ _f64(A)


def adapted_direction(W0, A, B, s):
    """V' = W0 + s * B @ A ([DN] Alg. 1 with [SD]'s scale s)."""
    return _f64(W0) + float(s) * lora_update(A, B)


def row_norms(V):
    """n_i = sqrt(sum_k V_ik^2), one per output row ([DN] Alg. 1; [SD])."""
    V = _f64(V)
    return np.sqrt(np.sum(V * V, axis=1))


def magnitude_scale(m, n):
    """g_i = m_i / n_i, with n clamped at NORM_EPS ([DN] Alg. 1)."""
    return _f64(m) / np.maximum(_f64(n), NORM_EPS)


def dora_norm(W0, A, B, s):
    """Row norms of the dense adapted direction ([SD] abstract; [DN] eq. 6)."""
    return row_norms(adapted_direction(W0, A, B, s))


def merged_weight(W0, A, B, m, s):
    """W' = m * V' / ||V'||_row ([DN] eq. 6; Alg. 1)."""
    V = adapted_direction(W0, A, B, s)
    g = magnitude_scale(m, row_norms(V))
    return g[:, None] * V


def dora_forward(x, W0, A, B, m, s, norm=None):
    """y = x @ W'^T with W' the merged DoRA weight ([DN] Alg. 1).

    ``norm`` substitutes fixed row norms for the computed ones: the value a
    detached norm contributes while it is held constant ([DN] Sec. 3.4).
    Returns (y [T, d_out], n [d_out]).
    """
    V = adapted_direction(W0, A, B, s)
    n = row_norms(V) if norm is None else _f64(norm)
    Wp = magnitude_scale(m, n)[:, None] * V
    return _f64(x) @ Wp.T, n


def dora_backward(gy, x, W0, A, B, m, s, exact=False):
    """Gradients of L = sum(gy * y) for y = dora_forward(x, ...).

    With the norm detached ([DN] Sec. 3.4) the direction gradient is
    eq. (7): dV' = (m/n) * dW', and the magnitude gradient is eq. (8):
    dm_i = dW'_i . V'_i / n_i, where dW' = gy^T @ x is the gradient of the
    merged weight.  ``exact=True`` projects dW' off V' per row first
    (Appendix A.1).  B and A receive dV' through V' = W0 + s*B@A; W0 is frozen.

    Returns dict(dx [T, d_in], dA [r, d_in], dB [d_out, r], dm [d_out]).
    """
    gy, x, A, B, m = map(_f64, (gy, x, A, B, m))
    V = adapted_direction(W0, A, B, s)
    n = row_norms(V)
    g = magnitude_scale(m, n)
    dWp = gy.T @ x                                   # dL/dW', [d_out, d_in]
    along = np.sum(dWp * V, axis=1)                  # dW'_i . V'_i
    dm = along / np.maximum(n, NORM_EPS)             # eq. (8)
    if exact:
        proj = dWp - (along / np.maximum(n, NORM_EPS) ** 2)[:, None] * V
        dV = g[:, None] * proj                       # eq. (A.1)
    else:
        dV = g[:, None] * dWp                        # eq. (7)
    dB = float(s) * dV @ A.T
    dA = float(s) * B.T @ dV
    dx = gy @ (g[:, None] * V)                       # y = x W'^T  =>  dx = gy W'
    return dict(dx=dx, dA=dA, dB=dB, dm=dm)


def scaled_down_projection(x, A, s):
    """s * (x @ A^T): the rank-r activations of the low-rank branch, scaled.

    The forward's output splits as y = g * (x W0^T + s (x A^T) B^T) because
    V' = W0 + s B A ([DN] Alg. 1); this is the factor
    s (x A^T) that a fast implementation keeps for the backward.
    """
    return float(s) * (_f64(x) @ _f64(A).T)


def norm_terms(W0, A, B, s):
    """The three terms of the factored squared norm ([SD] abstract).

    base_i  = ||W0_i||^2
    cross_i = 2 s B_i . (W0 A^T)_i
    gram_i  = s^2 B_i (A A^T) B_i^T
    so that base + cross + gram = ||W0_i + s (BA)_i||^2 by expanding the square.
    Used by the tests as an independent route to the same norm.
    """
    W0, A, B = map(_f64, (W0, A, B))
    s = float(s)
    base = np.sum(W0 * W0, axis=1)
    U = W0 @ A.T
    cross = 2.0 * s * np.sum(B * U, axis=1)
    G = A @ A.T
    gram = s * s * np.sum((B @ G) * B, axis=1)
    return base, cross, gram


# ---------------------------------------------------------------------------
# Sampled forms for layers too large to materialise in float64 at once.  Each
# evaluates the same definitions as above on a subset of rows / entries.
# ---------------------------------------------------------------------------

def dora_norm_rows(W0, A, B, s, rows):
    """n_i for the given output rows only (same definition as dora_norm)."""
    rows = np.asarray(rows)
    V = _f64(W0[rows]) + float(s) * (_f64(B[rows]) @ _f64(A))
    return row_norms(V)


def dora_forward_entries(x, W0, A, B, m, s, tok, rows):
    """y[tok[j], rows[j]] for paired index arrays (same definition as forward)."""
    tok, rows = np.asarray(tok), np.asarray(rows)
    ur, inv = np.unique(rows, return_inverse=True)
    V = _f64(W0[ur]) + float(s) * (_f64(B[ur]) @ _f64(A))
    g = magnitude_scale(_f64(m[ur]), row_norms(V))
    Wp = g[:, None] * V
    return np.einsum("jk,jk->j", _f64(x[tok]), Wp[inv])


def dora_backward_sampled(gy, x, W0, A, B, m, s, tok, rows, cols, exact=False):
    """Detached (or exact) backward evaluated on samples of every output.

    Returns dx[tok, :], dA[:, cols], dB[rows, :], dm[rows].  Uses the full
    dense V' (one [d_out, d_in] float64 matrix) but only the sampled slices of
    dW' = gy^T x, so it stays cheap at the largest layer shapes.
    """
    tok, rows, cols = map(np.asarray, (tok, rows, cols))
    gy, x = _f64(gy), _f64(x)
    A, B, m = _f64(A), _f64(B), _f64(m)
    s = float(s)
    V = adapted_direction(W0, A, B, s)
    n = row_norms(V)
    g = magnitude_scale(m, n)
    out = {}
    out["dx"] = gy[tok] @ (g[:, None] * V)
    # rows of dW' (for dB and dm)
    dWr = gy[:, rows].T @ x                               # [len(rows), d_in]
    along_r = np.sum(dWr * V[rows], axis=1)
    out["dm"] = along_r / np.maximum(n[rows], NORM_EPS)
    if exact:
        dVr = g[rows, None] * (dWr - (along_r / np.maximum(n[rows], NORM_EPS) ** 2)[:, None] * V[rows])
    else:
        dVr = g[rows, None] * dWr
    out["dB"] = s * dVr @ A.T
    # columns of dW' (for dA); the exact form needs every row's dW'_i . V'_i
    dWc = gy.T @ x[:, cols]                               # [d_out, len(cols)]
    if exact:
        along = np.sum((gy.T @ x) * V, axis=1)
        dVc = g[:, None] * (dWc - (along / np.maximum(n, NORM_EPS) ** 2)[:, None] * V[:, cols])
    else:
        dVc = g[:, None] * dWc
    out["dA"] = s * B.T @ dVc
    return out


# ---- DVoRA ([DN] Sec. 3.5) -----------------------------------------------------
# The direction update is VeRA's: a pair of frozen random matrices shared by all
# layers, A_sh [r, d_in] and B_sh [d_out, r], and two trainable vectors per
# layer, b [d_out] and d [r]:  Delta W = diag(b) B_sh diag(d) A_sh.  With the
# scale s of the rest of this oracle: V' = W0 + s * Delta W.

def vera_update(A_sh, B_sh, b, d):
    """diag(b) @ B_sh @ diag(d) @ A_sh, formed densely ([DN] Sec. 3.5)."""
    return np.diag(_f64(b)) @ _f64(B_sh) @ np.diag(_f64(d)) @ _f64(A_sh)


def dvora_forward(x, W0, A_sh, B_sh, b, d, m, s):
    """y = x @ W'^T with W' = m * V' / ||V'||_row and V' = W0 + s * vera_update.

    Returns (y, n).  Forms V' directly from the VeRA product, not through an
    effective B, so that the reduction to DoRA with B = diag(b) B_sh diag(d)
    is something the pins check rather than assume.
    """
    V = _f64(W0) + float(s) * vera_update(A_sh, B_sh, b, d)
    n = row_norms(V)
    Wp = magnitude_scale(m, n)[:, None] * V
    return _f64(x) @ Wp.T, n


def dvora_backward(gy, x, W0, A_sh, B_sh, b, d, m, s, exact=False):
    """Gradients of L = sum(gy * y) w.r.t. x, m and the VeRA vectors b, d.

    A_sh and B_sh are frozen (shared, not trained).  dV' follows eq. (7) (or
    A.1 with ``exact``), and Delta W = diag(b) B_sh diag(d) A_sh gives
      db_i = s * sum_k dV'_ik (B_sh diag(d) A_sh)_ik
      dd_j = s * sum_ik dV'_ik b_i B_sh_ij A_sh_jk.
    Returns a dict with dx, dm, db, dd.
    """
    gy, x, W0 = _f64(gy), _f64(x), _f64(W0)
    A_sh, B_sh, b, d, m = _f64(A_sh), _f64(B_sh), _f64(b), _f64(d), _f64(m)
    s = float(s)
    V = W0 + s * vera_update(A_sh, B_sh, b, d)
    n = row_norms(V)
    g = magnitude_scale(m, n)
    dWp = gy.T @ x
    along = np.sum(dWp * V, axis=1)
    dm = along / np.maximum(n, NORM_EPS)
    if exact:
        dV = g[:, None] * (dWp - (along / np.maximum(n, NORM_EPS) ** 2)[:, None] * V)
    else:
        dV = g[:, None] * dWp
    BdA = B_sh @ np.diag(d) @ A_sh
    db = s * np.sum(dV * BdA, axis=1)
    dd = s * np.einsum("ik,i,ij,jk->j", dV, b, B_sh, A_sh)
    dx = gy @ (g[:, None] * V)
    return {"dx": dx, "dm": dm, "db": db, "dd": dd}
