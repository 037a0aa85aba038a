"""Plant mistakes in copies of the oracle (on the CPU) and check a pin catches each.

Each mutant edits one expression of oracle/dora.py's source text and loads the
result as a separate module; the real oracle is untouched.
"""
import importlib.util
import os

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dora.py")

MUTANTS = {
    "sign_of_lora_update": ("return _f64(W0) + float(s) * lora_update(A, B)",
                            "return _f64(W0) - float(s) * lora_update(A, B)"),
    "scale_dropped": ("return _f64(W0) + float(s) * lora_update(A, B)",
                      "return _f64(W0) + lora_update(A, B)"),
    "norm_without_sqrt": ("return np.sqrt(np.sum(V * V, axis=1))", "return np.sum(V * V, axis=1)"),
    "magnitude_inverted": ("return _f64(m) / np.maximum(_f64(n), NORM_EPS)",
                           "return np.maximum(_f64(n), NORM_EPS) / _f64(m)"),
    "forward_drops_g": ("Wp = magnitude_scale(m, n)[:, None] * V\n    return _f64(x) @ Wp.T, n",
                        "Wp = magnitude_scale(m, n)[:, None] * V\n    return _f64(x) @ V.T, n"),
    "eq7_drops_m_over_n": ("dV = g[:, None] * dWp ", "dV = dWp "),
    "eq8_drops_norm": ("dm = along / np.maximum(n, NORM_EPS)", "dm = along"),
    "dB_drops_s": ("dB = float(s) * dV @ A.T", "dB = dV @ A.T"),
    "dA_uses_unscaled_grad": ("dA = float(s) * B.T @ dV", "dA = float(s) * B.T @ dWp"),
    "dx_drops_g": ("dx = gy @ (g[:, None] * V)", "dx = gy @ V"),
    "a1_projection_power": ("proj = dWp - (along / np.maximum(n, NORM_EPS) ** 2)[:, None] * V",
                            "proj = dWp - (along / np.maximum(n, NORM_EPS))[:, None] * V"),
    "cross_factor_two": ("cross = 2.0 * s * np.sum(B * U, axis=1)", "cross = s * np.sum(B * U, axis=1)"),
    "gram_single_s": ("gram = s * s * np.sum((B @ G) * B, axis=1)", "gram = s * np.sum((B @ G) * B, axis=1)"),
    "gram_transposed_operand": ("gram = s * s * np.sum((B @ G) * B, axis=1)",
                                "gram = s * s * np.sum((B @ (A.T @ A)[:B.shape[1], :B.shape[1]]) * B, axis=1)"),
    "merge_drops_g": ("    g = magnitude_scale(m, row_norms(V))\n    return g[:, None] * V",
                      "    g = magnitude_scale(m, row_norms(V))\n    return V"),
    "merge_scales_columns": ("    g = magnitude_scale(m, row_norms(V))\n    return g[:, None] * V",
                             "    g = magnitude_scale(m, row_norms(V))\n    return V * np.resize(g, V.shape[1])[None, :]"),
    "vera_drops_d": ("return np.diag(_f64(b)) @ _f64(B_sh) @ np.diag(_f64(d)) @ _f64(A_sh)",
                     "return np.diag(_f64(b)) @ _f64(B_sh) @ _f64(A_sh)"),
    "dvora_dd_drops_b": ('dd = s * np.einsum("ik,i,ij,jk->j", dV, b, B_sh, A_sh)',
                         'dd = s * np.einsum("ik,ij,jk->j", dV, B_sh, A_sh)'),
    "dvora_db_drops_d": ("BdA = B_sh @ np.diag(d) @ A_sh", "BdA = B_sh @ A_sh"),
    "sampled_rows_use_first_rows": ("V = _f64(W0[rows]) + float(s) * (_f64(B[rows]) @ _f64(A))\n    return row_norms(V)",
                                    "V = _f64(W0[:len(rows)]) + float(s) * (_f64(B[:len(rows)]) @ _f64(A))\n    return row_norms(V)"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new, 1)
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name):
    mod = _load_mutant(name, *MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
