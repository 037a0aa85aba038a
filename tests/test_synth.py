"""The seeded input generator: rounding, decoding, determinism, distributions."""
import numpy as np

import synth


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     -1.0 - 2.0 ** -8, 3.0e38, 1e-40], dtype=np.float32)
    got = synth.bf16_to_f64(synth.bf16_bits(vals))
    want = [1.0, 1.0, 1.0 + 4 * 2.0 ** -8, 1.0 + 2.0 ** -7, -1.0, None, None]
    assert got[0] == want[0]
    assert got[1] == want[1]                # tie -> even (mantissa 0)
    assert got[2] == want[2]                # tie -> even (rounds up to ...10)
    assert got[3] == want[3]                # above tie -> up
    assert got[4] == want[4]                # negative tie -> even
    assert np.isfinite(got[5]) and abs(got[5] - 3.0e38) / 3.0e38 < 2.0 ** -8
    assert 0 < got[6] and abs(got[6] - 1e-40) <= 2.0 ** -134  # subnormal, half a spacing


def test_bf16_exact_values_roundtrip():
    v = np.array([0.0, -2.5, 3.0, 0.15625, 65280.0], dtype=np.float32)
    assert np.array_equal(synth.bf16_to_f64(synth.bf16_bits(v)), v.astype(np.float64))


def test_make_layer_deterministic_and_shaped():
    sh = synth.LayerShape(40, 24, 8, 13, 2.0, "bf16")
    a = synth.make_layer(sh, 3, grad=True)
    b = synth.make_layer(sh, 3, grad=True)
    for k in a:
        assert np.array_equal(a[k], b[k])
        assert a[k].dtype == np.uint16
    assert a["W0"].shape == (40, 24) and a["A"].shape == (8, 24) and a["B"].shape == (40, 8)
    assert a["m"].shape == (40,) and a["x"].shape == (13, 24) and a["gy"].shape == (13, 40)
    c = synth.make_layer(sh, 4)
    assert not np.array_equal(a["W0"], c["W0"])


def test_make_layer_distributions():
    sh = synth.LayerShape(512, 1024, 64, 256, 2.0, "f32")
    L = synth.make_layer(sh, 0)
    assert abs(L["W0"].std() - 0.02) < 0.002
    assert abs(L["B"].std() - 0.01) < 0.001
    bound = 1 / np.sqrt(1024)
    assert L["A"].max() <= bound and L["A"].min() >= -bound
    assert abs(L["x"].std() - 1.0) < 0.02
    ratio = L["m"] / np.linalg.norm(L["W0"].astype(np.float64), axis=1)
    assert ratio.min() > 0.95 - 1e-6 and ratio.max() < 1.05 + 1e-6
    z = synth.make_layer(sh, 0, zero_b=True)
    assert not z["B"].any()
