"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_exact_gradient_projection_is_orthogonal():
    """Appendix A.1's projection removes the component of the gradient along V'_i.

    It exists because y does not change when (W0, B) are scaled together, so L
    has zero derivative along that direction.  Check that invariance by finite
    differences, and that the detached gradient (which skips the projection)
    differs from the exact one along B.
    """
    g = np.random.Generator(np.random.PCG64(21))
    W0 = g.standard_normal((5, 8)); A = g.uniform(-1, 1, (3, 8)); B = g.standard_normal((5, 3))
    m = g.uniform(0.5, 2, 5); x = g.standard_normal((4, 8)); gy = g.standard_normal((4, 5))
    s = 2.0
    eps = 1e-6
    lp = np.sum(gy * oracle.dora_forward(x, (1 + eps) * W0, A, (1 + eps) * B, m, s)[0])
    lm = np.sum(gy * oracle.dora_forward(x, (1 - eps) * W0, A, (1 - eps) * B, m, s)[0])
    assert abs(lp - lm) / (2 * eps) < 1e-8
    # ... while the detached gradient does see that direction (it is not projected).
    gd = oracle.dora_backward(gy, x, W0, A, B, m, s, exact=False)
    ge = oracle.dora_backward(gy, x, W0, A, B, m, s, exact=True)
    # d/de L((1+e)B) through B alone: exact and detached differ by the dropped term
    assert not np.allclose(np.sum(gd["dB"] * B), np.sum(ge["dB"] * B))


def test_detached_and_exact_agree_on_dm_and_dx():
    g = np.random.Generator(np.random.PCG64(22))
    W0 = g.standard_normal((5, 8)); A = g.uniform(-1, 1, (3, 8)); B = g.standard_normal((5, 3))
    m = g.uniform(0.5, 2, 5); x = g.standard_normal((4, 8)); gy = g.standard_normal((4, 5))
    gd = oracle.dora_backward(gy, x, W0, A, B, m, 2.0)
    ge = oracle.dora_backward(gy, x, W0, A, B, m, 2.0, exact=True)
    np.testing.assert_allclose(gd["dm"], ge["dm"], rtol=1e-14)
    np.testing.assert_allclose(gd["dx"], ge["dx"], rtol=1e-14)
