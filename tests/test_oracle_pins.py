"""The float64 oracle against the pins (pages' worked example, closed forms,
invariants, brute force in floating point and exact rationals)."""

import pytest

from oracle import default
from pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_oracle_refuses_inputs_outside_the_domain():
    """The oracle's tripwire: non-finite inputs and log-decays outside
    [g_min, 0] = [-5, 0] raise instead of producing numbers."""
    import numpy as np
    import pytest
    from oracle import default
    rng = np.random.default_rng(0)
    B, T, H, d = 1, 4, 1, 3
    q, k, g = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    v = rng.standard_normal((B, T, H, d))
    beta = np.full((B, T, H), 0.5)
    g = -5.0 * (1.0 / (1.0 + np.exp(-g)))
    orc = default()
    orc.fwd(q, k, v, g, beta)                                   # in the domain: runs
    for bad_g in (g - 0.5 - 5.0 * (g > -4.5), -g - 0.01):       # below -5 somewhere; above 0
        with pytest.raises(ValueError):
            orc.fwd(q, k, v, bad_g, beta)
    g_edge = g.copy()
    g_edge[0, 0, 0, 0] = -5.0                                   # the floor itself is allowed
    orc.fwd(q, k, v, g_edge, beta)
    for name in ("q", "k", "v", "beta"):
        x = {"q": q, "k": k, "v": v, "beta": beta}
        x[name] = x[name].copy()
        x[name].flat[1] = np.nan
        with pytest.raises(ValueError):
            orc.fwd(x["q"], x["k"], x["v"], g, x["beta"])
    S = np.zeros((B, H, d, d))
    S[0, 0, 1, 2] = np.inf
    with pytest.raises(ValueError):
        orc.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S)
