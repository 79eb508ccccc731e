"""Pins of the oracle's gate mapping g = -5 sigmoid(exp(A_h) z) (test
infrastructure: the oracle against closed forms and the bound, not against a
retyped formula).

"Kimi K3 - Lesson 3 of 14 - Sequence axis": the scaled sigmoid keeps every
log-decay in (-5, 0), so 16 tokens accumulate at most 80 and 1/Gamma stays
below e^80; A_h is a per-head log-scale initialised to 0.
"""

import math

import numpy as np

from oracle import gate_log_decay


def g1(z, a=0.0):
    return float(gate_log_decay(np.array([[z]]), np.array([a]))[0, 0])


def test_closed_form_values():
    assert g1(0.0) == -2.5                                  # sigmoid(0) = 1/2
    assert abs(g1(math.log(3.0)) - (-3.75)) < 1e-15          # sigmoid(ln 3) = 3/4
    assert abs(g1(-math.log(3.0)) - (-1.25)) < 1e-15
    assert abs(g1(math.log(9.0)) - (-4.5)) < 1e-15           # sigmoid(ln 9) = 9/10


def test_head_scale_multiplies_the_logit():
    # exp(ln 2) = 2: a logit of ln(3)/2 at A = ln 2 is the logit ln 3 at A = 0
    assert abs(g1(math.log(3.0) / 2, math.log(2.0)) - (-3.75)) < 1e-15
    # A = 0 is the plain scaled sigmoid; a large A sharpens towards the step -5 [z > 0]
    assert abs(g1(0.3, 0.0) - g1(0.3)) == 0.0
    assert g1(0.3, 8.0) < -4.999 and g1(-0.3, 8.0) > -1e-3


def test_symmetry_limits_and_range():
    rng = np.random.default_rng(0)
    z = rng.normal(0.0, 4.0, size=(64, 3, 16))
    A = rng.normal(0.0, 1.0, size=3)
    g = gate_log_decay(z, A)
    gm = gate_log_decay(-z, A)
    assert np.max(np.abs(g + gm + 5.0)) < 1e-14             # sigmoid(-x) = 1 - sigmoid(x)
    assert np.all(g <= 0.0) and np.all(g >= -5.0)
    big = gate_log_decay(np.array([[-1e4, 1e4, -800.0, 800.0]]), np.array([0.0]))
    assert np.all(np.isfinite(big))
    assert big[0, 0] == 0.0 and big[0, 1] == -5.0
    # strictly decreasing in z for a fixed head
    zs = np.linspace(-20, 20, 401)[:, None]
    gs = gate_log_decay(zs, np.array([0.4]))[:, 0]
    assert np.all(np.diff(gs) < 0)


def test_sixteen_token_tiles_stay_within_the_bound():
    # the e^80 bound of the pages: any 16 consecutive gates sum to at least -80
    rng = np.random.default_rng(1)
    z = rng.normal(3.0, 3.0, size=(4096, 2, 8))
    g = gate_log_decay(z, np.array([0.7, -0.4]))
    tiles = g.reshape(256, 16, 2, 8).sum(axis=1)
    assert tiles.min() >= -80.0
    assert math.exp(80.0) < 3.4e38
