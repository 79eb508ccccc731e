"""Pins of the oracle's output epilogue y = RMSNorm(o) * weight * sigmoid(z)
(test infrastructure: the oracle against hand-computed values, closed forms
and invariances, not against a retyped formula).

"Kimi K3 - Lesson 3 of 14 - Sequence axis": after the recurrent read a
full-rank, input-dependent gate decides which channels pass; "K3
Architecture Illustrated" (KDA section): the module holds normalisation and
output gating.  Each pin is chosen so that a plausible slip fails it: the
wrong normalisation axis, a sum in place of the mean, a missing square root,
eps outside the root, a per-head weight, another activation, the gate applied
before the normalisation.
"""

import math

import numpy as np

from oracle import output_gate

BIG = 60.0   # sigmoid(60) = 1 - 9e-27: 1.0 in float64


def test_hand_computed_row():
    # o = (3, 4): mean square 12.5, so o / rms = (3, 4) * sqrt(2) / 5
    y = output_gate(np.array([3.0, 4.0]), np.full(2, BIG), np.ones(2), 0.0)
    assert np.allclose(y, [0.6 * math.sqrt(2.0), 0.8 * math.sqrt(2.0)], rtol=1e-15, atol=0)
    # the weight scales channels, not rows
    y = output_gate(np.array([3.0, 4.0]), np.full(2, BIG), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(y, [0.6 * math.sqrt(2.0), 1.6 * math.sqrt(2.0)], rtol=1e-15, atol=0)


def test_eps_sits_inside_the_root_and_sigmoid_values():
    # o = 1 everywhere, eps = 3: 1 / sqrt(1 + 3) = 1/2;  sigmoid(ln 3) = 3/4;  weight 2
    y = output_gate(np.ones(8), np.full(8, math.log(3.0)), np.full(8, 2.0), 3.0)
    assert np.allclose(y, 0.75, rtol=1e-15, atol=0)
    # sigmoid(0) = 1/2 exactly, sigmoid(-ln 9) = 1/10
    y0 = output_gate(np.ones(4), np.zeros(4), np.ones(4), 0.0)
    assert np.all(y0 == 0.5)
    y1 = output_gate(np.ones(4), np.full(4, -math.log(9.0)), np.ones(4), 0.0)
    assert np.allclose(y1, 0.1, rtol=1e-14, atol=0)


def test_open_gate_gives_unit_rms_rows():
    rng = np.random.default_rng(0)
    o = rng.normal(0.0, 3.0, size=(5, 7, 3, 64))
    y = output_gate(o, np.full(o.shape, BIG), np.ones(64), 0.0)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    assert np.allclose(rms, 1.0, rtol=1e-14, atol=0)


def test_scale_invariance_and_oddness_at_zero_eps():
    rng = np.random.default_rng(1)
    o = rng.normal(size=(4, 2, 32))
    z = rng.normal(size=o.shape)
    w = rng.normal(1.0, 0.2, size=32)
    y = output_gate(o, z, w, 0.0)
    assert np.allclose(output_gate(17.5 * o, z, w, 0.0), y, rtol=1e-13, atol=1e-15)
    assert np.allclose(output_gate(-o, z, w, 0.0), -y, rtol=0, atol=0)
    # with eps > 0 small rows are damped: the ratio is sqrt(ms / (ms + eps))
    ye = output_gate(o, z, w, 0.25)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    assert np.allclose(ye / y, np.sqrt(ms / (ms + 0.25)), rtol=1e-13, atol=0)


def test_rows_are_independent():
    # each (token, head) row is normalised over its own channels only
    rng = np.random.default_rng(2)
    o = rng.normal(size=(3, 4, 16))
    z = rng.normal(size=o.shape)
    w = np.ones(16)
    y = output_gate(o, z, w, 1e-6)
    o2 = o.copy()
    o2[1, 2] *= 100.0
    y2 = output_gate(o2, z, w, 1e-6)
    mask = np.ones((3, 4), dtype=bool)
    mask[1, 2] = False
    assert np.array_equal(y2[mask], y[mask])


def test_gate_applies_after_the_normalisation():
    # a gate that varies across channels changes the output's profile; if the
    # gate were applied before normalising, halving every gate value uniformly
    # would cancel out -- here it must halve the output
    rng = np.random.default_rng(3)
    o = rng.normal(size=(6, 32))
    w = np.ones(32)
    y_open = output_gate(o, np.full(o.shape, BIG), w, 0.0)
    y_half = output_gate(o, np.zeros(o.shape), w, 0.0)
    assert np.allclose(y_half, 0.5 * y_open, rtol=1e-15, atol=0)


def test_extreme_logits_stay_finite():
    y = output_gate(np.ones(4), np.array([-1e4, 1e4, -800.0, 800.0]), np.ones(4), 0.0)
    assert np.all(np.isfinite(y))
    assert y[0] == 0.0 and y[1] == 1.0


# ------------------------------------------------ the pins catch planted slips

PINS = [test_hand_computed_row, test_eps_sits_inside_the_root_and_sigmoid_values,
        test_open_gate_gives_unit_rms_rows, test_scale_invariance_and_oddness_at_zero_eps,
        test_rows_are_independent, test_gate_applies_after_the_normalisation,
        test_extreme_logits_stay_finite]

MUTANTS = {
    "sum, not mean": ("np.mean(o * o, axis=-1, keepdims=True)", "np.sum(o * o, axis=-1, keepdims=True)"),
    "no square root": ("1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)",
                       "1.0 / (np.mean(o * o, axis=-1, keepdims=True) + eps)"),
    "eps outside the root": ("np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)",
                             "(np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + eps)"),
    "normalised over all rows": ("np.mean(o * o, axis=-1, keepdims=True)", "np.mean(o * o)"),
    "normalised over heads": ("np.mean(o * o, axis=-1, keepdims=True)", "np.mean(o * o, axis=-2, keepdims=True)"),
    "silu gate": ("return o * inv_rms * w * sig", "return o * inv_rms * w * sig * z"),
    "no gate": ("return o * inv_rms * w * sig", "return o * inv_rms * w"),
    "gate before the norm": ("inv_rms = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)",
                             "inv_rms = 1.0 / np.sqrt(np.mean((o * (1 / (1 + np.exp(-z)))) ** 2, axis=-1, keepdims=True) + eps) / (1 / (1 + np.exp(-z)))"),
    "weight ignored": ("return o * inv_rms * w * sig", "return o * inv_rms * sig"),
    "sigmoid of -z": ("sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))",
                      "sig = np.where(z >= 0, e / (1.0 + e), 1.0 / (1.0 + e))"),
}


def _variant(old, new):
    import inspect
    import oracle.kda_oracle as ko
    src = inspect.getsource(ko.output_gate)
    assert old in src, old
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    return ns["output_gate"]


def test_each_planted_slip_fails_a_pin():
    global output_gate
    original = output_gate
    try:
        for name, (old, new) in MUTANTS.items():
            output_gate = _variant(old, new)
            failed = 0
            for pin in PINS:
                try:
                    with np.errstate(all="ignore"):
                        pin()
                except (AssertionError, ValueError, IndexError):
                    failed += 1
            assert failed >= 1, name
    finally:
        output_gate = original
