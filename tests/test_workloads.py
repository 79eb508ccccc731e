"""The seeded generators: determinism, shapes, dtypes and distributions."""

import numpy as np
import pytest

from kda_workloads import configs, gen


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.3895e38], np.float32)
    r = gen.round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0            # tie -> even
    assert r[2] == np.float32(1.0 + 2 ** -6)       # tie -> even (up)
    assert r[3] == -2.5
    u = r.view(np.uint32)
    assert np.all(u & 0xFFFF == 0)


def test_deterministic_and_independent_streams():
    w = configs.TINY_F32
    a = gen.fwd_inputs(w, seed=0)
    b = gen.fwd_inputs(w, seed=0)
    c = gen.fwd_inputs(w, seed=1)
    for n in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(a[n].values, b[n].values)
        assert not np.array_equal(a[n].values, c[n].values)
    assert a["S0"] is None


@pytest.mark.parametrize("w", [configs.TINY_F32, configs.HEADGROUP_BF16,
                               configs.TRAIN_BF16.scaled(B=1, H=2, T=512)])
def test_shapes_dtypes_distributions(w):
    x = gen.fwd_inputs(w)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    assert x["q"].shape == (B, T, H, dk) and x["v"].shape == (B, T, H, dv)
    assert x["beta"].shape == (B, T, H)
    assert x["q"].dtype == w.qkv and x["g"].dtype == w.gate
    if w.qkv == "bf16":
        assert np.all(x["q"].values.view(np.uint32) & 0xFFFF == 0)
    n = np.linalg.norm(x["k"].f64(), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-2 if w.qkv == "bf16" else 1e-6)
    beta = x["beta"].f64()
    assert beta.min() > 0.0 and beta.max() < 1.0
    assert abs(beta.mean() - 0.5) < 0.05
    if w.s0_sd is not None:
        assert abs(x["S0"].f64().std() - w.s0_sd) < 0.1 * w.s0_sd


def test_decode_inputs():
    w = configs.DECODE_BF16.scaled(B=4, H=3)
    S = gen.decode_initial_state(w)
    assert S.shape == (4, 3, 128, 128) and S.dtype == "f32"
    s0 = gen.decode_step_inputs(w, 0)
    s1 = gen.decode_step_inputs(w, 1)
    assert s0["q"].shape == (4, 3, 128) and s0["beta"].shape == (4, 3)
    assert not np.array_equal(s0["k"].values, s1["k"].values)
    assert np.array_equal(s0["k"].values, gen.decode_step_inputs(w, 0)["k"].values)
