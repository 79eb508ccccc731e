"""The g_min = -5 bound that makes every 16-token tile safe (pin P12).

Checks the pages' numbers (golden/gmin_bound.json), that float32 (the
kernels' factor precision) really holds e^80 and overflows just past 88.7,
that the two 'one step over the line' co-designs the pages name overflow,
and that every generated workload's log-decay respects the bound.
"""

import json
import math
import os

import numpy as np
import pytest

from kda_workloads import configs, gen

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "gmin_bound.json")))


def test_page_numbers():
    assert GOLD["tile"] * -GOLD["g_min"] == GOLD["max_tile_log_decay"]
    e80 = math.exp(GOLD["max_tile_log_decay"])
    assert abs(e80 / GOLD["e80_approx"] - 1) < GOLD["e80_rel_tol"]
    assert e80 < GOLD["bf16_ceiling_approx"]
    # largest finite bfloat16 is (2 - 2^-7) * 2^127; its log is the overflow threshold
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    assert abs(bf16_max / GOLD["bf16_ceiling_approx"] - 1) < 0.01
    assert abs(math.log(bf16_max) - GOLD["overflow_log_decay_approx"]) < GOLD["overflow_abs_tol"]
    for d in GOLD["breaking_designs"]:
        assert d["floor"] * d["tile"] == d["cumulative"]
        assert d["cumulative"] > math.log(bf16_max) > GOLD["max_tile_log_decay"]


def _tile_reciprocal_f32(g_row, tile):
    """1/Gamma over one tile at a constant per-token log-decay, in float32."""
    b = np.cumsum(np.full(tile, np.float32(g_row), np.float32), dtype=np.float32)
    with np.errstate(over="ignore"):
        return np.exp(-b).astype(np.float32)


def test_float32_margin():
    assert np.all(np.isfinite(_tile_reciprocal_f32(-5.0, 16)))
    assert float(_tile_reciprocal_f32(-5.0, 16)[-1]) == pytest.approx(math.exp(80), rel=1e-5)
    assert not np.all(np.isfinite(_tile_reciprocal_f32(-6.0, 16)))   # floor 6
    assert not np.all(np.isfinite(_tile_reciprocal_f32(-5.0, 24)))   # tile 24
    # the forward factor e^-80 stays a normal float32 (no flush to zero)
    assert np.float32(math.exp(-80)) >= np.finfo(np.float32).tiny


SMALL = [configs.TINY_F32, configs.HEADGROUP_BF16,
         configs.TRAIN_BF16.scaled(B=1, H=4, T=1024),
         configs.TRAIN_BF16_LITERAL.scaled(B=1, H=4, T=1024),
         configs.LONG_BF16.scaled(H=4, T=1024)]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_generated_log_decay_within_bound(w):
    g = gen.fwd_tensor(w, "g").f64()
    assert g.max() <= 0.0 and g.min() >= -5.0
    T = w.T
    tiles = g[:, : T - T % 16].reshape(w.B, T // 16, 16, w.H, w.dk).sum(axis=2)
    assert tiles.min() >= -80.0
    if w.forced_channels:
        # the forced channels push tiles close to the bound: that is the point of the stress
        assert tiles.min() < (-79.0 if w.forced_z > 0 else -70.0)
