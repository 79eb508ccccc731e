"""GPU parity of the output epilogue y = o / sqrt(mean(o^2) + eps) * weight *
sigmoid(z) against the float64 oracle ("Kimi K3 - Lesson 3 of 14", the
output-gate paragraph; "K3 Architecture Illustrated", the KDA module's
normalisation and output gating), alone and fused into the decode step.

Bound: max |err| <= 1e-4 * RMS(oracle) (float32 arithmetic throughout; the
oracle receives the exact stored inputs), plus 2^-8 |oracle| when y is
stored in bfloat16 (its own rounding).
"""

import numpy as np
import pytest
import torch

from gpu_support import f64, say, spread_heads, to_dev
from kda_workloads import configs, gen, gen_torch

pytestmark = pytest.mark.gpu

TAU = 1e-4
EPS = 1e-6


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_101_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def orc():
    import types

    import oracle
    inst = oracle.default()
    return types.SimpleNamespace(fwd=inst.fwd, decode_step=inst.decode_step,
                                 output_gate=oracle.output_gate, gate_log_decay=oracle.gate_log_decay)


def _check(got, ref, y_bf16):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = TAU * rms + (2.0 ** -8 * np.abs(ref) if y_bf16 else 0.0)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    worst = float(np.max(err - bound))
    say(f"      max err/rms={float(np.max(err)) / rms:.3e}")
    assert worst <= 0.0


CASES = [  # rows, dv, o, z, y
    (37, 128, "f32", "f32", "f32"),
    (1, 64, "f32", "bf16", "f32"),
    (1000, 128, "bf16", "bf16", "bf16"),
    (16, 192, "f32", "bf16", "bf16"),
    (333, 256, "bf16", "f32", "f32"),
    (65, 512, "f32", "f32", "f32"),
]


@pytest.mark.parametrize("rows,dv,od,zd,yd", CASES, ids=[f"r{r}_dv{d}_{a}{b}{c}" for r, d, a, b, c in CASES])
def test_output_gate_matches_oracle(kda, orc, rows, dv, od, zd, yd):
    o = gen.read_rows(rows, dv, od, seed=rows)
    z = gen.output_gate_logits((rows, dv), zd, seed=rows)
    w = gen.output_norm_weight(dv)
    say(f"[epilogue] rows={rows} dv={dv} o={od} z={zd} y={yd}")
    y = kda.kda_output_gate(to_dev(o), to_dev(z), to_dev(w), EPS,
                            out_dtype=torch.bfloat16 if yd == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = orc.output_gate(o.f64(), z.f64(), w.f64(), EPS)
    _check(f64(y), ref, yd == "bf16")
    # the all-zero rows stay exactly zero
    assert torch.count_nonzero(y[3::7]).item() == 0


def test_output_gate_in_place_and_eps(kda, orc):
    rows, dv = 129, 128
    o = gen.read_rows(rows, dv, "f32", seed=4)
    z = gen.output_gate_logits((rows, dv), "f32", seed=4)
    w = gen.output_norm_weight(dv)
    od = to_dev(o)
    y = kda.kda_output_gate(od, to_dev(z), to_dev(w), 0.5, y=od)
    torch.cuda.synchronize()
    assert y.data_ptr() == od.data_ptr()
    _check(f64(od), orc.output_gate(o.f64(), z.f64(), w.f64(), 0.5), False)


def test_output_gate_after_chunk_forward(kda, orc):
    """The forward's reads, then the epilogue: against the oracle forward's
    reads through the oracle epilogue."""
    wl = configs.HEADGROUP_BF16.scaled(B=2, H=3, T=200, name="epilogue_after_fwd")
    x = gen.fwd_inputs(wl, 3)
    d = {n: to_dev(x[n]) for n in ("q", "k", "v", "g", "beta", "S0")}
    z = gen.output_gate_logits((wl.B, wl.T, wl.H, wl.dv), "bf16", seed=3)
    w = gen.output_norm_weight(wl.dv)
    o, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], output_final_state=False)
    y = kda.kda_output_gate(o, to_dev(z), to_dev(w), EPS)
    torch.cuda.synchronize()
    o_ref, _ = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")], x["S0"].f64(),
                         want_state=False)
    ref = orc.output_gate(o_ref, z.f64(), w.f64(), EPS)
    # the forward's own bf16-input error carries through the normalisation
    err = float(np.max(np.abs(f64(y) - ref))) / float(np.sqrt(np.mean(ref * ref)))
    say(f"[epilogue after fwd] err/rms={err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("dk,dv,qkv,logits", [(128, 128, "bf16", False), (64, 64, "f32", False),
                                              (128, 64, "bf16", True), (64, 128, "f32", True)])
def test_decode_with_fused_epilogue(kda, orc, dk, dv, qkv, logits):
    w = configs.DECODE_BF16.scaled(B=3, H=5, dk=dk, dv=dv, qkv=qkv, steps=4)
    S = gen.decode_initial_state(w)
    S_fused, S_plain = to_dev(S), to_dev(S)
    S_ref = S.f64().copy()
    wt = gen.output_norm_weight(dv)
    say(f"[decode+epilogue] dk={dk} dv={dv} qkv={qkv} gate logits={logits}")
    for step in range(w.steps):
        if logits:
            x = gen.decode_gate_logit_inputs(w, step)
            g_name, A = "z", x["A_log"]
            g64 = orc.gate_log_decay(x["z"].f64(), A.f64())
        else:
            x = gen.decode_step_inputs(w, step)
            g_name, A = "g", None
            g64 = x["g"].f64()
        d = {n: to_dev(x[n]) for n in x}
        zo = gen.output_gate_logits((w.B, w.H, dv), qkv, seed=step, stream=1)
        y = kda.kda_decode_step_gated(d["q"], d["k"], d["v"], d[g_name], d["beta"], S_fused, to_dev(zo),
                                      to_dev(wt), EPS, A_log=None if A is None else d["A_log"])
        if logits:
            o = kda.kda_decode_step_gate(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["beta"], S_plain)
        else:
            o = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S_plain)
        y2 = kda.kda_output_gate(o, to_dev(zo), to_dev(wt), EPS)
        o_ref = orc.decode_step(x["q"].f64(), x["k"].f64(), x["v"].f64(), g64, x["beta"].f64(), S_ref)
        torch.cuda.synchronize()
        ref = orc.output_gate(o_ref, zo.f64(), wt.f64(), EPS)
        tol = 1e-4 if qkv == "f32" else 2e-2
        err = float(np.max(np.abs(f64(y) - ref))) / float(np.sqrt(np.mean(ref * ref)))
        assert err <= tol, step
        # fused and separate agree to float32 rounding; the state is the same bits
        assert float(np.max(np.abs(f64(y) - f64(y2)))) <= 1e-5 * float(np.sqrt(np.mean(ref * ref)))
        assert torch.equal(S_fused, S_plain)


def test_output_gate_full_training_shape(kda, orc):
    """The epilogue over the training-shape forward output (B4 T16384 H32
    dv128, float32 reads, bf16 logits), sampled heads against the oracle."""
    wl = configs.TRAIN_BF16
    shape = (wl.B, wl.T, wl.H, wl.dv)
    say("[epilogue full] generating")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    o = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    z = gen_torch.output_gate_logits(shape, "bf16")
    w = gen_torch.output_norm_weight(wl.dv)
    y = kda.kda_output_gate(o, z, w, EPS)
    torch.cuda.synchronize()
    for b, h in spread_heads(wl.B, wl.H, 6):
        for t0 in (0, wl.T // 2, wl.T - 64):
            sl = (b, slice(t0, t0 + 64), h)
            ref = orc.output_gate(f64(o[sl]), f64(z[sl]), f64(w), EPS)
            _check(f64(y[sl]), ref, False)
