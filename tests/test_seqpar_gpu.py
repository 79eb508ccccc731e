"""GPU parity of the sequence-parallel forward (kda_chunk_fwd_seqpar) against
the float64 oracle: element by element on every output for several segment
counts (segments of whole and of ragged chunks, down to 2 tokens), S0 given
or not, both gate dtypes, dk != dv and a bfloat16 output; the one-head-group
workload in full on sampled heads; in-place continuation; argument errors.
Bound as the other bfloat16 parity tests: max |err| <= 2e-2 * RMS(oracle),
separately for o and S_final.
"""

import numpy as np
import pytest
import torch

from gpu_support import (err_ratio, f64, gpu_heads, oracle_heads, say, spread_heads, tau_for, to_dev)
from kda_workloads import configs, gen, gen_torch

pytestmark = pytest.mark.gpu

H8, T = configs.HEADGROUP_BF16, configs.TRAIN_BF16


@pytest.fixture(scope="module")
def orc():
    from oracle import default
    return default()


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_101_amd as m
    m.load_library()
    return m


CASES = [
    (H8.scaled(H=2, T=1024, name="headgroup_H2_T1024"), 8),          # two chunks per segment
    (H8.scaled(H=2, T=1000, name="headgroup_H2_T1000"), 8),          # 125 tokens: ragged chunks
    (T.scaled(B=2, H=3, T=768, name="bf16gates_B2_H3_T768"), 3),
    (T.scaled(B=1, H=2, T=96, dk=64, dv=128, name="dk64_dv128_T96"), 4),
    (T.scaled(B=1, H=2, T=640, dk=128, dv=256, name="dk128_dv256_T640"), 5),
    (T.scaled(B=1, H=2, T=256, dk=64, dv=64, name="d64_T256"), 16),
    (H8.scaled(H=1, T=128, name="two_tokens_per_segment"), 64),
    (H8.scaled(H=2, T=333, gate="bf16", name="bf16_gates_S0_T333"), 3),
    (H8.scaled(H=2, T=300, name="one_segment"), 1),
    # B H dv / 8 >= 256: the combine's 8-column workgroups (4 below that)
    (T.scaled(B=2, H=16, T=192, dk=64, dv=64, name="cw8_d64_B2_H16_T192"), 3),
    (H8.scaled(H=16, T=256, name="cw8_d128_H16_T256"), 4),
]


@pytest.mark.parametrize("w,P", CASES, ids=[f"{w.name}_P{P}" for w, P in CASES])
def test_seqpar_matches_oracle(kda, orc, w, P):
    x = gen.fwd_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[seqpar] {w.name} B={w.B} T={w.T} H={w.H} dk={w.dk} dv={w.dv} gate={w.gate} segments={P}")
    o, S = kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], segments=P)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")],
                           x["S0"].f64() if x["S0"] is not None else None)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms  o={eo:.3e}  S={es:.3e}")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv), (eo, es)


def test_seqpar_bf16_output_and_plain_forward(kda, orc):
    """bfloat16 o (bound as the plain forward's bfloat16-output test), and the
    same call's results against kda_chunk_fwd's within the bound."""
    w = H8.scaled(H=3, T=1536, name="bf16_out")
    x = gen.fwd_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[seqpar bf16 out] {w.name}")
    o, S = kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], segments=6,
                                    out_dtype=torch.bfloat16)
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    o_ref, S_ref = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")],
                           x["S0"].f64() if x["S0"] is not None else None)
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    slack = tau_for(w.qkv) * rms + np.abs(o_ref) * 2.0 ** -8
    assert np.all(np.abs(f64(o) - o_ref) <= slack)
    assert err_ratio(f64(S), S_ref) <= tau_for(w.qkv)
    assert err_ratio(f64(o), f64(o2)) <= tau_for(w.qkv) and err_ratio(f64(S), f64(S2)) <= tau_for(w.qkv)


def test_seqpar_full_head_group(kda, orc):
    """The one-head-group workload (B1 H8 T4096) in 8 segments, in full, on
    three sampled heads against the oracle over all 4096 tokens."""
    w = configs.HEADGROUP_BF16
    d = gen_torch.fwd_inputs(w)
    say(f"[seqpar full] {w.name} segments=8")
    o, S = kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], segments=8)
    torch.cuda.synchronize()
    heads = spread_heads(w.B, w.H, 3)
    o_ref, S_ref = oracle_heads(orc, d, heads)
    og, Sg = gpu_heads(o, S, heads)
    eo, es = err_ratio(og, o_ref), err_ratio(Sg, S_ref)
    say(f"      err/rms  o={eo:.3e}  S_final={es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())


def test_seqpar_in_place_continuation(kda, orc):
    """S_final may be S0: the state is carried over in place, as for kda_chunk_fwd."""
    w = H8.scaled(H=2, T=512, name="in_place")
    x = gen.fwd_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    S = d["S0"].clone()
    o, S_out = kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], S, S_final=S, segments=4)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    o_ref, S_ref = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")], x["S0"].f64())
    assert err_ratio(f64(o), o_ref) <= 2e-2 and err_ratio(f64(S), S_ref) <= 2e-2


def test_seqpar_argument_errors(kda):
    w = H8.scaled(H=2, T=300, name="errors")
    d = gen_torch.fwd_inputs(w)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    for P in (0, 7, 65):   # out of range, or not dividing T = 300
        with pytest.raises(kda.KdaError) as e:
            kda.kda_chunk_fwd_seqpar(*args, segments=P)
        assert e.value.status == kda.KDA_ERR_INVALID_ARG, P
    short = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_fwd_seqpar(*args, segments=4, workspace=short)
    assert e.value.status == kda.KDA_ERR_INVALID_ARG
    f = [t.float() for t in args[:3]]
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_fwd_seqpar(*f, *args[3:], segments=4)
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED


def test_seqpar_segment_count_from_the_library(kda, orc):
    """segments=None takes kda_chunk_fwd_seqpar_segments' choice (a divisor of T)."""
    w = H8.scaled(H=2, T=2048, name="auto_segments")
    P = kda.kda_chunk_fwd_seqpar_segments(w.B, w.T, w.H, w.dk, w.dv)
    assert P > 1 and w.T % P == 0, P
    x = gen.fwd_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[seqpar auto] {w.name} segments={P}")
    o, S = kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")], x["S0"].f64())
    assert err_ratio(f64(o), o_ref) <= 2e-2 and err_ratio(f64(S), S_ref) <= 2e-2


def test_seqpar_without_final_state(kda, orc):
    """output_final_state=False: no S_final is written (the combine skips it) and
    o is unchanged."""
    w = H8.scaled(H=2, T=640, name="no_final_state")
    x = gen.fwd_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    o, S = kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], segments=5,
                                    output_final_state=False)
    torch.cuda.synchronize()
    assert S is None
    o_ref, _ = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")], x["S0"].f64())
    assert err_ratio(f64(o), o_ref) <= 2e-2


GATE_CASES = [
    (H8.scaled(H=2, T=1024, gate="bf16", name="gate_logits_bf16_T1024"), 8),
    (H8.scaled(H=3, T=390, name="gate_logits_f32_T390_S0"), 5),
    (T.scaled(B=2, H=2, T=256, dk=64, dv=128, name="gate_logits_dk64_T256"), 4),
]


@pytest.mark.parametrize("w,P", GATE_CASES, ids=[f"{w.name}_P{P}" for w, P in GATE_CASES])
def test_seqpar_with_gate_logits(kda, orc, w, P):
    """kda_chunk_fwd_gate_seqpar against the oracle's gate mapping followed by
    its forward, as the plain gate-logit forward is checked."""
    from oracle import gate_log_decay
    x = gen.gate_logit_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[seqpar gate] {w.name} B={w.B} T={w.T} H={w.H} dk={w.dk} gate={w.gate} segments={P}")
    o, S = kda.kda_chunk_fwd_gate_seqpar(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["beta"], d["S0"], segments=P)
    torch.cuda.synchronize()
    g = gate_log_decay(x["z"].f64(), x["A_log"].f64())
    S0 = x["S0"].f64() if x["S0"] is not None else None
    o_ref, S_ref = orc.fwd(x["q"].f64(), x["k"].f64(), x["v"].f64(), g, x["beta"].f64(), S0)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms  o={eo:.3e}  S={es:.3e}")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv), (eo, es)


def test_seqpar_long_sequence_share(kda, orc):
    """One GPU's share of the long sequence under 8-way head sharding (B1 H12
    T131072) at the library's segment count, the first and the last head
    against the oracle over all 131072 tokens."""
    w = configs.LONG_SHARE_BF16
    P = kda.kda_chunk_fwd_seqpar_segments(w.B, w.T, w.H, w.dk, w.dv)
    d = gen_torch.fwd_inputs(w)
    say(f"[seqpar long share] {w.name} segments={P}")
    o, S = kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], segments=P)
    torch.cuda.synchronize()
    heads = spread_heads(w.B, w.H, 2)
    o_ref, S_ref = oracle_heads(orc, d, heads)
    og, Sg = gpu_heads(o, S, heads)
    eo, es = err_ratio(og, o_ref), err_ratio(Sg, S_ref)
    say(f"      err/rms  o={eo:.3e}  S_final={es:.3e}")
    assert P > 1 and eo <= 2e-2 and es <= 2e-2
