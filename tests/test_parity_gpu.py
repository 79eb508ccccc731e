"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Element-by-element on every output for cases the oracle finishes in
seconds (several chunks, ragged tails, both dtypes, dk != dv, the decay
floor), and on sampled heads at the full workload sizes in the launch
configuration the benchmark times.  Bound: max |err| <= tau * RMS(oracle)
separately for o and S_final, tau = 1e-4 (float32 q/k/v) or 2e-2 (bfloat16).
"""

import numpy as np
import pytest
import torch

from gpu_support import (err_ratio, f64, gpu_heads, oracle_heads, say, spread_heads, tau_for, to_dev)
from kda_workloads import configs, gen, gen_torch

pytestmark = pytest.mark.gpu


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


def _fwd_host_case(kda, orc, w, seed=0):
    x = gen.fwd_inputs(w, seed)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[fwd] {w.name} B={w.B} T={w.T} H={w.H} dk={w.dk} dv={w.dv} qkv={w.qkv} gate={w.gate}")
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    args = [x[n].f64() for n in ("q", "k", "v", "g", "beta")]
    S0 = x["S0"].f64() if x["S0"] is not None else None
    o_ref, S_ref = orc.fwd(*args, S0)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms  o={eo:.3e}  S={es:.3e}  (tau {tau_for(w.qkv):.0e})")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv), (eo, es)
    return o, S


T, H8, BF = configs.TRAIN_BF16, configs.HEADGROUP_BF16, configs.TINY_F32
SMALL_CASES = [
    configs.TINY_F32,
    configs.HEADGROUP_BF16,
    T.scaled(B=2, H=3, T=1000, name="train_bf16_B2_H3_T1000_ragged"),
    configs.TRAIN_BF16_LITERAL.scaled(B=1, H=2, T=777, name="train_literal_B1_H2_T777"),
    configs.LONG_BF16.scaled(H=4, T=2048, name="long_bf16_H4_T2048"),
    T.scaled(B=2, H=8, T=512, name="train_bf16_BH16_T512"),          # XCD-aware block mapping
    BF.scaled(B=1, H=3, T=200, dk=128, dv=128, name="f32_d128_T200"),
    BF.scaled(B=2, H=1, T=130, dk=64, dv=128, name="f32_dk64_dv128"),
    T.scaled(B=1, H=2, T=300, dk=128, dv=64, name="bf16_dk128_dv64"),
    T.scaled(B=1, H=2, T=192, dk=128, dv=192, name="bf16_dk128_dv192"),
    T.scaled(B=1, H=2, T=256, dk=64, dv=64, name="bf16_d64"),
    T.scaled(B=1, H=1, T=150, dk=128, dv=512, name="bf16_dk128_dv512"),   # largest dv: 8 value slabs
    BF.scaled(B=1, H=1, T=70, dk=64, dv=512, name="f32_dk64_dv512"),
    H8.scaled(H=2, T=333, gate="bf16", name="bf16_gates_S0"),
    BF.scaled(H=2, T=300, qkv="f32", gate="bf16", s0_sd=0.5, name="f32_qkv_bf16_gates_S0"),
] + [BF.scaled(B=1, H=2, T=t, name=f"f32_T{t}") for t in (1, 15, 16, 17, 63, 64, 65)] \
  + [T.scaled(B=1, H=2, T=t, name=f"bf16_T{t}") for t in (1, 17, 64, 65, 129)]


@pytest.mark.parametrize("w", SMALL_CASES, ids=[w.name for w in SMALL_CASES])
def test_fwd_matches_oracle(kda, orc, w):
    _fwd_host_case(kda, orc, w)


@pytest.mark.parametrize("w", [configs.HEADGROUP_BF16.scaled(H=3, T=1000, name="bf16_out_headgroup"),
                               configs.TRAIN_BF16_LITERAL.scaled(B=1, H=2, T=500, name="bf16_out_literal")],
                         ids=lambda w: w.name)
def test_fwd_bf16_output(kda, orc, w):
    """bfloat16 output: the bound adds the output's own rounding, |o| * 2^-8,
    to tau * RMS(o) (the product is computed at the float32-output precision,
    then rounded once)."""
    x = gen.fwd_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[fwd bf16 out] {w.name}")
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    o_ref, S_ref = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")],
                           x["S0"].f64() if x["S0"] is not None else None)
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    slack = tau_for(w.qkv) * rms + np.abs(o_ref) * 2.0 ** -8
    assert np.all(np.abs(f64(o) - o_ref) <= slack)
    assert err_ratio(f64(S), S_ref) <= tau_for(w.qkv)


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_fwd_at_the_decay_floor(kda, orc, qkv):
    """Half the key channels at g = -5 on every token: 1/f reaches e^80 in every tile."""
    rng = np.random.default_rng(5)
    B, T_, H, d = 1, 192, 2, 128
    q = rng.standard_normal((B, T_, H, d)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T_, H, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T_, H, d))
    g = np.full((B, T_, H, d), -5.0); g[..., ::2] = -0.02
    beta = rng.random((B, T_, H))
    dt = torch.float32 if qkv == "f32" else torch.bfloat16
    dq = [torch.tensor(a, dtype=torch.float32).to(dt).cuda() for a in (q, k, v)]
    dg = [torch.tensor(a, dtype=torch.float32).cuda() for a in (g, beta)]
    say(f"[fwd] decay floor qkv={qkv}")
    o, S = kda.kda_chunk_fwd(*dq, *dg)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.fwd(*[f64(t) for t in dq], *[f64(t) for t in dg])
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms  o={eo:.3e}  S={es:.3e}")
    assert np.all(np.isfinite(f64(o))) and eo <= tau_for(qkv) and es <= tau_for(qkv)


def test_fwd_empty_sequence(kda):
    S0 = torch.randn(2, 3, 128, 128, device="cuda")
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device="cuda")  # noqa: E731
    o, S = kda.kda_chunk_fwd(z(2, 0, 3, 128), z(2, 0, 3, 128), z(2, 0, 3, 128),
                             z(2, 0, 3, 128, dt=torch.float32), z(2, 0, 3, dt=torch.float32), S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128) and torch.equal(S, S0)
    o, S = kda.kda_chunk_fwd(z(2, 0, 3, 128), z(2, 0, 3, 128), z(2, 0, 3, 128),
                             z(2, 0, 3, 128, dt=torch.float32), z(2, 0, 3, dt=torch.float32), None)
    torch.cuda.synchronize()
    assert not torch.any(S)


def _dev_inputs(w, seed=0):
    x = gen.fwd_inputs(w, seed)
    return x, {n: to_dev(x[n]) for n in x}


def test_fwd_in_place_state_and_determinism(kda):
    w = configs.HEADGROUP_BF16.scaled(H=4, T=700)
    _, d = _dev_inputs(w)
    o1, S1 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    S_inplace = d["S0"].clone()
    o3, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S_inplace, S_final=S_inplace)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)          # bitwise rerun determinism
    assert torch.equal(o1, o3) and torch.equal(S1, S_inplace)   # S_final may alias S0


@pytest.mark.parametrize("T1", [128, 100])
def test_fwd_state_carry_composes(kda, T1):
    """fwd(T) equals fwd(T1) followed by fwd(T - T1) from its final state;
    bitwise when the split falls on a chunk boundary."""
    w = configs.TRAIN_BF16.scaled(B=2, H=3, T=300)
    _, d = _dev_inputs(w)
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    cut = lambda t, a, b: t[:, a:b].contiguous()  # noqa: E731
    o1, S1 = kda.kda_chunk_fwd(*(cut(d[n], 0, T1) for n in ("q", "k", "v", "g", "beta")))
    o2, S2 = kda.kda_chunk_fwd(*(cut(d[n], T1, w.T) for n in ("q", "k", "v", "g", "beta")), S1)
    torch.cuda.synchronize()
    if T1 % 64 == 0:
        assert torch.equal(o[:, :T1], o1) and torch.equal(o[:, T1:], o2) and torch.equal(S, S2)
    else:
        assert err_ratio(f64(torch.cat([o1, o2], 1)), f64(o)) <= 2e-2
        assert err_ratio(f64(S2), f64(S)) <= 2e-2


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_decode_after_prefill_equals_next_token(kda, orc, qkv):
    w = configs.TINY_F32.scaled(B=2, H=3, T=131, dk=128, dv=128, qkv=qkv)
    x, d = _dev_inputs(w)
    T_ = w.T
    head = lambda t: t[:, : T_ - 1].contiguous()  # noqa: E731
    _, Sp = kda.kda_chunk_fwd(*(head(d[n]) for n in ("q", "k", "v", "g", "beta")))
    last = {n: d[n][:, T_ - 1].contiguous() for n in ("q", "k", "v", "g", "beta")}
    od = kda.kda_decode_step(last["q"], last["k"], last["v"], last["g"], last["beta"], Sp)
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    o_ref, S_ref = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")])
    tau = tau_for(qkv)
    assert err_ratio(f64(od), o_ref[:, -1]) <= tau
    assert err_ratio(f64(Sp), S_ref) <= tau
    assert err_ratio(f64(o[:, -1]), f64(od)) <= tau


def test_write_then_read_same_key_returns_v(kda):
    """Unit keys, beta = 1, q = k: every output equals its value, whatever the state."""
    rng = np.random.default_rng(3)
    B, T_, H, d = 1, 256, 2, 64
    k = rng.standard_normal((B, T_, H, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T_, H, d))
    g = -5.0 * rng.random((B, T_, H, d))
    S0 = rng.standard_normal((B, H, d, d))
    t = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda")  # noqa: E731
    o, _ = kda.kda_chunk_fwd(t(k), t(k), t(v), t(g), t(np.ones((B, T_, H))), t(S0))
    torch.cuda.synchronize()
    assert err_ratio(f64(o), f64(t(v))) <= 1e-4


DECODE_CASES = [(dk, dv, qkv) for dk in (64, 128) for dv in (64, 128) for qkv in ("f32", "bf16")]


@pytest.mark.parametrize("dk,dv,qkv", DECODE_CASES, ids=[f"dk{a}_dv{b}_{c}" for a, b, c in DECODE_CASES])
def test_decode_matches_oracle(kda, orc, dk, dv, qkv):
    w = configs.DECODE_BF16.scaled(B=3, H=5, dk=dk, dv=dv, qkv=qkv, steps=6)
    S = gen.decode_initial_state(w)
    S_dev = to_dev(S)
    S_ref = S.f64().copy()
    say(f"[decode] dk={dk} dv={dv} qkv={qkv}")
    for step in range(w.steps):
        x = gen.decode_step_inputs(w, step)
        d = {n: to_dev(x[n]) for n in x}
        o = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S_dev)
        o_ref = orc.decode_step(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")], S_ref)
        torch.cuda.synchronize()
        assert err_ratio(f64(o), o_ref) <= tau_for(qkv), step
    assert err_ratio(f64(S_dev), S_ref) <= tau_for(qkv)


# ---------------------------------------------------------------- full sizes

def _full_fwd(kda, orc, w, n_heads):
    say(f"[fwd full] {w.name}: generating on device")
    d = gen_torch.fwd_inputs(w)
    say(f"[fwd full] {w.name}: kernel")
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    heads = spread_heads(w.B, w.H, n_heads)
    say(f"[fwd full] {w.name}: oracle on heads {heads}")
    o_full_ref, S_ref = oracle_heads(orc, d, heads)
    og, Sg = gpu_heads(o, S, heads)
    eo = err_ratio(og, o_full_ref)
    es = err_ratio(Sg, S_ref)
    say(f"      err/rms  o={eo:.3e}  S_final={es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())


@pytest.mark.parametrize("w", [configs.TRAIN_BF16, configs.TRAIN_BF16_LITERAL], ids=lambda w: w.name)
def test_full_training_shape(kda, orc, w):
    _full_fwd(kda, orc, w, n_heads=4)


def test_full_long_context(kda, orc):
    _full_fwd(kda, orc, configs.LONG_BF16, n_heads=2)


def test_full_decode(kda, orc):
    w = configs.DECODE_BF16
    say(f"[decode full] {w.name}")
    S = gen_torch.decode_initial_state(w)
    picks = spread_heads(w.B, w.H, 12)
    idx_b = torch.tensor([p[0] for p in picks]); idx_h = torch.tensor([p[1] for p in picks])
    S_ref = f64(S[idx_b, idx_h]).reshape(1, len(picks), w.dk, w.dv).copy()
    worst = 0.0
    for step in range(w.steps):
        d = gen_torch.decode_step_inputs(w, step)
        o = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
        sl = lambda t: f64(t[idx_b, idx_h]).reshape((1, len(picks)) + tuple(t.shape[2:]))  # noqa: E731
        o_ref = orc.decode_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), S_ref)
        worst = max(worst, err_ratio(sl(o), o_ref))
    torch.cuda.synchronize()
    es = err_ratio(f64(S[idx_b, idx_h]).reshape(S_ref.shape), S_ref)
    say(f"      err/rms  o(worst step)={worst:.3e}  S after {w.steps} steps={es:.3e}")
    assert worst <= 2e-2 and es <= 2e-2


# ------------------------------------------- prep/state ring kernel vs pipelined kernel

BF16_CASES = [w for w in SMALL_CASES if w.qkv == "bf16"]


@pytest.mark.parametrize("w", BF16_CASES, ids=[w.name for w in BF16_CASES])
def test_fwd_matches_oracle_without_workspace(kda, orc, w):
    """kda_chunk_fwd with no workspace (the single-workgroup pipelined kernel)."""
    x = gen.fwd_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[fwd no ring] {w.name}")
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], ring=False)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.fwd(*[x[n].f64() for n in ("q", "k", "v", "g", "beta")],
                           x["S0"].f64() if x["S0"] is not None else None)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms  o={eo:.3e}  S={es:.3e}")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv), (eo, es)


RING_CASES = BF16_CASES + [
    T.scaled(B=1, H=3, T=64 * 9 + 5, dk=128, dv=256, name="bf16_dv256_two_state_groups"),
    T.scaled(B=1, H=2, T=64 * 7 + 3, dk=128, dv=192, name="bf16_dv192_three_slabs"),
    T.scaled(B=1, H=2, T=64 * 11 + 60, dk=128, dv=512, name="bf16_dv512_eight_slabs"),
    T.scaled(B=1, H=2, T=64 * 3, dk=128, dv=512, name="bf16_dv512_fewer_chunks_than_slabs"),
    T.scaled(B=3, H=50, T=200, name="bf16_BH150_two_launches"),     # more heads than one launch holds
    H8.scaled(H=5, T=640, gate="bf16", name="bf16_gates_S0_T640"),
]


@pytest.mark.parametrize("w", RING_CASES, ids=[w.name for w in RING_CASES])
def test_ring_kernel_equals_pipelined_kernel(kda, w):
    """The workspace path runs the same steps as the pipelined kernel: the
    outputs and final states agree bit for bit."""
    _, d = _dev_inputs(w)
    say(f"[ring vs pipe] {w.name} B={w.B} T={w.T} H={w.H} dv={w.dv} gate={w.gate}")
    need = kda.kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv)
    assert (need > 0) == (w.dk == 128 and w.dv >= 128)   # one slab per head (dv = 64): no ring
    o1, S1 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], ring=True)
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], ring=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_ring_kernel_gate_logits_equals_pipelined(kda):
    w = T.scaled(B=2, H=4, T=333)
    _, d = _dev_inputs(w)
    A_log = torch.linspace(-1.0, 1.0, w.H, device="cuda")
    z = d["g"].float().mul(-1.0).to(d["g"].dtype)
    o1, S1 = kda.kda_chunk_fwd_gate(d["q"], d["k"], d["v"], z, A_log, d["beta"], ring=True)
    o2, S2 = kda.kda_chunk_fwd_gate(d["q"], d["k"], d["v"], z, A_log, d["beta"], ring=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_ring_workspace_reuse_and_uninitialised(kda):
    """One workspace reused across calls of different shapes, first filled with
    bytes that look like flags: results stay those of the pipelined kernel."""
    ws = torch.full((kda.kda_chunk_fwd_workspace_bytes(2, 1, 8, 128, 128),), 0xFF, dtype=torch.uint8, device="cuda")
    for i, (B, H, T_) in enumerate([(2, 8, 700), (1, 3, 130), (2, 8, 64)]):
        _, d = _dev_inputs(T.scaled(B=B, H=H, T=T_), seed=i)
        o1, S1 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], workspace=ws)
        o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], ring=False)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S1, S2), (B, H, T_)


@pytest.mark.parametrize("ring", [True, False])
def test_expired_wait_is_loud(kda, ring):
    """A wait inside the chunk kernels that runs out of spins (forced from the
    host with a zero bound) never yields finite wrong numbers: every finite
    output equals the normal run's bit for bit, and the rest is NaN."""
    w = T.scaled(B=2, H=4, T=64 * 12)
    _, d = _dev_inputs(w)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    o_ref, S_ref = kda.kda_chunk_fwd(*args, ring=ring)
    torch.cuda.synchronize()
    old = kda.debug_set_spin_limit(0)
    try:
        say(f"[expired wait] ring={ring}: spin bound 0")
        o, S = kda.kda_chunk_fwd(*args, ring=ring)
        torch.cuda.synchronize()
    finally:
        kda.debug_set_spin_limit(old)
    bad_o = ~torch.isfinite(o)
    say(f"      NaN outputs: {int(bad_o.sum())} of {o.numel()}; NaN state: {int((~torch.isfinite(S)).sum())}")
    assert bool(bad_o.any()), "a zero spin bound must make some wait expire"
    assert bool(torch.isnan(o[bad_o]).all())
    assert torch.equal(o[~bad_o], o_ref[~bad_o])
    bad_s = ~torch.isfinite(S)
    assert bool(bad_s.any()) and torch.equal(S[~bad_s], S_ref[~bad_s])
    # the bound is restored: the next call is whole again
    o2, S2 = kda.kda_chunk_fwd(*args, ring=ring)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(S2, S_ref)
