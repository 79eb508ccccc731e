"""GPU parity of the follow-on entry points against the float64 oracle.

* Speculative decoding ("K3 Architecture Illustrated", the speculative
  decoding section: the recurrent state needs rollback after rejected
  proposals): kda_verify_step must give, for K draft tokens, exactly the
  outputs the recurrence gives from the current state, and leave the state
  untouched; kda_commit_step must leave each sequence's state where the
  recurrence is after its accepted prefix (composability, fwd(T1 + T2) =
  fwd(T2, fwd(T1).S)).
* Gate logits ("Kimi K3 - Lesson 3 of 14", the scaled-sigmoid gate): the
  kernels' g = -5 sigmoid(exp(A_h) z) against the oracle's float64 mapping
  followed by the oracle recurrence.

Bound: max |err| <= tau * RMS(oracle), tau = 1e-4 (float32 q/k/v) or 2e-2.
"""

import numpy as np
import pytest
import torch

from gpu_support import err_ratio, f64, say, tau_for, to_dev
from kda_workloads import configs, gen

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


NAMES = ("q", "k", "v", "g", "beta")


def _draft_case(w, seed):
    """A state (from a prefix) and K draft tokens per sequence."""
    x = gen.fwd_inputs(w, seed)
    S0 = x["S0"].f64() if x["S0"] is not None else np.zeros((w.B, w.H, w.dk, w.dv))
    return x, S0


SPEC_CASES = [
    configs.HEADGROUP_BF16.scaled(B=3, H=2, T=16, name="spec_bf16_K16"),
    configs.HEADGROUP_BF16.scaled(B=2, H=3, T=5, dv=64, name="spec_bf16_K5_dv64"),
    configs.TRAIN_BF16.scaled(B=2, H=2, T=64, s0_sd=0.02, name="spec_bf16_K64_bf16gates"),
    configs.TINY_F32.scaled(B=3, H=2, T=16, dk=128, dv=128, s0_sd=0.3, name="spec_f32_K16"),
    configs.TINY_F32.scaled(B=2, H=2, T=1, s0_sd=0.3, name="spec_f32_K1"),
    configs.HEADGROUP_BF16.scaled(B=2, H=3, T=37, dk=64, dv=128, name="spec_bf16_K37_dk64"),
    configs.TINY_F32.scaled(B=2, H=2, T=7, dv=256, s0_sd=0.3, name="spec_f32_K7_dv256"),  # chunk-kernel route
    # up to 16 drafts with dk = 64 (the matrix-core tile, two 32-channel pairs)
    configs.HEADGROUP_BF16.scaled(B=3, H=2, T=12, dk=64, dv=64, name="spec_bf16_K12_dk64_dv64"),
    configs.TINY_F32.scaled(B=3, H=2, T=9, dk=64, dv=128, s0_sd=0.3, name="spec_f32_K9_dk64_dv128"),
    # bf16 with dv > 128: verify and commit take the pipelined chunk kernel (commit with
    # per-sequence lengths = the accepted counts, so its identity-token path runs)
    configs.HEADGROUP_BF16.scaled(B=3, H=2, T=9, dv=192, name="spec_bf16_K9_dv192"),
    configs.HEADGROUP_BF16.scaled(B=3, H=2, T=16, dv=256, name="spec_bf16_K16_dv256"),
]


@pytest.mark.parametrize("w", SPEC_CASES, ids=[w.name for w in SPEC_CASES])
def test_verify_outputs_and_state_untouched(kda, orc, w):
    x, S0 = _draft_case(w, seed=5)
    d = {n: to_dev(x[n]) for n in NAMES}
    S = torch.tensor(S0, dtype=torch.float32, device="cuda")
    S_before = S.clone()
    say(f"[verify] {w.name} B={w.B} K={w.T} H={w.H} dk={w.dk} dv={w.dv}")
    o = kda.kda_verify_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    torch.cuda.synchronize()
    o_ref, _ = orc.fwd(*[x[n].f64() for n in NAMES], S0, want_state=False)
    eo = err_ratio(f64(o), o_ref)
    say(f"      err/rms o={eo:.3e}")
    assert eo <= tau_for(w.qkv)
    assert torch.equal(S, S_before)


@pytest.mark.parametrize("w", SPEC_CASES, ids=[w.name for w in SPEC_CASES])
def test_commit_keeps_the_accepted_prefix(kda, orc, w):
    x, S0 = _draft_case(w, seed=6)
    K = w.T
    d = {n: to_dev(x[n]) for n in NAMES}
    rng = np.random.default_rng(7)
    acc = rng.integers(0, K + 1, size=w.B).astype(np.int32)
    acc[0] = K                       # everything accepted
    if w.B > 1:
        acc[1] = 0                   # nothing accepted
    S = torch.tensor(S0, dtype=torch.float32, device="cuda")
    say(f"[commit] {w.name} accepted={acc.tolist()}")
    kda.kda_commit_step(d["k"], d["v"], d["g"], d["beta"], torch.tensor(acc, device="cuda"), S)
    torch.cuda.synchronize()
    args = [x[n].f64() for n in NAMES]
    for b in range(w.B):
        n = int(acc[b])
        if n == 0:
            ref = S0[b:b + 1]
            assert torch.equal(S[b:b + 1].cpu(), torch.tensor(S0[b:b + 1], dtype=torch.float32))
            continue
        sl = [a[b:b + 1, :n] for a in args]
        _, ref = orc.fwd(*sl, S0[b:b + 1])
        es = err_ratio(f64(S[b:b + 1]), ref)
        say(f"      b={b} n={n} err/rms S={es:.3e}")
        assert es <= tau_for(w.qkv), (b, n)


def test_clamped_acceptance_counts(kda, orc):
    """Counts outside [0, K] are clamped: negative keeps S, above K applies all K."""
    w = configs.HEADGROUP_BF16.scaled(B=2, H=2, T=8, name="spec_clamp")
    x, S0 = _draft_case(w, seed=8)
    d = {n: to_dev(x[n]) for n in NAMES}
    S = torch.tensor(S0, dtype=torch.float32, device="cuda")
    kda.kda_commit_step(d["k"], d["v"], d["g"], d["beta"], torch.tensor([-3, 99], dtype=torch.int32, device="cuda"), S)
    torch.cuda.synchronize()
    assert torch.equal(S[0].cpu(), torch.tensor(S0[0], dtype=torch.float32))
    _, ref = orc.fwd(*[x[n].f64()[1:2] for n in NAMES], S0[1:2])
    assert err_ratio(f64(S[1:2]), ref) <= 2e-2


def test_speculative_rounds_compose(kda, orc):
    """Several verify/commit rounds with varying acceptance equal one forward
    over the concatenation of the accepted tokens, and each round's verified
    outputs of the accepted tokens equal that forward's outputs."""
    w = configs.HEADGROUP_BF16.scaled(B=3, H=2, T=12, name="spec_rounds")
    rng = np.random.default_rng(11)
    S0 = gen.fwd_inputs(w, 0)["S0"].f64()
    S = torch.tensor(S0, dtype=torch.float32, device="cuda")
    kept = {n: [[] for _ in range(w.B)] for n in NAMES}
    outs = [[] for _ in range(w.B)]
    for rnd in range(4):
        x = gen.fwd_inputs(w, 100 + rnd)
        d = {n: to_dev(x[n]) for n in NAMES}
        o = kda.kda_verify_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
        acc = rng.integers(0, w.T + 1, size=w.B).astype(np.int32)
        kda.kda_commit_step(d["k"], d["v"], d["g"], d["beta"], torch.tensor(acc, device="cuda"), S)
        torch.cuda.synchronize()
        for b in range(w.B):
            n = int(acc[b])
            for name in NAMES:
                kept[name][b].append(x[name].f64()[b, :n])
            outs[b].append(f64(o)[b, :n])
    for b in range(w.B):
        args = [np.concatenate(kept[n][b], axis=0)[None] for n in NAMES]
        if args[0].shape[1] == 0:
            assert np.allclose(f64(S[b]), S0[b])
            continue
        o_ref, S_ref = orc.fwd(*args, S0[b:b + 1])
        eo = err_ratio(np.concatenate(outs[b], axis=0)[None], o_ref)
        es = err_ratio(f64(S[b:b + 1]), S_ref)
        say(f"[rounds] b={b} tokens={args[0].shape[1]} err/rms o={eo:.3e} S={es:.3e}")
        assert eo <= 2e-2 and es <= 2e-2


# ---------------------------------------------------------------- gate logits

GATE_CASES = [
    configs.HEADGROUP_BF16.scaled(H=3, T=300, name="gate_headgroup_bf16"),
    configs.TRAIN_BF16.scaled(B=2, H=2, T=200, name="gate_train_bf16_gates"),
    configs.TINY_F32.scaled(B=1, H=2, T=200, name="gate_tiny_f32"),
    configs.TINY_F32.scaled(B=1, H=2, T=130, dk=128, dv=128, gate="bf16", name="gate_f32_qkv_bf16_gates"),
]


@pytest.mark.parametrize("w", GATE_CASES, ids=[w.name for w in GATE_CASES])
def test_chunk_fwd_with_gate_logits(kda, orc, w):
    from oracle import gate_log_decay
    x = gen.gate_logit_inputs(w)
    d = {n: to_dev(x[n]) for n in x}
    say(f"[gate fwd] {w.name} B={w.B} T={w.T} H={w.H} dk={w.dk} qkv={w.qkv} gate={w.gate}")
    o, S = kda.kda_chunk_fwd_gate(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    g = gate_log_decay(x["z"].f64(), x["A_log"].f64())
    S0 = x["S0"].f64() if x["S0"] is not None else None
    o_ref, S_ref = orc.fwd(x["q"].f64(), x["k"].f64(), x["v"].f64(), g, x["beta"].f64(), S0)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms o={eo:.3e} S={es:.3e}")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv)


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_decode_with_gate_logits(kda, orc, qkv):
    from oracle import gate_log_decay
    w = configs.DECODE_BF16.scaled(B=3, H=4, qkv=qkv, steps=4)
    S = gen.decode_initial_state(w)
    S_dev, S_ref = to_dev(S), S.f64().copy()
    for step in range(w.steps):
        x = gen.decode_gate_logit_inputs(w, step)
        d = {n: to_dev(x[n]) for n in x}
        o = kda.kda_decode_step_gate(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["beta"], S_dev)
        g = gate_log_decay(x["z"].f64(), x["A_log"].f64())
        o_ref = orc.decode_step(x["q"].f64(), x["k"].f64(), x["v"].f64(), g, x["beta"].f64(), S_ref)
        torch.cuda.synchronize()
        assert err_ratio(f64(o), o_ref) <= tau_for(qkv), step
    assert err_ratio(f64(S_dev), S_ref) <= tau_for(qkv)


# ------------------------------------------------------------- full sizes

def test_full_size_verify_and_commit(kda, orc):
    """The benchmark's speculative workload: 256 x 96 states (dk = dv = 128,
    bf16 drafts, fp32 gates), 16 drafts, 8 accepted; sampled states against
    the oracle (verify outputs of all 16 drafts, committed state)."""
    from gpu_support import head_slices, spread_heads
    from kda_workloads import gen_torch
    w = configs.DECODE_BF16
    fw = configs.Workload(name="spec_drafts", kind="fwd", B=w.B, H=w.H, dk=w.dk, dv=w.dv, T=16,
                          qkv=w.qkv, gate=w.gate, s0_sd=None)
    say("[spec full] generating 256 x 96 states and 16 drafts each")
    S = gen_torch.decode_initial_state(w)
    x = gen_torch.fwd_inputs(fw)
    heads = spread_heads(w.B, w.H, 6, seed=3)
    S_sel = f64(torch.stack([S[b, h] for b, h in heads]).unsqueeze(0))
    o = kda.kda_verify_step(x["q"], x["k"], x["v"], x["g"], x["beta"], S)
    acc = torch.full((w.B,), 8, dtype=torch.int32, device="cuda")
    kda.kda_commit_step(x["k"], x["v"], x["g"], x["beta"], acc, S)
    torch.cuda.synchronize()
    s = head_slices(x, heads)
    say(f"[spec full] oracle on {heads}")
    o_ref, _ = orc.fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], S_sel, want_state=False)
    _, S_ref = orc.fwd(*(s[n][:, :8] for n in NAMES), S_sel)
    og = f64(torch.stack([o[b, :, h] for b, h in heads], dim=1).unsqueeze(0))
    Sg = f64(torch.stack([S[b, h] for b, h in heads]).unsqueeze(0))
    eo, es = err_ratio(og, o_ref), err_ratio(Sg, S_ref)
    say(f"      err/rms o={eo:.3e} S={es:.3e}")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv)
