"""Edges of the bf16 path and of beta on the GPU, against the float64 oracle.

* Value scale: the fp16 operands of the forward (the state slab, the
  two-term U) hold values up to 65504.  Values scaled so that |o| and |S|
  reach 1e3..1e4 stay within the bf16 bound; values past the fp16 range make
  the outputs non-finite (loud), never finite and wrong.
* beta outside (0, 1): the erase/write is S <- (I - beta k k^T) S + beta k v^T
  ("K3 Architecture Illustrated", "Under what conditions are RoPE, PaTH, and
  KDA related?": the delta rule contains I - beta k k^T).  beta = 0 leaves only
  the fade; beta = 2 with a unit key makes I - 2 k k^T an orthogonal
  reflection, so with no fade (g = 0) and no write (v = 0) the state's
  Frobenius norm is preserved exactly.
* A NaN input stays visible: it reaches the outputs and state it feeds and
  leaves every other output bit-identical.

Bound: max |err| <= 2e-2 * RMS(oracle) (bf16 inputs).
"""

import numpy as np
import pytest
import torch

from gpu_support import err_ratio, f64, say, tau_for, to_dev
from kda_workloads import configs, gen
from kda_workloads.gen import HostTensor

pytestmark = pytest.mark.gpu

T_ = configs.TRAIN_BF16
H8 = configs.HEADGROUP_BF16
DEC = configs.DECODE_BF16
NAMES = ("q", "k", "v", "g", "beta")


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


def _with(x, name, values):
    """x with tensor `name` replaced by `values` (already exact in its dtype)."""
    y = dict(x)
    y[name] = HostTensor(np.ascontiguousarray(values, dtype=np.float32), x[name].dtype)
    return y


def _unit_keys(shape, seed):
    """Unit keys exact in bf16: four entries of +-0.5 at random channels."""
    rng = np.random.default_rng(seed)
    dk = shape[-1]
    k = np.zeros(shape, np.float32).reshape(-1, dk)
    for row in k:
        idx = rng.choice(dk, 4, replace=False)
        row[idx] = rng.choice([-0.5, 0.5], 4)
    return k.reshape(shape)


def _run_fwd(kda, x, ring):
    d = {n: to_dev(x[n]) for n in x}
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], ring=ring)
    torch.cuda.synchronize()
    return o, S


def _oracle_fwd(orc, x):
    return orc.fwd(*[x[n].f64() for n in NAMES], x["S0"].f64() if x["S0"] is not None else None)


RINGS = [True, False]


@pytest.mark.parametrize("ring", RINGS, ids=["ring", "pipelined"])
def test_large_values_within_bound(kda, orc, ring):
    """v scaled by 2^13 (exact in bf16): |o| and |S| reach the thousands (the
    largest values stay inside the fp16 range of the operands)."""
    w = T_.scaled(B=1, H=2, T=64 * 6 + 9, name="edge_large_v")
    x = gen.fwd_inputs(w, seed=21)
    x = _with(x, "v", x["v"].values * np.float32(8192.0))
    say(f"[large v] ring={ring} {w.name}")
    o, S = _run_fwd(kda, x, ring)
    o_ref, S_ref = _oracle_fwd(orc, x)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      max|o|={np.abs(o_ref).max():.3e} max|S|={np.abs(S_ref).max():.3e} err/rms o={eo:.3e} S={es:.3e}")
    assert np.abs(o_ref).max() > 1e3 and np.abs(S_ref).max() > 1e3
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv)


@pytest.mark.parametrize("ring", RINGS, ids=["ring", "pipelined"])
def test_values_past_fp16_range_are_loud(kda, orc, ring):
    """v scaled by 2^17 (about 1.3e5 per unit): the fp16 operands overflow and
    the outputs turn non-finite; whatever stays finite still matches."""
    w = T_.scaled(B=1, H=2, T=64 * 3, name="edge_overflow_v")
    x = gen.fwd_inputs(w, seed=22)
    x = _with(x, "v", x["v"].values * np.float32(131072.0))
    say(f"[overflow v] ring={ring}")
    o, S = _run_fwd(kda, x, ring)
    o_ref, _ = _oracle_fwd(orc, x)
    got = f64(o)
    bad = ~np.isfinite(got)
    say(f"      non-finite outputs: {int(bad.sum())} of {bad.size}")
    assert bad.any()
    ok = ~bad
    if ok.any():
        rms = float(np.sqrt(np.mean(o_ref * o_ref)))
        assert float(np.max(np.abs(got[ok] - o_ref[ok]))) <= tau_for(w.qkv) * rms


@pytest.mark.parametrize("ring", RINGS, ids=["ring", "pipelined"])
@pytest.mark.parametrize("beta", [0.0, 2.0], ids=["beta0", "beta2"])
def test_forward_beta_edges(kda, orc, ring, beta):
    w = H8.scaled(B=1, H=3, T=64 * 3 + 17, gate="bf16", name=f"edge_fwd_beta{beta:g}")
    x = gen.fwd_inputs(w, seed=23)
    x = _with(x, "beta", np.full(x["beta"].shape, beta, np.float32))
    say(f"[fwd beta={beta}] ring={ring}")
    o, S = _run_fwd(kda, x, ring)
    o_ref, S_ref = _oracle_fwd(orc, x)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms o={eo:.3e} S={es:.3e}")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv)


@pytest.mark.parametrize("ring", RINGS, ids=["ring", "pipelined"])
def test_forward_householder_keeps_the_norm(kda, orc, ring):
    """g = 0, beta = 2, v = 0, unit keys: S_T = R_T ... R_1 S_0 with each R an
    orthogonal reflection, so ||S_T||_F = ||S_0||_F for every head."""
    w = H8.scaled(B=1, H=3, T=64 * 4 + 11, gate="bf16", name="edge_householder")
    x = gen.fwd_inputs(w, seed=24)
    x = _with(x, "k", _unit_keys(x["k"].shape, 25))
    x = _with(x, "g", np.zeros(x["g"].shape, np.float32))
    x = _with(x, "v", np.zeros(x["v"].shape, np.float32))
    x = _with(x, "beta", np.full(x["beta"].shape, 2.0, np.float32))
    say(f"[householder fwd] ring={ring}")
    o, S = _run_fwd(kda, x, ring)
    o_ref, S_ref = _oracle_fwd(orc, x)
    n0 = np.linalg.norm(x["S0"].f64().reshape(w.H, -1), axis=1)
    n_ref = np.linalg.norm(S_ref.reshape(w.H, -1), axis=1)
    n_gpu = np.linalg.norm(f64(S).reshape(w.H, -1), axis=1)
    say(f"      ||S0|| {n0} oracle {n_ref} gpu {n_gpu}")
    assert np.allclose(n_ref, n0, rtol=1e-12)
    assert np.allclose(n_gpu, n0, rtol=2e-3)
    eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
    say(f"      err/rms o={eo:.3e} S={es:.3e}")
    assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv)


@pytest.mark.parametrize("beta", [0.0, 2.0], ids=["beta0", "beta2"])
def test_decode_beta_edges(kda, orc, beta):
    w = DEC.scaled(B=4, H=3, steps=6, name=f"edge_decode_beta{beta:g}")
    S_host = gen.decode_initial_state(w).f64()
    S = torch.tensor(S_host, dtype=torch.float32, device="cuda")
    S_ref = S_host.copy()
    say(f"[decode beta={beta}]")
    for step in range(w.steps):
        x = gen.decode_step_inputs(w, step)
        x = _with(x, "beta", np.full(x["beta"].shape, beta, np.float32))
        d = {n: to_dev(x[n]) for n in NAMES}
        o = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
        torch.cuda.synchronize()
        o_ref = orc.decode_step(*[x[n].f64() for n in NAMES], S_ref)
        eo, es = err_ratio(f64(o), o_ref), err_ratio(f64(S), S_ref)
        assert eo <= tau_for(w.qkv) and es <= tau_for(w.qkv), (step, eo, es)


def test_decode_householder_keeps_the_norm(kda, orc):
    w = DEC.scaled(B=2, H=3, steps=8, name="edge_decode_householder")
    S_host = gen.decode_initial_state(w).f64()
    S = torch.tensor(S_host, dtype=torch.float32, device="cuda")
    n0 = np.linalg.norm(S_host.reshape(w.B * w.H, -1), axis=1)
    for step in range(w.steps):
        x = gen.decode_step_inputs(w, step)
        x = _with(x, "k", _unit_keys(x["k"].shape, 100 + step))
        x = _with(x, "g", np.zeros(x["g"].shape, np.float32))
        x = _with(x, "v", np.zeros(x["v"].shape, np.float32))
        x = _with(x, "beta", np.full(x["beta"].shape, 2.0, np.float32))
        d = {n: to_dev(x[n]) for n in NAMES}
        kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    torch.cuda.synchronize()
    n = np.linalg.norm(f64(S).reshape(w.B * w.H, -1), axis=1)
    say(f"[householder decode] ||S0|| {n0[:3]} after {w.steps} reflections {n[:3]}")
    assert np.allclose(n, n0, rtol=1e-5)


@pytest.mark.parametrize("w", [H8.scaled(B=3, H=2, T=16, name="edge_spec_K16"),
                               H8.scaled(B=2, H=2, T=7, dv=256, name="edge_spec_K7_dv256")],
                         ids=["K16", "K7_dv256"])
def test_verify_commit_beta_two(kda, orc, w):
    """Drafts with beta = 2: verify's outputs and commit's states match the
    recurrence; with g = 0, v = 0 and unit keys the committed state keeps its
    norm."""
    x = gen.fwd_inputs(w, seed=26)
    x = _with(x, "beta", np.full(x["beta"].shape, 2.0, np.float32))
    S0 = x["S0"].f64()
    d = {n: to_dev(x[n]) for n in NAMES}
    S = torch.tensor(S0, dtype=torch.float32, device="cuda")
    o = kda.kda_verify_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    acc = np.array([w.T] + [w.T // 2] * (w.B - 1), np.int32)
    kda.kda_commit_step(d["k"], d["v"], d["g"], d["beta"], torch.tensor(acc, device="cuda"), S)
    torch.cuda.synchronize()
    args = [x[n].f64() for n in NAMES]
    o_ref, _ = orc.fwd(*args, S0, want_state=False)
    eo = err_ratio(f64(o), o_ref)
    say(f"[verify beta=2] {w.name} err/rms o={eo:.3e}")
    assert eo <= tau_for(w.qkv)
    for b in range(w.B):
        n = int(acc[b])
        _, ref = orc.fwd(*[a[b:b + 1, :n] for a in args], S0[b:b + 1])
        es = err_ratio(f64(S[b:b + 1]), ref)
        assert es <= tau_for(w.qkv), (b, es)
    # the reflection case
    y = _with(x, "k", _unit_keys(x["k"].shape, 27))
    y = _with(y, "g", np.zeros(x["g"].shape, np.float32))
    y = _with(y, "v", np.zeros(x["v"].shape, np.float32))
    d = {n: to_dev(y[n]) for n in NAMES}
    S = torch.tensor(S0, dtype=torch.float32, device="cuda")
    kda.kda_commit_step(d["k"], d["v"], d["g"], d["beta"], torch.full((w.B,), w.T, dtype=torch.int32,
                                                                      device="cuda"), S)
    torch.cuda.synchronize()
    n0 = np.linalg.norm(S0.reshape(w.B * w.H, -1), axis=1)
    n = np.linalg.norm(f64(S).reshape(w.B * w.H, -1), axis=1)
    say(f"[householder commit] {w.name} ||S0|| {n0[:2]} after {n[:2]}")
    assert np.allclose(n, n0, rtol=1e-5)


@pytest.mark.parametrize("ring", RINGS, ids=["ring", "pipelined"])
def test_nan_input_propagates(kda, ring):
    """A NaN in one value of one token of one head: that value column of that
    head turns NaN from the token's chunk on (outputs and final state); every
    other head, every other column and every earlier chunk is bit-identical
    to the clean run."""
    w = T_.scaled(B=2, H=3, T=64 * 6 + 5, name="edge_nan")
    x = gen.fwd_inputs(w, seed=28)
    o0, S0 = _run_fwd(kda, x, ring)
    b, t, h, c = 1, 200, 2, 5
    v = x["v"].values.copy()
    v[b, t, h, c] = np.nan
    o1, S1 = _run_fwd(kda, _with(x, "v", v), ring)
    chunk0 = (t // 64) * 64
    say(f"[nan] ring={ring} v[{b},{t},{h},{c}] = NaN")
    o0, o1, S0, S1 = (z.cpu() for z in (o0, o1, S0, S1))
    assert torch.isnan(o1[b, t, h, c])
    assert torch.isnan(o1[b, chunk0 + 64:, h, c]).all()
    assert torch.isnan(S1[b, h, :, c]).all()
    keep = torch.ones_like(o1, dtype=torch.bool)
    keep[b, chunk0:, h, c] = False
    assert torch.equal(o1[keep], o0[keep])
    keep_s = torch.ones_like(S1, dtype=torch.bool)
    keep_s[b, h, :, c] = False
    assert torch.equal(S1[keep_s], S0[keep_s])


def test_nan_input_propagates_in_decode(kda):
    w = DEC.scaled(B=3, H=2, steps=1, name="edge_nan_decode")
    S = torch.tensor(gen.decode_initial_state(w).f64(), dtype=torch.float32, device="cuda")
    S_clean = S.clone()
    x = gen.decode_step_inputs(w, 0)
    d = {n: to_dev(x[n]) for n in NAMES}
    o0 = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S_clean)
    v = x["v"].values.copy()
    v[2, 1, 7] = np.nan
    d["v"] = to_dev(_with(x, "v", v)["v"])
    o1 = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    torch.cuda.synchronize()
    assert torch.isnan(o1[2, 1, 7]) and torch.isnan(S[2, 1, :, 7]).all()
    keep = torch.ones_like(o1, dtype=torch.bool)
    keep[2, 1, 7] = False
    assert torch.equal(o1[keep], o0[keep])
    keep_s = torch.ones_like(S, dtype=torch.bool)
    keep_s[2, 1, :, 7] = False
    assert torch.equal(S[keep_s], S_clean[keep_s])
