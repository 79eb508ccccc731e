"""Pins of the backward oracle (oracle/kda_oracle_bwd.py): its gradients
against central finite differences of the forward, closed forms at beta = 0,
a hand-computed single token, and its forward against the pinned C oracle.

The pages define the recurrence but print no gradients, so every pin here
follows from the recurrence itself ("Review A - Sequence and depth", Free
recall: fade, erase/write, read).
"""

import math

import numpy as np
import pytest

from oracle import default as c_oracle
from oracle.kda_oracle_bwd import forward, kda_bwd


def _inputs(rng, B, T, H, dk, dv, beta_zero=False):
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, H, dv))
    g = -5.0 / (1.0 + np.exp(-rng.normal(size=(B, T, H, dk))))
    beta = np.zeros((B, T, H)) if beta_zero else 1.0 / (1.0 + np.exp(-rng.normal(size=(B, T, H))))
    S0 = rng.normal(size=(B, H, dk, dv))
    dO = rng.normal(size=(B, T, H, dv))
    dS = rng.normal(size=(B, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0), dO, dS


def _loss(x, dO, dS):
    o, S = forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    return float(np.sum(o * dO) + np.sum(S * dS))


def test_gradients_match_central_differences():
    rng = np.random.default_rng(0)
    x, dO, dS = _inputs(rng, 1, 5, 2, 3, 2)
    grads = kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], dO, dS)
    h = 1e-6
    for name in ("q", "k", "v", "g", "beta", "S0"):
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (_loss(xp, dO, dS) - _loss(xm, dO, dS)) / (2 * h)
        err = np.max(np.abs(grads["d" + name] - fd)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_single_token_by_hand():
    # dk = dv = 1: S0 = 2, alpha = 1/2, k = 0.6, v = 3, beta = 1/2, q = 1.5, dO = 2.
    # p = alpha S0 k = 0.6;  S1 = alpha S0 + beta k (v - p) = 1.72;  o = 2.58
    one = lambda a: np.full((1, 1, 1, 1), a)  # noqa: E731
    gr = kda_bwd(one(1.5), one(0.6), one(3.0), one(math.log(0.5)), np.full((1, 1, 1), 0.5),
                 np.full((1, 1, 1, 1), 2.0), one(2.0))
    assert abs(gr["dq"].item() - 1.72 * 2.0) < 1e-14                      # S1 dO
    assert abs(gr["dv"].item() - 0.5 * 0.6 * 1.5 * 2.0) < 1e-14           # beta k q dO
    assert abs(gr["dbeta"].item() - 0.6 * 2.4 * 1.5 * 2.0) < 1e-14        # k (v - p) q dO
    assert abs(gr["dk"].item() - 0.5 * 1.5 * 2.0 * (3.0 - 2 * 0.6)) < 1e-14   # beta q dO (v - 2 alpha S0 k)
    assert abs(gr["dg"].item() - 1.0 * (1 - 0.5 * 0.36) * 3.0) < 1e-14    # alpha S0 (1 - beta k^2) q dO
    assert abs(gr["dS0"].item() - 0.5 * (1 - 0.5 * 0.36) * 3.0) < 1e-14   # alpha (1 - beta k^2) q dO


def test_closed_forms_without_writes():
    """beta = 0: S_t = Diag(exp G_t) S0 with G_t = sum_{s<=t} g_s, so
    dq_t = S_t dO_t, dS0 = sum_t Diag(e^G_t) q_t dO_t^T + Diag(e^G_T) dS_T,
    dg_s,c = sum_{t>=s} e^{G_t,c} q_t,c (S0[c,:] . dO_t) + e^{G_T,c} (S0[c,:] . dS_T[c,:]),
    dk = dv = 0, and dbeta_s = sum_{t>=s} (q_t . e^{G_t - G_s} k_s) (v_s - S0^T e^{G_s} k_s) . dO_t
    + (e^{G_T - G_s} k_s)^T dS_T (v_s - S0^T e^{G_s} k_s)."""
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 1, 6, 1, 4, 3
    x, dO, dS = _inputs(rng, B, T, H, dk, dv, beta_zero=True)
    gr = kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], dO, dS)
    q, k, v, g, S0 = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["g"][0, :, 0], x["S0"][0, 0]
    dOt, dSt = dO[0, :, 0], dS[0, 0]
    G = np.cumsum(g, axis=0)
    assert np.all(gr["dk"] == 0.0) and np.all(gr["dv"] == 0.0)
    for t in range(T):
        assert np.allclose(gr["dq"][0, t, 0], (np.exp(G[t])[:, None] * S0) @ dOt[t], rtol=1e-13, atol=1e-13)
    dS0 = sum(np.outer(np.exp(G[t]) * q[t], dOt[t]) for t in range(T)) + np.exp(G[-1])[:, None] * dSt
    assert np.allclose(gr["dS0"][0, 0], dS0, rtol=1e-13, atol=1e-13)
    dg = np.zeros((T, dk))
    for s in range(T):
        for t in range(s, T):
            dg[s] += np.exp(G[t]) * q[t] * (S0 @ dOt[t])
        dg[s] += np.exp(G[-1]) * np.sum(S0 * dSt, axis=1)
    assert np.allclose(gr["dg"][0, :, 0], dg, rtol=1e-12, atol=1e-12)
    db = np.zeros(T)
    for s in range(T):
        resid = v[s] - S0.T @ (np.exp(G[s]) * k[s])
        for t in range(s, T):
            db[s] += (q[t] @ (np.exp(G[t] - G[s]) * k[s])) * (resid @ dOt[t])
        db[s] += (np.exp(G[-1] - G[s]) * k[s]) @ dSt @ resid
    assert np.allclose(gr["dbeta"][0, :, 0], db, rtol=1e-12, atol=1e-12)


def test_torch_forward_equals_the_c_oracle():
    rng = np.random.default_rng(2)
    x, _, _ = _inputs(rng, 2, 37, 2, 8, 5)
    o, S = forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    o2, S2 = c_oracle().fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, S2, rtol=1e-12, atol=1e-12)


def test_zero_upstream_gives_zero_gradients():
    rng = np.random.default_rng(3)
    x, dO, _ = _inputs(rng, 1, 4, 1, 3, 3)
    gr = kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], np.zeros_like(dO), None)
    for n, a in gr.items():
        assert np.all(a == 0.0), n


@pytest.mark.parametrize("seed", [4, 5])
def test_final_state_gradient_alone_is_the_transposed_transition(seed):
    """With dO = 0 the gradient of <S_T, dS_T> with respect to S0 is the
    transpose of the (linear in S0) map S0 -> S_T applied to dS_T:
    <S_T(S0 + E) - S_T(S0), dS_T> = <E, dS0> for any E."""
    rng = np.random.default_rng(seed)
    x, dO, dS = _inputs(rng, 1, 7, 1, 4, 3)
    gr = kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], np.zeros_like(dO), dS)
    E = rng.normal(size=x["S0"].shape)
    _, S1 = forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    _, S2 = forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"] + E)
    assert abs(np.sum((S2 - S1) * dS) - np.sum(E * gr["dS0"])) < 1e-11
