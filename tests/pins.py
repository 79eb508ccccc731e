"""Pins of the float64 oracle: facts fixed by the pages or by mathematics.

Each pin takes an `Oracle` handle and raises AssertionError when the oracle
disagrees.  None of them retypes the oracle's token loop: each checks a
worked example printed on the pages, a closed form, an invariant, or a
brute-force evaluation by a different route (products of explicit
transition matrices, in floating point and in exact rationals).

test_oracle_pins.py runs them on the real oracle; test_oracle_mutants.py
runs them on copies of the oracle with planted mistakes and requires every
mutant to fail at least one pin.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _unit(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max |err| {err:.3e} > {tol:.1e} * {scale:.3g}"


# --- P1: the pages' worked example -----------------------------------------

def pin_teaching_case(orc):
    """K3 Architecture Illustrated, 'Combining KDA and MLA': 1 + (3 - 1) = 3."""
    c = _load("delta_teaching_case.json")
    q = np.array(c["q"]).reshape(1, 1, 1, 1)
    k = np.array(c["k"]).reshape(1, 1, 1, 1)
    v = np.array(c["v"]).reshape(1, 1, 1, 1)
    g = np.array(c["g"]).reshape(1, 1, 1, 1)
    beta = np.array([c["beta"]]).reshape(1, 1, 1)
    S0 = np.array(c["S0"]).reshape(1, 1, 1, 1)
    o, S = orc.fwd(q, k, v, g, beta, S0)
    assert S[0, 0, 0, 0] == c["expected_S_final"][0][0], S
    assert o[0, 0, 0, 0] == c["expected_o"][0], o
    assert S[0, 0, 0, 0] != c["additive_memory_would_give"]


# --- P2: write then read under the same unit key returns v -----------------

def pin_write_read_same_key(orc, seed=1):
    """Unit k, beta = 1, q = k: o_t = v_t for ANY previous state and ANY decay.

    S_t^T k = (D S)^T (I - k k^T) k + v = v because (I - k k^T) k = 0.
    """
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 24, 2, 6, 5
    k = _unit(rng, B, T, H, dk)
    q = k.copy()
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 * rng.random((B, T, H, dk))
    beta = np.ones((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, _ = orc.fwd(q, k, v, g, beta, S0)
    _close(o, v, 1e-12, "write-then-read o vs v")


# --- P3: no write and no decay keeps the state ------------------------------

def pin_no_write_no_decay(orc, seed=2):
    """g = 0 and beta = 0: S_t = S0 for every t and o_t = S0^T q_t."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 9, 2, 5, 3
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = np.zeros((B, T, H, dk))
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = orc.fwd(q, k, v, g, beta, S0)
    assert np.array_equal(S, S0)
    ref = np.einsum("bhij,bthi->bthj", S0, q)
    _close(o, ref, 1e-13, "o = S0^T q")


# --- P4: reduction to (causal) linear attention -----------------------------

def pin_linear_attention(orc, seed=3):
    """g = 0, S0 = 0, mutually orthogonal unit keys: the erase term vanishes, so
    S_T = sum_t beta_t k_t v_t^T and o_t = sum_{s<=t} beta_s (q_t . k_s) v_s;
    with beta = 1 this is plain causal linear attention."""
    rng = np.random.default_rng(seed)
    B, H, dk, dv = 1, 2, 8, 6
    T = dk
    q = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    k = np.empty((B, T, H, dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k[0, :, h, :] = Qm.T          # rows are orthonormal
    g = np.zeros((B, T, H, dk))
    for beta in (np.ones((B, T, H)), rng.random((B, T, H))):
        o, S = orc.fwd(q, k, v, g, beta, None)
        S_ref = np.einsum("bth,bthi,bthj->bhij", beta, k, v)
        scores = np.einsum("bthi,bshi->bhts", q, k)
        mask = np.tril(np.ones((T, T)))
        o_ref = np.einsum("bhts,ts,bsh,bshj->bthj", scores, mask, beta, v)
        _close(S, S_ref, 1e-12, "linear-attention state")
        _close(o, o_ref, 1e-12, "linear-attention output")


# --- P5: pure channel-wise decay has a closed form --------------------------

def pin_pure_decay(orc, seed=4):
    """beta = 0: S_t = Diag(exp(sum_{s<=t} g_s)) S0, decaying each KEY channel
    (row of S) by its own factor; o_t = S_t^T q_t.  dk != dv exposes axis mix-ups."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 11, 2, 6, 4
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 * rng.random((B, T, H, dk))
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = orc.fwd(q, k, v, g, beta, S0)
    cum = np.cumsum(g, axis=1)                             # [B,T,H,dk]
    S_ref = np.exp(cum[:, -1])[..., None] * S0             # [B,H,dk,dv]
    o_ref = np.einsum("bthi,bhij,bthi->bthj", np.exp(cum), S0, q)
    _close(S, S_ref, 1e-13, "pure-decay state")
    _close(o, o_ref, 1e-13, "pure-decay output")


# --- P6: beta = 2 with a unit key is a Householder reflection ---------------

def pin_householder(orc, seed=5):
    """g = 0, v = 0, beta = 2, unit k: S <- (I - 2 k k^T) S, an orthogonal
    reflection ('RoPE, PaTH, and KDA' section: I - beta k k^T).  Frobenius norm
    is preserved and the same key applied twice restores the state."""
    rng = np.random.default_rng(seed)
    B, H, dk, dv = 1, 1, 7, 3
    T = 6
    kk = _unit(rng, T // 2, dk)
    k = np.concatenate([kk, kk[::-1]], 0).reshape(B, T, H, dk)   # palindrome of keys
    q = rng.standard_normal((B, T, H, dk))
    v = np.zeros((B, T, H, dv))
    g = np.zeros((B, T, H, dk))
    beta = np.full((B, T, H), 2.0)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = orc.fwd(q, k, v, g, beta, S0)
    # palindromic product of involutions is the identity
    _close(S, S0, 1e-12, "reflections undo themselves")
    # norm preserved after the first reflection
    o1, S1 = orc.fwd(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1], S0)
    assert abs(np.linalg.norm(S1) - np.linalg.norm(S0)) <= 1e-12 * np.linalg.norm(S0)
    Hm = np.eye(dk) - 2.0 * np.outer(kk[0], kk[0])
    _close(S1[0, 0], Hm @ S0[0, 0], 1e-12, "one reflection")


# --- P7: the transition is non-expansive -----------------------------------

def pin_non_expansive(orc, seed=6):
    """For g <= 0 and 0 <= beta |k|^2 <= 2 the map S -> (I - b k k^T) D S has
    spectral norm <= 1, so ||S_t||_2 <= ||S_{t-1}||_2 + |beta| |k| |v|."""
    rng = np.random.default_rng(seed)
    B, H, dk, dv, T = 1, 1, 6, 5, 40
    S = rng.standard_normal((B, H, dk, dv)) * 3.0
    for t in range(T):
        k = rng.standard_normal((B, 1, H, dk))
        kn2 = float(np.sum(k * k))
        beta = np.array([[[rng.uniform(0.0, 2.0 / kn2)]]])
        q = rng.standard_normal((B, 1, H, dk))
        v = rng.standard_normal((B, 1, H, dv))
        g = -5.0 * rng.random((B, 1, H, dk))
        _, S_new = orc.fwd(q, k, v, g, beta, S)
        lhs = np.linalg.norm(S_new[0, 0], 2)
        rhs = np.linalg.norm(S[0, 0], 2) + abs(beta.item()) * math.sqrt(kn2) * np.linalg.norm(v)
        assert lhs <= rhs * (1 + 1e-12), (t, lhs, rhs)
        S = S_new


# --- P8: brute force by products of transition matrices ---------------------

def _product_form(Ms, Ws, S0):
    """S_T = M_T ... M_1 S0 + sum_t M_T ... M_{t+1} W_t, generic over number types."""
    S = S0
    states = []
    for M, W in zip(Ms, Ws):
        S = _mm(M, S)
        S = _add(S, W)
        states.append(S)
    return states


def _mm(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), start=A[i][0] * 0) for j in range(p)]
            for i in range(n)]


def _add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _transition(alpha, k, beta):
    """M = (I - beta k k^T) Diag(alpha) as an explicit dk x dk matrix."""
    dk = len(k)
    one = alpha[0] * 0 + 1
    return [[((one if i == j else one * 0) - beta * k[i] * k[j]) * alpha[j] for j in range(dk)]
            for i in range(dk)]


def pin_brute_force_float(orc, seed=7):
    """Random tiny inputs (dk != dv): the oracle's o and S_final equal the
    product-of-transition-matrices evaluation M_t = (I - b_t k_t k_t^T) Diag(e^{g_t}),
    W_t = b_t k_t v_t^T, o_t = S_t^T q_t."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 7, 2, 4, 3
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk)) * 0.7
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 * rng.random((B, T, H, dk))
    beta = rng.random((B, T, H)) * 1.5
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = orc.fwd(q, k, v, g, beta, S0)
    for h in range(H):
        Ms, Ws = [], []
        for t in range(T):
            Ms.append(_transition(list(np.exp(g[0, t, h])), list(k[0, t, h]), beta[0, t, h]))
            Ws.append((beta[0, t, h] * np.outer(k[0, t, h], v[0, t, h])).tolist())
        states = _product_form(Ms, Ws, S0[0, h].tolist())
        for t in range(T):
            o_ref = np.array(states[t]).T @ q[0, t, h]
            _close(o[0, t, h], o_ref, 1e-12, f"brute-force o t={t} h={h}")
        _close(S[0, h], np.array(states[-1]), 1e-12, f"brute-force S h={h}")


def pin_brute_force_exact(orc):
    """Exact rational brute force.  Retentions 1, 1/2, 1/4 (g = -j ln 2), keys
    with rational entries (3/5, 4/5, ...), rational v, beta, q, S0.  The oracle
    (float64, exp(-j ln 2) rounded) must agree to a few ulps."""
    dk, dv, T = 3, 2, 5
    F = Fraction
    keys = [[F(3, 5), F(4, 5), F(0)], [F(0), F(3, 5), F(-4, 5)], [F(1, 2), F(1, 2), F(1, 2)],
            [F(-4, 5), F(0), F(3, 5)], [F(2, 3), F(-1, 3), F(2, 3)]]
    vals = [[F(3), F(-1)], [F(1, 2), F(2)], [F(-3, 2), F(1)], [F(5, 4), F(-2)], [F(1), F(1, 3)]]
    qs = [[F(1), F(-1, 2), F(1, 4)], [F(0), F(1), F(2)], [F(-1), F(1, 3), F(1)],
          [F(1, 2), F(1, 2), F(-1)], [F(2), F(0), F(1)]]
    betas = [F(1), F(1, 2), F(3, 4), F(2), F(1, 4)]
    jexp = [[0, 1, 2], [1, 0, 0], [2, 2, 1], [0, 0, 0], [1, 2, 0]]   # alpha = 2^-j
    S0 = [[F(1), F(2)], [F(-1), F(1, 2)], [F(0), F(3)]]
    Ms, Ws = [], []
    for t in range(T):
        alpha = [F(1, 2 ** j) for j in jexp[t]]
        Ms.append(_transition(alpha, keys[t], betas[t]))
        Ws.append([[betas[t] * keys[t][i] * vals[t][j] for j in range(dv)] for i in range(dk)])
    states = _product_form(Ms, Ws, S0)
    o_exact = [[sum((states[t][i][j] * qs[t][i] for i in range(dk)), F(0)) for j in range(dv)]
               for t in range(T)]

    def arr(x, shape):
        return np.array([[float(e) for e in row] for row in x]).reshape(shape)

    q = arr(qs, (1, T, 1, dk))
    k = arr(keys, (1, T, 1, dk))
    v = arr(vals, (1, T, 1, dv))
    g = np.array([[-j * math.log(2.0) for j in row] for row in jexp]).reshape(1, T, 1, dk)
    beta = np.array([float(b) for b in betas]).reshape(1, T, 1)
    o, S = orc.fwd(q, k, v, g, beta, arr(S0, (1, 1, dk, dv)))
    _close(o[0, :, 0], arr(o_exact, (T, dv)), 1e-14, "exact o")
    _close(S[0, 0], arr(states[-1], (dk, dv)), 1e-14, "exact S")


# --- P10: composability of the state carry, and decode vs. forward ----------

def pin_composable(orc, seed=8):
    """fwd(T1 + T2, S0) equals fwd(T2, S_final of fwd(T1, S0)) on the second part;
    one decode step after a T-token forward equals token T+1 of fwd(T+1)."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 13, 3, 5, 4
    q = rng.standard_normal((B, T, H, dk))
    k = _unit(rng, B, T, H, dk)
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 * rng.random((B, T, H, dk))
    beta = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = orc.fwd(q, k, v, g, beta, S0)
    T1 = 6
    o1, S1 = orc.fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
    o2, S2 = orc.fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], S1)
    assert np.array_equal(o1, o[:, :T1])
    assert np.array_equal(o2, o[:, T1:]) and np.array_equal(S2, S)
    _, Sp = orc.fwd(q[:, :-1], k[:, :-1], v[:, :-1], g[:, :-1], beta[:, :-1], S0)
    Sd = Sp.copy()
    od = orc.decode_step(q[:, -1], k[:, -1], v[:, -1], g[:, -1], beta[:, -1], Sd)
    assert np.array_equal(od, o[:, -1]) and np.array_equal(Sd, S)


# --- P11: identity (padding) tokens ----------------------------------------

def pin_identity_tokens(orc, seed=9):
    """Tokens with g = 0, beta = 0 and q = k = v = 0 leave the state untouched
    and read zero: padding a ragged tail with them changes nothing."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 1, 5, 2, 4, 3
    q = rng.standard_normal((B, T, H, dk))
    k = _unit(rng, B, T, H, dk)
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 * rng.random((B, T, H, dk))
    beta = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = orc.fwd(q, k, v, g, beta, S0)
    P = 7
    pad = lambda x: np.concatenate([x, np.zeros((B, P) + x.shape[2:])], axis=1)  # noqa: E731
    op, Sp = orc.fwd(pad(q), pad(k), pad(v), pad(g), pad(beta), S0)
    assert np.array_equal(Sp, S) and np.array_equal(op[:, :T], o)
    assert not np.any(op[:, T:])


ALL_PINS = [
    pin_teaching_case, pin_write_read_same_key, pin_no_write_no_decay,
    pin_linear_attention, pin_pure_decay, pin_householder, pin_non_expansive,
    pin_brute_force_float, pin_brute_force_exact, pin_composable, pin_identity_tokens,
]
