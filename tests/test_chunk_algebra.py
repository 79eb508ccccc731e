"""Executable specification of the chunkwise algebra the GPU kernel uses (pin P9).

A float64 numpy rendering of the chunk form ("Kimi K3 - Lesson 3 of 14 -
Sequence axis": sequential between chunks, parallel within; output
O = (Gamma . Q) S + A V~; keys rescaled by 1/Gamma inside 16-token tiles),
with the tile-local reference points the kernel uses, the blocked
forward-substitution solve of the unit-lower erase system, and identity
padding for a ragged tail.  It must reproduce the token-by-token oracle to
1e-12 of the output RMS.  It lives in the tests only: neither the oracle nor
the GPU library imports it.

Derivation in brief.  Inside a chunk, with b_r the within-chunk cumulative
log-decay (per key channel) and u_r = beta_r (v_r - k_r^T D_r S_{r-1}) the
corrected value written at token r, the state is
S_r = Diag(e^{b_r}) S_0 + sum_{s<=r} Diag(e^{b_r - b_s}) k_s u_s^T.  So
  (I + A_kk) U = Diag(beta) (V - K~ S_0),  A_kk(r,s) = beta_r sum_c k_rc k_sc e^{b_rc-b_sc} (s<r)
  O = Q~ S_0 + A_qk U,                     A_qk(r,s) = sum_c q_rc k_sc e^{b_rc-b_sc}     (s<=r)
  S_C = Diag(e^{b_C}) S_0 + K-bar^T U,      K-bar_s = k_s e^{b_C - b_s}
with Q~ = e^{b} . Q and K~ = e^{b} . K.
"""

import numpy as np
import pytest

from kda_workloads import configs, gen
from oracle import default

C, TILE = 64, 16
NT = C // TILE


def chunk_form_head(q, k, v, g, beta, S):
    """One head: q, k, g [T, dk]; v [T, dv]; beta [T]; S [dk, dv] (copied)."""
    T, dk = q.shape
    dv = v.shape[1]
    S = S.copy()
    o = np.zeros((T, dv))
    Tp = -(-T // C) * C
    pad = Tp - T

    def padz(x):
        return np.concatenate([x, np.zeros((pad,) + x.shape[1:])], 0) if pad else x

    q, k, v, g, beta = (padz(x) for x in (q, k, v, g, beta))
    for c0 in range(0, Tp, C):
        Q, K, V, G, Bt = (x[c0:c0 + C] for x in (q, k, v, g, beta))
        # tile-local decay factors: all <= 1 except 1/f <= e^80
        bl = np.concatenate([np.cumsum(G[m * TILE:(m + 1) * TILE], 0) for m in range(NT)], 0)
        f = np.exp(bl)
        D = np.stack([f[(m + 1) * TILE - 1] for m in range(NT)])          # [NT, dk]
        tile_of = np.repeat(np.arange(NT), TILE)
        invf = 1.0 / f
        h = D[tile_of] * invf
        E = np.stack([np.prod(D[:m], 0) for m in range(NT)])              # decay before tile m
        A_ = np.stack([np.prod(D[m + 1:], 0) for m in range(NT)])         # decay after tile m
        Gam = E[tile_of] * f
        GamC = np.prod(D, 0)
        Qf, Kf, Kinv, Kh = Q * f, K * f, K * invf, K * h
        Aqk = np.zeros((C, C))
        L = np.zeros((C, C))
        for m in range(NT):
            rm = slice(m * TILE, (m + 1) * TILE)
            for n in range(m + 1):
                rn = slice(n * TILE, (n + 1) * TILE)
                if n == m:
                    blk_q = Qf[rm] @ Kinv[rn].T
                    blk_k = Kf[rm] @ Kinv[rn].T
                    Aqk[rm, rn] = np.tril(blk_q)
                    L[rm, rn] = np.tril(blk_k, -1) * Bt[rm, None]
                else:
                    P = np.prod(D[n + 1:m], 0)
                    Aqk[rm, rn] = (Qf[rm] * P) @ Kh[rn].T
                    L[rm, rn] = ((Kf[rm] * P) @ Kh[rn].T) * Bt[rm, None]
        X = V - (K * Gam) @ S
        U = np.zeros((C, dv))
        for m in range(NT):
            rm = slice(m * TILE, (m + 1) * TILE)
            inv_m = np.linalg.inv(np.eye(TILE) + L[rm, rm])
            rhs = Bt[rm, None] * X[rm]
            for n in range(m):
                rn = slice(n * TILE, (n + 1) * TILE)
                rhs = rhs - L[rm, rn] @ U[rn]
            U[rm] = inv_m @ rhs
        O = (Q * Gam) @ S + Aqk @ U
        Kbar = K * h * A_[tile_of]
        S = GamC[:, None] * S + Kbar.T @ U
        take = min(C, T - c0)
        if take > 0:
            o[c0:c0 + take] = O[:take]
    return o, S


def chunk_form(q, k, v, g, beta, S0):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for hh in range(H):
            S = S0[b, hh] if S0 is not None else np.zeros((dk, dv))
            o[b, :, hh], Sf[b, hh] = chunk_form_head(q[b, :, hh], k[b, :, hh], v[b, :, hh],
                                                     g[b, :, hh], beta[b, :, hh], S)
    return o, Sf


def _rms(x):
    return float(np.sqrt(np.mean(x * x)))


CASES = [
    configs.TINY_F32,
    configs.TRAIN_BF16.scaled(B=1, H=2, T=320, name="train_stress_small"),
    configs.TRAIN_BF16_LITERAL.scaled(B=1, H=2, T=200, name="train_literal_ragged"),
    configs.HEADGROUP_BF16.scaled(H=2, T=256, name="headgroup_small"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_chunk_form_matches_oracle(w):
    x = gen.fwd_inputs(w)
    args = [x[n].f64() for n in ("q", "k", "v", "g", "beta")]
    S0 = x["S0"].f64() if x["S0"] is not None else None
    o_ref, S_ref = default().fwd(*args, S0)
    o, S = chunk_form(*args, S0)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * _rms(o_ref)
    assert np.max(np.abs(S - S_ref)) <= 1e-12 * _rms(S_ref)


def test_chunk_form_at_the_decay_floor():
    """Every channel at g = -5 on every token: 1/f reaches e^80 in every tile."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 1, 128, 1, 16, 8
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = np.full((B, T, H, dk), -5.0)
    g[..., : dk // 2] = -0.01
    beta = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o_ref, S_ref = default().fwd(q, k, v, g, beta, S0)
    o, S = chunk_form(q, k, v, g, beta, S0)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * _rms(o_ref)
    assert np.max(np.abs(S - S_ref)) <= 1e-12 * _rms(S_ref)
