"""Executable float64 specification of the chunkwise backward the GPU
kernels compute, checked against the autograd oracle.

Per 64-token chunk (chunk-local inclusive cumsum b of g, Gamma = e^b, the
chunkwise form of "Kimi K3 - Lesson 3 of 14 - Sequence axis"):
  A_qk = tril(sum_c q_rc k_sc e^{b_rc - b_sc}),  A_kk0 = strict_tril(same with k, k)
  N = (I + Diag(beta) A_kk0)^-1,  T = N Diag(beta)
  W = T (Gamma . K),  U_v = T V                       (S-independent, per chunk)
forward state pass:   U = U_v - W S,  S' = Diag(Gamma_C) S + K-bar^T U
reverse state pass:   dU = K-bar dS' + A_qk^T dO,
                      dS = Diag(Gamma_C) dS' + (Gamma . Q)^T dO - W^T dU
and the per-chunk gradients (dQ~ = dO S^T, dA_qk = tril(dO U^T),
dK-bar = U dS'^T, dW = -dU S^T, dT = dW K~^T + dU V^T, dN = dT Diag(beta),
dA_kk = -N^T dN N^T, the pairwise e^{b_r - b_s} products differentiated in
both roles, then dg = reverse cumsum of db).  The pairwise products use the
kernels' tile-local references: a row tile m scales its rows by
e^{b - rho_m} and the keys by e^{rho_m - b}, rho_m = b at the end of tile
m - 1, so no factor exceeds e^80 when g >= -5.
"""

import numpy as np
import pytest

from oracle.kda_oracle_bwd import kda_bwd

C, TILE = 64, 16


def _rowpart(D, X, b):
    """out[r] = sum_s D[r, s] X[s] e^{b_r - b_s} with tile-local references."""
    out = np.zeros((D.shape[0], X.shape[1]))
    for m in range(C // TILE):
        rows = slice(m * TILE, (m + 1) * TILE)
        rho = b[m * TILE - 1] if m else np.zeros(X.shape[1])
        keys = X[: (m + 1) * TILE] * np.exp(rho - b[: (m + 1) * TILE])   # <= e^80
        out[rows] = np.exp(b[rows] - rho) * (D[rows, : (m + 1) * TILE] @ keys)
    return out


def _colpart(D, X, b):
    """out[s] = sum_r D[r, s] X[r] e^{b_r - b_s} with tile-local references."""
    out = np.zeros((D.shape[1], X.shape[1]))
    for m in range(C // TILE):
        rows = slice(m * TILE, (m + 1) * TILE)
        rho = b[m * TILE - 1] if m else np.zeros(X.shape[1])
        xs = X[rows] * np.exp(b[rows] - rho)                               # in [e^-80, 1]
        part = D[rows, : (m + 1) * TILE].T @ xs
        out[: (m + 1) * TILE] += np.exp(rho - b[: (m + 1) * TILE]) * part
    return out


def _pairwise(X, Y, b, strict):
    """A[r, s] = sum_c X_rc Y_sc e^{b_rc - b_sc} for s <= r (s < r if strict)."""
    mask = np.tril(np.ones((C, C)), -1 if strict else 0)[..., None] > 0
    E = np.where(mask, np.exp(np.where(mask, b[:, None, :] - b[None, :, :], 0.0)), 0.0)   # [r, s, c]
    return np.einsum("rc,sc,rsc->rs", X, Y, E)


def chunk_bwd_head(q, k, v, g, beta, S0, dO, dST):
    """One head: [T, d] arrays; returns dq, dk, dv, dg, dbeta, dS0 (float64)."""
    T, dk = q.shape
    dv = v.shape[1]
    NC = -(-T // C)
    pad = NC * C - T
    P = lambda a: np.concatenate([a, np.zeros((pad,) + a.shape[1:])]) if pad else a  # noqa: E731
    q, k, v, g, beta, dO = P(q), P(k), P(v), P(g), P(beta), P(dO)
    low = np.tril(np.ones((C, C)))
    slow = np.tril(np.ones((C, C)), -1)
    pre = []
    for c in range(NC):
        sl = slice(c * C, (c + 1) * C)
        b = np.cumsum(g[sl], axis=0)
        Aqk = _pairwise(q[sl], k[sl], b, False)
        Akk0 = _pairwise(k[sl], k[sl], b, True)
        N = np.linalg.inv(np.eye(C) + beta[sl][:, None] * Akk0)
        Tm = N * beta[sl][None, :]
        Kt = np.exp(b) * k[sl]
        pre.append(dict(b=b, Aqk=Aqk, Akk0=Akk0, N=N, Tm=Tm, Qt=np.exp(b) * q[sl], Kt=Kt,
                        Kb=np.exp(b[-1] - b) * k[sl], W=Tm @ Kt, Uv=Tm @ v[sl]))
    # forward state pass
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    hs, Us = [], []
    for c in range(NC):
        p = pre[c]
        hs.append(S)
        U = p["Uv"] - p["W"] @ S
        Us.append(U)
        S = np.exp(p["b"][-1])[:, None] * S + p["Kb"].T @ U
    # reverse state pass with the per-chunk gradients
    dS = np.zeros((dk, dv)) if dST is None else dST.copy()
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    for c in reversed(range(NC)):
        p, S_c, U = pre[c], hs[c], Us[c]
        sl = slice(c * C, (c + 1) * C)
        b, GamC = p["b"], np.exp(p["b"][-1])
        dU = p["Kb"] @ dS + p["Aqk"].T @ dO[sl]
        dS_prev = GamC[:, None] * dS + p["Qt"].T @ dO[sl] - p["W"].T @ dU
        dQt = dO[sl] @ S_c.T
        dAqk = (dO[sl] @ U.T) * low
        dKb = U @ dS.T
        dGamC = np.sum(S_c * dS, axis=1)
        dW = -dU @ S_c.T
        dT = (dW @ p["Kt"].T + dU @ v[sl].T) * low
        dKt = p["Tm"].T @ dW
        dvv = p["Tm"].T @ dU
        dN = dT * beta[sl][None, :]
        dbeta = np.sum(dT * p["N"], axis=0)
        dAkk = -(p["N"].T @ dN @ p["N"].T) * slow
        dbeta += np.sum(dAkk * p["Akk0"], axis=1)
        dGkk = beta[sl][:, None] * dAkk
        rq = _rowpart(dAqk, k[sl], b)
        cq = _colpart(dAqk, q[sl], b)
        rk = _rowpart(dGkk, k[sl], b)
        ck = _colpart(dGkk, k[sl], b)
        dq = np.exp(b) * dQt + rq
        dkk = np.exp(b) * dKt + np.exp(b[-1] - b) * dKb + cq + rk + ck
        db = p["Qt"] * dQt + p["Kt"] * dKt - p["Kb"] * dKb + q[sl] * rq - k[sl] * cq + k[sl] * rk - k[sl] * ck
        db[-1] += np.sum(p["Kb"] * dKb, axis=0) + GamC * dGamC
        dg = np.cumsum(db[::-1], axis=0)[::-1]
        out["dq"][sl], out["dk"][sl], out["dv"][sl], out["dg"][sl], out["dbeta"][sl] = dq, dkk, dvv, dg, dbeta
        dS = dS_prev
    res = {n: a[:T] for n, a in out.items()}
    res["dS0"] = dS
    return res


def _case(rng, T, dk, dv, gmode="normal", s0=True, dst=True):
    q = rng.normal(size=(T, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.normal(size=(T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(T, dv))
    z = rng.normal(size=(T, dk))
    if gmode == "floor":
        z[:, :3] = 30.0                     # g = -5: tiles reach the e^80 bound
    g = -5.0 / (1.0 + np.exp(-z))
    beta = 1.0 / (1.0 + np.exp(-rng.normal(size=T)))
    S0 = rng.normal(size=(dk, dv)) * 0.3 if s0 else None
    dO = rng.normal(size=(T, dv))
    dST = rng.normal(size=(dk, dv)) if dst else None
    return q, k, v, g, beta, S0, dO, dST


@pytest.mark.parametrize("T,dk,dv,gmode,s0,dst", [
    (64, 8, 6, "normal", True, True),
    (150, 8, 5, "normal", True, False),     # ragged tail (identity padding)
    (128, 6, 4, "floor", False, True),      # decay floor, zero initial state
    (37, 4, 4, "normal", False, False),     # one partial chunk
])
def test_chunk_backward_equals_autograd(T, dk, dv, gmode, s0, dst):
    rng = np.random.default_rng(T + dk)
    q, k, v, g, beta, S0, dO, dST = _case(rng, T, dk, dv, gmode, s0, dst)
    got = chunk_bwd_head(q, k, v, g, beta, S0, dO, dST)
    E = lambda a: a[None, :, None]  # noqa: E731  -> [1, T, 1, d]
    ref = kda_bwd(E(q), E(k), E(v), E(g), beta[None, :, None],
                  None if S0 is None else S0[None, None], E(dO), None if dST is None else dST[None, None])
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        r = ref[n][0, :, 0]
        err = np.max(np.abs(got[n] - r)) / max(np.sqrt(np.mean(r * r)), 1e-300)
        assert err < 1e-9, (n, err)
    r = ref["dS0"][0, 0]
    assert np.max(np.abs(got["dS0"] - r)) / np.sqrt(np.mean(r * r)) < 1e-9
