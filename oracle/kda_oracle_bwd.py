"""float64 gradients of the KDA token recurrence -- TEST INFRASTRUCTURE ONLY.

Imported by the tests (and nothing in the GPU library).  The forward here is
the plain definition, token by token, in float64 PyTorch on the CPU:

    S <- Diag(exp g_t) S                      fade each key channel
    S <- S + beta_t k_t (v_t - S^T k_t)^T      erase what k_t retrieves, write v_t
    o_t = S^T q_t                              read the updated state

("Review A - Sequence and depth", Free recall, the question on KDA's three
operations; "K3 Architecture Illustrated", FIG 21 and the delta-rule factor
I - beta k k^T in "Under what conditions are RoPE, PaTH, and KDA related?"),
and the gradients are taken by reverse-mode automatic differentiation of that
loop (torch.autograd, a library primitive) of the scalar

    L = sum(o * dO) + sum(S_T * dS_T),

so (dq, dk, dv, dg, dbeta, dS0) are the vector-Jacobian products of the
forward with the upstream gradients dO (and dS_T of the final state).  The
pages describe training of the layer but give no gradients; these are the
derivatives of the recurrence they define.  Pinned by central finite
differences and by closed forms at beta = 0 (tests/test_bwd_pins.py).

Layouts as the forward: q, k, g [B, T, H, dk]; v, dO [B, T, H, dv];
beta [B, T, H]; S0, dS_T [B, H, dk, dv].
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch


def _t(x) -> torch.Tensor:
    return torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64, requires_grad=True)


def forward_torch(q, k, v, g, beta, S0):
    """The token recurrence in float64 torch ops; returns (o [B,T,H,dv], S_T)."""
    B, T, H, dk = q.shape
    S = S0
    outs = []
    for t in range(T):
        S = torch.exp(g[:, t])[..., None] * S                          # fade
        p = torch.einsum("bhkv,bhk->bhv", S, k[:, t])                  # what k retrieves
        S = S + beta[:, t, :, None, None] * k[:, t, :, :, None] * (v[:, t] - p)[:, :, None, :]
        outs.append(torch.einsum("bhkv,bhk->bhv", S, q[:, t]))         # read after the write
    o = torch.stack(outs, dim=1) if outs else torch.zeros(B, 0, H, S.shape[-1], dtype=torch.float64)
    return o, S


def kda_bwd(q, k, v, g, beta, S0, dO, dS_T=None) -> Dict[str, np.ndarray]:
    """Gradients of sum(o * dO) + sum(S_T * dS_T) with respect to q, k, v, g,
    beta and S0 (S0 = None means a zero initial state; its gradient is still
    returned).  All float64 numpy arrays."""
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    ins = {n: _t(x) for n, x in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta))}
    ins["S0"] = _t(np.zeros((B, H, dk, dv)) if S0 is None else S0)
    with torch.enable_grad():
        o, S = forward_torch(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"])
        L = (o * torch.tensor(np.asarray(dO, np.float64))).sum()
        if dS_T is not None:
            L = L + (S * torch.tensor(np.asarray(dS_T, np.float64))).sum()
        names = ("q", "k", "v", "g", "beta", "S0")
        grads = torch.autograd.grad(L, [ins[n] for n in names], allow_unused=True)
    out = {}
    for n, gr in zip(names, grads):
        out["d" + n] = np.zeros(ins[n].shape) if gr is None else gr.detach().numpy()
    return out


def forward(q, k, v, g, beta, S0=None):
    """float64 forward through the same torch loop (for the finite-difference pins)."""
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    S0 = np.zeros((B, H, dk, dv)) if S0 is None else S0
    with torch.no_grad():
        o, S = forward_torch(*(torch.tensor(np.asarray(x, np.float64)) for x in (q, k, v, g, beta, S0)))
    return o.numpy(), S.numpy()
