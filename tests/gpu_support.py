"""Shared plumbing for the GPU parity tests: moving seeded inputs to the
device, running the oracle on sampled heads, and the error measure.

Tolerance (both outputs and final states, each against its own scale):
max |gpu - oracle| <= tau * RMS(oracle), with tau = 1e-4 when q/k/v are
float32 and tau = 2e-2 when they are bfloat16.
"""

from __future__ import annotations

import sys
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

TAU_F32 = 1e-4
TAU_BF16 = 2e-2

_TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def tau_for(qkv: str) -> float:
    return TAU_BF16 if qkv == "bf16" else TAU_F32


def to_dev(ht, device="cuda") -> Optional[torch.Tensor]:
    if ht is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(ht.values)).to(device).to(_TORCH[ht.dtype])


def f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_ratio(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    if not np.isfinite(err):
        return float("inf")
    return err / rms if rms > 0 else err


def head_slices(x: Dict[str, torch.Tensor], heads: Sequence[Tuple[int, int]], T: Optional[int] = None):
    """Gather the inputs of the listed (b, h) heads as one oracle batch with B = 1, H = len(heads)."""
    out = {}
    for n in ("q", "k", "v", "g", "beta"):
        t = x[n]
        parts = [t[b, :T, h] for b, h in heads]                 # [T, d] or [T]
        out[n] = f64(torch.stack(parts, dim=1).unsqueeze(0))     # [1, T, n, d]
    S0 = x.get("S0")
    out["S0"] = None if S0 is None else f64(torch.stack([S0[b, h] for b, h in heads]).unsqueeze(0))
    return out


def oracle_heads(orc, x: Dict[str, torch.Tensor], heads, T: Optional[int] = None, nthreads: int = 0):
    s = head_slices(x, heads, T)
    return orc.fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["S0"], nthreads=nthreads)


def gpu_heads(o: torch.Tensor, S: Optional[torch.Tensor], heads, T: Optional[int] = None):
    og = f64(torch.stack([o[b, :T, h] for b, h in heads], dim=1).unsqueeze(0))
    Sg = None if S is None else f64(torch.stack([S[b, h] for b, h in heads]).unsqueeze(0))
    return og, Sg


def spread_heads(B: int, H: int, n: int, seed: int = 0) -> List[Tuple[int, int]]:
    """n distinct (b, h) pairs, always including the first and the last head."""
    rng = np.random.default_rng(seed)
    picks = {(0, 0), (B - 1, H - 1)}
    while len(picks) < min(n, B * H):
        picks.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(picks)
