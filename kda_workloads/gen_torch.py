"""Device-side generators for the full-size workloads (same recipe as gen.py).

The full-size forward and decode workloads hold up to 1.6e9 elements per
tensor; drawing them with numpy on the host takes minutes.  These functions
draw the same distributions with torch's seeded Philox generator directly on
the GPU and round with torch's round-to-nearest-even casts.  The random
streams differ from gen.py's (which the small cases use), the recipe does
not.  As with gen.py, nothing here touches the layer's arithmetic; the
oracle side receives the exact device values (copied back for the sampled
heads it checks).
"""

from __future__ import annotations

from typing import Dict, Optional

import torch

from .configs import Workload

_STREAM = {"q": 1, "k": 2, "v": 3, "g": 4, "beta": 5, "S0": 6}
_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(seed: int, stream: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed((int(seed) * 1_000_003 + int(stream)) & 0x7FFF_FFFF_FFFF_FFFF)
    return gen


def _normal(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    n = torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    return x.div_(n.clamp_min_(1e-30))


def _log_decay(shape, w: Workload, gen, device, bh_shape) -> torch.Tensor:
    z = _normal(shape, gen, device)
    if w.z_sd != 1.0 or w.z_mu != 0.0:
        z.mul_(w.z_sd).add_(w.z_mu)
    if w.forced_channels:
        B, H, dk = bh_shape
        pick = torch.rand((B, H, dk), generator=gen, device=device).argsort(dim=-1)[..., : w.forced_channels]
        mask = torch.zeros((B, H, dk), dtype=torch.bool, device=device)
        mask.scatter_(-1, pick, True)
        if z.dim() == 4:   # [B, T, H, dk]
            z.masked_fill_(mask[:, None, :, :], w.forced_z)
        else:
            z.masked_fill_(mask, w.forced_z)
    return torch.sigmoid(z).mul_(-5.0)


def fwd_tensor(w: Workload, name: str, seed: int = 0, device="cuda") -> Optional[torch.Tensor]:
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    gen = _gen(seed, _STREAM[name], device)
    if name in ("q", "k"):
        return _unit_rows(_normal((B, T, H, dk), gen, device)).to(_DTYPE[w.qkv])
    if name == "v":
        return _normal((B, T, H, dv), gen, device).to(_DTYPE[w.qkv])
    if name == "g":
        return _log_decay((B, T, H, dk), w, gen, device, (B, H, dk)).to(_DTYPE[w.gate])
    if name == "beta":
        return torch.sigmoid(_normal((B, T, H), gen, device)).to(_DTYPE[w.gate])
    if name == "S0":
        if w.s0_sd is None:
            return None
        return _normal((B, H, dk, dv), gen, device).mul_(w.s0_sd)
    raise KeyError(name)


def fwd_inputs(w: Workload, seed: int = 0, device="cuda") -> Dict[str, Optional[torch.Tensor]]:
    return {n: fwd_tensor(w, n, seed, device) for n in ("q", "k", "v", "g", "beta", "S0")}


def decode_initial_state(w: Workload, seed: int = 0, device="cuda") -> torch.Tensor:
    if w.s0_sd is None:
        return torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=device)
    return _normal((w.B, w.H, w.dk, w.dv), _gen(seed, 99, device), device).mul_(w.s0_sd)


def decode_step_inputs(w: Workload, step: int, seed: int = 0, device="cuda") -> Dict[str, torch.Tensor]:
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    base = 1000 + 8 * step
    out = {}
    out["q"] = _unit_rows(_normal((B, H, dk), _gen(seed, base + 1, device), device)).to(_DTYPE[w.qkv])
    out["k"] = _unit_rows(_normal((B, H, dk), _gen(seed, base + 2, device), device)).to(_DTYPE[w.qkv])
    out["v"] = _normal((B, H, dv), _gen(seed, base + 3, device), device).to(_DTYPE[w.qkv])
    out["g"] = _log_decay((B, H, dk), w, _gen(seed, base + 4, device), device, (B, H, dk)).to(_DTYPE[w.gate])
    out["beta"] = torch.sigmoid(_normal((B, H), _gen(seed, base + 5, device), device)).to(_DTYPE[w.gate])
    return out


_OUT_GATE_STREAM = 8
_OUT_WEIGHT_STREAM = 9


def output_gate_logits(shape, dtype: str, seed: int = 0, device="cuda") -> torch.Tensor:
    """Output-gate logits z_out ~ N(0, 1) (same recipe as gen.output_gate_logits)."""
    return _normal(tuple(shape), _gen(seed, _OUT_GATE_STREAM, device), device).to(_DTYPE[dtype])


def output_norm_weight(dv: int, seed: int = 0, device="cuda") -> torch.Tensor:
    """Per-channel normalisation weight 1 + 0.1 N(0, 1), float32 [dv]."""
    return _normal((dv,), _gen(seed, _OUT_WEIGHT_STREAM, device), device).mul_(0.1).add_(1.0)
