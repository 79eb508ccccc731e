"""Seeded synthetic input generators for the KDA workloads.

This module only draws random inputs and rounds them to their storage
dtype.  It contains none of the layer's own arithmetic (no decay
products, no state update, no read).  Both the oracle side and the GPU
side of every test take their inputs from here, so the two always see
bit-identical values.

Recipe (shared by every workload, sizes and parameters in configs.py):
  * q, k ~ N(0, 1) per element, then L2-normalised along the key axis per
    (b, t, h); v ~ N(0, 1).
  * log-decay g = -5 * sigmoid(z), z ~ N(z_mu, z_sd) per (b, t, h, key
    channel); optionally `forced_channels` key channels per (b, h), picked
    at random once, get z = forced_z at every token.
  * beta = sigmoid(N(0, 1)) per (b, t, h).
  * S0 ~ N(0, s0_sd) in fp32, or absent (zero state).
  * Values are drawn in float32 (normalisation and sigmoid in float64),
    then rounded once, round-to-nearest-even, to the storage dtype.

Every tensor has its own random stream, seeded by (seed, tensor id), so
tensors can be generated one at a time to bound host memory.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from .configs import Workload

# Stream ids: one independent numpy PCG64 stream per tensor.
_STREAM = {"q": 1, "k": 2, "v": 3, "g": 4, "beta": 5, "S0": 6}
_DECODE_STATE_STREAM = 99
_DECODE_STEP_BASE = 1000

_ROW_BLOCK = 1 << 22  # rows per block when normalising big tensors


@dataclass
class HostTensor:
    """A host array whose float32 values are exactly representable in `dtype`."""
    values: np.ndarray
    dtype: str  # "f32" | "bf16"

    @property
    def shape(self):
        return self.values.shape

    def f64(self) -> np.ndarray:
        return self.values.astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _to_dtype(x: np.ndarray, dtype: str) -> HostTensor:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return HostTensor(round_to_bf16(x), "bf16")
    if dtype == "f32":
        return HostTensor(x, "f32")
    raise ValueError(f"unknown dtype {dtype!r}")


def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), *[int(s) for s in stream]])


def _normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2_normalise_last(x: np.ndarray) -> np.ndarray:
    """Divide each vector along the last axis by its Euclidean norm (in place, float32 out)."""
    flat = x.reshape(-1, x.shape[-1])
    for r0 in range(0, flat.shape[0], _ROW_BLOCK):
        blk = flat[r0:r0 + _ROW_BLOCK].astype(np.float64)
        nrm = np.sqrt(np.einsum("ij,ij->i", blk, blk))[:, None]
        nrm[nrm == 0.0] = 1.0
        flat[r0:r0 + _ROW_BLOCK] = (blk / nrm).astype(np.float32)
    return x


def _sigmoid_f64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def _gate_logits(rng: np.random.Generator, shape, w: Workload, chan_axis_bh) -> np.ndarray:
    """The workload's gate logits z (float32), forced channels included."""
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if w.z_sd != 1.0 or w.z_mu != 0.0:
        z *= np.float32(w.z_sd)
        z += np.float32(w.z_mu)
    if w.forced_channels:
        B, H, dk = chan_axis_bh
        pick = np.argsort(rng.random((B, H, dk)), axis=-1)[..., : w.forced_channels]
        for b in range(B):
            for h in range(H):
                if z.ndim == 4:          # [B, T, H, dk]
                    z[b, :, h, pick[b, h]] = np.float32(w.forced_z)
                else:                    # [B, H, dk]
                    z[b, h, pick[b, h]] = np.float32(w.forced_z)
    return z


def _log_decay(rng: np.random.Generator, shape, w: Workload, chan_axis_bh) -> np.ndarray:
    """g = -5 * sigmoid(z) with the workload's logit distribution, float32."""
    z = _gate_logits(rng, shape, w, chan_axis_bh)
    out = np.empty(shape, dtype=np.float32)
    zf = z.reshape(-1)
    of = out.reshape(-1)
    step = _ROW_BLOCK * 16
    for i0 in range(0, zf.size, step):
        of[i0:i0 + step] = (-5.0 * _sigmoid_f64(zf[i0:i0 + step])).astype(np.float32)
    return out


def fwd_tensor(w: Workload, name: str, seed: int = 0) -> Optional[HostTensor]:
    """One input tensor of a forward workload, in the library's layout.

    q, k, g : [B, T, H, dk];  v : [B, T, H, dv];  beta : [B, T, H];
    S0 : [B, H, dk, dv] fp32, or None when the workload starts from zero.
    """
    assert w.kind == "fwd"
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    rng = _rng(seed, _STREAM[name])
    if name in ("q", "k"):
        return _to_dtype(_l2_normalise_last(_normal_f32(rng, (B, T, H, dk))), w.qkv)
    if name == "v":
        return _to_dtype(_normal_f32(rng, (B, T, H, dv)), w.qkv)
    if name == "g":
        return _to_dtype(_log_decay(rng, (B, T, H, dk), w, (B, H, dk)), w.gate)
    if name == "beta":
        z = _normal_f32(rng, (B, T, H))
        return _to_dtype(_sigmoid_f64(z).astype(np.float32), w.gate)
    if name == "S0":
        if w.s0_sd is None:
            return None
        s = _normal_f32(rng, (B, H, dk, dv)) * np.float32(w.s0_sd)
        return _to_dtype(s, "f32")
    raise KeyError(name)


def fwd_inputs(w: Workload, seed: int = 0) -> Dict[str, Optional[HostTensor]]:
    return {n: fwd_tensor(w, n, seed) for n in ("q", "k", "v", "g", "beta", "S0")}


_HEAD_SCALE_STREAM = 7


def head_log_scales(H: int, sd: float = 0.5, seed: int = 0) -> HostTensor:
    """Per-head gate log-scales A_h ~ N(0, sd), float32 [H] (A_h = 0 at initialisation)."""
    return HostTensor(_normal_f32(_rng(seed, _HEAD_SCALE_STREAM), (H,)) * np.float32(sd), "f32")


def gate_logit_inputs(w: Workload, seed: int = 0) -> Dict[str, Optional[HostTensor]]:
    """fwd_inputs with the raw gate logits "z" (same stream and distribution as
    the logits behind g, gate dtype) in place of g, plus per-head "A_log"."""
    assert w.kind == "fwd"
    out = {n: fwd_tensor(w, n, seed) for n in ("q", "k", "v", "beta", "S0")}
    B, T, H, dk = w.B, w.T, w.H, w.dk
    out["z"] = _to_dtype(_gate_logits(_rng(seed, _STREAM["g"]), (B, T, H, dk), w, (B, H, dk)), w.gate)
    out["A_log"] = head_log_scales(H, seed=seed)
    return out


def decode_gate_logit_inputs(w: Workload, step: int, seed: int = 0) -> Dict[str, HostTensor]:
    """decode_step_inputs with raw gate logits "z" in place of g, plus "A_log"."""
    assert w.kind == "decode"
    out = decode_step_inputs(w, step, seed)
    del out["g"]
    B, H, dk = w.B, w.H, w.dk
    out["z"] = _to_dtype(_gate_logits(_rng(seed, _DECODE_STEP_BASE + 8 * step + 4), (B, H, dk), w, (B, H, dk)),
                         w.gate)
    out["A_log"] = head_log_scales(H, seed=seed)
    return out


_OUT_GATE_STREAM = 8
_OUT_WEIGHT_STREAM = 9
_OUT_ROWS_STREAM = 10


def output_gate_logits(shape, dtype: str, seed: int = 0, stream: int = 0) -> HostTensor:
    """Output-gate logits z_out ~ N(0, 1) of any shape, rounded to `dtype`."""
    return _to_dtype(_normal_f32(_rng(seed, _OUT_GATE_STREAM, stream), tuple(shape)), dtype)


def output_norm_weight(dv: int, seed: int = 0) -> HostTensor:
    """Per-channel normalisation weight 1 + 0.1 N(0, 1), float32 [dv]."""
    return HostTensor(np.float32(1.0) + np.float32(0.1) * _normal_f32(_rng(seed, _OUT_WEIGHT_STREAM), (dv,)),
                      "f32")


def read_rows(rows: int, dv: int, dtype: str, seed: int = 0) -> HostTensor:
    """Stand-in reads o [rows, dv] for the output epilogue: N(0, 1) rows each
    scaled by exp(N(0, 1.5)), so row norms span several orders of magnitude;
    rows 3, 10, 17, ... are all zero (the eps-only case)."""
    rng = _rng(seed, _OUT_ROWS_STREAM)
    x = _normal_f32(rng, (rows, dv)) * np.exp(np.float32(1.5) * _normal_f32(rng, (rows, 1)))
    x[3::7] = 0.0
    return _to_dtype(x, dtype)


_GRAD_OUT_STREAM = 11
_GRAD_STATE_STREAM = 12


def grad_outputs(w: Workload, seed: int = 0, dtype: Optional[str] = None):
    """Upstream gradients for a forward workload: dO [B, T, H, dv] ~ N(0, 1)
    (rounded to `dtype`, default the q/k/v dtype) and dS_T [B, H, dk, dv] ~
    N(0, 1) float32."""
    assert w.kind == "fwd"
    dO = _to_dtype(_normal_f32(_rng(seed, _GRAD_OUT_STREAM), (w.B, w.T, w.H, w.dv)), dtype or w.qkv)
    dS = _to_dtype(_normal_f32(_rng(seed, _GRAD_STATE_STREAM), (w.B, w.H, w.dk, w.dv)), "f32")
    return dO, dS


def decode_initial_state(w: Workload, seed: int = 0) -> HostTensor:
    """S before the first decode step: [B, H, dk, dv] fp32, N(0, s0_sd) (zero if s0_sd is None)."""
    assert w.kind == "decode"
    if w.s0_sd is None:
        return HostTensor(np.zeros((w.B, w.H, w.dk, w.dv), np.float32), "f32")
    rng = _rng(seed, _DECODE_STATE_STREAM)
    return _to_dtype(_normal_f32(rng, (w.B, w.H, w.dk, w.dv)) * np.float32(w.s0_sd), "f32")


def decode_step_inputs(w: Workload, step: int, seed: int = 0) -> Dict[str, HostTensor]:
    """Token inputs of decode step `step`: q, k, g [B, H, dk]; v [B, H, dv]; beta [B, H]."""
    assert w.kind == "decode"
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    base = _DECODE_STEP_BASE + 8 * step
    out = {}
    out["q"] = _to_dtype(_l2_normalise_last(_normal_f32(_rng(seed, base + 1), (B, H, dk))), w.qkv)
    out["k"] = _to_dtype(_l2_normalise_last(_normal_f32(_rng(seed, base + 2), (B, H, dk))), w.qkv)
    out["v"] = _to_dtype(_normal_f32(_rng(seed, base + 3), (B, H, dv)), w.qkv)
    out["g"] = _to_dtype(_log_decay(_rng(seed, base + 4), (B, H, dk), w, (B, H, dk)), w.gate)
    zb = _normal_f32(_rng(seed, base + 5), (B, H))
    out["beta"] = _to_dtype(_sigmoid_f64(zb).astype(np.float32), w.gate)
    return out
