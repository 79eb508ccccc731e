"""Python front end of the float64 KDA oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg; never by the GPU library.  It marshals
numpy arrays into the C oracle and compiles that C file with gcc when no
built copy is present.

The C file's header states, with citations, what is computed: per token,
fade S <- Diag(exp g) S, erase/write S <- S + beta k (v - S^T k)^T, then the
read o = S^T q from the updated state.  Every function here takes and
returns float64 arrays in the library's layouts:
  q, k, g [B, T, H, dk];  v, o [B, T, H, dv];  beta [B, T, H];
  S0, S_final [B, H, dk, dv]  (decode drops the T axis).
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import tempfile
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "kda_oracle.c")
LIBRARY = os.path.join(HERE, "libkda_oracle.so")

_DP = ctypes.POINTER(ctypes.c_double)


def compile_oracle(source: str = SOURCE, out: str = LIBRARY, extra=()) -> str:
    """Build the oracle with gcc (IEEE double, no fast-math).  Returns the path."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", *extra,
           "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(_DP)


def _c64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


G_MIN = -5.0


def check_preconditions(q, k, v, g, beta, S=None) -> None:
    """The method's input domain: every input finite, and every log-decay in
    [g_min, 0] = [-5, 0] ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the g_min
    paragraphs: the scaled-sigmoid mapping holds each channel's log-decay
    between -5 and 0, which is what bounds the in-tile 1/Gamma rescale by e^80).
    The recurrence itself is defined for any g; this is a tripwire for inputs
    the GPU path does not accept.  Raises ValueError."""
    for name, x in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("S", S)):
        if x is not None and not np.all(np.isfinite(x)):
            raise ValueError(f"oracle input {name} holds a non-finite value")
    if g.size and (np.min(g) < G_MIN or np.max(g) > 0.0):
        raise ValueError(f"oracle log-decay outside [{G_MIN}, 0]: [{np.min(g)}, {np.max(g)}]")


class Oracle:
    """Handle on one built copy of the C oracle."""

    def __init__(self, lib_path: str = LIBRARY):
        if lib_path == LIBRARY and (not os.path.exists(LIBRARY)
                                    or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            compile_oracle()
        self.path = lib_path
        self.lib = ctypes.CDLL(lib_path)
        i = ctypes.c_int
        self.lib.kda_oracle_fwd.argtypes = [_DP] * 8 + [i] * 6
        self.lib.kda_oracle_fwd.restype = i
        self.lib.kda_oracle_decode.argtypes = [_DP] * 7 + [i] * 5
        self.lib.kda_oracle_decode.restype = i
        self.lib.kda_oracle_max_threads.argtypes = []
        self.lib.kda_oracle_max_threads.restype = i

    def max_threads(self) -> int:
        return int(self.lib.kda_oracle_max_threads())

    def fwd(self, q, k, v, g, beta, S0=None, *, want_state: bool = True,
            nthreads: int = 0, check: bool = True) -> Tuple[np.ndarray, Optional[np.ndarray]]:
        """Token-by-token forward.  Returns (o [B,T,H,dv], S_final [B,H,dk,dv] or None).
        With `check`, inputs outside the method's domain raise (check_preconditions)."""
        q, k, v, g, beta = (_c64(x) for x in (q, k, v, g, beta))
        if check:
            check_preconditions(q, k, v, g, beta, S0)
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and g.shape == q.shape
        assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
        if S0 is not None:
            S0 = _c64(S0)
            assert S0.shape == (B, H, dk, dv)
        o = np.zeros((B, T, H, dv), np.float64)
        Sf = np.zeros((B, H, dk, dv), np.float64) if want_state else None
        rc = self.lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(S0), _ptr(o), _ptr(Sf), B, T, H, dk, dv,
                                     int(nthreads))
        if rc != 0:
            raise RuntimeError("kda_oracle_fwd failed")
        return o, Sf

    def decode_step(self, q, k, v, g, beta, S, *, nthreads: int = 0, check: bool = True) -> np.ndarray:
        """One token for every (b, h): S [B,H,dk,dv] float64 updated IN PLACE; returns o [B,H,dv].
        With `check`, inputs outside the method's domain raise (check_preconditions)."""
        q, k, v, g, beta = (_c64(x) for x in (q, k, v, g, beta))
        if check:
            check_preconditions(q, k, v, g, beta, S)
        assert isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous
        B, H, dk = q.shape
        dv = v.shape[-1]
        assert S.shape == (B, H, dk, dv)
        o = np.zeros((B, H, dv), np.float64)
        rc = self.lib.kda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(S), _ptr(o), B, H, dk, dv, int(nthreads))
        if rc != 0:
            raise RuntimeError("kda_oracle_decode failed")
        return o


_DEFAULT: Optional[Oracle] = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        # KDA_ORACLE_LIBRARY: another build of the oracle (the sanitizer build of its tests)
        alt = os.environ.get("KDA_ORACLE_LIBRARY")
        _DEFAULT = Oracle(alt) if alt else Oracle()
    return _DEFAULT


def kda_fwd(q, k, v, g, beta, S0=None, **kw):
    return default().fwd(q, k, v, g, beta, S0, **kw)


def kda_decode_step(q, k, v, g, beta, S, **kw):
    return default().decode_step(q, k, v, g, beta, S, **kw)


def gate_log_decay(z, A_log, head_axis: int = -2) -> np.ndarray:
    """Log-decay from gate logits, float64: g = g_min * sigmoid(exp(A_h) * z)
    with g_min = -5 ("Kimi K3 - Lesson 3 of 14 - Sequence axis", the
    scaled-sigmoid mapping: sigmoid bounded in (0, 1) scaled by g_min bounds
    the log-decay in (-5, 0); A_h a per-head learnable log-scale initialised
    to 0).  The page omits the formula; the log-scale is read as scaling the
    logit inside the sigmoid, the one placement that keeps g in (-5, 0) for
    every A_h and reduces to -5 sigmoid(z) at A_h = 0.

    z: [..., H, dk] (H on `head_axis`), A_log: [H].  Written with exp of a
    non-positive argument on both branches, so no overflow for any finite z.
    """
    z = np.asarray(z, dtype=np.float64)
    shape = [1] * z.ndim
    shape[head_axis] = -1
    x = np.exp(np.asarray(A_log, dtype=np.float64)).reshape(shape) * z
    e = np.exp(-np.abs(x))
    sig = np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return -5.0 * sig


def output_gate(o, z, weight, eps: float) -> np.ndarray:
    """The output epilogue after the read, float64:
    y = o / sqrt(mean_j o_j^2 + eps) * weight * sigmoid(z), per (token, head)
    row over the dv value channels.

    "Kimi K3 - Lesson 3 of 14 - Sequence axis", the output-gate paragraph: after
    the recurrent read a gate decides which channels of the result pass through,
    full-rank and input-dependent per token; "K3 Architecture Illustrated", the
    KDA section under FIG 21: the module also holds a normalisation and output
    gating.  Neither page gives the form.  Reading: RMS normalisation of each
    head's read over its dv channels with a learnable per-channel weight
    [dv], then a sigmoid gate (a value in (0, 1) per channel, "which channels
    pass") from per-token logits z with o's shape.

    o, z: [..., dv]; weight: [dv]; eps >= 0.
    """
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    inv_rms = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return o * inv_rms * w * sig


def build_variant(source_text: str) -> Oracle:
    """Compile a modified copy of the oracle source into a temporary library.

    Used by the mutation tests, which plant mistakes into a copy of the oracle
    on the CPU to show that the pins catch them.
    """
    d = tempfile.mkdtemp(prefix="kda_oracle_variant_")
    try:
        src = os.path.join(d, "variant.c")
        with open(src, "w") as f:
            f.write(source_text)
        # once loaded, the library stays mapped after its file is removed
        return Oracle(compile_oracle(src, os.path.join(d, "libvariant.so")))
    finally:
        shutil.rmtree(d, ignore_errors=True)
