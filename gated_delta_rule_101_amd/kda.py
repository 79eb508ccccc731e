"""Python binding of libkda.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/kda.h).  PyTorch supplies device memory and the current stream;
nothing here computes any part of the layer, and there is no fallback: if
the library is missing or a call fails, an exception is raised.

    o, S_final = kda_chunk_fwd(q, k, v, g, beta, S0=None)
    o = kda_decode_step(q, k, v, g, beta, S)        # S updated in place
    y = kda_output_gate(o, z_out, weight, eps)      # RMS-normalised, sigmoid-gated

The output is float32 unless out_dtype=torch.bfloat16 is asked for: a
bfloat16 output carries only 8 significant bits, which for heavy-tailed
outputs is already a few percent of their RMS.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY selects another build of the library (a sanitizer build, say)
LIBRARY = os.environ.get("KDA_LIBRARY") or os.path.join(HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_LAUNCH, KDA_ERR_SCRATCH = 0, 1, 2, 3, 4

# Every symbol include/kda.h declares.
EXPORTS = ("kda_chunk_fwd", "kda_chunk_fwd_gate", "kda_chunk_fwd_ws", "kda_chunk_fwd_gate_ws",
           "kda_chunk_fwd_noalloc", "kda_chunk_fwd_seqpar", "kda_chunk_fwd_seqpar_workspace_bytes",
           "kda_chunk_fwd_seqpar_segments", "kda_chunk_fwd_gate_seqpar",
           "kda_chunk_fwd_workspace_bytes", "kda_debug_set_spin_limit", "kda_verify_step", "kda_commit_step",
           "kda_decode_step", "kda_decode_step_gate", "kda_decode_step_gated", "kda_output_gate",
           "kda_chunk_bwd", "kda_chunk_bwd_workspace_bytes", "kda_status_string", "kda_abi_version")

_lib: Optional[ctypes.CDLL] = None


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libkda.so (built by gated_delta_rule_101_amd.build_lib); raise if absent."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m gated_delta_rule_101_amd.build_lib` "
                          "(hipcc, gfx950) first")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [vp] * 8 + [i] * 8 + [vp]
    lib.kda_chunk_fwd.restype = i
    lib.kda_decode_step.argtypes = [vp] * 7 + [i] * 7 + [vp]
    lib.kda_decode_step.restype = i
    lib.kda_chunk_fwd_gate.argtypes = [vp] * 9 + [i] * 8 + [vp]
    lib.kda_chunk_fwd_gate.restype = i
    sz = ctypes.c_size_t
    lib.kda_chunk_fwd_ws.argtypes = [vp] * 9 + [sz] + [i] * 8 + [vp]
    lib.kda_chunk_fwd_noalloc.argtypes = [vp] * 8 + [i] * 8 + [vp]
    lib.kda_chunk_fwd_noalloc.restype = i
    lib.kda_chunk_fwd_ws.restype = i
    lib.kda_chunk_fwd_gate_ws.argtypes = [vp] * 10 + [sz] + [i] * 8 + [vp]
    lib.kda_chunk_fwd_gate_ws.restype = i
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i] * 5
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd_seqpar.argtypes = [vp] * 9 + [sz] + [i] * 9 + [vp]
    lib.kda_chunk_fwd_gate_seqpar.argtypes = [vp] * 10 + [sz] + [i] * 9 + [vp]
    lib.kda_chunk_fwd_gate_seqpar.restype = i
    lib.kda_chunk_fwd_seqpar.restype = i
    lib.kda_chunk_fwd_seqpar_workspace_bytes.argtypes = [i] * 6
    lib.kda_chunk_fwd_seqpar_workspace_bytes.restype = sz
    lib.kda_chunk_fwd_seqpar_segments.argtypes = [i] * 6
    lib.kda_chunk_fwd_seqpar_segments.restype = i
    lib.kda_debug_set_spin_limit.argtypes = [ctypes.c_uint]
    lib.kda_debug_set_spin_limit.restype = ctypes.c_uint
    lib.kda_decode_step_gate.argtypes = [vp] * 8 + [i] * 7 + [vp]
    lib.kda_decode_step_gate.restype = i
    lib.kda_verify_step.argtypes = [vp] * 7 + [i] * 8 + [vp]
    lib.kda_verify_step.restype = i
    lib.kda_commit_step.argtypes = [vp] * 6 + [i] * 7 + [vp]
    lib.kda_commit_step.restype = i
    f = ctypes.c_float
    lib.kda_output_gate.argtypes = [vp, vp, vp, f, vp, ctypes.c_int64, i, i, i, i, vp]
    lib.kda_output_gate.restype = i
    lib.kda_decode_step_gated.argtypes = [vp] * 9 + [f, vp] + [i] * 7 + [vp]
    lib.kda_decode_step_gated.restype = i
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [i] * 5
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd.argtypes = [vp] * 15 + [sz] + [i] * 8 + [vp]
    lib.kda_chunk_bwd.restype = i
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = i
    if path == LIBRARY:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _stream_handle(stream, device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _raise(status: int, what: str):
    if status != KDA_OK:
        raise KdaError(status, f"{what}: {status_string(status)}")


def kda_chunk_fwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int) -> int:
    """Bytes of device workspace kda_chunk_fwd_ws needs (0: it uses none)."""
    return int(load_library().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv))


def debug_set_spin_limit(limit: int) -> int:
    """Test hook: bound on the chunk kernels' internal waits; returns the old bound."""
    return int(load_library().kda_debug_set_spin_limit(int(limit)))


def _workspace(lib, workspace, B, T, H, dk, dv, device):
    need = int(lib.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv))
    if need == 0:
        return None
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return workspace


def _ring_pays(q: torch.Tensor, B: int, H: int, dk: int, dv: int) -> bool:
    """Whether the workspace (ring) kernel is the faster choice for this call:
    its workgroups share each head's state-independent chunk work, which pays
    for dv of 256 and more while the grid (B H dv/64 workgroups) fills at most
    half the device; at dv = 128 the two kernels measure the same
    (include/kda.h states the measured ratios)."""
    if q.dtype != torch.bfloat16 or dk != 128 or dv < 256 or dv % 64 or dv > 512 or not q.is_cuda:
        return False
    cus = torch.cuda.get_device_properties(q.device).multi_processor_count
    return 2 * B * H * (dv // 64) <= cus


def _use_ring(ring: Optional[bool], workspace, q, B, H, dk, dv) -> bool:
    if ring is not None:
        return ring
    return workspace is not None or _ring_pays(q, B, H, dk, dv)


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, S0: Optional[torch.Tensor] = None, *,
                  output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                  S_final: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  ring: Optional[bool] = None, workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA forward.  Shapes as in include/kda.h:
    q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; S0 [B,H,dk,dv] float32 or None.
    Returns (o [B,T,H,dv], S_final [B,H,dk,dv] float32 or None).  o is float32
    unless out_dtype (or a passed `o`) says bfloat16.  `S_final` may be passed
    (and may be S0 itself for an in-place continuation).  With ring=True the
    call goes through kda_chunk_fwd_ws with `workspace` (device bytes; allocated
    here when not given), ring=False calls kda_chunk_fwd; ring=None (default)
    takes the workspace path when a workspace is passed or the ring kernel is
    the faster one for the shape."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch between q, k, v, g, beta")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != g.dtype:
        raise TypeError("q, k, v share one dtype; g and beta share one dtype")
    if S0 is not None and (S0.shape != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("S0 must be float32 [B,H,dk,dv]")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif o.shape != (B, T, H, dv):
        raise ValueError("o must be [B,T,H,dv]")
    if S_final is None and output_final_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    ring = _use_ring(ring, workspace, q, B, H, dk, dv)
    ws = _workspace(lib, workspace, B, T, H, dk, dv, q.device) if ring else None
    dev = _check_dev(q, k, v, g, beta, S0, o, S_final, ws)
    if ring:
        st = lib.kda_chunk_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                  _ptr(S_final), _ptr(ws), _nbytes(ws), B, T, H, dk, dv, _dtype_code(q),
                                  _dtype_code(g), _dtype_code(o), _stream_handle(stream, dev))
        _raise(st, "kda_chunk_fwd_ws")
    else:
        st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                               _ptr(S_final), B, T, H, dk, dv, _dtype_code(q), _dtype_code(g),
                               _dtype_code(o), _stream_handle(stream, dev))
        _raise(st, "kda_chunk_fwd")
    return o, S_final


def kda_chunk_fwd_seqpar_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, segments: int) -> int:
    """Device bytes kda_chunk_fwd_seqpar needs (0: the shape or segment count is invalid)."""
    return int(load_library().kda_chunk_fwd_seqpar_workspace_bytes(B, T, H, dk, dv, segments))


def kda_chunk_fwd_seqpar_segments(B: int, T: int, H: int, dk: int, dv: int, cus: int = 0) -> int:
    """Segment count for kda_chunk_fwd_seqpar (1: the plain forward is expected
    faster); cus <= 0 takes the current device's compute-unit count."""
    return int(load_library().kda_chunk_fwd_seqpar_segments(B, T, H, dk, dv, cus))


def kda_chunk_fwd_seqpar(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                         beta: torch.Tensor, S0: Optional[torch.Tensor] = None, *, segments: Optional[int] = None,
                         output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                         S_final: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                         workspace: Optional[torch.Tensor] = None,
                         stream: Optional[torch.cuda.Stream] = None
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd_seqpar: the forward as `segments` pieces of the sequence run
    side by side and joined through their linear maps on the state (bfloat16
    q, k, v; `segments` divides T, and None takes
    kda_chunk_fwd_seqpar_segments' choice).  Shapes, dtypes and results as
    kda_chunk_fwd; `workspace` (device bytes) is allocated here when not given."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if segments is None:
        segments = int(lib.kda_chunk_fwd_seqpar_segments(B, T, H, dk, dv, 0))
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch between q, k, v, g, beta")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != g.dtype:
        raise TypeError("q, k, v share one dtype; g and beta share one dtype")
    if S0 is not None and (S0.shape != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("S0 must be float32 [B,H,dk,dv]")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif o.shape != (B, T, H, dv):
        raise ValueError("o must be [B,T,H,dv]")
    if S_final is None and output_final_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if workspace is None and T > 0:
        need = int(lib.kda_chunk_fwd_seqpar_workspace_bytes(B, T, H, dk, dv, int(segments)))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dev = _check_dev(q, k, v, g, beta, S0, o, S_final, workspace)
    st = lib.kda_chunk_fwd_seqpar(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                  _ptr(S_final), _ptr(workspace), _nbytes(workspace), B, T, H, dk, dv,
                                  int(segments), _dtype_code(q), _dtype_code(g), _dtype_code(o),
                                  _stream_handle(stream, dev))
    _raise(st, "kda_chunk_fwd_seqpar")
    return o, S_final


def kda_chunk_fwd_gate_seqpar(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, z: torch.Tensor,
                              A_log: torch.Tensor, beta: torch.Tensor, S0: Optional[torch.Tensor] = None, *,
                              segments: Optional[int] = None, output_final_state: bool = True,
                              o: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                              out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
                              stream: Optional[torch.cuda.Stream] = None
                              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd_gate_seqpar: kda_chunk_fwd_seqpar with the log-decay formed in
    the kernels from gate logits z [B,T,H,dk] and A_log [H] float32."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or z.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch between q, k, v, z, beta")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != z.dtype:
        raise TypeError("q, k, v share one dtype; z and beta share one dtype")
    if A_log.shape != (H,) or A_log.dtype != torch.float32:
        raise ValueError("A_log must be float32 [H]")
    if S0 is not None and (S0.shape != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("S0 must be float32 [B,H,dk,dv]")
    if segments is None:
        segments = int(lib.kda_chunk_fwd_seqpar_segments(B, T, H, dk, dv, 0))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif o.shape != (B, T, H, dv):
        raise ValueError("o must be [B,T,H,dv]")
    if S_final is None and output_final_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if workspace is None and T > 0:
        need = int(lib.kda_chunk_fwd_seqpar_workspace_bytes(B, T, H, dk, dv, int(segments)))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dev = _check_dev(q, k, v, z, A_log, beta, S0, o, S_final, workspace)
    st = lib.kda_chunk_fwd_gate_seqpar(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(beta), _ptr(S0),
                                       _ptr(o), _ptr(S_final), _ptr(workspace), _nbytes(workspace), B, T, H, dk,
                                       dv, int(segments), _dtype_code(q), _dtype_code(z), _dtype_code(o),
                                       _stream_handle(stream, dev))
    _raise(st, "kda_chunk_fwd_gate_seqpar")
    return o, S_final


def kda_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, S0: Optional[torch.Tensor], o: torch.Tensor,
                          S_final: Optional[torch.Tensor], stream: Optional[torch.cuda.Stream] = None) -> None:
    """kda_chunk_fwd_noalloc: the workspace forward with the library's own fixed
    scratch as the ring; o and S_final are the caller's (shapes as
    kda_chunk_fwd).  Raises KdaError (status KDA_ERR_SCRATCH) for inputs beyond
    the scratch."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch between q, k, v, g, beta")
    if o.shape != (B, T, H, dv) or (S_final is not None and S_final.shape != (B, H, dk, dv)):
        raise ValueError("o must be [B,T,H,dv], S_final [B,H,dk,dv]")
    dev = _check_dev(q, k, v, g, beta, S0, o, S_final)
    st = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                   _ptr(S_final), B, T, H, dk, dv, _dtype_code(q), _dtype_code(g),
                                   _dtype_code(o), _stream_handle(stream, dev))
    _raise(st, "kda_chunk_fwd_noalloc")


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, S: torch.Tensor, *, o: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One KDA token for every (b, h): q, k, g [B,H,dk]; v [B,H,dv]; beta [B,H];
    S [B,H,dk,dv] float32 updated IN PLACE.  Returns o [B,H,dv] (float32 unless
    out_dtype or a passed `o` says bfloat16)."""
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, H, dv) or beta.shape != (B, H):
        raise ValueError("shape mismatch between q, k, v, g, beta")
    if S.shape != (B, H, dk, dv) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,dk,dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != g.dtype:
        raise TypeError("q, k, v share one dtype; g and beta share one dtype")
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif o.shape != (B, H, dv):
        raise ValueError("o must be [B,H,dv]")
    dev = _check_dev(q, k, v, g, beta, S, o)
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                             B, H, dk, dv, _dtype_code(q), _dtype_code(g), _dtype_code(o),
                             _stream_handle(stream, dev))
    _raise(st, "kda_decode_step")
    return o


def _check_chunk_shapes(q, k, v, g, beta):
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    if (q is not None and q.shape != k.shape) or g.shape != k.shape or v.shape != (B, T, H, dv) \
            or beta.shape != (B, T, H):
        raise ValueError("shape mismatch between q, k, v, g, beta")
    if (q is not None and q.dtype != k.dtype) or v.dtype != k.dtype or beta.dtype != g.dtype:
        raise TypeError("q, k, v share one dtype; g and beta share one dtype")
    return B, T, H, dk, dv


def _check_head_scale(A_log: torch.Tensor, H: int):
    if A_log.shape != (H,) or A_log.dtype != torch.float32:
        raise ValueError("A_log must be float32 [H]")


def kda_chunk_fwd_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, z: torch.Tensor,
                       A_log: torch.Tensor, beta: torch.Tensor, S0: Optional[torch.Tensor] = None, *,
                       output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                       S_final: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                       ring: Optional[bool] = None, workspace: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd with the log-decay formed in the kernel from gate logits:
    g = -5 sigmoid(exp(A_log[h]) z).  z [B,T,H,dk] (gate dtype), A_log [H] float32.
    ring / workspace as kda_chunk_fwd (kda_chunk_fwd_gate_ws or kda_chunk_fwd_gate)."""
    lib = load_library()
    B, T, H, dk, dv = _check_chunk_shapes(q, k, v, z, beta)
    _check_head_scale(A_log, H)
    if S0 is not None and (S0.shape != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("S0 must be float32 [B,H,dk,dv]")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif o.shape != (B, T, H, dv):
        raise ValueError("o must be [B,T,H,dv]")
    if S_final is None and output_final_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    ring = _use_ring(ring, workspace, q, B, H, dk, dv)
    ws = _workspace(lib, workspace, B, T, H, dk, dv, q.device) if ring else None
    dev = _check_dev(q, k, v, z, A_log, beta, S0, o, S_final, ws)
    if ring:
        st = lib.kda_chunk_fwd_gate_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(beta), _ptr(S0),
                                       _ptr(o), _ptr(S_final), _ptr(ws), _nbytes(ws), B, T, H, dk, dv,
                                       _dtype_code(q), _dtype_code(z), _dtype_code(o), _stream_handle(stream, dev))
        _raise(st, "kda_chunk_fwd_gate_ws")
    else:
        st = lib.kda_chunk_fwd_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(beta), _ptr(S0),
                                    _ptr(o), _ptr(S_final), B, T, H, dk, dv, _dtype_code(q), _dtype_code(z),
                                    _dtype_code(o), _stream_handle(stream, dev))
        _raise(st, "kda_chunk_fwd_gate")
    return o, S_final


def kda_decode_step_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, z: torch.Tensor,
                         A_log: torch.Tensor, beta: torch.Tensor, S: torch.Tensor, *,
                         o: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                         stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """kda_decode_step with g = -5 sigmoid(exp(A_log[h]) z) formed in the kernel."""
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or z.shape != q.shape or v.shape != (B, H, dv) or beta.shape != (B, H):
        raise ValueError("shape mismatch between q, k, v, z, beta")
    if S.shape != (B, H, dk, dv) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,dk,dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != z.dtype:
        raise TypeError("q, k, v share one dtype; z and beta share one dtype")
    _check_head_scale(A_log, H)
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif o.shape != (B, H, dv):
        raise ValueError("o must be [B,H,dv]")
    dev = _check_dev(q, k, v, z, A_log, beta, S, o)
    st = lib.kda_decode_step_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(beta), _ptr(S),
                                  _ptr(o), B, H, dk, dv, _dtype_code(q), _dtype_code(z), _dtype_code(o),
                                  _stream_handle(stream, dev))
    _raise(st, "kda_decode_step_gate")
    return o


def kda_verify_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, S: torch.Tensor, *, o: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Outputs of K draft tokens per sequence ([B,K,H,*] inputs) through the
    state S [B,H,dk,dv], which is left unchanged.  Returns o [B,K,H,dv]."""
    lib = load_library()
    B, K, H, dk, dv = _check_chunk_shapes(q, k, v, g, beta)
    if S.shape != (B, H, dk, dv) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,dk,dv]")
    if o is None:
        o = torch.empty((B, K, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif o.shape != (B, K, H, dv):
        raise ValueError("o must be [B,K,H,dv]")
    dev = _check_dev(q, k, v, g, beta, S, o)
    st = lib.kda_verify_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                             B, K, H, dk, dv, _dtype_code(q), _dtype_code(g), _dtype_code(o),
                             _stream_handle(stream, dev))
    _raise(st, "kda_verify_step")
    return o


def kda_commit_step(k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                    accepted: torch.Tensor, S: torch.Tensor, *,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Advance S [B,H,dk,dv] IN PLACE by the first accepted[b] (int32 [B],
    clamped to [0, K]) of the K draft tokens of each sequence.  Returns S."""
    lib = load_library()
    B, K, H, dk, dv = _check_chunk_shapes(None, k, v, g, beta)
    if S.shape != (B, H, dk, dv) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,dk,dv]")
    if accepted.shape != (B,) or accepted.dtype != torch.int32:
        raise ValueError("accepted must be int32 [B]")
    dev = _check_dev(k, v, g, beta, accepted, S)
    st = lib.kda_commit_step(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(accepted), _ptr(S),
                             B, K, H, dk, dv, _dtype_code(k), _dtype_code(g), _stream_handle(stream, dev))
    _raise(st, "kda_commit_step")
    return S


def kda_output_gate(o: torch.Tensor, z: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, *,
                    y: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The output epilogue y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z)
    over the last axis (dv) of o [..., dv]; z has o's shape, weight is float32
    [dv].  y may be passed (o itself for in place, same dtype); otherwise it is
    allocated with out_dtype (default o's dtype)."""
    lib = load_library()
    dv = o.shape[-1]
    if z.shape != o.shape:
        raise ValueError("z must have o's shape")
    if weight.shape != (dv,) or weight.dtype != torch.float32:
        raise ValueError("weight must be float32 [dv]")
    if y is None:
        y = torch.empty(o.shape, dtype=out_dtype or o.dtype, device=o.device)
    elif y.shape != o.shape:
        raise ValueError("y must have o's shape")
    dev = _check_dev(o, z, weight, y)
    rows = o.numel() // dv if dv else 0
    st = lib.kda_output_gate(_ptr(o), _ptr(z), _ptr(weight), float(eps), _ptr(y), rows, dv,
                             _dtype_code(o), _dtype_code(z), _dtype_code(y), _stream_handle(stream, dev))
    _raise(st, "kda_output_gate")
    return y


def kda_decode_step_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, S: torch.Tensor, z_out: torch.Tensor, weight: torch.Tensor,
                          eps: float = 1e-6, *, A_log: Optional[torch.Tensor] = None,
                          y: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                          stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """kda_decode_step followed, in the same kernel, by the output epilogue:
    returns y [B,H,dv] = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z_out)
    (z_out [B,H,dv] in q's dtype, weight float32 [dv]); S is updated in place.
    With A_log [H] given, g holds gate logits as in kda_decode_step_gate."""
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, H, dv) or beta.shape != (B, H):
        raise ValueError("shape mismatch between q, k, v, g, beta")
    if S.shape != (B, H, dk, dv) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,dk,dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != g.dtype:
        raise TypeError("q, k, v share one dtype; g and beta share one dtype")
    if z_out.shape != (B, H, dv) or z_out.dtype != q.dtype:
        raise ValueError("z_out must be [B,H,dv] in q's dtype")
    if weight.shape != (dv,) or weight.dtype != torch.float32:
        raise ValueError("weight must be float32 [dv]")
    if A_log is not None:
        _check_head_scale(A_log, H)
    if y is None:
        y = torch.empty((B, H, dv), dtype=out_dtype or torch.float32, device=q.device)
    elif y.shape != (B, H, dv):
        raise ValueError("y must be [B,H,dv]")
    dev = _check_dev(q, k, v, g, beta, S, z_out, weight, A_log, y)
    st = lib.kda_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(A_log), _ptr(beta), _ptr(S),
                                   _ptr(z_out), _ptr(weight), float(eps), _ptr(y), B, H, dk, dv,
                                   _dtype_code(q), _dtype_code(g), _dtype_code(y), _stream_handle(stream, dev))
    _raise(st, "kda_decode_step_gated")
    return y


def kda_chunk_bwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int) -> int:
    """Bytes of device workspace kda_chunk_bwd needs for these sizes."""
    return int(load_library().kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv))


def kda_chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                  S0: Optional[torch.Tensor], dO: torch.Tensor, dS_final: Optional[torch.Tensor] = None, *,
                  want_dS0: bool = True, workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None):
    """Gradients of kda_chunk_fwd(q, k, v, g, beta, S0) for upstream dO
    [B,T,H,dv] (and dS_final [B,H,dk,dv] float32 or None).  Returns float32
    (dq, dk, dv, dg, dbeta, dS0) with the inputs' shapes (dS0 None unless
    want_dS0).  `workspace` (bytes, on the device) is allocated if not given."""
    lib = load_library()
    B, T, H, dk, dv = _check_chunk_shapes(q, k, v, g, beta)
    if dO.shape != (B, T, H, dv):
        raise ValueError("dO must be [B,T,H,dv]")
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None and (t.shape != (B, H, dk, dv) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [B,H,dk,dv]")
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk_, dg = (torch.empty((B, T, H, dk), **f32) for _ in range(3))
    dv_ = torch.empty((B, T, H, dv), **f32)
    dbeta = torch.empty((B, T, H), **f32)
    dS0 = torch.empty((B, H, dk, dv), **f32) if want_dS0 else None
    need = int(lib.kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    dev = _check_dev(q, k, v, g, beta, S0, dO, dS_final, workspace)
    st = lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_final),
                           _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(dbeta), _ptr(dS0),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           B, T, H, dk, dv, _dtype_code(q), _dtype_code(g), _dtype_code(dO),
                           _stream_handle(stream, dev))
    _raise(st, "kda_chunk_bwd")
    return dq, dk_, dv_, dg, dbeta, dS0
