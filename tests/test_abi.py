"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/kda.h declares, and rejects bad arguments before any HIP call.

Only calls that fail validation (or have nothing to do) are made here: no
call reaches a kernel launch.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
PKG = os.path.join(ROOT, "gated_delta_rule_101_amd")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_101_amd import kda
    if not os.path.exists(kda.LIBRARY):
        from gated_delta_rule_101_amd.build_lib import build_library
        build_library()
    return kda.load_library()


def test_header_matches_binding():
    from gated_delta_rule_101_amd import kda
    assert _declared() == sorted(kda.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    from gated_delta_rule_101_amd import kda
    assert lib.kda_abi_version() == 6
    for st in (kda.KDA_OK, kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_ERR_LAUNCH,
               kda.KDA_ERR_SCRATCH):
        assert lib.kda_status_string(st).decode().startswith("KDA_")
    assert lib.kda_status_string(77).decode() == "KDA_ERR_UNKNOWN"


FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced (validation fails first)


def _fwd(lib, q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, beta=FAKE * 5, S0=None, o=FAKE * 6,
         Sf=None, B=1, T=64, H=1, dk=64, dv=64, qd=1, gd=0, od=0):
    return lib.kda_chunk_fwd(q, k, v, g, beta, S0, o, Sf, B, T, H, dk, dv, qd, gd, od, None)


def _dec(lib, q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, beta=FAKE * 5, S=FAKE * 6, o=FAKE * 7,
         B=1, H=1, dk=64, dv=64, qd=1, gd=0, od=0):
    return lib.kda_decode_step(q, k, v, g, beta, S, o, B, H, dk, dv, qd, gd, od, None)


def test_chunk_fwd_validation(lib):
    from gated_delta_rule_101_amd import kda
    INV, UNS, OK = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_OK
    big = 1 << 24   # spaced far enough apart that the fake buffers do not overlap
    base = dict(q=big, k=2 * big, v=3 * big, g=4 * big, beta=5 * big, o=6 * big)
    assert _fwd(lib, **{**base, "q": None}) == INV
    assert _fwd(lib, **{**base, "o": None}) == INV
    assert _fwd(lib, **{**base, "beta": None}) == INV
    assert _fwd(lib, **base, B=-1) == INV
    assert _fwd(lib, **base, T=-5) == INV
    assert _fwd(lib, **base, dk=0) == INV
    assert _fwd(lib, **base, qd=7) == INV
    assert _fwd(lib, **base, gd=-1) == INV
    assert _fwd(lib, **base, od=2) == INV
    assert _fwd(lib, **{**base, "q": big + 2}) == INV          # misaligned
    assert _fwd(lib, **{**base, "o": 2 * big + 64}) == INV     # o overlaps k
    assert _fwd(lib, **base, Sf=big + 128) == INV              # S_final overlaps q
    assert _fwd(lib, **base, S0=7 * big, Sf=7 * big + 256) == INV   # partial S0/S_final overlap
    assert _fwd(lib, **base, dk=96) == UNS
    assert _fwd(lib, **base, dk=256) == UNS
    assert _fwd(lib, **base, dv=96) == UNS
    assert _fwd(lib, **base, dv=576) == UNS
    # nothing to do: returns before touching the device
    assert _fwd(lib, **base, B=0) == OK
    assert _fwd(lib, **base, H=0) == OK
    assert _fwd(lib, q=None, k=None, v=None, g=None, beta=None, o=None, T=0) == OK   # T=0, no S_final


def test_decode_validation(lib):
    from gated_delta_rule_101_amd import kda
    INV, UNS, OK = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_OK
    big = 1 << 24
    base = dict(q=big, k=2 * big, v=3 * big, g=4 * big, beta=5 * big, S=6 * big, o=8 * big)
    assert _dec(lib, **{**base, "S": None}) == INV
    assert _dec(lib, **{**base, "S": 6 * big + 4}) == INV      # misaligned state
    assert _dec(lib, **{**base, "o": 6 * big + 512}) == INV    # o inside S
    assert _dec(lib, **{**base, "S": big}) == INV              # S over q
    assert _dec(lib, **base, H=-1) == INV
    assert _dec(lib, **base, od=5) == INV
    assert _dec(lib, **base, dk=32) == UNS
    assert _dec(lib, **base, dv=256) == UNS
    assert _dec(lib, **base, B=0) == OK


def test_missing_library_fails_loudly(tmp_path):
    from gated_delta_rule_101_amd import kda
    with pytest.raises(ImportError):
        kda.load_library(str(tmp_path / "libkda.so"))


def test_product_path_never_touches_the_oracle():
    """No source of the library or its binding imports, loads or names the oracle."""
    for dirpath, _, files in os.walk(PKG):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, fn)


def test_follow_on_entry_points_validation(lib):
    from gated_delta_rule_101_amd import kda
    INV, UNS, OK = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_OK
    big = 1 << 24
    q, k, v, g, b, S, o, A, acc = (i * big for i in range(1, 10))
    # verify: S is read-only and required; o must not overlap it
    verify = lambda **kw: lib.kda_verify_step(*(kw.get(n, d) for n, d in (  # noqa: E731
        ("q", q), ("k", k), ("v", v), ("g", g), ("beta", b), ("S", S), ("o", o))),
        kw.get("B", 2), kw.get("K", 16), 3, 128, 128, 1, 0, 0, None)
    assert verify(S=None) == INV
    assert verify(o=S + 256) == INV
    assert verify(K=-1) == INV
    assert verify(B=0) == OK
    assert verify(K=0) == OK
    # commit: accepted and S required, S must not overlap the drafts or the counts
    commit = lambda **kw: lib.kda_commit_step(*(kw.get(n, d) for n, d in (  # noqa: E731
        ("k", k), ("v", v), ("g", g), ("beta", b), ("acc", acc), ("S", S))),
        kw.get("B", 2), kw.get("K", 16), 3, 128, 128, 1, 0, None)
    assert commit(acc=None) == INV
    assert commit(S=None) == INV
    assert commit(acc=S + 64) == INV
    assert commit(acc=acc + 2) == INV          # misaligned int32 array
    assert commit(S=k + 512) == INV            # S over the keys
    assert commit(K=0) == OK
    # gate-logit forward and decode: A_log required and 4-byte aligned
    fwdg = lambda **kw: lib.kda_chunk_fwd_gate(*(kw.get(n, d) for n, d in (  # noqa: E731
        ("q", q), ("k", k), ("v", v), ("z", g), ("A", A), ("beta", b), ("S0", None), ("o", o), ("Sf", None))),
        1, 64, 2, kw.get("dk", 64), 64, 1, 0, 0, None)
    assert fwdg(A=None) == INV
    assert fwdg(A=A + 1) == INV
    assert fwdg(o=A) == INV                    # o over A_log
    assert fwdg(dk=96) == UNS
    decg = lambda **kw: lib.kda_decode_step_gate(*(kw.get(n, d) for n, d in (  # noqa: E731
        ("q", q), ("k", k), ("v", v), ("z", g), ("A", A), ("beta", b), ("S", S), ("o", o))),
        1, 2, 64, 64, 1, 0, 0, None)
    assert decg(A=None) == INV
    assert decg(S=A) == INV                    # S over A_log


def test_output_epilogue_validation(lib):
    from gated_delta_rule_101_amd import kda
    INV, UNS, OK = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_OK
    big = 1 << 24
    o, z, w, y = big, 2 * big, 3 * big, 4 * big
    gate = lambda o=o, z=z, w=w, y=y, eps=1e-6, rows=10, dv=128, od=0, zd=1, yd=0: \
        lib.kda_output_gate(o, z, w, eps, y, rows, dv, od, zd, yd, None)  # noqa: E731
    assert gate(o=None) == INV
    assert gate(z=None) == INV
    assert gate(w=None) == INV
    assert gate(y=None) == INV
    assert gate(w=w + 4) == INV                  # misaligned weight
    assert gate(y=y + 8) == INV                  # misaligned output
    assert gate(eps=-1.0) == INV
    assert gate(eps=float("nan")) == INV
    assert gate(eps=float("inf")) == INV
    assert gate(rows=-1) == INV
    assert gate(od=3) == INV
    assert gate(y=z + 256) == INV                # y overlaps z
    assert gate(y=o + 256) == INV                # partial overlap with o
    assert gate(y=w) == INV                      # y over the weight
    assert gate(dv=96) == UNS
    assert gate(dv=1024) == UNS
    assert gate(rows=0) == OK
    # fused decode: the epilogue's arguments are checked with the decode's
    q, k, v, g, b, S, zo, wt, yy = (i * big for i in range(1, 10))
    dec = lambda **kw: lib.kda_decode_step_gated(*(kw.get(n, d) for n, d in (  # noqa: E731
        ("q", q), ("k", k), ("v", v), ("g", g), ("A", None), ("beta", b), ("S", S), ("z", zo), ("w", wt))),
        kw.get("eps", 1e-6), kw.get("y", yy), kw.get("B", 2), 3, 128, 128, 1, 0, 0, None)
    assert dec(z=None) == INV
    assert dec(w=None) == INV
    assert dec(eps=-0.5) == INV
    assert dec(z=zo + 4) == INV                  # misaligned logits
    assert dec(y=zo + 128) == INV                # y over the logits
    assert dec(y=wt) == INV                      # y over the weight
    assert dec(y=yy + 4) == INV                  # misaligned y (vector stores)
    assert dec(B=0) == OK


def test_backward_validation(lib):
    from gated_delta_rule_101_amd import kda
    INV, UNS, OK = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_OK
    big = 1 << 28
    B, T, H, d = 1, 64, 2, 64
    need = lib.kda_chunk_bwd_workspace_bytes(B, T, H, d, d)
    assert need > 0 and need % 4 == 0
    assert lib.kda_chunk_bwd_workspace_bytes(B, 0, H, d, d) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(B, T, H, 96, d) == 0
    names = ("q", "k", "v", "g", "beta", "S0", "dO", "dS", "dq", "dk", "dv", "dg", "dbeta", "dS0", "ws")
    base = {n: (i + 1) * big for i, n in enumerate(names)}
    base["S0"] = base["dS"] = None

    def call(size=need, B=B, T=T, kdim=d, vdim=d, qd=1, **kw):
        p = {**base, **kw}
        return lib.kda_chunk_bwd(*(p[n] for n in names[:-1]), p["ws"], size, B, T, H, kdim, vdim, qd, 0, 0, None)

    assert call(q=None) == INV
    assert call(dq=None) == INV
    assert call(ws=None) == INV
    assert call(size=need - 4) == INV                    # workspace too small
    assert call(dk=base["q"] + 64) == INV                # a gradient over an input
    assert call(dg=base["dq"] + 256) == INV              # two gradients overlap
    assert call(ws=base["dv"] + 1024) == INV             # workspace over a gradient
    assert call(dS0=base["dO"]) == INV
    assert call(T=-1) == INV
    assert call(qd=4) == INV
    assert call(kdim=96) == UNS
    assert call(vdim=256) == UNS
    assert call(B=0) == OK
    assert call(T=0, dS0=None) == OK                     # nothing to write


def test_workspace_forward_validation(lib):
    """kda_chunk_fwd_ws / kda_chunk_fwd_gate_ws: the forward's own checks, plus
    the workspace's size, alignment and overlap."""
    from gated_delta_rule_101_amd import kda
    INV, UNS, OK = kda.KDA_ERR_INVALID_ARG, kda.KDA_ERR_UNSUPPORTED, kda.KDA_OK
    big = 1 << 30
    B, T, H, d = 2, 640, 3, 128
    need = lib.kda_chunk_fwd_workspace_bytes(B, T, H, d, d)
    assert need > 0 and need % 16 == 0
    assert lib.kda_chunk_fwd_workspace_bytes(B, 0, H, d, d) == 0     # nothing to run
    assert lib.kda_chunk_fwd_workspace_bytes(B, T, H, 64, 64) == 0   # dk = 64: no workspace used
    assert lib.kda_chunk_fwd_workspace_bytes(B, T, H, d, 96) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(B, T, H, d, 64) == 0    # one slab per head: nothing to share
    # more heads than one launch holds: the ring is sized for one launch
    assert lib.kda_chunk_fwd_workspace_bytes(4, T, 64, d, d) == lib.kda_chunk_fwd_workspace_bytes(4, T, 32, d, d)
    names = ("q", "k", "v", "g", "beta", "S0", "o", "Sf", "ws")
    base = {n: (i + 1) * big for i, n in enumerate(names)}
    base["S0"] = base["Sf"] = None

    def call(size=need, B=B, T=T, dk=d, dv=d, qd=1, **kw):
        p = {**base, **kw}
        return lib.kda_chunk_fwd_ws(*(p[n] for n in names), size, B, T, H, dk, dv, qd, 1, 0, None)

    assert call(q=None) == INV
    assert call(size=need - 16) == INV                   # workspace too small
    assert call(ws=base["ws"] + 8) == INV                # misaligned workspace
    assert call(ws=base["o"] + 4096) == INV              # workspace over the output
    assert call(ws=base["q"]) == INV                     # workspace over an input
    assert call(dk=96) == UNS
    assert call(B=0) == OK
    assert call(T=0) == OK                               # no S_final: nothing to write
    gate = lambda A=FAKE, **kw: lib.kda_chunk_fwd_gate_ws(  # noqa: E731
        *(kw.get(n, base[n]) for n in ("q", "k", "v", "g")), A, base["beta"], None, base["o"], None,
        kw.get("ws", base["ws"]), kw.get("size", need), B, T, H, d, d, 1, 1, 0, None)
    assert gate(A=None) == INV
    assert gate(size=1) == INV
    # kda_chunk_fwd_noalloc: the forward's checks, and inputs beyond its fixed scratch
    # (the ring of 64 heads) refused before anything is enqueued
    SCR = kda.KDA_ERR_SCRATCH
    na = lambda B=B, H=H, dv=d, qd=1, q=base["q"]: lib.kda_chunk_fwd_noalloc(  # noqa: E731
        q, base["k"], base["v"], base["g"], base["beta"], None, base["o"], None, B, T, H, d, dv, qd, 1, 0, None)
    assert na(q=None) == INV
    assert na(B=0) == OK
    assert na(B=5, H=13) == SCR                          # 65 heads with the ring
    assert na(B=4, H=16, dv=96) == UNS
    # the spin-bound hook returns the previous bound
    old = lib.kda_debug_set_spin_limit(123)
    assert lib.kda_debug_set_spin_limit(old) == 123


def test_seqpar_workspace_bytes_and_validation(lib):
    """Workspace size of the sequence-parallel forward (N, M and the segments'
    starting states, float32), 0 for invalid shapes; argument errors before
    any launch."""
    f = lib.kda_chunk_fwd_seqpar_workspace_bytes
    assert f(1, 4096, 8, 128, 128, 8) == 8 * 8 * (2 * 128 * 128 + 128 * 128) * 4
    assert f(2, 300, 3, 64, 128, 3) == 2 * 3 * 3 * (2 * 64 * 128 + 64 * 64) * 4
    for args in [(1, 4096, 8, 128, 128, 0), (1, 4096, 8, 128, 128, 65), (1, 4095, 8, 128, 128, 2),
                 (1, 4096, 8, 96, 128, 2), (1, 4096, 8, 128, 96, 2), (0, 4096, 8, 128, 128, 2)]:
        assert f(*args) == 0, args
    from gated_delta_rule_101_amd import kda
    INV = kda.KDA_ERR_INVALID_ARG
    # distinct, aligned, never dereferenced: each call fails validation first
    q, k, v, g, beta, o, ws = (ctypes.c_void_p((i + 1) << 36) for i in range(7))

    def call(segments, T=256, nbytes=1 << 30, qkv=kda.KDA_BF16):
        return lib.kda_chunk_fwd_seqpar(q, k, v, g, beta, None, o, None, ws, nbytes, 1, T, 2, 128, 128, segments,
                                        qkv, kda.KDA_F32, kda.KDA_F32, None)
    assert call(0) == INV and call(65) == INV and call(3) == INV          # range, not dividing T
    assert call(4, qkv=kda.KDA_F32) == kda.KDA_ERR_UNSUPPORTED
    assert call(4, nbytes=1024) == INV                                     # short workspace
    # the gate-logit form: a NULL A_log is an argument error before anything else
    assert lib.kda_chunk_fwd_gate_seqpar(q, k, v, g, None, beta, None, o, None, ws, 1 << 30, 1, 256, 2, 128, 128, 4,
                                         kda.KDA_BF16, kda.KDA_F32, kda.KDA_F32, None) == INV


def test_seqpar_segment_choice(lib):
    """kda_chunk_fwd_seqpar_segments (host arithmetic, with the compute-unit
    count given) picks what measured fastest on MI355X for the one-head-group
    shape (8 segments), two heads (16), a longer head group (16, its first
    pass in two rounds) and one long head (64); shapes whose plain grid already fills the device, and
    invalid shapes, take 1; the count always divides T."""
    f = lib.kda_chunk_fwd_seqpar_segments
    assert f(1, 4096, 8, 128, 128, 256) == 8            # 0.119 ms (16: 0.122, 4: 0.177, plain 0.317)
    assert f(1, 4096, 2, 128, 128, 256) == 16           # 0.096 ms (8: 0.113, 32: 0.108)
    assert f(1, 16384, 8, 128, 128, 256) == 16          # 0.267 ms (8: 0.326)
    assert f(1, 32768, 1, 128, 128, 256) == 64          # 0.215 ms (32: 0.224, plain 2.379)
    assert f(4, 16384, 32, 128, 128, 256) == 1          # training shape: 256 workgroups already
    assert f(1, 131072, 96, 128, 128, 256) == 1         # long sequence: 2 segments would need 768
    assert f(1, 64, 8, 128, 128, 256) == 1              # one chunk: nothing to gain
    for args in [(0, 4096, 8, 128, 128, 256), (1, 4096, 8, 96, 128, 256), (1, 0, 8, 128, 128, 256)]:
        assert f(*args) == 1, args
    for T in (1000, 4096, 333, 8192, 130):
        P = f(1, T, 2, 64, 64, 256)
        assert 1 <= P <= 64 and T % P == 0, (T, P)
