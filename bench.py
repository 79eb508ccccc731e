"""Throughput of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one kda_chunk_fwd over the training-shape workload
(B=4, H=32, T=16384, dk=dv=128, bf16 q/k/v/g/beta, fp32 state), inputs
already resident in HBM.  `value` is tokens/s (B*T tokens per step, each
token carrying all H heads).  The decode path is timed on its own workload
(B=256 sequences x H=96, d=128, 64 consecutive steps) and reported under
"decode" in GB/s.  Speculative decoding on the same states (verify 16 draft
tokens, commit 8 of them) is reported under "speculative", the output
epilogue (alone over the training-shape reads, and fused into decode) under
"epilogue", the chunkwise backward under "backward", and two secondary
forward workloads (one head group B1 H8 T4096, a latency figure; the long
sequence B1 H96 T131072, and one GPU's share of it under 8-way head sharding,
B1 H12 T131072; the first and the third also sequence-parallel) under
"forward_secondary", and the forward and decode with the log-decay formed
in the kernel from gate logits under "gate_prologue".  Each carries a
roofline object for its kernel, with the kernel's average duration measured
by HIP events on the launch stream, and `traffic`: the HBM bytes per launch
that the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
profiles/traffic.json, or null when the kernel's source has changed since
(for the backward, one launch is one call: the sum over its five kernels).
"peaks" holds what plain kernels reach on the same device (a streaming copy,
a loop of independent bf16 matrix-core products); every roofline also states
its fraction of that achievable peak.

Prints ONE JSON line on stdout (progress goes to stderr).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA chunk-fwd tokens/s + TFLOP/s (H=32,d=128,T=16K); decode GB/s vs roofline"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix, published
CHUNK = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic counts

def fwd_bytes(B, T, H, dk, dv, s_qkv, s_g, s_o, s0: bool, sfinal: bool) -> int:
    """Compulsory HBM bytes of one forward: read q, k, v, g, beta once, write o
    once; the fp32 state is read (S0) and written (S_final) once when present."""
    per_tok = s_qkv * (2 * dk + dv) + s_g * (dk + 1) + s_o * dv
    return B * T * H * per_tok + (int(s0) + int(sfinal)) * 4 * B * H * dk * dv


def fwd_executed_flops(B, T, H, dk, dv, C=CHUNK, tile=16) -> int:
    """Matrix-core FLOP the bf16 forward kernels execute, counted per 16x16
    tile product as issued (2 x 16 x 16 x K per instruction), including the
    zero halves of triangular tiles, the second terms of two-term operands and
    the state-independent work each dv/64 slab workgroup repeats:
      per chunk and slab (value columns 64): (Gamma.Q) S and (Gamma.K) S,
        2 x (C/16) x (dk/32) 16x16x32 products per 16 columns; the blocked
        solve, 6 strict tiles + 4 inverses x 2 terms, 16x16x16; the outputs,
        10 lower tiles x 2 terms, 16x16x16; the state update, (dk/16) x 2 x 2
        16x16x32;
      per chunk and slab, the prep: the in-tile cumsum, (C/16) x (dk/16)
        16x16x16; the diagonal Gram tiles, (C/16) x (dk/32) x 4 16x16x32; the
        6 off-diagonal tiles, 6 x (dk/32) x 2 16x16x32."""
    nt, kb, kt = C // tile, dk // 32, dk // 16
    m32, m16 = 2 * 16 * 16 * 32, 2 * 16 * 16 * 16
    cols = dv // 16
    state = cols * ((2 * nt * kb + kt * 2 * 2) * m32 + (6 + 4 * 2 + 10 * 2) * m16)
    nslab = max(1, dv // 64)
    prep = nslab * ((nt * kb * 4 + 6 * kb * 2) * m32 + nt * kt * m16)
    chunks = B * H * ((T + C - 1) // C)
    return chunks * (state + prep)


def fwd_flops(B, T, H, dk, dv, C=CHUNK) -> int:
    """Algorithmic FLOP of the chunkwise form per token-head: three C x d x d
    products (Gamma.Q S, Gamma.K S, K-bar^T U) = 6 dk dv; the four C x C x d
    triangular products at their non-zero half = 2 C (dk + dv); the unit-lower
    inverse ~ C^2 / 3."""
    return B * T * H * (6 * dk * dv + 2 * C * (dk + dv) + (C * C) // 3)


def decode_bytes(B, H, dk, dv, s_qkv, s_g, s_o) -> int:
    """One decode step: fp32 state read + written, q, k, v, g, beta read, o written."""
    return B * H * (8 * dk * dv + s_qkv * (2 * dk + dv) + s_g * (dk + 1) + s_o * dv)


def epilogue_bytes(rows, dv, s_o, s_z, s_y) -> int:
    """Output epilogue: each read and gate logit read once, each result written
    once, plus the fp32 weight vector."""
    return rows * dv * (s_o + s_z + s_y) + 4 * dv


def gated_decode_bytes(B, H, dk, dv, s_qkv, s_g, s_o) -> int:
    """A decode step with the epilogue fused: the decode's bytes plus the
    output-gate logits (q's dtype) and the weight vector."""
    return decode_bytes(B, H, dk, dv, s_qkv, s_g, s_o) + B * H * dv * s_qkv + 4 * dv


BWD_CHUNK = 32   # the backward kernels' chunk length


def bwd_flops(B, T, H, dk, dv, C=BWD_CHUNK) -> int:
    """Algorithmic FLOP of the chunkwise backward per token-head: eight
    C x d x d products with the state or its gradient (recomputed W S and
    K-bar^T U; K-bar dS', (Gamma.Q)^T dO, W^T dU; dO S^T, dU S^T, U dS'^T)
    = 16 dk dv; the C x C x d products at their non-zero half (A_qk, A_kk,
    W, dT's key part, dK~ and four pairwise-gradient products on the key
    side = 9 C dk; U_v, A_qk^T dO, dA_qk, dT's value part, dV = 5 C dv);
    the inverse and N^T dN N^T ~ C^2."""
    return B * T * H * (16 * dk * dv + 9 * C * dk + 5 * C * dv + C * C)


def bwd_bytes(B, T, H, dk, dv, s_qkv, s_g, s_do) -> int:
    """Compulsory HBM bytes of one backward: read q, k, v, g, beta, dO once,
    write float32 dq, dk, dv, dg, dbeta once (no initial or final state)."""
    return B * T * H * (s_qkv * (2 * dk + dv) + s_g * (dk + 1) + s_do * dv + 4 * (3 * dk + dv + 1))


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the kernel's source, its device helpers and the build script (compile flags)
CHUNK_SOURCES = ["gated_delta_rule_101_amd/csrc/kda_chunk_pipe.hip", "gated_delta_rule_101_amd/csrc/kda_device.h",
                 "gated_delta_rule_101_amd/build_lib.py"]
DECODE_SOURCES = ["gated_delta_rule_101_amd/csrc/kda_decode.hip", "gated_delta_rule_101_amd/csrc/kda_device.h",
                  "gated_delta_rule_101_amd/build_lib.py"]
RING_SOURCES = ["gated_delta_rule_101_amd/csrc/kda_chunk_ps.hip", "gated_delta_rule_101_amd/csrc/kda_chunk_tiles.h",
                "gated_delta_rule_101_amd/csrc/kda_device.h", "gated_delta_rule_101_amd/build_lib.py"]
BWD_SOURCES = ["gated_delta_rule_101_amd/csrc/kda_bwd.hip", "gated_delta_rule_101_amd/csrc/kda_device.h",
               "gated_delta_rule_101_amd/build_lib.py"]
VERIFY_SOURCES = ["gated_delta_rule_101_amd/csrc/kda_verify.hip", "gated_delta_rule_101_amd/csrc/kda_device.h",
                  "gated_delta_rule_101_amd/build_lib.py"]
EPILOGUE_SOURCES = ["gated_delta_rule_101_amd/csrc/kda_epilogue.hip", "gated_delta_rule_101_amd/csrc/kda_device.h",
                    "gated_delta_rule_101_amd/build_lib.py"]
# kernel record -> (substrings its rocprofv3 kernel name must all contain, sources);
# verify and commit are the two instantiations of one tile kernel (its last
# template argument), the output epilogue is the stand-alone one
SINGLE_KERNELS = (
    ("kda_chunk_fwd", ("kda_chunk_pipe_kernel",), CHUNK_SOURCES),
    ("kda_chunk_fwd_ws", ("kda_chunk_ps_kernel",), RING_SOURCES),
    ("kda_decode_step", ("kda_decode_kernel",), DECODE_SOURCES),
    ("kda_verify_step", ("kda_verify_tile_kernel<", "false>("), VERIFY_SOURCES),
    ("kda_commit_step", ("kda_verify_tile_kernel<", "true>("), VERIFY_SOURCES),
    ("kda_output_gate", ("kda_output_gate_kernel",), EPILOGUE_SOURCES),
)
# the five kernels of one backward call, in launch order
BWD_KERNELS = ("kda_bwd_prep_kernel", "kda_bwd_states_kernel", "kda_bwd_dstates_kernel",
               "kda_bwd_sgrads_kernel", "kda_bwd_intra_kernel")


def stored_traffic(kernel: str, sources) -> "dict | None":
    """HBM bytes per launch from the committed counter runs, if the kernel
    source is unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(sources):
        return None
    return rec


# ------------------------------------------------------------------- timing

def time_launches(fn, steps, warmup, stream, per_launch=False):
    """Wall time of `steps` back-to-back calls and the mean kernel duration
    from HIP events recorded around each launch on `stream` (and, with
    per_launch, the list of the launches' durations in seconds)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    each = [a.elapsed_time(b) * 1e-3 for a, b in ev]
    ker = sum(each) / steps
    return (wall, ker, each) if per_launch else (wall, ker)


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


# achievable peaks measured by bench_peaks (None until measured)
ACHIEVABLE = {"hbm_GBs": None, "bf16_TFLOPs": None}


def roofline(algo_bytes_per_launch, kernel_s, traffic_rec):
    achieved = algo_bytes_per_launch / kernel_s / 1e9
    traffic = None
    if traffic_rec:
        traffic = traffic_rec["hbm_bytes_per_launch"]
    out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    if ACHIEVABLE["hbm_GBs"]:
        out["achievable_peak"] = ACHIEVABLE["hbm_GBs"]
        out["frac_of_achievable"] = round(achieved / ACHIEVABLE["hbm_GBs"], 4)
    return out


def bench_peaks(reps=10):
    """What plain kernels reach here: a 1 GiB streaming device copy (bytes read
    plus bytes written per second) and a loop of independent bf16 16x16x32
    matrix-core products on every CU (FLOP per second)."""
    import ctypes
    import torch
    from gated_delta_rule_101_amd.build_lib import PROBE_LIBRARY
    lib = ctypes.CDLL(PROBE_LIBRARY)
    lib.kda_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.kda_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def copy():
        assert lib.kda_probe_copy(src.data_ptr(), dst.data_ptr(), n, sh) == 0

    _, ker, each = time_launches(copy, reps, 3, stream, per_launch=True)
    probe_gbs = 2 * n / min(each) / 1e9
    _, ker, each = time_launches(lambda: dst.copy_(src), reps, 3, stream, per_launch=True)
    runtime_gbs = 2 * n / min(each) / 1e9
    lib.kda_probe_update.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p]

    def update():
        assert lib.kda_probe_update(src.data_ptr(), n, 0, sh) == 0

    _, ker, each = time_launches(update, reps, 3, stream, per_launch=True)
    update_gbs = 2 * n / min(each) / 1e9
    copy_gbs = max(probe_gbs, runtime_gbs, update_gbs)
    del src, dst
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 4 * cus, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    rates = {}
    for big, shape, flop_per in ((0, "16x16x32", 8 * 16384), (1, "32x32x16", 4 * 32768)):
        def mfma():
            assert lib.kda_probe_mfma(out.data_ptr(), blocks, iters, big, sh) == 0

        _, ker_m, each_m = time_launches(mfma, reps, 3, stream, per_launch=True)
        rates[shape] = blocks * 4 * iters * flop_per / min(each_m) / 1e12
    tfs = max(rates.values())
    ACHIEVABLE["hbm_GBs"] = round(copy_gbs, 1)
    ACHIEVABLE["bf16_TFLOPs"] = round(tfs, 1)
    log(f"[bench] peaks: device copy {copy_gbs:.0f} GB/s, bf16 MFMA loop {tfs:.0f} TFLOP/s")
    return {"hbm_copy": {"GB/s": round(copy_gbs, 1), "frac_of_published": round(copy_gbs / HBM_PEAK_GBS, 4),
                         "by_kernel_GB/s": {"probe_copy": round(probe_gbs, 1), "torch_copy": round(runtime_gbs, 1),
                                            "probe_in_place": round(update_gbs, 1)},
                         "sample": f"1 GiB moved each way: a streaming copy (the probe kernel: 16 KB per "
                                   f"workgroup, non-temporal loads and stores), torch's copy_, and the same probe "
                                   f"read-modify-writing in place; the fastest, read + write bytes, best of {reps}"},
            "mfma_bf16": {"TFLOP/s": round(tfs, 1), "frac_of_published": round(tfs / BF16_MFMA_PEAK_TFLOPS, 4),
                          "by_shape_TFLOP/s": {k: round(v, 1) for k, v in rates.items()},
                          "sample": f"{blocks} workgroups x 4 waves x {iters} rounds of independent bf16 products "
                                    f"(8 of 16x16x32 or 4 of 32x32x16), the faster shape, best of {reps}"}}


# --------------------------------------------------------------- workloads

def bench_fwd(kda, steps, warmup):
    import torch
    from kda_workloads import configs, gen_torch
    w = configs.TRAIN_BF16
    log(f"[bench] generating {w.name} on the device")
    d = gen_torch.fwd_inputs(w)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, o=o, S_final=Sf)

    log(f"[bench] chunk_fwd: {warmup} warmup + {steps} timed launches")
    wall, ker, each = time_launches(step, steps, warmup, stream, per_launch=True)
    nbytes = fwd_bytes(w.B, w.T, w.H, w.dk, w.dv, 2, 2, 4, s0=False, sfinal=True)
    nbytes_bf16_o = fwd_bytes(w.B, w.T, w.H, w.dk, w.dv, 2, 2, 2, s0=False, sfinal=True)
    flops = fwd_flops(w.B, w.T, w.H, w.dk, w.dv)
    executed = fwd_executed_flops(w.B, w.T, w.H, w.dk, w.dv)
    ms = wall / steps * 1e3
    tok_s = w.B * w.T / (wall / steps)
    log(f"[bench] chunk_fwd {ms:.3f} ms/step (kernel mean {ker * 1e3:.3f}, median {median(each) * 1e3:.3f}, "
        f"min {min(each) * 1e3:.3f} ms), {tok_s:.3e} tokens/s")
    rf = roofline(nbytes, ker, stored_traffic("kda_chunk_fwd", CHUNK_SOURCES))
    # the same kernel time against the byte count with a bfloat16 o (the
    # survey's count; the kernel writes float32 o here)
    rf["frac_bf16_o_count"] = round(nbytes_bf16_o / ker / 1e9 / HBM_PEAK_GBS, 4)
    rf["bytes_bf16_o_count"] = nbytes_bf16_o
    tflops = flops / ker / 1e12
    ex_tflops = executed / ker / 1e12
    extra = {
        "tflops": round(flops / (wall / steps) / 1e12, 2),
        "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "executed_mfma_flop_per_step": executed,
        "executed_mfma_tflops": round(ex_tflops, 2),
        "executed_mfma_frac": round(ex_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "algorithmic_flop_per_step": flops,
        "algorithmic_bytes_per_step": nbytes,
        "kernel": "kda_chunk_pipe_kernel (no workspace: the ring kernel is slower on a full-device grid)",
        "kernel_ms": round(ker * 1e3, 4),
        "kernel_ms_median": round(median(each) * 1e3, 4),
        "kernel_ms_min": round(min(each) * 1e3, 4),
        "timed_launches": steps,
    }
    if ACHIEVABLE["bf16_TFLOPs"]:
        extra["executed_mfma_frac_of_achievable"] = round(ex_tflops / ACHIEVABLE["bf16_TFLOPs"], 4)
    return w, d, ms, tok_s, rf, extra


def bench_fwd_secondary(kda, w, steps, warmup):
    """Secondary forward workloads, timed like the headline one: the single
    head group (B1 H8 T4096: eight sequential carries, a latency figure) and
    the long single sequence (B1 H96 T131072: 2048 chunks per carry).  Both
    forward kernels are timed: the pipelined one (kda_chunk_fwd) and the ring
    one (kda_chunk_fwd_ws, its workspace allocated before timing), and, where
    the plain grid has at most 64 workgroups, the sequence-parallel forward
    (kda_chunk_fwd_seqpar) at 4, 8 and 16 segments and at the count
    kda_chunk_fwd_seqpar_segments picks; the figures at the top of the record
    are the fastest one's.  The third workload is one GPU's share of the long
    sequence under 8-way head sharding (B1 H12 T131072)."""
    import torch
    from kda_workloads import gen_torch
    log(f"[bench] generating {w.name} on the device")
    d = gen_torch.fwd_inputs(w)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    need = kda.kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    s_q, s_g = (2 if w.qkv == "bf16" else 4), (2 if w.gate == "bf16" else 4)
    nbytes = fwd_bytes(w.B, w.T, w.H, w.dk, w.dv, s_q, s_g, 4, s0=d["S0"] is not None, sfinal=True)
    flops = fwd_flops(w.B, w.T, w.H, w.dk, w.dv)
    runs = {}
    for name, ring in (("pipelined", False), ("ring", True)):
        if ring and ws is None:
            continue

        def step():
            kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o=o, S_final=Sf,
                              ring=ring, workspace=ws if ring else None)

        wall, ker, each = time_launches(step, steps, warmup, stream, per_launch=True)
        ms = wall / steps * 1e3
        log(f"[bench] {w.name} {name}: {ms:.3f} ms/step (kernel mean {ker * 1e3:.3f}, min {min(each) * 1e3:.3f} ms)")
        runs[name] = {"ms": round(ms, 4), "kernel_ms": round(ker * 1e3, 4),
                      "kernel_ms_median": round(median(each) * 1e3, 4), "kernel_ms_min": round(min(each) * 1e3, 4),
                      "tokens_per_s": round(w.B * w.T / (wall / steps), 1),
                      "tflops": round(flops / (wall / steps) / 1e12, 2),
                      "roofline": roofline(nbytes, ker, stored_traffic("kda_chunk_fwd_ws", RING_SOURCES)
                                           if ring and w.name == "kda_fwd_B1_H8_T4096_d128_bf16" else None)}
    # sequence-parallel forward where the plain grid leaves most CUs idle
    # (the three launches of one call timed together)
    if w.B * w.H * (w.dv // 64) <= 64:
        picked = kda.kda_chunk_fwd_seqpar_segments(w.B, w.T, w.H, w.dk, w.dv)
        for P in sorted({4, 8, 16, picked} - {1}):
            if w.T % P:
                continue
            wsp = torch.empty(kda.kda_chunk_fwd_seqpar_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, P),
                              dtype=torch.uint8, device="cuda")

            def step():
                kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o=o, S_final=Sf,
                                         segments=P, workspace=wsp)

            wall, ker, each = time_launches(step, steps, warmup, stream, per_launch=True)
            ms = wall / steps * 1e3
            log(f"[bench] {w.name} sequence-parallel P={P}: {ms:.3f} ms/step (kernels mean {ker * 1e3:.3f}, "
                f"min {min(each) * 1e3:.3f} ms)")
            runs[f"sequence_parallel_P{P}"] = {
                "ms": round(ms, 4), "kernel_ms": round(ker * 1e3, 4),
                "kernel_ms_median": round(median(each) * 1e3, 4), "kernel_ms_min": round(min(each) * 1e3, 4),
                "tokens_per_s": round(w.B * w.T / (wall / steps), 1),
                "tflops": round(flops / (wall / steps) / 1e12, 2),
                "workspace_bytes": int(wsp.numel()),
                "roofline": roofline(nbytes, ker, None)}
            del wsp
    best = min(runs, key=lambda k: runs[k]["ms"])
    out = {"workload": w.name, "faster_kernel": best, **runs[best], "algorithmic_bytes": nbytes,
           "kernels": runs,
           "library_segment_choice": kda.kda_chunk_fwd_seqpar_segments(w.B, w.T, w.H, w.dk, w.dv)}
    del d, o, Sf, ws
    torch.cuda.empty_cache()
    return out


def bench_gate_prologue(kda, steps=10, decode_reps=1):
    """The gate prologue: the log-decay formed inside the kernels from gate
    logits z and per-head scales A_log, g = -5 sigmoid(exp(A_log) z).  The
    chunked forward on the training shape (bf16 z; it reads z where the plain
    forward reads g) and the decode step on the decode workload."""
    import torch
    from kda_workloads import configs, gen_torch
    w = configs.TRAIN_BF16
    d = gen_torch.fwd_inputs(w)
    z = d["g"].float().mul_(-1.0).to(d["g"].dtype)   # logits of the same shape and dtype as g
    del d["g"]
    A_log = torch.linspace(-1.0, 1.0, w.H, device="cuda")
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fwd():
        kda.kda_chunk_fwd_gate(d["q"], d["k"], d["v"], z, A_log, d["beta"], None, o=o, S_final=Sf, ring=False)

    wall, ker, each = time_launches(fwd, steps, 2, stream, per_launch=True)
    nbytes = fwd_bytes(w.B, w.T, w.H, w.dk, w.dv, 2, 2, 4, s0=False, sfinal=True) + 4 * w.H
    ms = wall / steps * 1e3
    log(f"[bench] chunk_fwd_gate {ms:.3f} ms/step (kernel mean {ker * 1e3:.3f} ms)")
    out = {"chunk_fwd_gate": {"workload": w.name + "_gate_logits", "ms": round(ms, 4), "kernel_ms": round(ker * 1e3, 4),
                              "kernel_ms_min": round(min(each) * 1e3, 4),
                              "tokens_per_s": round(w.B * w.T / (wall / steps), 1),
                              "algorithmic_bytes": nbytes, "roofline": roofline(nbytes, ker, None)}}
    del d, z, o, Sf
    torch.cuda.empty_cache()

    dw = configs.DECODE_BF16
    S = gen_torch.decode_initial_state(dw)
    xs = [gen_torch.decode_step_inputs(dw, s) for s in range(dw.steps)]
    zs = [x["g"].float().mul(-1.0).to(x["g"].dtype) for x in xs]
    A_d = torch.linspace(-1.0, 1.0, dw.H, device="cuda")
    od = torch.empty((dw.B, dw.H, dw.dv), dtype=torch.float32, device="cuda")
    it = {"i": 0}

    def one():
        i = it["i"] % dw.steps
        it["i"] += 1
        x = xs[i]
        kda.kda_decode_step_gate(x["q"], x["k"], x["v"], zs[i], A_d, x["beta"], S, o=od)

    n = dw.steps * decode_reps
    wall, ker = time_launches(one, n, dw.steps // 4, stream)
    per_step = decode_bytes(dw.B, dw.H, dw.dk, dw.dv, 2, 4, 4) + 4 * dw.H
    gbs = per_step * n / wall / 1e9
    log(f"[bench] decode_step_gate {wall / n * 1e3:.3f} ms/step (kernel {ker * 1e3:.3f} ms), {gbs:.1f} GB/s")
    out["decode_step_gate"] = {"workload": dw.name + "_gate_logits", "ms_per_step": round(wall / n * 1e3, 4),
                               "GB/s": round(gbs, 1), "algorithmic_bytes_per_step": per_step,
                               "roofline": roofline(per_step, ker, None)}
    return out


def bench_decode(kda, reps):
    import torch
    from kda_workloads import configs, gen_torch
    w = configs.DECODE_BF16
    log(f"[bench] generating {w.name} on the device")
    S = gen_torch.decode_initial_state(w)
    xs = [gen_torch.decode_step_inputs(w, s) for s in range(w.steps)]
    o = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    it = {"i": 0}

    def one():
        x = xs[it["i"] % w.steps]
        it["i"] += 1
        kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], S, o=o)

    log(f"[bench] decode: {w.steps} steps x {reps} repetitions")
    wall, ker = time_launches(one, w.steps * reps, w.steps, stream)
    per_step = decode_bytes(w.B, w.H, w.dk, w.dv, 2, 4, 4)
    n = w.steps * reps
    gbs = per_step * n / wall / 1e9
    log(f"[bench] decode {wall / n * 1e3:.3f} ms/step (kernel {ker * 1e3:.3f} ms), {gbs:.1f} GB/s")
    return {
        "workload": w.name, "value": round(gbs, 1), "unit": "GB/s",
        "ms_per_step": round(wall / n * 1e3, 4), "steps": n,
        "algorithmic_bytes_per_step": per_step,
        "roofline": roofline(per_step, ker, stored_traffic("kda_decode_step", DECODE_SOURCES)),
    }


def spec_bytes(B, H, K, n, dk, dv, s_qkv, s_g, s_o):
    """Algorithmic bytes of one speculative verify of K draft tokens per state
    (reads the state once, the drafts' q, k, v, g, beta, writes K outputs)
    and one commit of n accepted tokens per state (reads and writes the state
    once, reads the accepted tokens' k, v, g, beta and the counts)."""
    state = B * H * dk * dv * 4
    verify = state + B * K * H * ((2 * dk + dv) * s_qkv + (dk + 1) * s_g + dv * s_o)
    commit = 2 * state + B * n * H * ((dk + dv) * s_qkv + (dk + 1) * s_g) + 4 * B
    return verify, commit


def bench_speculative(kda, reps, K=16):
    """Verify + commit of K draft tokens on the decode workload's states."""
    import torch
    from kda_workloads import configs, gen_torch
    w = configs.DECODE_BF16
    fw = configs.Workload(name="spec_drafts", kind="fwd", B=w.B, H=w.H, dk=w.dk, dv=w.dv, T=K,
                          qkv=w.qkv, gate=w.gate, s0_sd=None)
    log(f"[bench] speculative: {w.B}x{w.H} states, {K} draft tokens")
    S = gen_torch.decode_initial_state(w)
    x = gen_torch.fwd_inputs(fw)
    o = torch.empty((w.B, K, w.H, w.dv), dtype=torch.float32, device="cuda")
    n = K // 2
    acc = torch.full((w.B,), n, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    verify_b, commit_b = spec_bytes(w.B, w.H, K, n, w.dk, w.dv, 2, 4, 4)
    out = {"workload": f"kda_spec_B{w.B}_H{w.H}_d{w.dk}_bf16_K{K}", "draft_tokens": K, "accepted": n}
    calls = (("verify", lambda: kda.kda_verify_step(x["q"], x["k"], x["v"], x["g"], x["beta"], S, o=o), verify_b),
             ("commit", lambda: kda.kda_commit_step(x["k"], x["v"], x["g"], x["beta"], acc, S), commit_b))
    for name, fn, nbytes in calls:
        wall, ker = time_launches(fn, reps, 2, stream)
        gbs = nbytes * reps / wall / 1e9
        log(f"[bench] {name} {wall / reps * 1e3:.3f} ms (kernel {ker * 1e3:.3f} ms), {gbs:.1f} GB/s")
        out[name] = {"ms": round(wall / reps * 1e3, 4), "GB/s": round(gbs, 1), "algorithmic_bytes": nbytes,
                     "roofline": roofline(nbytes, ker, stored_traffic(f"kda_{name}_step", VERIFY_SOURCES))}
    return out


def bench_epilogue(kda, reps=10, fused=True):
    """The output epilogue over the training-shape reads (float32 o, bf16
    logits, float32 y), and (`fused`) the decode step with the epilogue fused."""
    import torch
    from kda_workloads import configs, gen_torch
    w = configs.TRAIN_BF16
    shape = (w.B, w.T, w.H, w.dv)
    rows = w.B * w.T * w.H
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    o = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    z = gen_torch.output_gate_logits(shape, "bf16")
    wt = gen_torch.output_norm_weight(w.dv)
    y = torch.empty_like(o)
    stream = torch.cuda.current_stream()
    wall, ker = time_launches(lambda: kda.kda_output_gate(o, z, wt, 1e-6, y=y), reps, 2, stream)
    nbytes = epilogue_bytes(rows, w.dv, 4, 2, 4)
    gbs = nbytes * reps / wall / 1e9
    log(f"[bench] output_gate {wall / reps * 1e3:.3f} ms (kernel {ker * 1e3:.3f} ms), {gbs:.1f} GB/s")
    out = {"output_gate": {"workload": f"kda_output_gate_B{w.B}_T{w.T}_H{w.H}_dv{w.dv}_f32o_bf16z",
                           "ms": round(wall / reps * 1e3, 4), "GB/s": round(gbs, 1),
                           "algorithmic_bytes": nbytes,
                           "roofline": roofline(nbytes, ker, stored_traffic("kda_output_gate", EPILOGUE_SOURCES))}}
    del o, z, y
    if not fused:
        return out

    dw = configs.DECODE_BF16
    S = gen_torch.decode_initial_state(dw)
    xs = [gen_torch.decode_step_inputs(dw, s) for s in range(dw.steps)]
    zs = [gen_torch.output_gate_logits((dw.B, dw.H, dw.dv), dw.qkv, seed=s) for s in range(dw.steps)]
    wd = gen_torch.output_norm_weight(dw.dv)
    yd = torch.empty((dw.B, dw.H, dw.dv), dtype=torch.float32, device="cuda")
    it = {"i": 0}

    def one():
        i = it["i"] % dw.steps
        it["i"] += 1
        x = xs[i]
        kda.kda_decode_step_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], S, zs[i], wd, 1e-6, y=yd)

    wall, ker = time_launches(one, dw.steps, dw.steps // 4, stream)
    per_step = gated_decode_bytes(dw.B, dw.H, dw.dk, dw.dv, 2, 4, 4)
    gbs = per_step * dw.steps / wall / 1e9
    log(f"[bench] decode+epilogue {wall / dw.steps * 1e3:.3f} ms/step (kernel {ker * 1e3:.3f} ms), {gbs:.1f} GB/s")
    out["decode_gated"] = {"workload": dw.name + "_gated", "ms_per_step": round(wall / dw.steps * 1e3, 4),
                           "GB/s": round(gbs, 1), "algorithmic_bytes_per_step": per_step,
                           "roofline": roofline(per_step, ker, None)}
    return out


def bench_backward(kda, reps=3):
    """kda_chunk_bwd on the training shape (bf16 q, k, v, g, beta; float32
    upstream gradient dO; zero initial state, no final-state gradient)."""
    import torch
    from kda_workloads import configs, gen_torch
    w = configs.TRAIN_BF16
    d = gen_torch.fwd_inputs(w)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    dO = torch.randn((w.B, w.T, w.H, w.dv), generator=gen, device="cuda", dtype=torch.float32)
    ws = torch.empty(kda.kda_chunk_bwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device="cuda")
    log(f"[bench] backward workspace {ws.numel() / 1e9:.2f} GB")
    stream = torch.cuda.current_stream()
    fn = lambda: kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, dO, None,  # noqa: E731
                                   want_dS0=False, workspace=ws)
    if reps == 0:   # the counter pass: one call, nothing timed
        fn()
        torch.cuda.synchronize()
        return None
    wall, ker = time_launches(fn, reps, 1, stream)
    flops = bwd_flops(w.B, w.T, w.H, w.dk, w.dv)   # at the kernels' 32-token chunks
    nbytes = bwd_bytes(w.B, w.T, w.H, w.dk, w.dv, 2, 2, 4)
    tfs = flops / ker / 1e12
    log(f"[bench] backward {wall / reps * 1e3:.3f} ms (kernels {ker * 1e3:.3f} ms), {tfs:.1f} TFLOP/s, "
        f"{w.B * w.T / (wall / reps):.3e} tokens/s")
    rec = stored_traffic("kda_chunk_bwd", BWD_SOURCES)
    return {"workload": w.name + "_bwd", "ms": round(wall / reps * 1e3, 4),
            "tokens_per_s": round(w.B * w.T / (wall / reps), 1),
            "algorithmic_flop": flops, "algorithmic_bytes": nbytes,
            "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tfs / FP32_MFMA_PEAK_TFLOPS, 4),
                         "traffic": rec["hbm_bytes_per_launch"] if rec else None}}


def cpu_baseline(w, d, batch=32):
    """The float64 oracle on the same workload, every head over the full
    sequence, on all host threads, `batch` heads per call (only the recurrence
    is timed, not the copies to float64)."""
    import numpy as np
    import torch
    from oracle import default
    orc = default()
    threads = orc.max_threads()
    n_all = w.B * w.H
    log(f"[bench] cpu baseline: oracle on {n_all} heads x {w.T} tokens, {threads} threads")

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    dt = 0.0
    for i0 in range(0, n_all, batch):
        heads = [(i // w.H, i % w.H) for i in range(i0, min(n_all, i0 + batch))]
        x = {nm: f64(torch.stack([d[nm][b, :, h] for b, h in heads], dim=1).unsqueeze(0))
             for nm in ("q", "k", "v", "g", "beta")}
        t0 = time.perf_counter()
        orc.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, nthreads=threads)
        dt += time.perf_counter() - t0
        del x
    tok_s = w.B * w.T / dt
    log(f"[bench] cpu baseline: {dt:.2f} s -> {tok_s:.3e} tokens/s")
    # the per-core rate: one head over the whole sequence on one thread
    x1 = {nm: f64(d[nm][0:1, :, 0:1]) for nm in ("q", "k", "v", "g", "beta")}
    t0 = time.perf_counter()
    orc.fwd(x1["q"], x1["k"], x1["v"], x1["g"], x1["beta"], None, nthreads=1)
    dt1 = time.perf_counter() - t0
    flop_head_tok = 7 * w.dk * w.dv   # fade, the two state-vector products and the rank-one update
    log(f"[bench] cpu baseline, one thread: {w.T} tokens of one head in {dt1:.2f} s")
    try:
        affinity = sorted(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(tok_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host": {"nproc": os.cpu_count(), "affinity_cpus": len(affinity) if affinity is not None else None,
                     "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
                     "oracle_threads": threads},
            "sample": f"all {n_all} heads x {w.T} tokens of {w.name} (the full step), float64 "
                      f"token recurrence, {batch} heads per call, {dt:.2f} s wall",
            "gflops_f64": round(w.B * w.T * w.H * flop_head_tok / dt / 1e9, 2),
            "one_thread": {"token_heads_per_s": round(w.T / dt1, 1),
                           "gflops_f64": round(w.T * flop_head_tok / dt1 / 1e9, 3),
                           "sample": f"one head x {w.T} tokens, {dt1:.2f} s"}}


# ------------------------------------------------------------ counter passes

COPY_BYTES = 1 << 30   # the calibration copy moves 1 GiB each way


def profile_pass(kda, reps=3):
    """A short run for `rocprofv3 --pmc`: a plain device copy of known size
    (calibrates the byte counters), then the chunked forward and the decode
    step of the benchmark workloads, `reps` launches each, the ring forward
    on the head-group workload (`reps` launches), verify and commit
    of the speculative workload and the output epilogue (three launches
    each), and one backward call (its five kernels) on the training shape."""
    import torch
    from kda_workloads import configs, gen_torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w, d, *_ = bench_fwd(kda, reps, 1)
    del d
    torch.cuda.empty_cache()
    # the ring kernel on the workload where it is the faster one (one head group)
    hw = configs.HEADGROUP_BF16
    hd = gen_torch.fwd_inputs(hw)
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(hw.B, hw.T, hw.H, hw.dk, hw.dv), dtype=torch.uint8,
                     device="cuda")
    for _ in range(reps):
        kda.kda_chunk_fwd(hd["q"], hd["k"], hd["v"], hd["g"], hd["beta"], hd["S0"], workspace=ws)
    torch.cuda.synchronize()
    del hd, ws
    bench_decode(kda, 1)
    bench_speculative(kda, 1)
    bench_epilogue(kda, reps=1, fused=False)   # the fused decode would mix into the decode record
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    bench_backward(kda, reps=0)


def profile_pass_seqpar(kda, P=8, reps=3):
    """The one-head-group forward (B1 H8 T4096) through kda_chunk_fwd_seqpar
    in P segments: one warm-up call, then `reps` calls (each three launches:
    transition and value slabs, combine, re-run)."""
    import torch
    from kda_workloads import configs, gen_torch
    w = configs.HEADGROUP_BF16
    d = gen_torch.fwd_inputs(w)
    ws = torch.empty(kda.kda_chunk_fwd_seqpar_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, P), dtype=torch.uint8,
                     device="cuda")
    for _ in range(1 + reps):
        kda.kda_chunk_fwd_seqpar(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], segments=P, workspace=ws)
    torch.cuda.synchronize()
    log(f"[profile-pass-seqpar] {w.name}, {P} segments, {1 + reps} calls done")


def _counter_rows(directory, counter):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append(r)
    return rows


def _per_dispatch(rows, *name_parts):
    acc = {}
    for r in rows:
        if all(p in r["Kernel_Name"] for p in name_parts):
            acc[r["Dispatch_Id"]] = acc.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(acc.values())


def counters_to_traffic(fetch_dir, write_dir, out=TRAFFIC_FILE):
    """Turn FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of a profile pass into
    HBM bytes per launch of each KDA kernel, scaled by what the same counters
    read for the 1 GiB calibration copy, and store them with the kernels'
    source hashes."""
    fr, wr = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    copy_f = _per_dispatch(fr, "copyBuffer")   # the runtime's device-to-device copy kernel
    copy_w = _per_dispatch(wr, "copyBuffer")
    if not copy_f or not copy_w:
        raise SystemExit("no calibration copy dispatch found in the counter files")
    cf = COPY_BYTES / (max(copy_f) * 1024.0)
    cw = COPY_BYTES / (max(copy_w) * 1024.0)
    rec = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_KiB": max(copy_f), "write_KiB": max(copy_w),
                           "fetch_scale": round(cf, 4), "write_scale": round(cw, 4)}}
    for kernel, parts, sources in SINGLE_KERNELS:
        f, w_ = _per_dispatch(fr, *parts), _per_dispatch(wr, *parts)
        if not f or not w_:
            continue
        fb = sum(f) / len(f) * 1024.0 * cf
        wb = sum(w_) / len(w_) * 1024.0 * cw
        rec[kernel] = {"source_hash": kernel_source_hash(sources), "fetch_bytes_per_launch": round(fb),
                       "write_bytes_per_launch": round(wb), "hbm_bytes_per_launch": round(fb + wb),
                       "dispatches": len(f)}
    # the backward: bytes of one call, the sum over its five kernels
    parts = {}
    for part in BWD_KERNELS:
        f, w_ = _per_dispatch(fr, part), _per_dispatch(wr, part)
        if f and w_:
            parts[part] = (sum(f) / len(f) * 1024.0 * cf, sum(w_) / len(w_) * 1024.0 * cw)
    if len(parts) == len(BWD_KERNELS):
        fb = sum(x[0] for x in parts.values())
        wb = sum(x[1] for x in parts.values())
        rec["kda_chunk_bwd"] = {"source_hash": kernel_source_hash(BWD_SOURCES),
                                "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                                "hbm_bytes_per_launch": round(fb + wb),
                                "per_kernel": {k: {"fetch_bytes": round(a), "write_bytes": round(b)}
                                               for k, (a, b) in parts.items()}}
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-reps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for rocprofv3 --pmc: calibration copy, then each kernel a few times")
    ap.add_argument("--profile-pass-fwd", action="store_true",
                    help="short run for rocprofv3 --pmc: the headline forward only, three launches")
    ap.add_argument("--profile-pass-seqpar", action="store_true",
                    help="short run for rocprofv3: the one-head-group forward, sequence-parallel in 8 segments, "
                         "three calls after one warm-up")
    ap.add_argument("--only-backward", action="store_true",
                    help="run only the backward leg (two calls) and print its JSON object")
    ap.add_argument("--counters-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs of --profile-pass")
    args = ap.parse_args()
    if args.counters_from:
        counters_to_traffic(*args.counters_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): every workload here "
              "runs on a single GPU (heads would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_101_amd as kda
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kda.load_library()
    if args.profile_pass:
        profile_pass(kda)
        return
    if args.profile_pass_fwd:
        bench_fwd(kda, 3, 1)
        return
    if args.profile_pass_seqpar:
        profile_pass_seqpar(kda)
        return
    if args.only_backward:
        print(json.dumps(bench_backward(kda, reps=2)), flush=True)
        return

    peaks = bench_peaks()
    w, d, ms, tok_s, rf, extra = bench_fwd(kda, args.steps, args.warmup)
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "chunk": CHUNK, "tile": 16, "qkv": w.qkv, "gate": w.gate, "out": "f32",
                   "state": "f32"},
        **extra,
        "roofline": rf,
        "peaks": peaks,
    }
    if not args.no_decode:
        from kda_workloads import configs
        out["forward_secondary"] = [bench_fwd_secondary(kda, configs.HEADGROUP_BF16, 20, 3),
                                    bench_fwd_secondary(kda, configs.LONG_BF16, 3, 1),
                                    bench_fwd_secondary(kda, configs.LONG_SHARE_BF16, 5, 1)]
        out["decode"] = bench_decode(kda, args.decode_reps)
        out["speculative"] = bench_speculative(kda, 10)
        out["epilogue"] = bench_epilogue(kda)
        out["backward"] = bench_backward(kda)
        out["gate_prologue"] = bench_gate_prologue(kda)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
