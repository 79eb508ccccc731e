"""The benchmark's algorithmic byte and FLOP counts, checked by hand counts.

The roofline fractions the benchmark reports divide these counts by measured
kernel times, so a wrong count would misstate every fraction.
"""

import bench


def test_forward_counts_at_training_shape():
    # B4 H32 T16384 d128, bf16 q/k/v/g/beta, fp32 outputs, final state written:
    # per token-head 2*(128+128+128) + 2*129 + 4*128 bytes, plus one fp32 state per head
    per_tok = 2 * 384 + 2 * 129 + 4 * 128
    tok_heads = 4 * 16384 * 32
    state = 4 * 32 * 128 * 128 * 4
    assert bench.fwd_bytes(4, 16384, 32, 128, 128, 2, 2, 4, False, True) == tok_heads * per_tok + state
    assert bench.fwd_bytes(4, 16384, 32, 128, 128, 2, 2, 4, True, True) == tok_heads * per_tok + 2 * state
    # 6 d^2 + 2 C (2 d) + C^2/3 at C = 64, d = 128
    assert bench.fwd_flops(1, 1, 1, 128, 128) == 6 * 16384 + 128 * 256 + 4096 // 3 == 132437


def test_decode_counts():
    # B256 H96 d128: fp32 state read and written, bf16 q, k, v, fp32 g, beta, fp32 o
    per_state = 2 * 128 * 128 * 4 + 2 * 384 + 4 * 129 + 4 * 128
    assert bench.decode_bytes(256, 96, 128, 128, 2, 4, 4) == 256 * 96 * per_state


def test_speculative_counts():
    B, H, K, n, d = 2, 3, 16, 5, 64
    state = B * H * d * d * 4
    # verify: the state once, K drafts of q, k, v (bf16), g, beta (fp32), K fp32 outputs
    verify = state + B * H * K * (2 * 3 * d + 4 * (d + 1) + 4 * d)
    # commit: the state read and written, n accepted drafts of k, v, g, beta, B int32 counts
    commit = 2 * state + B * H * n * (2 * 2 * d + 4 * (d + 1)) + 4 * B
    assert bench.spec_bytes(B, H, K, n, d, d, 2, 4, 4) == (verify, commit)


def test_epilogue_counts():
    # rows of dv = 128: fp32 read, bf16 logit, fp32 result per channel, plus the weight
    assert bench.epilogue_bytes(10, 128, 4, 2, 4) == 10 * 128 * 10 + 4 * 128
    # fused decode: the decode step plus bf16 output-gate logits and the weight
    assert bench.gated_decode_bytes(256, 96, 128, 128, 2, 4, 4) == \
        bench.decode_bytes(256, 96, 128, 128, 2, 4, 4) + 256 * 96 * 128 * 2 + 4 * 128


def test_executed_forward_flops():
    # one chunk of one head, dk = dv = 128 (two 64-column slabs, eight 16-column state waves).
    # per state wave: (Gamma.Q) S and (Gamma.K) S, 4 row tiles x 4 k-blocks x 2; the state
    # update, 8 row tiles x 2 token halves x 2 terms (16x16x32); the solve, 6 strict tiles
    # + 4 inverses x 2 terms, and the outputs, 10 lower tiles x 2 terms (16x16x16)
    m32, m16 = 2 * 16 * 16 * 32, 2 * 16 * 16 * 16
    state = 8 * ((32 + 32) * m32 + (6 + 8 + 20) * m16)
    # per slab: cumsum 4 tiles x 8 channel tiles (16x16x16), diagonal Gram 4 tiles x 4
    # k-blocks x 4 products, off-diagonal 6 tiles x 4 k-blocks x 2 (16x16x32)
    prep = 2 * ((4 * 4 * 4 + 6 * 4 * 2) * m32 + 4 * 8 * m16)
    assert bench.fwd_executed_flops(1, 64, 1, 128, 128) == state + prep == 14811136
    # a ragged last chunk still runs whole tiles
    assert bench.fwd_executed_flops(1, 65, 1, 128, 128) == 2 * 14811136


def test_backward_counts():
    # per token-head at the kernels' C = 32, d = 128: 16 d^2 + 9 C d + 5 C d + C^2
    assert bench.bwd_flops(1, 1, 1, 128, 128) == 16 * 16384 + 14 * 32 * 128 + 1024 == 320512
    # bf16 q, k, v, g, beta and fp32 dO read; fp32 dq, dk, dg (d each), dv (d), dbeta written
    per = 2 * 384 + 2 * 129 + 4 * 128 + 4 * (3 * 128 + 128 + 1)
    assert bench.bwd_bytes(4, 16384, 32, 128, 128, 2, 2, 4) == 4 * 16384 * 32 * per


def _write_counters(path, counter, rows):
    """A rocprofv3 counter_collection.csv with the columns the benchmark reads."""
    import csv
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "p_counter_collection.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for disp, name, kib in rows:
            # counters are reported per shader engine: split each value in two rows
            wr.writerow([disp, name, counter, kib / 2])
            wr.writerow([disp, name, counter, kib / 2])


def test_counters_to_traffic(tmp_path):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch, summed over rows) become
    bytes per launch, scaled by what the calibration copy of 1 GiB reads, and
    the backward's five kernels add up to one call."""
    import json
    copy = "void copyBuffer(...)"
    fwd = "kda_chunk_pipe_kernel<128, true, false, false>"
    fetch = [(1, copy, 524288.0), (2, fwd, 1000.0), (3, fwd, 3000.0)]
    write = [(1, copy, 1048576.0), (2, fwd, 500.0), (3, fwd, 500.0)]
    ver = "void kda::kda_verify_tile_kernel<128, 128, unsigned short, unsigned short, float, false>(float*)"
    com = "void kda::kda_verify_tile_kernel<128, 128, unsigned short, unsigned short, float, true>(float*)"
    fetch += [(4, ver, 100.0), (5, com, 300.0), (6, "kda_output_gate_kernel<float>", 50.0)]
    write += [(4, ver, 10.0), (5, com, 30.0), (6, "kda_output_gate_kernel<float>", 5.0)]
    for i, part in enumerate(bench.BWD_KERNELS):
        fetch.append((10 + i, part + "<128, 128>", 100.0 * (i + 1)))
        write.append((10 + i, part + "<128, 128>", 10.0 * (i + 1)))
    _write_counters(tmp_path / "f", "FETCH_SIZE", fetch)
    _write_counters(tmp_path / "w", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    bench.counters_to_traffic(str(tmp_path / "f"), str(tmp_path / "w"), out=str(out))
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    f = rec["kda_chunk_fwd"]
    assert f["fetch_bytes_per_launch"] == 2 * 2000 * 1024 and f["write_bytes_per_launch"] == 500 * 1024
    assert f["dispatches"] == 2 and f["source_hash"] == bench.kernel_source_hash(bench.CHUNK_SOURCES)
    assert "kda_decode_step" not in rec   # no decode dispatch in these files
    # the two instantiations of the tile kernel are told apart by their last template argument
    assert rec["kda_verify_step"]["hbm_bytes_per_launch"] == (2 * 100 + 10) * 1024
    assert rec["kda_commit_step"]["hbm_bytes_per_launch"] == (2 * 300 + 30) * 1024
    assert rec["kda_verify_step"]["source_hash"] == bench.kernel_source_hash(bench.VERIFY_SOURCES)
    assert rec["kda_output_gate"]["hbm_bytes_per_launch"] == (2 * 50 + 5) * 1024
    b = rec["kda_chunk_bwd"]
    assert b["fetch_bytes_per_launch"] == 2 * 1500 * 1024 and b["write_bytes_per_launch"] == 150 * 1024
    assert b["hbm_bytes_per_launch"] == (3000 + 150) * 1024
    assert b["source_hash"] == bench.kernel_source_hash(bench.BWD_SOURCES)
    # a stored record counts only while the source hash matches
    orig = bench.TRAFFIC_FILE
    try:
        bench.TRAFFIC_FILE = str(out)
        assert bench.stored_traffic("kda_chunk_bwd", bench.BWD_SOURCES)["hbm_bytes_per_launch"] == 3150 * 1024
        assert bench.stored_traffic("kda_chunk_bwd", bench.DECODE_SOURCES) is None
    finally:
        bench.TRAFFIC_FILE = orig
