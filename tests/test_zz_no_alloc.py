"""kda_chunk_fwd_noalloc: the workspace forward with the library's own fixed
scratch as its ring.  Called through the C ABI (ctypes), compared bit for bit
with kda_chunk_fwd_ws on a caller workspace (the same kernel and arithmetic),
on consecutive calls whose second input is smaller than the first, so a stale
ring left by the first call is present during the second."""
import pytest
import torch

from gpu_support import say, to_dev
from kda_workloads import configs, gen

pytestmark = pytest.mark.gpu

T = configs.TRAIN_BF16


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_101_amd as m
    m.load_library()
    return m


def _inputs(w, seed):
    x = gen.fwd_inputs(w, seed)
    return {n: to_dev(x[n]) for n in x}


def _noalloc(kda, d, w):
    o = torch.full((w.B, w.T, w.H, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    S = torch.full((w.B, w.H, w.dk, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S)
    return o, S


def _with_workspace(kda, d, w):
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device="cuda")
    return kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], ring=True, workspace=ws)


# (first call, second smaller call): ring at 64 heads (the scratch's limit)
# then 3 heads at dv = 256; a ragged tail in each
PAIRS = [
    (T.scaled(B=4, H=16, T=64 * 6 + 17, name="noalloc_BH64_T401"),
     T.scaled(B=1, H=3, T=64 * 2 + 5, dv=256, name="noalloc_BH3_dv256_T133")),
    (T.scaled(B=2, H=8, T=64 * 5, dv=512, name="noalloc_BH16_dv512_T320"),
     T.scaled(B=1, H=2, T=70, name="noalloc_BH2_T70")),
]


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"{a.name}-then-{b.name}" for a, b in PAIRS])
def test_noalloc_equals_workspace_entry_point(kda, first, second):
    for i, w in enumerate((first, second)):
        say(f"[noalloc] call {i + 1}: {w.name} B={w.B} H={w.H} T={w.T} dv={w.dv}")
        d = _inputs(w, seed=10 + i)
        o1, S1 = _noalloc(kda, d, w)
        o2, S2 = _with_workspace(kda, d, w)
        torch.cuda.synchronize()
        assert torch.isfinite(o1).all() and torch.isfinite(S1).all()
        assert torch.equal(o1, o2) and torch.equal(S1, S2), w.name


def test_noalloc_without_ring_and_beyond_scratch(kda):
    # dv = 64 takes no ring: the kernels of kda_chunk_fwd, no scratch
    w = T.scaled(B=1, H=2, T=200, dv=64)
    d = _inputs(w, seed=3)
    say("[noalloc] dv = 64 (no ring)")
    o1, S1 = _noalloc(kda, d, w)
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], ring=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # 65 heads with the ring: more than the scratch holds; refused, nothing written
    w = T.scaled(B=5, H=13, T=64)
    d = _inputs(w, seed=4)
    say("[noalloc] 65 heads: beyond the scratch")
    o = torch.zeros((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    with pytest.raises(kda.KdaError) as err:
        kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, None)
    assert err.value.status == kda.KDA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert not o.any()
