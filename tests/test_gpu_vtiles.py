"""The V-tiled verify (KDA_SCHEDULE_V_TILES: several workgroups per request
and head, each on a block of state rows) against the one-workgroup-per-item
verify, bit for bit, and against the fp64 oracle on the single-request
workload; its per-item arrival counters are left at zero by every launch,
also under HIP-graph replay."""
import numpy as np
import pytest
import torch

import linear_attention_speculative_amd as kda
from linear_attention_speculative_amd import _abi
from tests.gpu_check import bits, check_verify, run_oracle_verify, snapshot
from tests.test_gpu_parity import _commit_case
from workloads import drive, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"
PER_ITEM, V_TILES = _abi.KDA_SCHEDULE_PER_ITEM, _abi.KDA_SCHEDULE_V_TILES


def _run(wl, page0, qkv, **kw):
    """Restore the pages, run one verify, return (out, pages, counter)."""
    L = wl.layers[0]
    L.page.copy_(page0)
    L.out.fill_(float("nan"))
    c = drive.counter(wl)
    if qkv:
        drive.verify_qkv(wl, 0, c, **kw)
    else:
        drive.verify(wl, 0, c, **kw)
    torch.cuda.synchronize()
    return bits(L.out), L.page.clone(), c


# name: (make_workload arguments, unfused verify)
CASES = {
    "d128_q4_bf16_dimfirst": (dict(B=6, H=5, D=128, Q=4, N=16,
                                   conv_dim_first=True), False),
    "d128_q8_f32_tokfirst_nulls": (dict(B=9, H=3, D=128, Q=8, N=24,
                                        act="f32", weight="f32",
                                        conv_dim_first=False,
                                        null_frac=0.3, gates=[None]), False),
    "d64_q4_ragged_kgact": (dict(B=11, H=4, D=64, Q=4, N=24,
                                 kg_dtype="act", out_dtype="act",
                                 null_frac=0.2), False),
    "d64_q7_f32_tokfirst": (dict(B=5, H=2, D=64, Q=7, N=12, act="f32",
                                 weight="f32", conv_dim_first=False), False),
    "d128_q3_unfused": (dict(B=7, H=3, D=128, Q=3, N=16), True),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_vtiles_bitwise_equal_per_item(case):
    sizes, qkv = CASES[case]
    wl = make_workload("ragged", DEV, **sizes)
    page0 = wl.layers[0].page.clone()
    ref_out, ref_page, _ = _run(wl, page0, qkv, schedule=PER_ITEM)
    assert not torch.isnan(wl.layers[0].out).any()
    for vt in (2, 4, 8):
        out, page, c = _run(wl, page0, qkv, schedule=V_TILES, v_tiles=vt)
        assert np.array_equal(out, ref_out), (case, vt)
        assert torch.equal(page, ref_page), (case, vt)
        assert int(c.abs().sum()) == 0, "arrival counters left non-zero"


def test_single_request_vtiles_matches_oracle():
    """The single-request workload (B=1, 32 heads, head dim 128, token-first
    conv) under each V-tile count (0: the library's count, 8 here) and the
    default schedule: outputs, records, conv roll and the commit against
    the oracle."""
    for vt in (0, 2, 4, 8):
        wl = make_workload("single", DEV)
        L = wl.layers[0]
        sample = snapshot(wl, 0)
        state0 = L.state.clone()
        c = drive.counter(wl)
        drive.verify(wl, 0, c, schedule=V_TILES, v_tiles=vt)
        torch.cuda.synchronize()
        assert int(c.abs().sum()) == 0
        assert torch.equal(L.state, state0), "verify wrote the checkpoint"
        ref = run_oracle_verify(sample)
        errs = check_verify(wl, 0, sample, ref)
        cerr = _commit_case(wl, {0: (sample, ref)})
        print("single vtiles", vt, errs, cerr)


def test_vtiles_graph_replay_and_counter_reuse():
    """One counter array reused by consecutive launches and by three replays
    of a captured graph: every launch leaves it at zero and gives the eager
    bytes."""
    wl = make_workload("ragged", DEV, B=4, H=8, D=128, Q=4, N=12)
    L = wl.layers[0]
    page0 = L.page.clone()
    c = drive.counter(wl)
    drive.verify(wl, 0, c, schedule=V_TILES, v_tiles=8)
    torch.cuda.synchronize()
    eager_out, eager_page = bits(L.out), L.page.clone()
    for _ in range(2):                       # the counter is reused as is
        L.page.copy_(page0)
        drive.verify(wl, 0, c, schedule=V_TILES, v_tiles=8)
        torch.cuda.synchronize()
        assert int(c.abs().sum()) == 0
        assert torch.equal(L.page, eager_page)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    L.page.copy_(page0)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            drive.verify(wl, 0, c, schedule=V_TILES, v_tiles=8)
    torch.cuda.synchronize()
    for _ in range(3):
        L.page.copy_(page0)
        L.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(c.abs().sum()) == 0
        assert np.array_equal(bits(L.out), eager_out)
        assert torch.equal(L.page, eager_page)


def test_vtiles_need_counter_room():
    """The default schedule runs whole items with a one-element counter and
    gives the same bytes as with a full counter array; the V-tile schedule
    refuses a counter without one arrival slot per item."""
    wl = make_workload("single", DEV)
    L = wl.layers[0]
    page0 = L.page.clone()
    one = torch.zeros(1, dtype=torch.int32, device=DEV)
    drive.verify(wl, 0, one)
    torch.cuda.synchronize()
    a_out, a_page = bits(L.out), L.page.clone()
    L.page.copy_(page0)
    drive.verify(wl, 0, drive.counter(wl))
    torch.cuda.synchronize()
    assert np.array_equal(bits(L.out), a_out)
    assert torch.equal(L.page, a_page)
    assert int(one.item()) == 0
    with pytest.raises(kda.KdaError):
        drive.verify(wl, 0, one, schedule=V_TILES, v_tiles=4)
