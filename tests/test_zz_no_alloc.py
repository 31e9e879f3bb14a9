"""The allocation-free verify entry point (kda_conv_update_verify_noalloc,
whose work counters live in the library's per-GPU scratch) against
kda_conv_update_verify with a caller-supplied counter array: the same bytes
under every schedule that uses counters and the default one, for two calls
in a row, the second on a smaller batch; the size limit of the scratch is
enforced before any device call."""
import numpy as np
import pytest
import torch

import linear_attention_speculative_amd as kda
from linear_attention_speculative_amd import _abi
from tests.gpu_check import bits
from workloads import drive, make_workload

DEV = "cuda"
SCHEDULES = [
    dict(schedule=_abi.KDA_SCHEDULE_DEFAULT),
    dict(schedule=_abi.KDA_SCHEDULE_TICKETS, max_workgroups=5),
    dict(schedule=_abi.KDA_SCHEDULE_TICKETS, items_per_ticket=3),
    dict(schedule=_abi.KDA_SCHEDULE_V_TILES, v_tiles=4),
]


def _pair(wl, sched):
    """(out bits, pages) of the existing entry point and of the
    allocation-free one, each from the same starting pages."""
    L = wl.layers[0]
    page0 = L.page.clone()
    res = []
    for noalloc in (False, True):
        L.page.copy_(page0)
        L.out.fill_(float("nan"))
        torch.cuda.synchronize()
        kw = drive.verify_kwargs(wl, 0, None if noalloc else drive.counter(wl),
                                 **sched)
        if noalloc:
            kda.conv_update_verify_noalloc(**kw)
        else:
            kda.conv_update_verify(**kw)
        torch.cuda.synchronize()
        res.append((bits(L.out), L.page.clone()))
    return res


@pytest.mark.gpu
@pytest.mark.parametrize("si", range(len(SCHEDULES)))
def test_noalloc_verify_matches_verify_twice(si):
    sched = SCHEDULES[si]
    big = make_workload("ragged", DEV, B=24, H=6, D=128, Q=4, N=40,
                        null_frac=0.1)
    small = make_workload("ragged", DEV, B=5, H=6, D=128, Q=4, N=12,
                          null_frac=0.0)
    for wl in (big, small):              # the second call: a smaller batch
        (o0, p0), (o1, p1) = _pair(wl, sched)
        assert np.array_equal(o0, o1), sched
        assert torch.equal(p0, p1), sched
        assert not torch.isnan(wl.layers[0].out).any()


def test_noalloc_refuses_batches_beyond_the_scratch():
    # V-tiles of more (request, head) items than the scratch has counters:
    # refused by the host checks (no device call; runs without a GPU).
    # Descriptors are edited directly: nothing of that size is allocated.
    wl = make_workload("ragged", B=4, H=2, D=64, Q=4, N=8)
    kw = drive.verify_kwargs(wl, 0, None, schedule=_abi.KDA_SCHEDULE_V_TILES,
                             v_tiles=2)
    a = kda.verify_args(**kw)
    a.batch = 32769                     # 32769 x 2 heads + 1 > 65537
    lib = _abi.load()
    rc = lib.kda_conv_update_verify_noalloc(a, None)
    assert rc == _abi.KDA_E_CAPACITY, lib.kda_last_error()
    assert b"scratch" in lib.kda_last_error()
