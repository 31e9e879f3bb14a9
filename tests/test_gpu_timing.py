"""Kernel timing through kda_set_launch_events: the armed launches record
the caller's events from their own dispatch, leave every result byte as an
unarmed launch does, and the library reports an arming that outlived its
launches."""
import numpy as np
import pytest
import torch

import linear_attention_speculative_amd as kda
from tests.gpu_check import bits
from workloads import drive, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _events(n):
    out = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in out:
        e.record()                       # creates the event
    torch.cuda.synchronize()
    return out


def test_armed_launches_time_kernels_and_change_nothing():
    wl = make_workload("large", DEV, B=16, H=4, N=40, gates=[None, -5.0])
    counter = drive.counter(wl)
    pages0 = [L.page.clone() for L in wl.layers]

    def run():
        for layer in range(2):
            drive.verify(wl, layer, counter)
        torch.cuda.synchronize()
        return [bits(L.out) for L in wl.layers[:2]], \
            [L.page.clone() for L in wl.layers[:2]]

    plain_out, plain_pages = run()
    for L, page in zip(wl.layers, pages0):
        L.page.copy_(page)
    a, b, c = _events(3)
    assert kda.set_launch_events(a, b, 2) == 0
    timed_out, timed_pages = run()
    assert kda.set_launch_events(None, None, 0) == 0    # both launches seen
    for x, y in zip(plain_out, timed_out):
        assert np.array_equal(x, y)
    for x, y in zip(plain_pages, timed_pages):
        assert torch.equal(x, y)
    two = a.elapsed_time(b)
    assert 0.0 < two < 1000.0, two
    # one launch, start and stop on the same kernel
    assert kda.set_launch_events(a, c, 1) == 0
    drive.verify(wl, 0, counter)
    torch.cuda.synchronize()
    assert kda.set_launch_events(None, None, 0) == 0
    one = a.elapsed_time(c)
    assert 0.0 < one < two, (one, two)


def test_arming_reports_launches_that_did_not_happen():
    wl = make_workload("ragged", DEV, B=4, H=2, D=64, Q=4, N=12)
    counter = drive.counter(wl)
    a, b = _events(2)
    assert kda.set_launch_events(a, b, 3) == 0
    drive.verify(wl, 0, counter)
    torch.cuda.synchronize()
    assert kda.set_launch_events(None, None, 0) == 2    # 1 of 3 happened
    with pytest.raises(kda.KdaError):
        kda.set_launch_events(None, None, -1)
