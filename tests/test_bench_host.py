"""Host-side pieces of bench.py (no GPU): the one-GPU guard and the
algorithmic byte counts the roofline divides by, checked against a count
written out per tensor for a small workload."""
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def _count(wl, pending=None, boundary=None, conv=True):
    """Bytes of every tensor a launch must touch, request by request
    (conv False: the unfused verify, which has no taps, history or roll)."""
    H, D, Q, W, B = wl.H, wl.D, wl.Q, wl.W, wl.B
    e = {"f32": 4, "bf16": 2}
    ea, ew, eo, ek = (e[wl.act], e[wl.weight], e[wl.out_dtype],
                      e[wl.kg_dtype])
    C = 3 * H * D
    qsl = wl.query_start_loc.numpy()
    slots = wl.state_indices.numpy()
    lens = wl.commit_lens.numpy()
    v = (C * W * ew if conv else 0) + 4 * H + 4 * H * D + 4 * (3 * B + 1)
    c = 4 * H + 4 * H * D + 8 * B
    fl = cp = 0
    for b in range(B):
        q = int(min(max(qsl[b + 1] - qsl[b], 0), Q))
        if q == 0:
            continue
        if not 0 < slots[b] < wl.N:
            v += q * H * D * eo                    # zero rows only
            continue
        v += H * D * D * 4                         # checkpoint read
        if conv:
            v += (W - 1) * C * ea + (W - 2 + q) * C * ea   # history, roll
        v += q * C * ea + q * H * D * ea + q * H * ea  # q|k|v, gate, beta
        v += q * H * D * eo                        # outputs
        v += q * (H * D * 4 + 2 * H * D * ek)      # records
        n = int(min(max(lens[b], 0), Q))
        if n:
            c += 2 * H * D * D * 4 + n * (H * D * 4 + 2 * H * D * ek)
            if boundary is not None:
                cp += 2 * (W - 1) * C * ea
                if boundary[b] > 0:
                    c += H * D * D * 4
                    cp += 2 * (W - 1) * C * ea
        if pending is not None and pending[b] > 0:
            m = int(min(pending[b], Q))
            fl += H * D * D * 4 + m * (H * D * 4 + 2 * H * D * ek)
    return v, c, fl, cp


def test_algorithmic_bytes_match_a_per_tensor_count():
    for name, kw in (("ragged", dict(B=9, H=2, D=16, Q=4, N=16,
                                     null_frac=0.3)),
                     ("deferred", dict(B=6, H=2, D=32, N=12)),
                     ("tiny", {})):
        wl = make_workload(name, out_dtype="act", **kw)
        rng = np.random.default_rng(1)
        pend = rng.integers(0, wl.Q + 1, size=wl.B)
        bnd = rng.integers(0, 2, size=wl.B)
        got = bench.algorithmic_bytes(wl, pending=pend, boundary=bnd)
        v, c, fl, cp = _count(wl, pend, bnd)
        assert (got["verify"], got["commit"], got["flush"],
                got["compact"]) == (v, c, fl, cp), name
        qsl = wl.query_start_loc.numpy()
        assert got["tokens"] == int(np.minimum(np.diff(qsl), wl.Q).sum())
        # the unfused verify: the same count without the conv terms
        got = bench.algorithmic_bytes(wl, conv=False)
        v, c, _, _ = _count(wl, conv=False)
        assert (got["verify"], got["commit"]) == (v, c), name


def test_running_block_tables():
    """The align workload's tables: column 0 is each request's source slot,
    column 1 a free slot no source uses (distinct across requests, null once
    the free slots run out); the tokens already in the running block lie in
    [0, block size)."""
    from workloads.gen import running_block_tables
    wl = make_workload("headline")
    src = wl.state_indices.numpy()
    table, computed = running_block_tables(src, wl.N, 16, seed=5)
    assert table.dtype == np.int32 and table.shape == (wl.B, 2)
    assert np.array_equal(table[:, 0], src)
    nxt = table[:, 1]
    live = nxt[nxt > 0]
    assert len(set(live.tolist())) == len(live)
    assert not set(live.tolist()) & set(src.tolist())
    assert live.max() < wl.N
    assert len(live) == min(wl.B, wl.N - 1 - len(set(src.tolist())))
    assert computed.min() >= 0 and computed.max() < 16
    # the same seed gives the same tables
    t2, c2 = running_block_tables(src, wl.N, 16, seed=5)
    assert np.array_equal(t2, table) and np.array_equal(c2, computed)
    # with too few free slots, the last rows' next block is null
    small, _ = running_block_tables(np.arange(1, 9), 12, 16, seed=1)
    assert small[:3, 1].tolist() == [9, 10, 11]
    assert (small[3:, 1] == 0).all()
