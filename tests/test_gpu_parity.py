"""Parity of the HIP verify/commit (called through the C ABI) with the fp64
oracle on seeded inputs: every workload at its full size with every request
compared (the 24-layer workload: three layers in full, every layer checked
for coverage), plus edge cases, sweeps over head dims and windows, the key
record in the activation dtype, determinism across grid sizes, the ticket
counter protocol and HIP-graph replay."""
import numpy as np
import pytest
import torch

import linear_attention_speculative_amd as kda
import oracle
from tests.gpu_check import (TOL, bits, check_commit, check_verify,
                             commit_layer_inputs, f64, kg_extra_tol, rel_err,
                             run_oracle_verify, run_oracle_verify_qkv,
                             snapshot)
from workloads import drive, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _counter():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _view_mask(wl, record_page=False):
    """Bool mask over a page row: True inside a tensor view."""
    L = wl.layers[0]
    page = L.record_page if record_page else L.page
    m = torch.zeros(page.shape[1], dtype=torch.bool, device=page.device)
    views = wl.meta["page_views"]
    names = ("correction", "key_gate") if record_page else \
        (("conv", "state") + (("correction", "key_gate")
                              if wl.meta["records_in_page"] else ()))
    for nm in names:
        off, n = views[nm]
        m[off:off + n] = True
    return m


def _check_pages(wl, layer, page_before, rec_before=None):
    """Pages of slots no live request names are bitwise unchanged; padding
    bytes of every page are unchanged."""
    L = wl.layers[layer]
    slots = wl.state_indices.cpu().numpy()
    live = sorted({int(s) for s in slots if 0 < s < wl.N})
    unused = torch.ones(wl.N, dtype=torch.bool, device=DEV)
    if live:
        unused[torch.tensor(live, device=DEV)] = False
    assert torch.equal(L.page[unused], page_before[unused])
    pad = ~_view_mask(wl)
    assert torch.equal(L.page[:, pad], page_before[:, pad])
    if rec_before is not None:
        pad = ~_view_mask(wl, record_page=True)
        assert torch.equal(L.record_page[:, pad], rec_before[:, pad])
        rows = wl.record_rows.cpu().numpy()
        used = {int(rows[b]) for b in range(wl.B) if 0 < slots[b] < wl.N}
        keep = torch.tensor([r not in used for r in range(wl.R)], device=DEV)
        assert torch.equal(L.record_page[keep], rec_before[keep])


def _verify_case(wl, layer=0, reqs=None, max_wg=0, kg_tol=None, sched=0):
    L = wl.layers[layer]
    sample = snapshot(wl, layer, reqs)
    state_before = L.state.clone()
    page_before = L.page.clone()
    rec_before = None if L.record_page is None else L.record_page.clone()
    counter = _counter()
    drive.verify(wl, layer, counter, max_workgroups=max_wg, schedule=sched)
    torch.cuda.synchronize()
    assert int(counter.item()) == 0, "ticket counter must be left at 0"
    assert torch.equal(L.state, state_before), "verify wrote the checkpoint"
    ref = run_oracle_verify(sample)
    errs = check_verify(wl, layer, sample, ref, kg_k_tol=kg_tol,
                        extra_tol=kg_extra_tol(wl))
    _check_pages(wl, layer, page_before, rec_before)
    return sample, ref, errs


def _commit_case(wl, samples_refs, layers=None, final=None, lens=None):
    """Run the GPU commit over `layers` and compare with the oracle commit of
    each sampled layer.  samples_refs: {layer: (sample, ref)}."""
    ctx = drive.commit_context(wl, layers)
    lens_t = wl.commit_lens if lens is None else lens
    before = {l: wl.layers[l].state.clone() for l in samples_refs}
    ctx.commit(wl.state_indices, lens_t, final_state_indices=final,
               record_rows=wl.record_rows)
    torch.cuda.synchronize()
    errs = {}
    lens_np = lens_t.cpu().numpy()
    final_np = None if final is None else final.cpu().numpy()
    for l, (sample, ref) in samples_refs.items():
        L = wl.layers[l]
        # A live final slot receives the same value as the source would, so
        # the oracle folds in place in its compact pool; a null final slot
        # stays null there.
        cfinal = None
        if final_np is not None:
            cfinal = np.array(
                [sample.new_slot[i] if 0 < final_np[b] < wl.N else 0
                 for i, b in enumerate(sample.reqs)])
        (new, written), = oracle.commit(
            layers=[commit_layer_inputs(sample, ref, L)],
            state_indices=sample.new_slot, commit_lens=lens_np[sample.reqs],
            spec_query_len=wl.Q, final_state_indices=cfinal,
            record_rows=None if wl.record_rows is None else sample.new_row)
        errs[l] = check_commit(wl, l, sample, new, written, final_np,
                               extra_tol=kg_extra_tol(wl))
        # every slot the commit had no reason to write is bitwise unchanged
        slots = wl.state_indices.cpu().numpy()
        targets = set()
        for b in range(wl.B):
            s = int(slots[b])
            n = min(max(int(lens_np[b]), 0), wl.Q)
            if 0 < s < wl.N and n > 0:
                f = s if final is None else int(final_np[b])
                if 0 < f < wl.N:
                    targets.add(f)
        keep = torch.tensor([s not in targets for s in range(wl.N)],
                            device=DEV)
        assert torch.equal(L.state[keep], before[l][keep])
    return errs


# ---- small workload, in full --------------------------------------------------

@pytest.mark.parametrize("gate", [None, -5.0])
@pytest.mark.parametrize("dim_first", [True, False])
def test_tiny_verify_commit(gate, dim_first):
    wl = make_workload("tiny", DEV, gates=[gate], conv_dim_first=dim_first)
    sample, ref, errs = _verify_case(wl)
    cerr = _commit_case(wl, {0: (sample, ref)})
    print("tiny", gate, dim_first, errs, cerr)


# ---- single request and ragged batch, in full ----------------------------------

def test_single_request_full_shape():
    wl = make_workload("single", DEV)
    sample, ref, errs = _verify_case(wl)
    cerr = _commit_case(wl, {0: (sample, ref)})
    print("single", errs, cerr)


def test_ragged_batch_with_null_slots():
    wl = make_workload("ragged", DEV)
    assert int((wl.state_indices == 0).sum()) == 6
    sample, ref, errs = _verify_case(wl)
    cerr = _commit_case(wl, {0: (sample, ref)})
    print("ragged", errs, cerr)


# ---- sweeps over head dim, window, dtypes, layouts -------------------------------

SWEEP = [(16, 1), (16, 4), (16, 7), (32, 3), (32, 8), (64, 4), (64, 6),
         (64, 12), (128, 1), (128, 2), (128, 5), (128, 8), (128, 16),
         (16, 16), (32, 16)]


@pytest.mark.parametrize("D,Q", SWEEP)
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_sweep_head_dim_and_window(D, Q, act):
    wl = make_workload("ragged", DEV, B=7, H=3, D=D, Q=Q, N=12, act=act,
                       weight=act, null_frac=0.15,
                       conv_dim_first=(D + Q) % 2 == 0,
                       gates=[-5.0 if Q % 2 else None], act_row_pad=8)
    # each schedule (per item, tickets) sees half of the shapes
    sched = (1, 2)[(D + Q + len(act)) % 2]
    sample, ref, errs = _verify_case(wl, sched=sched)
    _commit_case(wl, {0: (sample, ref)})


@pytest.mark.parametrize("out_dtype,kg_dtype", [("act", "f32"),
                                                ("f32", "act"),
                                                ("act", "act")])
@pytest.mark.parametrize("Q", [4, 8])
def test_activation_dtype_outputs_and_records(out_dtype, kg_dtype, Q):
    # (Q = 8 stores its results non-temporally, Q = 4 with plain stores)
    wl = make_workload("ragged", DEV, B=12, H=4, D=128, Q=Q, N=20,
                       out_dtype=out_dtype, kg_dtype=kg_dtype)
    # A bf16 key record (the ops page's layout): the oracle's verify rounds
    # its fp64 key to bf16 and its commit folds those records; the bounds
    # widen by one bf16 step (see kg_extra_tol).
    sample, ref, errs = _verify_case(wl)
    cerr = _commit_case(wl, {0: (sample, ref)})
    print("act records", out_dtype, kg_dtype, Q, errs, cerr)


def test_bf16_out_is_rne_of_fp32_out():
    wl = make_workload("ragged", DEV, B=16, H=4, D=128, Q=4, N=24)
    L = wl.layers[0]
    page0 = L.page.clone()
    drive.verify(wl, 0, _counter())
    out32 = L.out.clone()
    L.page.copy_(page0)
    out16 = torch.empty_like(out32, dtype=torch.bfloat16)
    kw = drive.verify_kwargs(wl, 0, _counter())
    kw["out"] = out16
    kda.conv_update_verify(**kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out16), bits(out32.to(torch.bfloat16)))


# ---- edge cases -----------------------------------------------------------------

def test_edge_cases_verify_and_commit():
    wl = make_workload("ragged", DEV, B=9, H=2, D=32, Q=4, N=16, act="f32",
                       weight="f32", null_frac=0.0)
    qsl = wl.query_start_loc.cpu().numpy()
    # request 1 has no tokens; request 4 points past the pool; request 6
    # has a negative slot (padding row)
    lens = np.diff(qsl)
    lens[1] = 0
    qsl = np.concatenate([[0], np.cumsum(lens)])
    wl.query_start_loc.copy_(torch.tensor(qsl, dtype=torch.int32))
    T = int(qsl[-1])
    for L in wl.layers:
        L.mixed_qkv = L.mixed_qkv[:T]
        L.raw_gate = L.raw_gate[:T]
        L.raw_beta = L.raw_beta[:T]
        L.out = L.out[:T]
    wl.T = T
    slots = wl.state_indices.clone()
    slots[4] = wl.N + 7
    slots[6] = -1
    wl.state_indices.copy_(slots)
    # accepted counts outside [1, Q] are clamped
    acc = wl.num_accepted_tokens.clone()
    acc[0], acc[2] = 0, 99
    wl.num_accepted_tokens.copy_(acc)
    sample, ref, _ = _verify_case(wl)
    # commit lengths: 0, over-long (clamped to Q), negative
    lens_c = wl.commit_lens.clone()
    lens_c[0], lens_c[2], lens_c[3] = 0, 50, -3
    _commit_case(wl, {0: (sample, ref)}, lens=lens_c)


def test_batch_beyond_one_grid_row():
    """65,636 requests, more than one grid row of 65,535 holds: the default
    schedule takes the ticket kernel and the commit its strided kernel. The
    requests on both sides of 65,535 and the last ones match the oracle, and
    every slot no request names is unchanged."""
    B = 65536 + 100
    wl = make_workload("ragged", DEV, B=B, H=1, D=16, Q=2, N=B + 64,
                       null_frac=0.05)
    reqs = (list(range(0, 8)) + list(range(65528, 65544)) +
            list(range(B - 8, B)))
    sample, ref, errs = _verify_case(wl, reqs=reqs)
    cerr = _commit_case(wl, {0: (sample, ref)})
    print("beyond one grid row", errs, cerr)


def test_commit_to_final_slots():
    wl = make_workload("ragged", DEV, B=6, H=2, D=64, Q=4, N=20,
                       null_frac=0.0)
    sample, ref, _ = _verify_case(wl)
    slots = wl.state_indices.cpu().numpy()
    free = [s for s in range(1, wl.N) if s not in set(slots.tolist())]
    final = torch.tensor(free[:wl.B], dtype=torch.int32, device=DEV)
    final[3] = 0                       # null final slot: skipped
    src_before = wl.layers[0].state.clone()
    _commit_case(wl, {0: (sample, ref)}, final=final)
    # sources are untouched when the result goes to the final slot
    si = torch.tensor(slots, device=DEV).long()
    assert torch.equal(wl.layers[0].state[si], src_before[si])


def test_record_rows_negative_row_writes_no_records():
    wl = make_workload("deferred", DEV, B=10, H=2, D=32, Q=4, N=24)
    rows = wl.record_rows.clone()
    rows[3] = -1
    wl.record_rows.copy_(rows)
    sample, ref, _ = _verify_case(wl)
    assert sample.new_row[3] == -1


# ---- scheduling: determinism, counter protocol, graph replay ----------------------

def test_results_independent_of_grid_size():
    wl = make_workload("ragged", DEV, B=20, H=8, D=128, Q=4, N=32)
    L = wl.layers[0]
    page0, rec0 = L.page.clone(), None
    outs = []
    # (schedule, max_workgroups, items_per_ticket)
    for sched, grid, per in ((0, 0, 0), (1, 0, 0), (2, 1, 0), (2, 3, 0),
                             (2, 0, 3), (2, 5, 7), (2, 2, 1000)):
        L.page.copy_(page0)
        c = _counter()
        drive.verify(wl, 0, c, max_workgroups=grid, items_per_ticket=per,
                     schedule=sched)
        torch.cuda.synchronize()
        assert int(c.item()) == 0
        outs.append((L.out.clone(), L.page.clone()))
    for o, p in outs[1:]:
        assert np.array_equal(bits(o), bits(outs[0][0]))
        assert torch.equal(p, outs[0][1])


def test_counter_protocol_and_reset():
    wl = make_workload("ragged", DEV, B=8, H=2, D=16, Q=4, N=12)
    c = _counter()
    for _ in range(3):
        drive.verify(wl, 0, c, max_workgroups=5, schedule=2)
        torch.cuda.synchronize()
        assert int(c.item()) == 0
    c.fill_(123)
    kda.reset_counter(c)
    torch.cuda.synchronize()
    assert int(c.item()) == 0


def test_verify_graph_replay_matches_eager():
    wl = make_workload("ragged", DEV, B=16, H=4, D=128, Q=4, N=24)
    L = wl.layers[0]
    page0 = L.page.clone()
    counter = _counter()
    drive.verify(wl, 0, counter)
    torch.cuda.synchronize()
    eager_out, eager_page = L.out.clone(), L.page.clone()
    L.page.copy_(page0)
    L.out.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            drive.verify(wl, 0, counter)
    torch.cuda.synchronize()
    for _ in range(3):
        L.page.copy_(page0)          # eager work between replays
        L.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(counter.item()) == 0
        assert np.array_equal(bits(L.out), bits(eager_out))
        assert torch.equal(L.page, eager_page)


def _graph_matches_eager(run, reset, outputs):
    """Capture run() in a HIP graph; replay it three times with eager
    resets in between and compare every replay with an eager run, bit for
    bit."""
    reset()
    torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    eager = [bits(t) for t in outputs()]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for _ in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs(), eager):
            assert np.array_equal(bits(a), b)


def test_commit_flush_and_align_graph_replay_matches_eager():
    wl = make_workload("ragged", DEV, B=16, H=4, D=128, Q=4, N=48,
                       null_frac=0.1)
    L = wl.layers[0]
    drive.verify(wl, 0, _counter())            # records to commit
    torch.cuda.synchronize()
    page0 = L.page.clone()

    def reset():
        L.page.copy_(page0)
        L.out.fill_(float("nan"))

    ctx = drive.commit_context(wl, conv=True)
    # the multi-layer commit
    _graph_matches_eager(
        lambda: ctx.commit(wl.state_indices, wl.commit_lens), reset,
        lambda: [L.page])
    # the fused deferred flush + verify
    _graph_matches_eager(
        lambda: drive.verify(wl, 0, _counter(), pending_lens=wl.commit_lens),
        reset, lambda: [L.page, L.out])
    # plan, compaction and align-mode commit in one call
    rng = np.random.default_rng(3)
    slots = wl.state_indices.cpu().numpy()
    free = [x for x in range(1, wl.N) if x not in set(slots.tolist())]
    table = np.zeros((wl.B, 2), dtype=np.int32)
    table[:, 0] = slots
    table[:, 1] = free[:wl.B]
    table_t = torch.as_tensor(table, device=DEV)
    computed = torch.as_tensor(rng.integers(0, 6, size=wl.B),
                               dtype=torch.int32, device=DEV)
    _graph_matches_eager(
        lambda: ctx.commit_step(wl.commit_lens, wl.state_indices,
                                wl.query_start_loc, block_table=table_t,
                                num_computed_tokens=computed,
                                mamba_block_size=6),
        reset, lambda: [L.page])


# ---- full-size workloads, every request compared ---------------------------------------

@pytest.mark.timeout(600)
def test_headline_workload_full():
    wl = make_workload("headline", DEV, out_dtype="act")
    sample, ref, errs = _verify_case(wl)
    cerr = _commit_case(wl, {0: (sample, ref)})
    print("headline", errs, cerr)


@pytest.mark.timeout(900)
def test_large_multilayer_commit_full():
    """24 verifies, then one commit launch over all 24 layers.  Layers 0,
    11 and 23 are compared with the oracle on every request; every layer is
    checked for coverage: no output left unwritten (the buffers start as
    NaN), every live request's record row written at each of its positions,
    and every committing request's checkpoint changed while every other slot
    keeps its bytes."""
    wl = make_workload("large", DEV)
    checked = {0: None, 11: None, 23: None}
    rec0 = {}
    for layer in range(len(wl.layers)):
        L = wl.layers[layer]
        rec0[layer] = (L.correction.clone(), L.key_gate.clone())
        if layer in checked:
            sample, ref, errs = _verify_case(wl, layer)
            checked[layer] = (sample, ref)
        else:
            drive.verify(wl, layer, _counter())
    torch.cuda.synchronize()
    slots = wl.state_indices.cpu().numpy()
    live = [b for b in range(wl.B) if 0 < slots[b] < wl.N]
    lens = wl.commit_lens.cpu().numpy()
    qsl = wl.query_start_loc.cpu().numpy()
    for layer, L in enumerate(wl.layers):
        assert not torch.isnan(L.out).any(), ("unwritten outputs", layer)
        c0, k0 = rec0[layer]
        for b in live:
            q = int(qsl[b + 1] - qsl[b])
            s = int(slots[b])
            # each written position differs from the noise it replaced
            assert bool((L.correction[s, :, :q] != c0[s, :, :q])
                        .any(dim=-1).all()), ("records", layer, b)
            assert bool((L.key_gate[s, :, :q] != k0[s, :, :q])
                        .any(dim=-1).all()), ("key records", layer, b)
    before = [L.state.clone() for L in wl.layers]
    errs = _commit_case(wl, checked)          # one launch, all 24 layers
    commits = torch.tensor([int(slots[b]) for b in live if lens[b] > 0],
                           device=DEV)
    keep = torch.ones(wl.N, dtype=torch.bool, device=DEV)
    keep[commits.long()] = False
    for layer, L in enumerate(wl.layers):
        changed = (L.state.index_select(0, commits) !=
                   before[layer].index_select(0, commits))
        assert bool(changed.flatten(2).any(dim=-1).all()), ("commit", layer)
        assert torch.equal(L.state[keep], before[layer][keep]), layer
    print("large", errs)


@pytest.mark.timeout(900)
def test_deferred_sequence_full():
    wl = make_workload("deferred", DEV)
    reqs = None
    # previous step: verify both layers, creating the records
    first = {}
    for layer in range(2):
        first[layer] = snapshot(wl, layer, reqs)
        drive.verify(wl, layer, _counter())
    torch.cuda.synchronize()
    # this step: fold the pending tokens of every layer in one launch,
    # then verify each layer from the committed checkpoints
    ctx = drive.commit_context(wl)
    ctx.commit(wl.state_indices, wl.commit_lens, record_rows=wl.record_rows)
    torch.cuda.synchronize()
    pending = wl.commit_lens.cpu().numpy()
    for layer in range(2):
        L = wl.layers[layer]
        s0 = first[layer]
        r0 = run_oracle_verify(s0)
        check_verify(wl, layer, s0, r0)       # the previous step's verify
        (new, written), = oracle.commit(
            layers=[commit_layer_inputs(s0, r0, L)],
            state_indices=s0.new_slot, commit_lens=pending[s0.reqs],
            spec_query_len=wl.Q, record_rows=s0.new_row)
        check_commit(wl, layer, s0, new, written)
        # second verify on the oracle side: committed state, rolled conv
        # state and the previous step's records as inputs
        inp = dict(s0.inputs)
        inp["state"] = new
        inp["conv_state"] = r0["conv_state"]
        inp["correction"] = r0["correction"]
        inp["key_gate"] = r0["key_gate"]
        s1 = snapshot(wl, layer, reqs)
        ref1 = oracle.conv_update_verify(**inp)
        counter = _counter()
        drive.verify(wl, layer, counter)
        torch.cuda.synchronize()
        errs = check_verify(wl, layer, s1, ref1)
        print("deferred", layer, errs)


def _flush_case(wl, reqs=None, layers=(0,)):
    """Previous step: verify (records); this step: the fused launch that
    folds the pending positions (wl.commit_lens) and verifies.  Oracle:
    commit, then verify from the committed state, rolled conv state and the
    previous records."""
    first = {}
    for layer in layers:
        first[layer] = snapshot(wl, layer, reqs)
        drive.verify(wl, layer, _counter())
    torch.cuda.synchronize()
    pending = wl.commit_lens.cpu().numpy()
    out = {}
    for layer in layers:
        L = wl.layers[layer]
        s0 = first[layer]
        r0 = run_oracle_verify(s0)
        (new, written), = oracle.commit(
            layers=[commit_layer_inputs(s0, r0, L)],
            state_indices=s0.new_slot, commit_lens=pending[s0.reqs],
            spec_query_len=wl.Q, record_rows=s0.new_row)
        inp = dict(s0.inputs)
        inp["state"] = new
        inp["conv_state"] = r0["conv_state"]
        inp["correction"] = r0["correction"]
        inp["key_gate"] = r0["key_gate"]
        s1 = snapshot(wl, layer, reqs)
        ref1 = oracle.conv_update_verify(**inp)
        state_before = L.state.clone()
        drive.verify(wl, layer, _counter(), pending_lens=wl.commit_lens)
        torch.cuda.synchronize()
        cerr = check_commit(wl, layer, s0, new, written,
                            extra_tol=kg_extra_tol(wl))
        errs = check_verify(wl, layer, s1, ref1, extra_tol=kg_extra_tol(wl))
        # slots with nothing pending (or null, or no record row) keep their
        # checkpoint bit for bit
        slots = wl.state_indices.cpu().numpy()
        rows = (slots if wl.record_rows is None
                else wl.record_rows.cpu().numpy())
        for b in range(wl.B):
            sl = int(slots[b])
            if 0 < sl < wl.N and (pending[b] <= 0 or not 0 <= rows[b] < wl.R):
                assert torch.equal(bits_t(L.state[sl]), bits_t(state_before[sl]))
        out[layer] = (cerr, errs)
    return out


def bits_t(t):
    return t.contiguous().view(torch.int32)


@pytest.mark.parametrize("D,Q,act,kg", [(128, 4, "bf16", "f32"),
                                        (64, 8, "f32", "f32"),
                                        (32, 3, "bf16", "f32"),
                                        (16, 16, "f32", "f32"),
                                        (128, 4, "bf16", "act"),
                                        (64, 8, "bf16", "act")])
def test_deferred_flush_fused(D, Q, act, kg):
    wl = make_workload("ragged", DEV, B=20, H=3, D=D, Q=Q, N=32, act=act,
                       weight=act, null_frac=0.15,
                       conv_dim_first=Q % 2 == 0, kg_dtype=kg)
    # pending positions: at most what the previous verify recorded, some 0
    rng = np.random.default_rng(D + Q)
    qlen = (wl.query_start_loc[1:] - wl.query_start_loc[:-1]).cpu().numpy()
    pend = np.minimum(rng.integers(0, Q + 1, size=wl.B), qlen)
    wl.commit_lens.copy_(torch.tensor(pend, dtype=torch.int32))
    print("flush", D, Q, act, kg, _flush_case(wl))


@pytest.mark.parametrize("all_empty", [False, True])
def test_deferred_flush_with_empty_windows(all_empty):
    """A request whose slot is live but whose window is empty this step
    still folds its pending positions into its checkpoint (the deferred
    commit does not depend on the new window); with no tokens at all the
    launch still runs for the flush.  Oracle: commit, then verify."""
    wl = make_workload("ragged", DEV, B=16, H=3, D=128, Q=4, N=32,
                       null_frac=0.15)
    L = wl.layers[0]
    s0 = snapshot(wl, 0)
    drive.verify(wl, 0, _counter())           # the previous step's records
    torch.cuda.synchronize()
    r0 = run_oracle_verify(s0)
    qlen = np.diff(wl.query_start_loc.cpu().numpy())
    rng = np.random.default_rng(11 + all_empty)
    pend = np.minimum(rng.integers(1, wl.Q + 1, size=wl.B), qlen)
    # this step's windows: every third request (or every request) is empty
    new_len = np.where(np.arange(wl.B) % 3 == 0, 0, qlen)
    if all_empty:
        new_len[:] = 0
    qsl = np.concatenate([[0], np.cumsum(new_len)])
    T = int(qsl[-1])
    wl.query_start_loc.copy_(torch.tensor(qsl, dtype=torch.int32))
    L.mixed_qkv, L.raw_gate = L.mixed_qkv[:T], L.raw_gate[:T]
    L.raw_beta, L.out = L.raw_beta[:T], L.out[:T]
    wl.T = T
    pend_t = torch.tensor(pend, dtype=torch.int32, device=DEV)
    (new, written), = oracle.commit(
        layers=[commit_layer_inputs(s0, r0, L)], state_indices=s0.new_slot,
        commit_lens=pend, spec_query_len=wl.Q)
    s1 = snapshot(wl, 0)
    inp = dict(s1.inputs)
    inp.update(state=new, conv_state=r0["conv_state"],
               correction=r0["correction"], key_gate=r0["key_gate"])
    ref1 = oracle.conv_update_verify(**inp)
    rec_before = (L.correction.clone(), L.key_gate.clone())
    drive.verify(wl, 0, _counter(), pending_lens=pend_t)
    torch.cuda.synchronize()
    live = [b for b in range(wl.B) if s0.valid[b]]
    assert any(new_len[b] == 0 and pend[b] > 0 for b in live)
    cerr = check_commit(wl, 0, s0, new, written)
    errs = check_verify(wl, 0, s1, ref1, rec_before=rec_before)
    print("flush, empty windows", all_empty, T, cerr, errs)


@pytest.mark.timeout(900)
def test_deferred_flush_fused_full():
    wl = make_workload("deferred", DEV)
    print("flush deferred", _flush_case(wl, layers=(0, 1)))


def test_commit_schedules_agree_bitwise():
    # The persistent strided schedule and the one-workgroup-per-item grid
    # compute every item with the same code: identical bytes.
    wl = make_workload("large", DEV, B=24, H=4, D=128, N=40,
                       gates=[None, -5.0, None])
    for layer in range(3):
        drive.verify(wl, layer, _counter())
    ctx = drive.commit_context(wl)
    pages0 = [L.page.clone() for L in wl.layers]
    results = []
    for grid in (0, 7, 1, 100000):
        for L, p0 in zip(wl.layers, pages0):
            L.page.copy_(p0)
        ctx.commit(wl.state_indices, wl.commit_lens, max_workgroups=grid)
        torch.cuda.synchronize()
        results.append([L.page.clone() for L in wl.layers])
    for other in results[1:]:
        for a, b in zip(results[0], other):
            assert torch.equal(a, b)


# ---- the unfused verify (q | k | v already convolved) ------------------------

def _qkv_case(wl, layer=0, reqs=None, sched=0):
    """The layer's activation rows are taken as convolved q | k | v: outputs
    and records match the oracle's unfused verify; the checkpoint and the
    conv state are not touched."""
    L = wl.layers[layer]
    sample = snapshot(wl, layer, reqs)
    state_before = L.state.clone()
    conv_before = L.conv_state.clone()
    page_before = L.page.clone()
    rec_before = None if L.record_page is None else L.record_page.clone()
    counter = _counter()
    drive.verify_qkv(wl, layer, counter, schedule=sched)
    torch.cuda.synchronize()
    assert int(counter.item()) == 0
    assert torch.equal(L.state, state_before), "verify wrote the checkpoint"
    assert torch.equal(L.conv_state, conv_before), "conv state was written"
    ref = run_oracle_verify_qkv(sample)
    errs = check_verify(wl, layer, sample, ref)
    _check_pages(wl, layer, page_before, rec_before)
    return sample, ref, errs


@pytest.mark.parametrize("D,Q,act,gate,sched",
                         [(128, 4, "bf16", None, 0), (64, 8, "f32", -5.0, 2),
                          (32, 3, "bf16", None, 1), (16, 16, "f32", -5.0, 0),
                          (128, 8, "f32", None, 2)])
def test_unfused_verify(D, Q, act, gate, sched):
    wl = make_workload("ragged", DEV, B=20, H=3, D=D, Q=Q, N=32, act=act,
                       weight=act, null_frac=0.15, gates=[gate])
    sample, ref, errs = _qkv_case(wl, sched=sched)
    # the records feed the commit exactly as the fused verify's do
    cerr = _commit_case(wl, {0: (sample, ref)})
    print("qkv", D, Q, act, gate, sched, errs, cerr)


def test_unfused_verify_tiny_and_record_rows():
    wl = make_workload("tiny", DEV)
    print("qkv tiny", _qkv_case(wl)[2])
    wl = make_workload("deferred", DEV, B=40, N=96, out_dtype="act",
                       kg_dtype="act")
    for layer in range(2):
        print("qkv rows", layer, _qkv_case(wl, layer)[2])


@pytest.mark.timeout(600)
def test_unfused_verify_headline_full():
    wl = make_workload("headline", DEV)
    sample, ref, errs = _qkv_case(wl)
    print("qkv headline", errs)


def test_deferred_flush_with_unfused_verify():
    # The fused flush in front of the unfused verify: commit of the pending
    # positions, then the verify of convolved q | k | v from the committed
    # state; the conv state is not touched.
    for D, Q, act in ((128, 4, "bf16"), (64, 8, "f32")):
        wl = make_workload("ragged", DEV, B=16, H=3, D=D, Q=Q, N=32, act=act,
                           weight=act, null_frac=0.15)
        rng = np.random.default_rng(D + 7 * Q)
        qlen = (wl.query_start_loc[1:] - wl.query_start_loc[:-1]).cpu().numpy()
        pend = np.minimum(rng.integers(0, Q + 1, size=wl.B), qlen)
        wl.commit_lens.copy_(torch.tensor(pend, dtype=torch.int32))
        L = wl.layers[0]
        s0 = snapshot(wl, 0)
        drive.verify_qkv(wl, 0, _counter())
        torch.cuda.synchronize()
        r0 = run_oracle_verify_qkv(s0)
        (new, written), = oracle.commit(
            layers=[commit_layer_inputs(s0, r0, L)],
            state_indices=s0.new_slot, commit_lens=pend[s0.reqs],
            spec_query_len=wl.Q, record_rows=s0.new_row)
        s1 = snapshot(wl, 0)
        inp = {k: v for k, v in s0.inputs.items()
               if k not in ("conv_state", "conv_weight", "num_accepted_tokens")}
        inp.update(state=new, correction=r0["correction"],
                   key_gate=r0["key_gate"])
        ref1 = oracle.verify_qkv(**inp)
        conv_before = L.conv_state.clone()
        drive.verify_qkv(wl, 0, _counter(), pending_lens=wl.commit_lens)
        torch.cuda.synchronize()
        assert torch.equal(L.conv_state, conv_before)
        cerr = check_commit(wl, 0, s0, new, written)
        errs = check_verify(wl, 0, s1, ref1)
        print("flush qkv", D, Q, act, cerr, errs)
