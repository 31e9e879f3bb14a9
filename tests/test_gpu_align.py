"""Parity of the HIP commit plan, conv compaction and align-mode commit
(called through the C ABI) with the fp64 oracle: the plan and the compaction
bit for bit, the boundary and final states to the commit's tolerance, and a
multi-step prefix-caching sequence (verify -> plan -> compaction -> commit)
checked against the oracle at every step."""
import numpy as np
import pytest
import torch

import linear_attention_speculative_amd as kda
import oracle
from linear_attention_speculative_amd.debug import check_slot_aliasing
from tests.gpu_check import (TOL, bits, check_verify, f64, full_inputs,
                             kg_extra_tol, rel_err, run_oracle_verify,
                             snapshot)
from workloads import drive, make_workload
from workloads.gen import (block_tables, running_block_tables,
                           step_activations)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.int32, device=DEV)


def _np(t):
    return t.cpu().numpy().astype(np.int64)


def _destinations(rng, sources, N):
    """Final and boundary slots that never collide with another request's
    source or destination: each is the request's own source, a fresh free
    slot, or null (boundary only)."""
    free = [s for s in range(1, N) if s not in set(sources.tolist())]
    rng.shuffle(free)
    final, bnd = [], []
    for s in sources:
        final.append(int(s) if rng.random() < 0.4 else free.pop())
        r = rng.random()
        bnd.append(0 if r < 0.3 else (int(s) if r < 0.5 else free.pop()))
    final, bnd = np.array(final), np.array(bnd)
    check_slot_aliasing(sources, num_slots=N, final_state_indices=final,
                        boundary_state_indices=bnd)
    return final, bnd


# ---- the plan ------------------------------------------------------------------

@pytest.mark.parametrize("align,mapped", [(False, False), (False, True),
                                          (True, False), (True, True)])
def test_plan_matches_oracle_bitwise(align, mapped):
    rng = np.random.default_rng(40 + 2 * align + mapped)
    wl = make_workload("ragged", DEV, B=4, H=2, D=16, Q=4, N=8)
    ctx = drive.commit_context(wl)
    B, Q, bs, width = 300, wl.Q, 6, 9
    rows = B + 7 if mapped else B
    acc = rng.integers(-1, Q + 3, size=rows)
    req = rng.permutation(rows)[:B]
    if mapped:
        req[:5] = [rows, rows + 3, -1, -2, rows - 1]   # rows out of range
    slots = rng.integers(0, 60, size=B)
    qlen = rng.integers(0, Q + 1, size=B)
    qsl = np.concatenate([[0], np.cumsum(qlen)])
    wide = rng.integers(-1, 60, size=(rows, 2 * width))
    table = wide[:, ::2]                               # a strided view
    computed = rng.integers(-3, width * bs + 5, size=rows)
    kw = dict(num_accepted_tokens=_i32(acc), state_indices=_i32(slots),
              query_start_loc=_i32(qsl),
              request_indices=_i32(req) if mapped else None)
    okw = dict(num_accepted_tokens=acc, state_indices=slots,
               query_start_loc=qsl, spec_query_len=Q,
               request_indices=req if mapped else None)
    if align:
        kw.update(block_table=_i32(wide)[:, ::2],
                  num_computed_tokens=_i32(computed), mamba_block_size=bs)
        okw.update(block_table=table, num_computed_tokens=computed,
                   mamba_block_size=bs)
    got = ctx.plan(**kw)
    torch.cuda.synchronize()
    ref = oracle.commit_plan(**okw)
    for name, g, r in zip(("lens", "final", "boundary", "blens"), got, ref):
        assert np.array_equal(_np(g), r), name
    if align:
        assert (ref[3] > 0).sum() > 20                 # boundaries occurred


# ---- the compaction ------------------------------------------------------------

@pytest.mark.parametrize("dim_first,act", [(True, "bf16"), (False, "f32"),
                                           (True, "f32"), (False, "bf16")])
def test_compaction_matches_oracle_bitwise(dim_first, act):
    rng = np.random.default_rng(50 + dim_first + 2 * (act == "f32"))
    wl = make_workload("large", DEV, B=24, H=2, D=32, Q=8, N=80, act=act,
                       weight=act, gates=[None, -5.0, None],
                       conv_dim_first=dim_first)
    ctx = drive.commit_context(wl, conv=True)
    src = _np(wl.state_indices)
    final, bnd = _destinations(rng, src, wl.N)
    lens = rng.integers(-1, wl.Q + 2, size=wl.B)
    blens = rng.integers(-1, wl.Q + 2, size=wl.B)
    src[3] = 0                                         # a null request
    si = _i32(src)
    before = [bits(wl.conv_state_dim_first(l)) for l in range(3)]
    pages = [L.page.clone() for L in wl.layers]
    ctx.compact(si, _i32(lens), _i32(final), _i32(bnd), _i32(blens))
    torch.cuda.synchronize()
    ref = oracle.compact_conv_state(
        conv_states=before, state_indices=src, commit_lens=lens,
        final_state_indices=final, boundary_state_indices=bnd,
        boundary_recovery_lens=blens)
    for l in range(3):
        assert np.array_equal(bits(wl.conv_state_dim_first(l)), ref[l])
        assert not np.array_equal(ref[l], before[l])
        # nothing outside the conv views changed
        L = wl.layers[l]
        off, n = wl.meta["page_views"]["conv"]
        keep = torch.ones(L.page.shape[1], dtype=torch.bool, device=DEV)
        keep[off:off + n] = False
        assert torch.equal(L.page[:, keep], pages[l][:, keep])


# ---- the align-mode commit ---------------------------------------------------------

def test_align_commit_matches_oracle():
    rng = np.random.default_rng(61)
    wl = make_workload("large", DEV, B=24, H=4, D=128, Q=8, N=80,
                       gates=[None, -5.0, None])
    # oracle inputs taken before any launch; the oracle verifies from them
    # and its commit folds its own records
    oin = []
    for layer in range(3):
        oin.append(full_inputs(wl, layer))
        drive.verify(wl, layer, torch.zeros(1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    src = _np(wl.state_indices)
    final, bnd = _destinations(rng, src, wl.N)
    lens = rng.integers(0, wl.Q + 1, size=wl.B)
    blens = rng.integers(-1, wl.Q + 2, size=wl.B)
    lens[:3] = wl.Q
    blens[:3] = [0, wl.Q, 3]                       # m = 0, m = n, m inside
    inputs = []
    for l, L in enumerate(wl.layers):
        v = oracle.conv_update_verify(**oin[l])
        inputs.append(dict(state=oin[l]["state"], correction=v["correction"],
                           key_gate=v["key_gate"], A_log=oin[l]["A_log"],
                           dt_bias=oin[l]["dt_bias"],
                           use_lower_bound=L.use_lower_bound,
                           lower_bound=L.lower_bound))
    before = [L.state.clone() for L in wl.layers]
    ctx = drive.commit_context(wl)
    ctx.commit(_i32(src), _i32(lens), final_state_indices=_i32(final),
               boundary_state_indices=_i32(bnd),
               boundary_recovery_lens=_i32(blens))
    torch.cuda.synchronize()
    refs = oracle.commit(layers=inputs, state_indices=src, commit_lens=lens,
                         spec_query_len=wl.Q, final_state_indices=final,
                         boundary_state_indices=bnd,
                         boundary_recovery_lens=blens)
    n_bnd = 0
    for l, (new, written) in enumerate(refs):
        L = wl.layers[l]
        w = written.any(axis=1)
        gpu = f64(L.state)
        err = rel_err(gpu[w], new[w])
        assert err <= TOL[wl.act], (l, err)
        keep = torch.as_tensor(~w, device=DEV)
        assert torch.equal(L.state[keep], before[l][keep])
        n_bnd += int(sum(1 for b in range(wl.B) if 0 < bnd[b] and
                         lens[b] > 0 and 0 < final[b] and written[bnd[b]].all()))
    assert n_bnd > 10


# ---- a prefix-caching sequence ----------------------------------------------------

def test_align_sequence_matches_oracle():
    """Eight requests, each with its own table of state blocks (6 tokens per
    block), through several speculative steps: verify the running block
    (accepted count 1: the history was compacted), then plan, compaction
    and commit of every layer in one call.  The oracle runs the same steps
    on its own pools (seeded like the GPU's, then carried from step to step
    on the oracle side); at every step each GPU result matches it."""
    rng = np.random.default_rng(71)
    B, H, D, Q, bs, width = 8, 2, 32, 4, 6, 8
    wl = make_workload("ragged", DEV, B=B, H=H, D=D, Q=Q, N=B * width + 1,
                       act="bf16", weight="bf16", gates=[None, -5.0])
    N = wl.N
    ctx = drive.commit_context(wl, conv=True)
    tables = block_tables(B, width, N, seed=7)
    table_t = _i32(tables)
    c = rng.integers(1, 2 * bs, size=B)
    tol = TOL["bf16"]
    crossings = 0
    # the oracle's own pools, from the seeded tensors before any launch; each
    # step's oracle results carry over to the next step on the oracle side
    opool = [dict(state=f64(L.state), conv_state=f64(wl.conv_state_dim_first(l)),
                  correction=f64(L.correction), key_gate=f64(L.key_gate))
             for l, L in enumerate(wl.layers)]
    for step in range(6):
        qlen = rng.integers(1, Q + 1, size=B)
        qsl = np.concatenate([[0], np.cumsum(qlen)])
        T = int(qsl[-1])
        acc = np.minimum(rng.integers(1, Q + 1, size=B), qlen)
        src = tables[np.arange(B), c // bs]
        meta = dict(query_start_loc=_i32(qsl), state_indices=_i32(src),
                    num_accepted_tokens=_i32(np.ones(B)))
        acts = step_activations(T, H, D, "bf16", seed=100 + step, device=DEV)
        oracle_in, outs, gpu_before = [], [], []
        for l, L in enumerate(wl.layers):
            gpu_before.append(f64(L.state))
            oracle_in.append(dict(
                mixed_qkv=f64(acts["mixed_qkv"]), raw_gate=f64(acts["raw_gate"]),
                raw_beta=f64(acts["raw_beta"]), A_log=f64(L.A_log),
                dt_bias=f64(L.dt_bias), state=opool[l]["state"],
                correction=opool[l]["correction"],
                key_gate=opool[l]["key_gate"],
                out=np.zeros((T, H * D)),
                conv_state=opool[l]["conv_state"],
                conv_weight=f64(L.conv_weight), query_start_loc=qsl,
                state_indices=src, num_accepted_tokens=np.ones(B, np.int64),
                spec_query_len=Q, use_lower_bound=L.use_lower_bound,
                lower_bound=L.lower_bound))
            kw = drive.verify_kwargs(wl, l, None, schedule=1)
            kw.update(acts)
            kw.update(meta)
            kw["out"] = torch.zeros(T, H * D, device=DEV)
            kda.conv_update_verify(**kw)
            outs.append(kw["out"])
        plan = ctx.commit_step(_i32(acc), meta["state_indices"],
                               meta["query_start_loc"], block_table=table_t,
                               num_computed_tokens=_i32(c),
                               mamba_block_size=bs)
        torch.cuda.synchronize()
        ref_plan = oracle.commit_plan(
            num_accepted_tokens=acc, state_indices=src, query_start_loc=qsl,
            spec_query_len=Q, block_table=tables, num_computed_tokens=c,
            mamba_block_size=bs)
        for g, r in zip(plan, ref_plan):
            assert np.array_equal(_np(g), r), step
        lens, final, bnd, blens = ref_plan
        crossings += int((bnd > 0).sum())
        for l, L in enumerate(wl.layers):
            v = oracle.conv_update_verify(**oracle_in[l])
            assert rel_err(f64(outs[l]), v["out"]) <= tol
            conv, = oracle.compact_conv_state(
                conv_states=[v["conv_state"]], state_indices=src,
                commit_lens=lens, final_state_indices=final,
                boundary_state_indices=bnd, boundary_recovery_lens=blens)
            assert np.array_equal(f64(wl.conv_state_dim_first(l)), conv), \
                (step, l)
            (new, written), = oracle.commit(
                layers=[dict(state=oracle_in[l]["state"],
                             correction=v["correction"],
                             key_gate=v["key_gate"], A_log=oracle_in[l]["A_log"],
                             dt_bias=oracle_in[l]["dt_bias"],
                             use_lower_bound=L.use_lower_bound,
                             lower_bound=L.lower_bound)],
                state_indices=src, commit_lens=lens, spec_query_len=Q,
                final_state_indices=final, boundary_state_indices=bnd,
                boundary_recovery_lens=blens)
            w = written.any(axis=1)
            gpu = f64(L.state)
            assert rel_err(gpu[w], new[w]) <= tol, (step, l)
            # slots the step does not commit keep their bytes, and every
            # slot still matches the oracle's chain
            assert np.array_equal(gpu[~w], gpu_before[l][~w])
            assert rel_err(gpu, new) <= tol, (step, l)
            opool[l] = dict(state=new, conv_state=conv,
                            correction=v["correction"],
                            key_gate=v["key_gate"])
        c = c + lens
    assert crossings >= 4


# ---- the align workload at full size -------------------------------------------------

@pytest.mark.timeout(600)
@pytest.mark.parametrize("kg", ["f32", "act"])
def test_align_workload_full(kg):
    """The headline batch under prefix caching, in the launches the align
    benchmark times: a two-block table per request (16 tokens per block),
    the verify with accepted count 1, then plan, compaction and commit in
    one call.  Every request against the oracle: the plan bit for bit,
    outputs and records, compacted conv histories bit for bit, boundary and
    final states to the tolerance.  `kg` = "act" stores the key record in
    the activation dtype (the ops page's layout): the oracle's verify rounds
    its key to bf16 and its commit folds those records."""
    wl = make_workload("headline", DEV, kg_dtype=kg)
    xtol = kg_extra_tol(wl)
    assert wl.record_rows is None          # records indexed by source slot
    L = wl.layers[0]
    bs = 16
    slots = _np(wl.state_indices)
    table, computed = running_block_tables(slots, wl.N, bs, seed=5)
    acc = _np(wl.commit_lens)
    ref_plan = oracle.commit_plan(
        num_accepted_tokens=acc, state_indices=slots,
        query_start_loc=_np(wl.query_start_loc), spec_query_len=wl.Q,
        block_table=table, num_computed_tokens=computed,
        mamba_block_size=bs)
    lens, final, bnd, blens = ref_plan
    crossing = np.nonzero(bnd > 0)[0].tolist()
    assert len(crossing) >= 10
    reqs = list(range(wl.B))

    wl.num_accepted_tokens.fill_(1)        # the history was compacted
    sample = snapshot(wl, 0, reqs)
    live = [i for i, ok in enumerate(sample.valid) if ok]
    # destinations that are no request's source: fresh blocks
    dest = sorted(({int(final[b]) for b in reqs} |
                   {int(bnd[b]) for b in reqs if bnd[b] > 0})
                  - set(slots.tolist()))
    dest_t = torch.tensor(dest, device=DEV)
    dest_state = f64(L.state.index_select(0, dest_t))
    dest_conv = f64(wl.conv_state_dim_first(0).index_select(0, dest_t))

    ctx = drive.commit_context(wl, conv=True)
    drive.verify(wl, 0, torch.zeros(1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ref = run_oracle_verify(sample)
    errs = check_verify(wl, 0, sample, ref,       # before the compaction
                        extra_tol=xtol)
    plan = ctx.commit_step(wl.commit_lens, wl.state_indices,
                           wl.query_start_loc, block_table=_i32(table),
                           num_computed_tokens=_i32(computed),
                           mamba_block_size=bs)
    torch.cuda.synchronize()
    for name, g, r in zip(("lens", "final", "boundary", "blens"), plan,
                          ref_plan):
        assert np.array_equal(_np(g), r), name

    # the compact pool: 0 null, then the sampled sources, then `dest`
    n_src = sample.inputs["state"].shape[0]
    cmap = {int(sample.slots[i]): int(sample.new_slot[i]) for i in live}
    cmap.update({s: n_src + j for j, s in enumerate(dest)})

    def compact(a):
        return np.array([cmap[int(a[b])] if a[b] > 0 else 0 for b in reqs])

    c_src, c_final, c_bnd = sample.new_slot, compact(final), compact(bnd)
    conv_ref, = oracle.compact_conv_state(
        conv_states=[np.concatenate([ref["conv_state"], dest_conv])],
        state_indices=c_src, commit_lens=lens[reqs],
        final_state_indices=c_final, boundary_state_indices=c_bnd,
        boundary_recovery_lens=blens[reqs])
    (new, written), = oracle.commit(
        layers=[dict(state=np.concatenate([sample.inputs["state"],
                                           dest_state]),
                     correction=ref["correction"], key_gate=ref["key_gate"],
                     A_log=sample.inputs["A_log"],
                     dt_bias=sample.inputs["dt_bias"],
                     use_lower_bound=L.use_lower_bound,
                     lower_bound=L.lower_bound)],
        state_indices=c_src, commit_lens=lens[reqs], spec_query_len=wl.Q,
        final_state_indices=c_final, boundary_state_indices=c_bnd,
        boundary_recovery_lens=blens[reqs])

    inv = {c: s for s, c in cmap.items()}
    pool = sorted(inv)
    gpu_conv = f64(wl.conv_state_dim_first(0).index_select(
        0, torch.tensor([inv[c] for c in pool], device=DEV)))
    assert np.array_equal(gpu_conv, conv_ref[pool])
    rows = np.nonzero(written.any(axis=1))[0]
    assert written[c_bnd[c_bnd > 0]].all()
    gpu = f64(L.state.index_select(
        0, torch.tensor([inv[int(c)] for c in rows], device=DEV)))
    err = rel_err(gpu, new[rows])
    assert err <= TOL[wl.act] + xtol, err
    print("align full size", kg, len(reqs), "requests,", len(crossing),
          "boundaries, verify", errs, "state", err)


# ---- the fused commit step ----------------------------------------------------------

# name: (workload, sizes, align, conv states, request mapping, max_workgroups)
STEP_CASES = {
    "align_bf16_dimfirst": ("large", dict(D=32, Q=8, act="bf16",
                                          conv_dim_first=True),
                            True, True, False, 0),
    "align_f32_tokfirst_mapped": ("large", dict(D=16, Q=4, act="f32",
                                                conv_dim_first=False),
                                  True, True, True, 0),
    "align_noconv_d128_strided": ("large", dict(D=128, Q=4, act="bf16",
                                                conv_dim_first=True),
                                  True, False, False, 7),
    "plain_conv_ragged_nulls": ("ragged", dict(D=64, Q=8, act="bf16",
                                               conv_dim_first=True,
                                               null_frac=0.2),
                                False, True, False, 0),
    "plain_noconv_q16_mapped": ("ragged", dict(D=128, Q=16, act="f32",
                                               conv_dim_first=False),
                                False, False, True, 0),
    # the pages' record layout: the key record in the activation dtype
    "align_bf16_keyrecord_d64": ("large", dict(D=64, Q=4, act="bf16",
                                               conv_dim_first=True,
                                               kg_dtype="act"),
                                 True, True, False, 0),
}


@pytest.mark.parametrize("case", sorted(STEP_CASES))
def test_fused_commit_step_matches_three_launches(case):
    """kda_recoverssm_commit_step against kda_commit_plan, then
    kda_compact_conv_state, then kda_recoverssm_commit on the same pools:
    the plan's four arrays and every byte of every layer's pages (states,
    conv states, records) are identical; the plan also equals the
    oracle's."""
    name, sizes, align, conv, mapped, max_wg = STEP_CASES[case]
    rng = np.random.default_rng(80 + sorted(STEP_CASES).index(case))
    B, width, bs = 24, 4, 8
    rows = B + 3 if mapped else B
    N = rows * width + 1 if align else 80
    gates = [None, -5.0, None] if name == "large" else [None, -5.0]
    wl = make_workload(name, DEV, B=B, H=2, N=N, weight=sizes["act"],
                       gates=gates, **sizes)
    Q = wl.Q
    req = rng.permutation(rows)[:B] if mapped else None
    acc = rng.integers(-1, Q + 2, size=rows)
    extra, oextra = {}, {}
    if align:
        tables = block_tables(rows, width, N, seed=9)
        computed = rng.integers(0, 2 * bs, size=rows)
        ridx = req if mapped else np.arange(B)
        src = tables[ridx, computed[ridx] // bs]
        src[3] = 0                                   # a null request
        wl.state_indices.copy_(_i32(src))
        extra = dict(block_table=_i32(tables),
                     num_computed_tokens=_i32(computed), mamba_block_size=bs)
        oextra = dict(block_table=tables, num_computed_tokens=computed,
                      mamba_block_size=bs)
    if mapped:
        extra["request_indices"] = _i32(req)
        oextra["request_indices"] = req
    counter = torch.zeros(1, dtype=torch.int32, device=DEV)
    for layer in range(len(wl.layers)):
        drive.verify(wl, layer, counter)
    ctx = drive.commit_context(wl, conv=conv)
    args = (_i32(acc), wl.state_indices, wl.query_start_loc)
    before = [L.page.clone() for L in wl.layers]
    plan_f = [t.clone() for t in ctx.commit_step(
        *args, fused=True, max_workgroups=max_wg, **extra)]
    torch.cuda.synchronize()
    after_f = [L.page.clone() for L in wl.layers]
    for L, page in zip(wl.layers, before):
        L.page.copy_(page)
    plan_s = ctx.commit_step(*args, fused=False, **extra)
    torch.cuda.synchronize()
    ref = oracle.commit_plan(
        num_accepted_tokens=acc, state_indices=_np(wl.state_indices),
        query_start_loc=_np(wl.query_start_loc), spec_query_len=Q, **oextra)
    for what, f, s, r in zip(("lens", "final", "boundary", "blens"), plan_f,
                             plan_s, ref):
        assert torch.equal(f, s), what
        assert np.array_equal(_np(f), r), what
    for layer, L in enumerate(wl.layers):
        assert torch.equal(L.page, after_f[layer]), layer
        assert not torch.equal(after_f[layer], before[layer]), layer
    assert (ref[0] > 0).sum() >= 5
    if align:
        assert (ref[2] > 0).sum() >= 3
