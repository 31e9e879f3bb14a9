"""The C-ABI library loads without a GPU, exports every function the header
declares, and its host-only checks map each rule of the pages' validation
to its status code (no launch, no device memory: descriptors point at CPU
tensors that are never dereferenced)."""
import ctypes
import os
import re

import pytest
import torch

import linear_attention_speculative_amd as kda
from linear_attention_speculative_amd import _abi
from workloads import make_workload
from workloads.drive import verify_kwargs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda_recoverssm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _abi.load()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert set(declared) == set(_abi.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert kda.abi_version() == 6
    assert lib.kda_status_string(_abi.KDA_E_UNALIGNED) == b"KDA_E_UNALIGNED"


def test_launch_events_arming_is_checked():
    """Arming the kernel timing takes launches >= 0; 0 (or NULL events)
    arms nothing, a negative count is an argument error."""
    lib = _abi.load()
    left = ctypes.c_int32(-1)
    assert lib.kda_set_launch_events(None, None, 0, None) == _abi.KDA_OK
    assert lib.kda_set_launch_events(None, None, 3, None) == _abi.KDA_OK
    assert lib.kda_set_launch_events(None, None, -1,
                                     ctypes.byref(left)) == _abi.KDA_E_ARG
    assert b"launches" in lib.kda_last_error()
    assert left.value == -1                  # untouched on error
    assert lib.kda_set_launch_events(None, None, 0,
                                     ctypes.byref(left)) == _abi.KDA_OK
    assert left.value == 3                   # none of the 3 happened
    assert lib.kda_set_launch_events(None, None, 0,
                                     ctypes.byref(left)) == _abi.KDA_OK
    assert left.value == 0


def _kw(**over):
    wl = make_workload(over.pop("cfg", "ragged"), B=4, H=2, D=16, Q=4, N=8,
                       **over)
    counter = torch.zeros(1, dtype=torch.int32)
    return wl, verify_kwargs(wl, 0, counter)


def _code(kw):
    return kda.check_verify(**kw)


def test_valid_arguments_pass_both_layouts_and_dtypes():
    for dim_first in (True, False):
        for act in ("f32", "bf16"):
            for out_dtype in ("f32", "act"):
                for kg in ("f32", "act"):
                    wl, kw = _kw(conv_dim_first=dim_first, act=act,
                                 weight=act, out_dtype=out_dtype,
                                 kg_dtype=kg)
                    assert _code(kw) == 0, kda.load().kda_last_error()


def test_tiny_and_deferred_configs_pass():
    wl = make_workload("tiny")
    assert _code(verify_kwargs(wl, 0, torch.zeros(1, dtype=torch.int32))) == 0
    wl = make_workload("deferred", B=8, H=2, D=32, N=16)
    for layer in range(2):
        assert _code(verify_kwargs(wl, layer,
                                   torch.zeros(1, dtype=torch.int32))) == 0


def test_shape_errors():
    wl, kw = _kw()
    kw["raw_gate"] = kw["raw_gate"][:, :-8]
    assert _code(kw) == _abi.KDA_E_SHAPE
    wl, kw = _kw()
    kw["out"] = torch.empty(wl.T, wl.H * wl.D + 4)
    assert _code(kw) == _abi.KDA_E_SHAPE
    wl, kw = _kw()
    kw["A_log"] = torch.zeros(wl.H + 1)
    assert _code(kw) == _abi.KDA_E_SHAPE
    wl, kw = _kw()
    kw["correction"] = kw["correction"][:, :, :2]
    assert _code(kw) == _abi.KDA_E_SHAPE
    wl, kw = _kw()
    kw["conv_weight"] = torch.zeros(3 * wl.H * wl.D, 3)
    assert _code(kw) == _abi.KDA_E_SHAPE


def test_dtype_errors():
    wl, kw = _kw(act="bf16", weight="bf16")
    kw["raw_beta"] = kw["raw_beta"].float()
    assert _code(kw) == _abi.KDA_E_DTYPE
    wl, kw = _kw()
    kw["correction"] = torch.zeros(kw["correction"].shape,
                                   dtype=torch.bfloat16)
    assert _code(kw) == _abi.KDA_E_DTYPE
    wl, kw = _kw()
    kw["state"] = torch.zeros(kw["state"].shape, dtype=torch.bfloat16)
    assert _code(kw) == _abi.KDA_E_DTYPE
    wl, kw = _kw()
    kw["mixed_qkv"] = kw["mixed_qkv"].half()
    assert _code(kw) == _abi.KDA_E_DTYPE


def test_layout_errors_on_static_tensors():
    wl, kw = _kw()
    st = kw["state"]
    kw["state"] = st.transpose(2, 3)   # heads no longer row-major
    assert _code(kw) == _abi.KDA_E_LAYOUT
    wl, kw = _kw()
    # a slot stride that is not a multiple of 16 bytes
    big = torch.zeros(wl.N * (wl.H * wl.D * wl.D + 1))
    kw["state"] = big.as_strided((wl.N, wl.H, wl.D, wl.D),
                                 (wl.H * wl.D * wl.D + 1, wl.D * wl.D, wl.D, 1))
    assert _code(kw) == _abi.KDA_E_LAYOUT
    wl, kw = _kw()
    buf = torch.zeros(kw["conv_weight"].numel() + 1)
    kw["conv_weight"] = buf[1:].view(kw["conv_weight"].shape)  # 4-byte offset
    assert _code(kw) == _abi.KDA_E_LAYOUT


def test_unaligned_activation_is_reported_without_launch():
    wl, kw = _kw()
    x = kw["mixed_qkv"]
    buf = torch.zeros(x.shape[0] * x.shape[1] + 1, dtype=x.dtype)
    kw["mixed_qkv"] = buf[1:].view(x.shape)    # one element past 16 bytes
    assert _code(kw) == _abi.KDA_E_UNALIGNED
    wl, kw = _kw()
    x = kw["out"]
    wide = torch.zeros(x.shape[0], x.shape[1] + 1, dtype=x.dtype)
    kw["out"] = wide[:, :x.shape[1]]           # row stride not 16-byte
    assert _code(kw) == _abi.KDA_E_UNALIGNED
    # the launch entry point refuses it the same way, before any device work
    with pytest.raises(kda.KdaUnaligned):
        kda.conv_update_verify(stream=0, **kw)


def test_unsupported_sizes():
    wl, kw = _kw()
    kw["spec_query_len"] = 17
    assert _code(kw) == _abi.KDA_E_UNSUPPORTED
    wl = make_workload("ragged", B=2, H=1, D=8, Q=4, N=4)
    kw = verify_kwargs(wl, 0, torch.zeros(1, dtype=torch.int32))
    assert _code(kw) == _abi.KDA_E_UNSUPPORTED            # head dim 8
    wl, kw = _kw()
    cs = kw["conv_state"]
    kw["conv_state"] = cs[:, :, :-1]                      # width-3 conv
    assert _code(kw) == _abi.KDA_E_UNSUPPORTED


def test_capacity_and_argument_errors():
    wl, kw = _kw()
    kw["spec_query_len"] = 1
    kw["correction"] = kw["correction"][:, :, :1]
    kw["key_gate"] = kw["key_gate"][:, :, :1]
    kw["conv_state"] = torch.zeros(wl.N, 3 * wl.H * wl.D, 3,
                                   dtype=kw["conv_state"].dtype)
    assert _code(kw) == _abi.KDA_E_CAPACITY
    wl, kw = _kw()
    kw["work_counter"] = None
    for sched in (_abi.KDA_SCHEDULE_DEFAULT, _abi.KDA_SCHEDULE_PER_ITEM):
        kw["schedule"] = sched       # no counter needed
        assert _code(kw) == 0
    kw["schedule"] = _abi.KDA_SCHEDULE_TICKETS
    assert _code(kw) == _abi.KDA_E_ARG
    for bad in (-1, 4):
        kw["schedule"] = bad
        assert _code(kw) == _abi.KDA_E_ARG
    kw["schedule"] = 0
    kw["max_workgroups"] = -1
    assert _code(kw) == _abi.KDA_E_ARG
    kw["max_workgroups"] = 0
    kw["items_per_ticket"] = -2
    assert _code(kw) == _abi.KDA_E_ARG


def test_zero_batch_is_a_valid_no_op():
    wl, kw = _kw()
    for k in ("mixed_qkv", "raw_gate", "raw_beta", "out"):
        kw[k] = kw[k][:0]
    kw["state_indices"] = kw["state_indices"][:0]
    kw["query_start_loc"] = kw["query_start_loc"][:1]
    kw["num_accepted_tokens"] = kw["num_accepted_tokens"][:0]
    assert _code(kw) == 0
    kda.conv_update_verify(stream=0, **kw)   # returns without launching


def _qkv_kw(**over):
    wl, kw = _kw(**over)
    for k in ("conv_state", "conv_weight", "num_accepted_tokens"):
        kw[k] = None
    return wl, kw


def test_unfused_verify_checks():
    for act in ("f32", "bf16"):
        wl, kw = _qkv_kw(act=act, weight=act)
        assert kda.check_verify_qkv(**kw) == 0, kda.load().kda_last_error()
    # the conv arguments are ignored, whatever they hold
    wl, kw = _kw()
    kw["conv_state"] = kw["conv_state"][:, :, :-1]
    assert kda.check_verify_qkv(**kw) == 0
    assert _code(kw) == _abi.KDA_E_UNSUPPORTED
    # the other rules still apply
    wl, kw = _qkv_kw()
    kw["query_start_loc"] = None
    assert kda.check_verify_qkv(**kw) == _abi.KDA_E_ARG
    wl, kw = _qkv_kw()
    kw["mixed_qkv"] = kw["mixed_qkv"][:, :-8]
    assert kda.check_verify_qkv(**kw) == _abi.KDA_E_SHAPE
    wl, kw = _qkv_kw()
    kw["state"] = torch.zeros(kw["state"].shape, dtype=torch.bfloat16)
    assert kda.check_verify_qkv(**kw) == _abi.KDA_E_DTYPE
    wl, kw = _qkv_kw()
    kw["schedule"] = _abi.KDA_SCHEDULE_TICKETS
    kw["work_counter"] = None
    assert kda.check_verify_qkv(**kw) == _abi.KDA_E_ARG
    wl, kw = _qkv_kw()
    x = kw["out"]
    wide = torch.zeros(x.shape[0], x.shape[1] + 1, dtype=x.dtype)
    kw["out"] = wide[:, :x.shape[1]]
    assert kda.check_verify_qkv(**kw) == _abi.KDA_E_UNALIGNED
    with pytest.raises(kda.KdaUnaligned):
        kda.verify_qkv(stream=0, **kw)


def _commit_ctx(**over):
    wl = make_workload(over.pop("cfg", "large"), B=4, H=2, D=16, Q=8, N=8,
                       gates=[None, -5.0, None], **over)
    layers = [dict(state=L.state, correction=L.correction,
                   key_gate=L.key_gate, A_log=L.A_log, dt_bias=L.dt_bias,
                   lower_bound=L.lower_bound if L.use_lower_bound else None)
              for L in wl.layers]
    return wl, layers


def test_commit_context_checks():
    wl, layers = _commit_ctx()
    # device tables on the CPU here: only the host-side checks run
    ctx = kda.CommitContext(layers, spec_query_len=wl.Q)
    assert ctx.check(wl.state_indices, wl.commit_lens) == 0
    assert ctx.check(wl.state_indices, wl.commit_lens,
                     final_state_indices=wl.state_indices) == 0
    with pytest.raises(ValueError):
        kda.CommitContext([], spec_query_len=wl.Q)
    bad = dict(layers[1])
    bad["state"] = bad["state"][:, :, :, :8]
    with pytest.raises(ValueError):
        kda.CommitContext([layers[0], bad], spec_query_len=wl.Q)
    bad = dict(layers[1])
    bad["key_gate"] = bad["key_gate"][:, :, :4]
    with pytest.raises(ValueError):
        kda.CommitContext([layers[0], bad], spec_query_len=wl.Q)


def test_commit_abi_codes():
    wl, layers = _commit_ctx()
    ctx = kda.CommitContext(layers, spec_query_len=wl.Q)
    lib = kda.load()

    def code(mut):
        a = ctx.args(wl.state_indices, wl.commit_lens)
        mut(a)
        return lib.kda_check_commit(ctypes.byref(a))

    assert code(lambda a: None) == 0
    assert code(lambda a: setattr(a, "num_layers", 0)) == _abi.KDA_E_ARG
    assert code(lambda a: setattr(a, "head_dim", 48)) == \
        _abi.KDA_E_UNSUPPORTED
    assert code(lambda a: setattr(a, "spec_query_len", 0)) == \
        _abi.KDA_E_UNSUPPORTED
    assert code(lambda a: a.state_strides.__setitem__(1, 17)) == \
        _abi.KDA_E_LAYOUT
    assert code(lambda a: setattr(a, "key_gate_dtype", 7)) == \
        _abi.KDA_E_DTYPE
    assert code(lambda a: setattr(a, "commit_lens", None)) == _abi.KDA_E_ARG
    # a misaligned layer base in the host copy of the tables
    host = ctx._host_tables.clone()
    host[0, 1] += 4
    keep = host.numpy()

    def mis(a):
        a.host_tables = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    assert code(mis) == _abi.KDA_E_LAYOUT
    assert b"layer 1" in lib.kda_last_error()


# ---- commit plan, conv compaction, align-mode commit ---------------------------

def _align_ctx():
    wl = make_workload("ragged", B=6, H=2, D=16, Q=4, N=12, act="bf16",
                       weight="bf16")
    layers = [dict(state=L.state, correction=L.correction,
                   key_gate=L.key_gate, A_log=L.A_log, dt_bias=L.dt_bias,
                   lower_bound=L.lower_bound if L.use_lower_bound else None,
                   conv_state=wl.conv_state_dim_first(i))
              for i, L in enumerate(wl.layers)]
    return wl, kda.CommitContext(layers, spec_query_len=wl.Q)


def test_plan_checks():
    wl, ctx = _align_ctx()
    lib = kda.load()
    acc = wl.num_accepted_tokens
    table = torch.zeros(wl.B, 5, dtype=torch.int32)
    computed = torch.zeros(wl.B, dtype=torch.int32)

    def code(**kw):
        base = dict(num_accepted_tokens=acc, state_indices=wl.state_indices,
                    query_start_loc=wl.query_start_loc)
        base.update(kw)
        a, _ = ctx.plan_args(**base)
        return lib.kda_check_commit_plan(ctypes.byref(a))

    assert code() == 0
    assert code(block_table=table, num_computed_tokens=computed,
                mamba_block_size=4) == 0
    # align arguments all or none
    assert code(block_table=table, mamba_block_size=4) == _abi.KDA_E_ARG
    assert code(num_computed_tokens=computed) == _abi.KDA_E_ARG
    # a block must cover one window
    assert code(block_table=table, num_computed_tokens=computed,
                mamba_block_size=3) == _abi.KDA_E_ARG
    a, _ = ctx.plan_args(num_accepted_tokens=acc,
                         state_indices=wl.state_indices,
                         query_start_loc=wl.query_start_loc,
                         block_table=table, num_computed_tokens=computed,
                         mamba_block_size=4)
    a.block_table_width = 0
    assert lib.kda_check_commit_plan(ctypes.byref(a)) == _abi.KDA_E_SHAPE
    # too few request rows for an identity mapping
    assert code(num_accepted_tokens=acc[:-1]) == _abi.KDA_E_ARG
    # with a mapping, the rows may be fewer or more than the batch
    assert code(num_accepted_tokens=acc[:2],
                request_indices=torch.zeros(wl.B, dtype=torch.int32)) == 0
    with pytest.raises(ValueError):
        ctx.plan_args(num_accepted_tokens=acc, state_indices=wl.state_indices,
                      query_start_loc=wl.query_start_loc,
                      request_indices=torch.zeros(wl.B - 1,
                                                  dtype=torch.int32))
    with pytest.raises(ValueError):
        ctx.plan_args(num_accepted_tokens=acc, state_indices=wl.state_indices,
                      query_start_loc=wl.query_start_loc,
                      block_table=table[0], num_computed_tokens=computed,
                      mamba_block_size=4)


def test_compaction_and_boundary_checks():
    wl, ctx = _align_ctx()
    lib = kda.load()
    si, lens = wl.state_indices, wl.commit_lens
    a = ctx.compact_args(si, lens)
    assert lib.kda_check_compact_conv(ctypes.byref(a)) == 0
    a = ctx.compact_args(si, lens, si, si, None)
    assert lib.kda_check_compact_conv(ctypes.byref(a)) == _abi.KDA_E_ARG
    a = ctx.compact_args(si, lens)
    a.conv_dtype = 9
    assert lib.kda_check_compact_conv(ctypes.byref(a)) == _abi.KDA_E_DTYPE
    a = ctx.compact_args(si, lens)
    a.num_layers = 0
    assert lib.kda_check_compact_conv(ctypes.byref(a)) == _abi.KDA_E_ARG
    # slots that would overlap in the host copy of the tables
    host = ctx._host_conv_tables.clone()
    host[1, 0] = 8
    keep = host.numpy()
    a = ctx.compact_args(si, lens)
    a.host_conv_tables = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    assert lib.kda_check_compact_conv(ctypes.byref(a)) == _abi.KDA_E_LAYOUT
    # the commit: boundary slots and lengths go together
    assert lib.kda_check_commit(ctypes.byref(ctx.args(si, lens))) == 0
    a = ctx.args(si, lens, boundary_state_indices=si)
    assert lib.kda_check_commit(ctypes.byref(a)) == _abi.KDA_E_ARG
    a = ctx.args(si, lens, boundary_state_indices=si,
                 boundary_recovery_lens=lens)
    assert lib.kda_check_commit(ctypes.byref(a)) == 0
    # a context without conv states cannot compact
    plain = kda.CommitContext([{k: v for k, v in L.items()
                                if k != "conv_state"} for L in ctx.layers],
                              spec_query_len=wl.Q)
    with pytest.raises(ValueError):
        plain.compact_args(si, lens)


def test_commit_step_checks():
    """The fused commit step takes the argument blocks of the three separate
    calls, linked through the plan's outputs; anything else is refused."""
    wl, ctx = _align_ctx()
    lib = kda.load()
    si, qsl = wl.state_indices, wl.query_start_loc
    acc = wl.num_accepted_tokens
    table = torch.zeros(wl.B, 5, dtype=torch.int32)
    computed = torch.zeros(wl.B, dtype=torch.int32)

    def blocks(align):
        extra = dict(block_table=table, num_computed_tokens=computed,
                     mamba_block_size=4) if align else {}
        pa, out = ctx.plan_args(acc, si, qsl, **extra)
        lens, fin, bnd, blen = out
        b2 = (bnd, blen) if align else (None, None)
        ca = ctx.args(si, lens, fin, None, 0, *b2)
        xa = ctx.compact_args(si, lens, fin, *b2)
        return pa, ca, xa, out

    def code(ca, pa, xa):
        return lib.kda_check_commit_step(
            ctypes.byref(ca), ctypes.byref(pa),
            None if xa is None else ctypes.byref(xa))

    for align in (False, True):
        pa, ca, xa, out = blocks(align)
        assert code(ca, pa, xa) == 0
        assert code(ca, pa, None) == 0               # no compaction
    pa, ca, xa, (lens, fin, bnd, blen) = blocks(True)
    # the commit must read the plan's outputs
    other = torch.zeros_like(lens)
    bad = ctx.args(si, other, fin, None, 0, bnd, blen)
    assert code(bad, pa, xa) == _abi.KDA_E_ARG
    bad = ctx.args(si, lens, fin)                    # align pair missing
    assert code(bad, pa, xa) == _abi.KDA_E_ARG
    bad = ctx.args(si.clone(), lens, fin, None, 0, bnd, blen)
    assert code(bad, pa, xa) == _abi.KDA_E_ARG
    # ... and so must the compaction
    bad = ctx.compact_args(si, lens, None, bnd, blen)
    assert code(ca, pa, bad) == _abi.KDA_E_ARG
    bad = ctx.compact_args(si, lens, fin, bnd, blen)
    bad.num_slots -= 1
    assert code(ca, pa, bad) == _abi.KDA_E_ARG
    bad = ctx.compact_args(si, lens, fin, bnd, blen)
    bad.conv_dim -= 1
    assert code(ca, pa, bad) == _abi.KDA_E_ARG
    # one batch and window for all three
    pa.spec_query_len = wl.Q - 1
    assert code(ca, pa, xa) == _abi.KDA_E_ARG
    # a non-align plan with a commit in align mode
    pa, ca, xa, (lens, fin, bnd, blen) = blocks(False)
    bad = ctx.args(si, lens, fin, None, 0, bnd, blen)
    assert code(bad, pa, None) == _abi.KDA_E_ARG
    # errors of the blocks themselves still come through
    ca.num_layers = 0
    assert code(ca, pa, xa) == _abi.KDA_E_ARG
    assert lib.kda_check_commit_step(None, ctypes.byref(pa), None) == \
        _abi.KDA_E_ARG


def test_byte_offsets_of_strided_outputs_fit_32_bits():
    # An fp32 `out` whose row stride keeps the element offsets of a window
    # under 2^31 but its byte offsets over it is refused (the kernel forms
    # those byte offsets in 32 bits).  Descriptors are edited directly: no
    # tensor of that extent is allocated.
    from linear_attention_speculative_amd.ops import verify_args
    wl, kw = _kw()
    a = verify_args(**kw)
    lib = _abi.load()
    assert lib.kda_check_verify(ctypes.byref(a)) == 0
    a.out.stride[0] = 1 << 28          # Q * stride = 2^30 elements, 2^32 B
    assert lib.kda_check_verify(ctypes.byref(a)) == _abi.KDA_E_LAYOUT
    assert b"byte offsets" in lib.kda_last_error()
    a = verify_args(**kw)
    a.correction.stride[2] = 1 << 28   # correction positions, fp32
    assert lib.kda_check_verify(ctypes.byref(a)) == _abi.KDA_E_LAYOUT


def test_vtile_schedule_checks():
    # explicit V-tiles: head dims 64 and 128, windows up to 8, no pending
    # records, and a counter with one arrival slot per (request, head)
    wl = make_workload("ragged", B=4, H=2, D=64, Q=4, N=8)
    big = torch.zeros(1 + wl.B * wl.H, dtype=torch.int32)
    kw = verify_kwargs(wl, 0, big, schedule=_abi.KDA_SCHEDULE_V_TILES,
                       v_tiles=4)
    assert _code(kw) == 0, kda.load().kda_last_error()
    kw["work_counter"] = big[:wl.B * wl.H]          # one element short
    assert _code(kw) == _abi.KDA_E_ARG
    assert b"1 + batch * heads" in kda.load().kda_last_error()
    kw["work_counter"] = big
    for bad in (1, 3, 16, -2):
        kw["v_tiles"] = bad
        assert _code(kw) == _abi.KDA_E_ARG
    kw["v_tiles"] = 0                               # library's choice
    assert _code(kw) == 0
    kw["pending_lens"] = torch.zeros(wl.B, dtype=torch.int32)
    assert _code(kw) == _abi.KDA_E_UNSUPPORTED
    wl = make_workload("ragged", B=4, H=2, D=16, Q=4, N=8)
    kw = verify_kwargs(wl, 0, torch.zeros(1 + 8, dtype=torch.int32),
                       schedule=_abi.KDA_SCHEDULE_V_TILES)
    assert _code(kw) == _abi.KDA_E_UNSUPPORTED       # head dim 16
    wl = make_workload("ragged", B=4, H=2, D=64, Q=12, N=8)
    kw = verify_kwargs(wl, 0, torch.zeros(1 + 8, dtype=torch.int32),
                       schedule=_abi.KDA_SCHEDULE_V_TILES)
    assert _code(kw) == _abi.KDA_E_UNSUPPORTED       # window 12
    # the unfused verify needs no counter for V-tiles
    wl = make_workload("ragged", B=4, H=2, D=64, Q=4, N=8)
    kw = verify_kwargs(wl, 0, None, schedule=_abi.KDA_SCHEDULE_V_TILES)
    for k in ("conv_state", "conv_weight", "num_accepted_tokens"):
        kw[k] = None
    assert kda.check_verify_qkv(**kw) == 0, kda.load().kda_last_error()


_TENSOR_FIELDS = ("mixed_qkv", "raw_gate", "raw_beta", "A_log", "dt_bias",
                  "state", "correction", "key_gate", "out", "conv_state",
                  "conv_weight")


def _fieldwise_tensor(t):
    d = _abi.KdaTensor()
    if t is not None:
        d.data = t.data_ptr()
        d.dtype = {torch.float32: _abi.KDA_F32,
                   torch.bfloat16: _abi.KDA_BF16}.get(t.dtype, -1)
        d.ndim = t.dim()
        for i in range(t.dim()):
            d.shape[i] = t.shape[i]
            d.stride[i] = t.stride(i)
    return d


def _fieldwise_verify_args(kw):
    """kda_verify_args built field by field through ctypes (the reference
    for the packed marshalling)."""
    a = _abi.KdaVerifyArgs()
    for name in _TENSOR_FIELDS:
        setattr(a, name, _fieldwise_tensor(kw.get(name)))
    for name in ("query_start_loc", "state_indices", "num_accepted_tokens",
                 "record_rows", "work_counter", "pending_lens"):
        t = kw.get(name)
        setattr(a, name, None if t is None else t.data_ptr())
    a.batch = kw["state_indices"].shape[0]
    a.spec_query_len = kw["spec_query_len"]
    a.null_block_id = kw.get("null_block_id", 0)
    a.conv_dim_first = 1 if kw["conv_dim_first"] else 0
    lb = kw.get("lower_bound")
    a.use_lower_bound = 0 if lb is None else 1
    a.lower_bound = 0.0 if lb is None else float(lb)
    a.max_workgroups = kw.get("max_workgroups", 0)
    a.items_per_ticket = kw.get("items_per_ticket", 0)
    a.schedule = kw.get("schedule", 0)
    wc = kw.get("work_counter")
    a.work_counter_len = 0 if wc is None else wc.numel()
    a.v_tiles = kw.get("v_tiles", 0)
    return a


def test_packed_verify_args_match_fieldwise_ctypes():
    """The one-call packed argument block is byte for byte the structure
    ctypes builds field by field (layouts, dtypes, optional tensors,
    scalars)."""
    from linear_attention_speculative_amd import ops
    cases = []
    for dim_first in (True, False):
        wl, kw = _kw(conv_dim_first=dim_first, act="f32", weight="f32")
        cases.append(kw)
    wl, kw = _kw(lower_bound=-5.0, kg_dtype="act", out_dtype="act")
    kw.update(record_rows=torch.arange(wl.B, dtype=torch.int32),
              pending_lens=torch.ones(wl.B, dtype=torch.int32),
              null_block_id=3, max_workgroups=7, items_per_ticket=2,
              schedule=2, v_tiles=4)
    cases.append(kw)
    kw2 = dict(kw, conv_state=None, conv_weight=None,
               num_accepted_tokens=None, work_counter=None)
    cases.append(kw2)
    # a transposed (strided) output view
    kw3 = dict(cases[0])
    kw3["out"] = kw3["out"].t().contiguous().t()
    cases.append(kw3)
    for kw in cases:
        packed = bytes(ops.verify_args(**kw))
        ref = bytes(_fieldwise_verify_args(kw))
        assert packed == ref
        for name in _TENSOR_FIELDS:
            t = kw.get(name)
            assert bytes(ops.describe(t)) == bytes(_fieldwise_tensor(t))
