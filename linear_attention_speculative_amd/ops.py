"""Python binding of the KDA RecoverSSM C ABI, taking torch tensors.

Argument marshalling only: tensors are described by pointer, dtype, sizes and
strides, and the current HIP stream is passed through.  Every step of the
path runs in the HIP library; if it is missing these functions raise.

Functions mirror the pages' host API:
  * `conv_update_verify` -- the kernels page's `CuteRecoverSSMVerify.__call__`
    (fused conv update + verify), with the ops page's record layout;
  * `CommitContext` -- the ops page's `KDARecoverSSMCommitContext` (per-layer
    address tables built once, then one commit launch per step).
"""
from __future__ import annotations

import ctypes
import struct
from typing import Optional, Sequence

import torch

from . import _abi

_DT = {torch.float32: _abi.KDA_F32, torch.bfloat16: _abi.KDA_BF16}


class KdaError(RuntimeError):
    """A failing library call: `status` is the kda_status code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class KdaUnaligned(KdaError):
    """An activation is not 16-byte aligned; nothing was launched."""


def _status_name(code: int) -> str:
    return _abi.load().kda_status_string(code).decode()


def _raise(code: int):
    msg = _abi.load().kda_last_error().decode()
    cls = KdaUnaligned if code == _abi.KDA_E_UNALIGNED else KdaError
    raise cls(code, msg)


_PAD = ((0, 0, 0, 0), (0, 0, 0), (0, 0), (0,), ())


def _pack_format(cls) -> str:
    """struct-module format of a ctypes type in its C layout (explicit
    padding bytes, little-endian, standard sizes)."""
    if issubclass(cls, ctypes.Structure):
        fmt, pos = "", 0
        for name, ftype in cls._fields_:
            off = getattr(cls, name).offset
            fmt += f"{off - pos}x" if off > pos else ""
            fmt += _pack_format(ftype)
            pos = off + ctypes.sizeof(ftype)
        end = ctypes.sizeof(cls)
        return fmt + (f"{end - pos}x" if end > pos else "")
    if issubclass(cls, ctypes.Array):
        return _pack_format(cls._type_) * cls._length_
    if cls is ctypes.c_void_p or issubclass(cls, ctypes._Pointer):
        return "Q"
    if cls is ctypes.c_float:
        return "f"
    return {4: "i", 8: "q"}[ctypes.sizeof(cls)]


# KdaTensor as 11 values: data, dtype, ndim, 4 sizes, 4 strides
_NO_TENSOR = (0, 0, 0) + (0,) * 8
_TENSOR_PACK = struct.Struct("<" + _pack_format(_abi.KdaTensor))


def _tensor_values(t: Optional[torch.Tensor]) -> tuple:
    if t is None:
        return _NO_TENSOR
    nd = t.dim()
    if nd > 4:
        raise ValueError("tensors of at most 4 dimensions")
    pad = _PAD[nd]
    return (t.data_ptr(), _DT.get(t.dtype, -1), nd, *t.shape, *pad,
            *t.stride(), *pad)


def describe(t: Optional[torch.Tensor]) -> _abi.KdaTensor:
    """Descriptor of a tensor view (sizes and strides in elements), for
    callers that fill an argument structure themselves."""
    return _abi.KdaTensor.from_buffer_copy(
        _TENSOR_PACK.pack(*_tensor_values(t)))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise TypeError("metadata tensors must be int32")
    if not t.is_contiguous():
        raise ValueError("metadata tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


_VERIFY_PACK = struct.Struct("<" + _pack_format(_abi.KdaVerifyArgs))


def verify_args(*, mixed_qkv, raw_gate, raw_beta, A_log, dt_bias,
                lower_bound, state, correction, key_gate, out, conv_state,
                conv_weight, query_start_loc, state_indices,
                num_accepted_tokens, spec_query_len, conv_dim_first,
                work_counter, record_rows=None, null_block_id=0,
                max_workgroups=0, items_per_ticket=0,
                schedule=0, pending_lens=None,
                v_tiles=0) -> _abi.KdaVerifyArgs:
    """kda_verify_args for these tensors, packed in one struct-module call
    (field order and layout of `_abi.KdaVerifyArgs`)."""
    vals = (*_tensor_values(mixed_qkv), *_tensor_values(raw_gate),
            *_tensor_values(raw_beta), *_tensor_values(A_log),
            *_tensor_values(dt_bias), *_tensor_values(state),
            *_tensor_values(correction), *_tensor_values(key_gate),
            *_tensor_values(out), *_tensor_values(conv_state),
            *_tensor_values(conv_weight),
            _ptr(query_start_loc) or 0, _ptr(state_indices) or 0,
            _ptr(num_accepted_tokens) or 0, _ptr(record_rows) or 0,
            _ptr(work_counter) or 0,
            state_indices.shape[0], spec_query_len, null_block_id,
            1 if conv_dim_first else 0,
            0 if lower_bound is None else 1,
            0.0 if lower_bound is None else float(lower_bound),
            max_workgroups, items_per_ticket, schedule,
            _ptr(pending_lens) or 0,
            0 if work_counter is None else work_counter.numel(),
            v_tiles)
    return _abi.KdaVerifyArgs.from_buffer_copy(_VERIFY_PACK.pack(*vals))


def check_verify(**kwargs) -> int:
    """Host-only validation (no launch); returns the kda_status code."""
    a = verify_args(**kwargs)
    return _abi.load().kda_check_verify(ctypes.byref(a))


def conv_update_verify(*, stream=None, **kwargs) -> None:
    """Fused conv update + speculative verify of one KDA layer on the current
    (or given) stream.  Arguments follow kda_verify_args in
    include/kda_recoverssm.h; `lower_bound=None` selects the softplus gate;
    `pending_lens` (int32 [batch]) first folds the previous step's pending
    record positions into the checkpoints (the deferred commit).
    Raises KdaUnaligned (nothing launched) for misaligned activations and
    KdaError for any other rejected argument."""
    a = verify_args(**kwargs)
    rc = _abi.load().kda_conv_update_verify(ctypes.byref(a),
                                           _stream(stream))
    if rc != _abi.KDA_OK:
        _raise(rc)


def conv_update_verify_noalloc(*, stream=None, **kwargs) -> None:
    """`conv_update_verify` without a caller-supplied counter array: the
    library's per-GPU scratch holds the work counters (the C entry point
    allocates nothing; `work_counter` is ignored).  Calls that overlap on
    one GPU race on that scratch."""
    kwargs.setdefault("work_counter", None)
    a = verify_args(**kwargs)
    rc = _abi.load().kda_conv_update_verify_noalloc(ctypes.byref(a),
                                                   _stream(stream))
    if rc != _abi.KDA_OK:
        _raise(rc)


def _qkv_args(kwargs) -> _abi.KdaVerifyArgs:
    for k in ("conv_state", "conv_weight", "num_accepted_tokens"):
        kwargs.setdefault(k, None)
    kwargs.setdefault("conv_dim_first", True)
    return verify_args(**kwargs)


def check_verify_qkv(**kwargs) -> int:
    """Host-only validation of the unfused verify (no launch)."""
    a = _qkv_args(kwargs)
    return _abi.load().kda_check_verify_qkv(ctypes.byref(a))


def verify_qkv(*, stream=None, **kwargs) -> None:
    """The unfused verify (ops page, `kda_recoverssm_verify`): `mixed_qkv`
    holds the already convolved q | k | v; conv_state, conv_weight and
    num_accepted_tokens are not used (pass None).  Otherwise as
    `conv_update_verify`."""
    a = _qkv_args(kwargs)
    rc = _abi.load().kda_recoverssm_verify_qkv(ctypes.byref(a),
                                              _stream(stream))
    if rc != _abi.KDA_OK:
        _raise(rc)


def reset_counter(counter: torch.Tensor, stream=None) -> None:
    rc = _abi.load().kda_reset_counter(_ptr(counter), counter.numel(),
                                      _stream(stream))
    if rc != _abi.KDA_OK:
        _raise(rc)


def set_launch_events(start=None, stop=None, launches: int = 1) -> int:
    """Time the next `launches` kernels that library calls on this thread
    launch: `start` (a torch.cuda.Event, created by one record beforehand,
    or None) records the start of the first, `stop` the end of the last,
    from the kernels' own dispatch (kda_set_launch_events).  Returns how
    many launches the previous arming was still waiting for."""
    def handle(ev):
        if ev is None:
            return None
        h = ev.cuda_event
        if not h:
            raise ValueError("record the event once before arming it")
        return h
    left = ctypes.c_int32(0)
    rc = _abi.load().kda_set_launch_events(handle(start), handle(stop),
                                           int(launches), ctypes.byref(left))
    if rc != _abi.KDA_OK:
        _raise(rc)
    return left.value


def abi_version() -> int:
    return _abi.load().kda_abi_version()


class CommitContext:
    """Per-layer address tables and stacked gate parameters for the
    multi-layer commit, built once (ops page,
    `KDARecoverSSMCommitContext.create`), then `commit` per step.

    `layers` is a sequence of dicts with `state` [N,H,D,D] f32,
    `correction` [R,H,Q,D] f32, `key_gate` [R,H,Q,2D], `A_log` [H],
    `dt_bias` [H,D] (or [H*D]) and `lower_bound` (None = softplus), and
    optionally `conv_state`, the layer's conv state seen dim-first
    [N, 3HD, Q+2] (a token-first state's `.transpose(1, 2)`), which enables
    the compaction.  Every layer must share sizes, dtypes and inner
    strides; slot strides may differ per layer.
    """

    def __init__(self, layers: Sequence[dict], *, spec_query_len: int,
                 null_block_id: int = 0):
        if not layers:
            raise ValueError("KDA RecoverSSM commit requires at least one "
                             "layer")
        ref = layers[0]
        st, corr, kg = ref["state"], ref["correction"], ref["key_gate"]
        if st.dim() != 4:
            raise ValueError("KDA RecoverSSM checkpoint must be "
                             "four-dimensional")
        N, H, V, K = st.shape
        if V != K:
            raise ValueError("key and value head dims must be equal")
        Q = spec_query_len
        for L in layers:
            s = L["state"]
            if (s.shape != st.shape or s.dtype != torch.float32 or
                    s.device != st.device or s.stride()[1:] != st.stride()[1:]):
                raise ValueError("KDA RecoverSSM layers need matching "
                                 "checkpoint layout")
            c = L["correction"]
            if (c.shape[1:] != (H, Q, V) or c.shape[0] != corr.shape[0] or
                    c.dtype != torch.float32 or c.device != st.device or
                    c.stride()[1:] != corr.stride()[1:]):
                raise ValueError("KDA RecoverSSM correction buffers need "
                                 f"float32 shape [rows, {H}, {Q}, {V}]")
            g = L["key_gate"]
            if (g.shape != (c.shape[0], H, Q, 2 * K) or g.dtype != kg.dtype or
                    g.device != st.device or g.stride()[1:] != kg.stride()[1:]):
                raise ValueError("KDA RecoverSSM key/gate buffers need shape "
                                 f"[rows, {H}, {Q}, {2 * K}]")
            if L["A_log"].shape != (H,):
                raise ValueError("KDA RecoverSSM A_log shape is incompatible")
            if L["dt_bias"].numel() != H * K:
                raise ValueError("KDA RecoverSSM dt_bias shape is "
                                 "incompatible")
        dev = st.device
        self.layers = list(layers)
        self.num_layers = len(layers)
        self.H, self.D, self.Q, self.N = H, K, Q, N
        self.R = corr.shape[0]
        self.null_block_id = null_block_id
        self.key_gate_dtype = _DT[kg.dtype]
        self.state_strides = st.stride()[1:3]
        self.correction_strides = corr.stride()[1:3]
        self.key_gate_strides = kg.stride()[1:3]

        def col(key, fn):
            return [fn(L[key]) for L in layers]

        host = torch.tensor(
            [col("state", lambda t: t.data_ptr()),
             col("state", lambda t: t.stride(0)),
             col("correction", lambda t: t.data_ptr()),
             col("correction", lambda t: t.stride(0)),
             col("key_gate", lambda t: t.data_ptr()),
             col("key_gate", lambda t: t.stride(0))], dtype=torch.int64)
        self._host_tables = host.contiguous()
        self.tables = self._host_tables.to(dev)
        self._fixed: Optional[bytes] = None   # constant argument fields
        self.A_log = torch.stack([L["A_log"].float() for L in layers]) \
            .contiguous().to(dev)
        self.dt_bias = torch.stack(
            [L["dt_bias"].float().reshape(H, K) for L in layers]) \
            .contiguous().to(dev)
        self.use_lower_bound = torch.tensor(
            [0 if L.get("lower_bound") is None else 1 for L in layers],
            dtype=torch.int32, device=dev)
        self.lower_bound = torch.tensor(
            [0.0 if L.get("lower_bound") is None else float(L["lower_bound"])
             for L in layers], dtype=torch.float32, device=dev)
        self.conv_tables = None
        convs = [L.get("conv_state") for L in layers]
        if any(c is not None for c in convs):
            if any(c is None for c in convs):
                raise ValueError("KDA RecoverSSM layers need matching conv "
                                 "state")
            c0 = convs[0]
            for c in convs:
                if (c.dim() != 3 or c.shape != c0.shape or
                        c.dtype != c0.dtype or c.shape[0] != N or
                        c.shape[2] != Q + 2 or c.dtype not in _DT):
                    raise ValueError("KDA RecoverSSM layers need matching "
                                     "conv state")
            self.conv_dim = c0.shape[1]
            self.conv_dtype = _DT[c0.dtype]
            self._host_conv_tables = torch.tensor(
                [[c.data_ptr() for c in convs],
                 [c.stride(0) for c in convs],
                 [c.stride(1) for c in convs],
                 [c.stride(2) for c in convs]], dtype=torch.int64)
            self.conv_tables = self._host_conv_tables.to(dev)

    def _constant_args(self) -> bytes:
        """The fields of kda_commit_args that do not change between steps
        (sizes, address tables, strides, gate parameters), built once."""
        a = _abi.KdaCommitArgs()
        a.num_layers = self.num_layers
        a.num_heads = self.H
        a.head_dim = self.D
        a.spec_query_len = self.Q
        a.null_block_id = self.null_block_id
        a.num_slots = self.N
        a.num_record_rows = self.R
        base = self.tables.data_ptr()
        L8 = self.num_layers * 8
        a.state_base_addrs = base
        a.state_block_strides = base + L8
        a.correction_base_addrs = base + 2 * L8
        a.correction_block_strides = base + 3 * L8
        a.key_gate_base_addrs = base + 4 * L8
        a.key_gate_block_strides = base + 5 * L8
        a.state_strides[:] = list(self.state_strides)
        a.correction_strides[:] = list(self.correction_strides)
        a.key_gate_strides[:] = list(self.key_gate_strides)
        a.key_gate_dtype = self.key_gate_dtype
        a.A_log = self.A_log.data_ptr()
        a.A_log_strides[:] = list(self.A_log.stride())
        a.dt_bias = self.dt_bias.data_ptr()
        a.dt_bias_strides[:] = list(self.dt_bias.stride())
        a.use_lower_bound = self.use_lower_bound.data_ptr()
        a.lower_bound = self.lower_bound.data_ptr()
        a.host_tables = self._host_tables.numpy().ctypes.data_as(
            ctypes.POINTER(ctypes.c_int64))
        return bytes(a)

    def args(self, state_indices, commit_lens, final_state_indices=None,
             record_rows=None, max_workgroups=0,
             boundary_state_indices=None,
             boundary_recovery_lens=None) -> _abi.KdaCommitArgs:
        if self._fixed is None:
            self._fixed = self._constant_args()
        a = _abi.KdaCommitArgs.from_buffer_copy(self._fixed)
        a.batch = state_indices.shape[0]
        a.max_workgroups = max_workgroups
        a.state_indices = _ptr(state_indices)
        a.commit_lens = _ptr(commit_lens)
        a.final_state_indices = _ptr(final_state_indices)
        a.record_rows = _ptr(record_rows)
        a.boundary_state_indices = _ptr(boundary_state_indices)
        a.boundary_recovery_lens = _ptr(boundary_recovery_lens)
        return a

    def check(self, state_indices, commit_lens, final_state_indices=None,
              record_rows=None) -> int:
        a = self.args(state_indices, commit_lens, final_state_indices,
                      record_rows)
        return _abi.load().kda_check_commit(ctypes.byref(a))

    def commit(self, state_indices, commit_lens, final_state_indices=None,
               record_rows=None, stream=None, max_workgroups=0,
               boundary_state_indices=None,
               boundary_recovery_lens=None) -> None:
        """Fold the first commit_lens[b] recorded positions of every request
        into its checkpoint (or final slot), for all layers, in one launch;
        with boundary slots and lengths (align mode), also store the state
        after the first boundary_recovery_lens[b] positions there.
        max_workgroups > 0 selects the persistent strided schedule."""
        a = self.args(state_indices, commit_lens, final_state_indices,
                      record_rows, max_workgroups, boundary_state_indices,
                      boundary_recovery_lens)
        rc = _abi.load().kda_recoverssm_commit(ctypes.byref(a),
                                              _stream(stream))
        if rc != _abi.KDA_OK:
            _raise(rc)

    # ---- commit plan and conv compaction -----------------------------------

    def plan_args(self, num_accepted_tokens, state_indices, query_start_loc,
                  request_indices=None, block_table=None,
                  num_computed_tokens=None, mamba_block_size=None,
                  out=None) -> tuple:
        """Arguments of kda_commit_plan and its four int32 [batch] outputs
        (allocated on the device of `state_indices` unless `out` is
        given)."""
        B = state_indices.shape[0]
        if out is None:
            out = tuple(torch.empty(B, dtype=torch.int32,
                                    device=state_indices.device)
                        for _ in range(4))
        a = _abi.KdaPlanArgs()
        a.batch = B
        a.spec_query_len = self.Q
        a.null_block_id = self.null_block_id
        a.mamba_block_size = mamba_block_size or 0
        rows = [num_accepted_tokens.shape[0]]
        if block_table is not None:
            if block_table.dim() != 2:
                raise ValueError("KDA RecoverSSM block table must be "
                                 "two-dimensional")
            if block_table.dtype != torch.int32:
                raise TypeError("the block table must be int32")
            rows.append(block_table.shape[0])
            a.block_table = block_table.data_ptr()
            a.block_table_width = block_table.shape[1]
            a.block_table_strides[:] = list(block_table.stride())
        if num_computed_tokens is not None:
            rows.append(num_computed_tokens.shape[0])
        a.num_request_rows = min(rows)
        if request_indices is not None and request_indices.shape[0] < B:
            raise ValueError("KDA RecoverSSM request mapping is too short")
        a.num_accepted_tokens = _ptr(num_accepted_tokens)
        a.request_indices = _ptr(request_indices)
        a.state_indices = _ptr(state_indices)
        a.query_start_loc = _ptr(query_start_loc)
        a.num_computed_tokens = _ptr(num_computed_tokens)
        a.commit_lens, a.final_state_indices, a.boundary_state_indices, \
            a.boundary_recovery_lens = (_ptr(t) for t in out)
        return a, out

    def plan(self, num_accepted_tokens, state_indices, query_start_loc,
             request_indices=None, block_table=None, num_computed_tokens=None,
             mamba_block_size=None, out=None, stream=None) -> tuple:
        """The commit plan (ops page `_prepare_commit_plan_kernel`): returns
        (commit_lens, final_state_indices, boundary_state_indices,
        boundary_recovery_lens), int32 [batch] on the device.  With a block
        table, num_computed_tokens and mamba_block_size (align mode) the
        final slot is the block of the next token and a completed block
        gets the boundary state."""
        a, out = self.plan_args(num_accepted_tokens, state_indices,
                                query_start_loc, request_indices, block_table,
                                num_computed_tokens, mamba_block_size, out)
        rc = _abi.load().kda_commit_plan(ctypes.byref(a), _stream(stream))
        if rc != _abi.KDA_OK:
            _raise(rc)
        return out

    def compact_args(self, state_indices, commit_lens,
                     final_state_indices=None, boundary_state_indices=None,
                     boundary_recovery_lens=None) -> _abi.KdaCompactArgs:
        if self.conv_tables is None:
            raise ValueError("this commit context has no conv states")
        a = _abi.KdaCompactArgs()
        a.num_layers = self.num_layers
        a.batch = state_indices.shape[0]
        a.spec_query_len = self.Q
        a.null_block_id = self.null_block_id
        a.num_slots = self.N
        a.conv_dim = self.conv_dim
        a.conv_dtype = self.conv_dtype
        a.conv_tables = self.conv_tables.data_ptr()
        a.host_conv_tables = self._host_conv_tables.numpy().ctypes.data_as(
            ctypes.POINTER(ctypes.c_int64))
        a.state_indices = _ptr(state_indices)
        a.commit_lens = _ptr(commit_lens)
        a.final_state_indices = _ptr(final_state_indices)
        a.boundary_state_indices = _ptr(boundary_state_indices)
        a.boundary_recovery_lens = _ptr(boundary_recovery_lens)
        return a

    def compact(self, state_indices, commit_lens, final_state_indices=None,
                boundary_state_indices=None, boundary_recovery_lens=None,
                stream=None) -> None:
        """Conv-state compaction of every layer (ops page
        `_compact_conv_state_kernel`): the three inputs before token n of
        each committing request's window go to the front of its final (and,
        in align mode, boundary) slot's conv state."""
        a = self.compact_args(state_indices, commit_lens, final_state_indices,
                              boundary_state_indices, boundary_recovery_lens)
        rc = _abi.load().kda_compact_conv_state(ctypes.byref(a),
                                               _stream(stream))
        if rc != _abi.KDA_OK:
            _raise(rc)

    def commit_step(self, num_accepted_tokens, state_indices, query_start_loc,
                    request_indices=None, block_table=None,
                    num_computed_tokens=None, mamba_block_size=None,
                    record_rows=None, stream=None, fused=True,
                    max_workgroups=0, out=None) -> tuple:
        """The ops page's `KDARecoverSSMCommitContext.commit`: plan, conv
        compaction (when the context has conv states), then the state
        commit of every layer.  Returns the plan's four arrays.  fused:
        all three in one launch (kda_recoverssm_commit_step); otherwise
        three launches."""
        align = block_table is not None
        if fused:
            pa, out = self.plan_args(num_accepted_tokens, state_indices,
                                     query_start_loc, request_indices,
                                     block_table, num_computed_tokens,
                                     mamba_block_size, out)
            lens, final, bnd, blens = out
            bnd_a, blens_a = (bnd, blens) if align else (None, None)
            ca = self.args(state_indices, lens, final, record_rows,
                           max_workgroups, bnd_a, blens_a)
            xa = None if self.conv_tables is None else self.compact_args(
                state_indices, lens, final, bnd_a, blens_a)
            rc = _abi.load().kda_recoverssm_commit_step(
                ctypes.byref(ca), ctypes.byref(pa),
                None if xa is None else ctypes.byref(xa), _stream(stream))
            if rc != _abi.KDA_OK:
                _raise(rc)
            return out
        lens, final, bnd, blens = self.plan(
            num_accepted_tokens, state_indices, query_start_loc,
            request_indices, block_table, num_computed_tokens,
            mamba_block_size, out=out, stream=stream)
        if self.conv_tables is not None:
            self.compact(state_indices, lens, final,
                         bnd if align else None, blens if align else None,
                         stream=stream)
        self.commit(state_indices, lens, final, record_rows, stream=stream,
                    max_workgroups=max_workgroups,
                    boundary_state_indices=bnd if align else None,
                    boundary_recovery_lens=blens if align else None)
        return lens, final, bnd, blens
