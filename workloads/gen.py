"""Seeded synthetic inputs shaped like the decode batches of a speculative KDA
layer (vLLM Kimi-K3 pages: the kernels page's `CuteRecoverSSMVerify.__call__`
argument list, the ops page's `KDARecoverSSMCommitContext.create` KV-cache
page of conv state, recurrent state, correction and key/gate records).

Only random draws and memory layout live here.  Every per-slot tensor is a
strided view into a per-slot "page" (one page per state slot, as a serving KV
cache lays them out), so slot strides differ from the tensors' own sizes, and
the page padding is filled with random bytes so that stray writes show up.

Value recipe (all seeded):
  mixed_qkv, raw_gate, raw_beta ~ N(0, 1) in the activation dtype (bf16 by
  round-to-nearest-even from fp32 draws);  A_log = log U(1, 16);
  dt_bias ~ N(0, 0.1);  conv weight ~ N(0, 0.5);  recurrent state ~ N(0, 0.02)
  in fp32;  conv state ~ N(0, 1) (past raw inputs);  records pre-filled with
  N(0, 1) noise.  Non-null slots are drawn without replacement from
  1 .. N-1; slot 0 is the null block.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

NULL_BLOCK_ID = 0
CONV_WIDTH = 4

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_ELEM = {"f32": 4, "bf16": 2}

# Per-config structure.  Sizes follow the decode batches the pages describe;
# `overrides` in make_workload shrinks them for CPU-sized parity cases.
CONFIGS = {
    # Two requests, two heads, head dim 16, three draft tokens, all fp32.
    "tiny": dict(B=2, H=2, D=16, Q=3, N=4, act="f32", weight="f32",
                 qlen="full", null_frac=0.0, conv_dim_first=True,
                 gates=[None], commit="tiny", record_rows=False),
    # One request at the full head shape; token-first conv state.
    "single": dict(B=1, H=32, D=128, Q=4, N=8, act="bf16", weight="bf16",
                   qlen="full", null_frac=0.0, conv_dim_first=False,
                   gates=[None], commit="const2", record_rows=False),
    # 64 requests with ragged query lengths and 10% null slots.
    "ragged": dict(B=64, H=32, D=128, Q=4, N=128, act="bf16", weight="bf16",
                   qlen="uniform", null_frac=0.1, conv_dim_first=True,
                   gates=[-5.0], commit="qlen", record_rows=False),
    # 256 requests, eight draft tokens, 24 layers folded by one commit.
    "large": dict(B=256, H=32, D=128, Q=8, N=512, act="bf16", weight="bf16",
                  qlen="full", null_frac=0.0, conv_dim_first=False,
                  gates=[None] * 24, commit="uniform0", record_rows=False),
    # 1024 requests, deferred commit of pending tokens, records by request
    # slot, a softplus layer and a lower-bound layer.
    "deferred": dict(B=1024, H=32, D=128, Q=4, N=2048, act="bf16",
                     weight="bf16", qlen="full", null_frac=0.0,
                     conv_dim_first=True, gates=[None, -5.0],
                     commit="pending", record_rows=True),
    # The throughput workload: 256 requests, four draft tokens, one layer.
    "headline": dict(B=256, H=32, D=128, Q=4, N=512, act="bf16",
                     weight="bf16", qlen="full", null_frac=0.0,
                     conv_dim_first=True, gates=[-5.0], commit="uniform1",
                     record_rows=False),
}


def _align(n: int, a: int = 256) -> int:
    return (n + a - 1) // a * a


@dataclass
class LayerTensors:
    """One KDA layer's cache page views, parameters and activations."""
    page: torch.Tensor                 # uint8 [N, page_bytes]
    conv_state: torch.Tensor           # as stored: [N,3HD,Lc] or [N,Lc,3HD]
    state: torch.Tensor                # f32 [N, H, D, D]
    correction: torch.Tensor           # f32 [R, H, Q, D]
    key_gate: torch.Tensor             # kg dtype [R, H, Q, 2D]
    record_page: Optional[torch.Tensor]  # uint8 [R, bytes] when not in page
    A_log: torch.Tensor                # f32 [H]
    dt_bias: torch.Tensor              # f32 [H, D]
    conv_weight: torch.Tensor          # weight dtype [3HD, W]
    use_lower_bound: bool
    lower_bound: float
    mixed_qkv: torch.Tensor            # act [T, 3HD] (possibly row-padded)
    raw_gate: torch.Tensor             # act [T, HD]
    raw_beta: torch.Tensor             # act [T, H]
    out: torch.Tensor                  # out dtype [T, HD]


@dataclass
class Workload:
    name: str
    B: int
    H: int
    D: int
    Q: int
    W: int
    N: int
    R: int
    T: int
    act: str
    weight: str
    out_dtype: str
    kg_dtype: str
    conv_dim_first: bool
    null_block_id: int
    query_start_loc: torch.Tensor      # int32 [B+1]
    state_indices: torch.Tensor        # int32 [B]
    num_accepted_tokens: torch.Tensor  # int32 [B]
    record_rows: Optional[torch.Tensor]  # int32 [B] or None
    commit_lens: torch.Tensor          # int32 [B]
    layers: list = field(default_factory=list)
    meta: dict = field(default_factory=dict)

    @property
    def Lc(self) -> int:
        return self.Q + self.W - 2

    def conv_state_dim_first(self, layer: int) -> torch.Tensor:
        """The conv state viewed as [N, 3HD, Lc] whatever the stored layout."""
        cs = self.layers[layer].conv_state
        return cs if self.conv_dim_first else cs.transpose(-1, -2)


def _randn(shape, std, gen, device):
    return torch.randn(shape, generator=gen, device=device,
                       dtype=torch.float32) * std


def _fill_(view: torch.Tensor, values_f32: torch.Tensor) -> None:
    view.copy_(values_f32.to(view.dtype))


def _draw_metadata(cfg: dict, B: int, Q: int, N: int, seed: int):
    rng = np.random.RandomState(seed)
    if cfg["qlen"] == "full":
        qlen = np.full(B, Q, dtype=np.int64)
    else:
        qlen = rng.randint(1, Q + 1, size=B).astype(np.int64)
    n_null = int(round(cfg["null_frac"] * B))
    null_pos = rng.choice(B, size=n_null, replace=False) if n_null else []
    if N - 1 < B - n_null:
        raise ValueError("state pool too small for the batch")
    is_null = np.zeros(B, dtype=bool)
    is_null[list(null_pos)] = True
    slots = np.full(B, NULL_BLOCK_ID, dtype=np.int64)
    slots[~is_null] = rng.choice(np.arange(1, N), size=int((~is_null).sum()),
                                 replace=False)
    kind = cfg["commit"]
    if kind == "tiny":
        commit = np.array([1, 3][:B] + [1] * max(0, B - 2), dtype=np.int64)
    elif kind == "const2":
        commit = np.full(B, min(2, Q), dtype=np.int64)
    elif kind == "qlen":
        commit = qlen.copy()
    elif kind == "uniform0":
        commit = rng.randint(0, Q + 1, size=B).astype(np.int64)
    elif kind == "uniform1":
        commit = rng.randint(1, Q + 1, size=B).astype(np.int64)
    elif kind == "pending":
        commit = rng.randint(0, Q + 1, size=B).astype(np.int64)
    else:
        raise ValueError(kind)
    if kind == "pending":
        accepted = np.maximum(commit, 1)
    else:
        accepted = rng.randint(1, Q + 1, size=B).astype(np.int64)
    record_rows = rng.permutation(B).astype(np.int64) \
        if cfg["record_rows"] else None
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int64)
    return qsl, slots, accepted, commit, record_rows


def make_workload(name: str, device="cpu", *, seed: Optional[int] = None,
                  out_dtype: str = "f32", kg_dtype: str = "f32",
                  conv_dim_first: Optional[bool] = None,
                  act_row_pad: int = 0, **overrides) -> Workload:
    """Build a seeded workload.

    `overrides` may replace B, H, D, Q, N, act, weight, qlen, null_frac,
    gates (list of per-layer lower bounds, None = softplus), commit kind and
    record_rows.  `out_dtype` / `kg_dtype` are "f32" or "act".
    `act_row_pad` > 0 makes the activations views into wider rows.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    if conv_dim_first is not None:
        cfg["conv_dim_first"] = conv_dim_first
    if seed is None:
        seed = sorted(CONFIGS).index(name) + 1
    B, H, D, Q, N = cfg["B"], cfg["H"], cfg["D"], cfg["Q"], cfg["N"]
    W = CONV_WIDTH
    Lc = Q + W - 2
    C = 3 * H * D
    act, weight = cfg["act"], cfg["weight"]
    out_dt = act if out_dtype == "act" else out_dtype
    kg_dt = act if kg_dtype == "act" else kg_dtype
    device = torch.device(device)
    dim_first = bool(cfg["conv_dim_first"])

    qsl, slots, accepted, commit, record_rows = _draw_metadata(cfg, B, Q, N,
                                                               seed)
    T = int(qsl[-1])
    R = B if record_rows is not None else N

    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 7919 + 17)

    def i32(a):
        return torch.as_tensor(np.asarray(a), dtype=torch.int32).to(device)

    wl = Workload(
        name=name, B=B, H=H, D=D, Q=Q, W=W, N=N, R=R, T=T, act=act,
        weight=weight, out_dtype=out_dt, kg_dtype=kg_dt,
        conv_dim_first=dim_first, null_block_id=NULL_BLOCK_ID,
        query_start_loc=i32(qsl), state_indices=i32(slots),
        num_accepted_tokens=i32(accepted),
        record_rows=None if record_rows is None else i32(record_rows),
        commit_lens=i32(commit), meta=dict(seed=seed, cfg=cfg))

    conv_bytes = _align(C * Lc * _ELEM[act])
    state_bytes = _align(H * D * D * 4)
    corr_bytes = _align(H * Q * D * 4)
    kg_bytes = _align(H * Q * 2 * D * _ELEM[kg_dt])
    rec_in_page = record_rows is None
    page_bytes = conv_bytes + state_bytes + (corr_bytes + kg_bytes
                                             if rec_in_page else 0) + 256
    tdt = _TORCH_DTYPE
    # Byte ranges the views cover inside a page (the rest is padding).
    used = {"conv": (0, C * Lc * _ELEM[act]),
            "state": (conv_bytes, H * D * D * 4)}
    rec_off = conv_bytes + state_bytes if rec_in_page else 0
    used["correction"] = (rec_off, H * Q * D * 4)
    used["key_gate"] = (rec_off + corr_bytes, H * Q * 2 * D * _ELEM[kg_dt])
    wl.meta["page_views"] = used
    wl.meta["records_in_page"] = rec_in_page

    for layer_idx, lb in enumerate(cfg["gates"]):
        page = torch.randint(0, 256, (N, page_bytes), generator=gen,
                             device=device, dtype=torch.uint8)

        def carve(buf, off, nbytes, dt, shape):
            raw = buf[:, off:off + nbytes]
            v = raw.view(tdt[dt])
            return v[:, :int(np.prod(shape))].unflatten(1, shape)

        conv_shape = (C, Lc) if dim_first else (Lc, C)
        conv_state = carve(page, 0, conv_bytes, act, conv_shape)
        state = carve(page, conv_bytes, state_bytes, "f32", (H, D, D))
        if rec_in_page:
            base = conv_bytes + state_bytes
            correction = carve(page, base, corr_bytes, "f32", (H, Q, D))
            key_gate = carve(page, base + corr_bytes, kg_bytes, kg_dt,
                             (H, Q, 2 * D))
            record_page = None
        else:
            record_page = torch.randint(
                0, 256, (R, corr_bytes + kg_bytes + 256), generator=gen,
                device=device, dtype=torch.uint8)
            correction = carve(record_page, 0, corr_bytes, "f32", (H, Q, D))
            key_gate = carve(record_page, corr_bytes, kg_bytes, kg_dt,
                             (H, Q, 2 * D))

        _fill_(conv_state, _randn(conv_state.shape, 1.0, gen, device))
        # The state pool is filled one slot group at a time to bound the
        # temporary fp32 buffer.
        step = max(1, (1 << 28) // (H * D * D * 4))
        for s0 in range(0, N, step):
            sl = state[s0:s0 + step]
            _fill_(sl, _randn(sl.shape, 0.02, gen, device))
        _fill_(correction, _randn(correction.shape, 1.0, gen, device))
        _fill_(key_gate, _randn(key_gate.shape, 1.0, gen, device))

        u = torch.rand((H,), generator=gen, device=device,
                       dtype=torch.float64)
        A_log = torch.log(1.0 + 15.0 * u).to(torch.float32)
        dt_bias = _randn((H, D), 0.1, gen, device)
        conv_weight = _randn((C, W), 0.5, gen, device).to(tdt[weight])

        def act_tensor(cols, std=1.0):
            full = _randn((T, cols + act_row_pad), std, gen, device)
            return full.to(tdt[act])[:, :cols]

        mixed_qkv = act_tensor(C)
        raw_gate = act_tensor(H * D)
        raw_beta = act_tensor(H)
        out = torch.full((T, H * D), float("nan"), device=device,
                         dtype=tdt[out_dt])

        wl.layers.append(LayerTensors(
            page=page, conv_state=conv_state, state=state,
            correction=correction, key_gate=key_gate,
            record_page=record_page, A_log=A_log, dt_bias=dt_bias,
            conv_weight=conv_weight, use_lower_bound=lb is not None,
            lower_bound=0.0 if lb is None else float(lb),
            mixed_qkv=mixed_qkv, raw_gate=raw_gate, raw_beta=raw_beta,
            out=out))
    return wl


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a tensor's values to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def step_activations(T: int, H: int, D: int, act: str, seed: int,
                     device="cpu") -> dict:
    """Fresh activations of one decode step: mixed_qkv [T, 3HD], raw_gate
    [T, HD] and raw_beta [T, H] ~ N(0, 1) in the activation dtype."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 104729 + 3)
    dt = _TORCH_DTYPE[act]
    return dict(
        mixed_qkv=_randn((T, 3 * H * D), 1.0, gen, device).to(dt),
        raw_gate=_randn((T, H * D), 1.0, gen, device).to(dt),
        raw_beta=_randn((T, H), 1.0, gen, device).to(dt))


def block_tables(B: int, width: int, N: int, seed: int,
                 null_block_id: int = 0) -> np.ndarray:
    """Every request's state blocks: int32 [B, width] of distinct live slots
    drawn without replacement from (null_block_id, N)."""
    rng = np.random.default_rng(seed)
    live = np.arange(null_block_id + 1, N)
    if live.size < B * width:
        raise ValueError("the pool is too small for the block tables")
    return rng.permutation(live)[:B * width].reshape(B, width) \
        .astype(np.int32)


def running_block_tables(state_indices: np.ndarray, N: int, block_size: int,
                         seed: int, null_block_id: int = 0):
    """Two-block tables for a decode batch under prefix caching: column 0
    is the request's current (running) state block, its source slot;
    column 1 a free slot for the block after it (null once the free slots
    run out).  Also draws the tokens already in the running block,
    uniform in [0, block_size).  Returns (table int32 [B, 2], computed
    int32 [B])."""
    rng = np.random.default_rng(seed)
    slots = np.asarray(state_indices)
    B = slots.shape[0]
    used = set(slots.tolist())
    free = [s for s in range(null_block_id + 1, N) if s not in used]
    table = np.full((B, 2), null_block_id, dtype=np.int32)
    table[:, 0] = slots
    nfree = min(len(free), B)
    table[:nfree, 1] = free[:nfree]
    computed = rng.integers(0, block_size, size=B).astype(np.int32)
    return table, computed
