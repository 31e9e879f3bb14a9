"""Selection of a request sample from a Workload, copied to the host and
remapped to a compact slot pool, as keyword arguments for the CPU oracle.

Index bookkeeping only (which rows and slots to copy, and where they land);
no arithmetic of the method.  Take a snapshot before the launch that
modifies the tensors.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a tensor's values to float64 on the host."""
    return t.detach().to("cpu").to(torch.float64).numpy()


@dataclass
class Sample:
    """Oracle inputs of a request sample, remapped to a compact pool."""
    reqs: list           # original request indices
    valid: list          # per sampled request: live (non-null) slot?
    slots: np.ndarray    # original slots of the sample
    rows: np.ndarray     # original record rows (or -1)
    tok: list            # per sampled request: original token rows
    inputs: dict         # oracle keyword arguments (compact)
    new_slot: np.ndarray  # compact slot per sampled request
    new_row: np.ndarray   # compact record row per sampled request


def snapshot(wl, layer: int, reqs=None) -> Sample:
    """Copy to the host everything the oracle needs for `reqs` (default: all
    requests).  Call before the launch that modifies the tensors."""
    L = wl.layers[layer]
    B, N, Q = wl.B, wl.N, wl.Q
    reqs = list(range(B)) if reqs is None else list(reqs)
    qsl = wl.query_start_loc.cpu().numpy().astype(np.int64)
    slots_all = wl.state_indices.cpu().numpy().astype(np.int64)
    acc_all = wl.num_accepted_tokens.cpu().numpy().astype(np.int64)
    rows_all = None if wl.record_rows is None else \
        wl.record_rows.cpu().numpy().astype(np.int64)
    R = L.correction.shape[0]

    valid, tok, orig_slots, orig_rows = [], [], [], []
    for b in reqs:
        s = int(slots_all[b])
        ok = wl.null_block_id < s < N
        valid.append(ok)
        tok.append(list(range(int(qsl[b]), int(qsl[b + 1]))))
        orig_slots.append(s)
        r = s if rows_all is None else int(rows_all[b])
        orig_rows.append(r if (ok and 0 <= r < R) else -1)
    live = [i for i, ok in enumerate(valid) if ok]
    live_slots = [orig_slots[i] for i in live]
    new_slot = np.zeros(len(reqs), dtype=np.int64)
    for j, i in enumerate(live):
        new_slot[i] = j + 1
    n_pool = len(live) + 1
    # A slot past the pool stays past the (compact) pool.
    for i, s in enumerate(orig_slots):
        if s >= N:
            new_slot[i] = n_pool + 5
    row_src = [orig_rows[i] for i in live if orig_rows[i] >= 0]
    new_row = np.full(len(reqs), -1, dtype=np.int64)
    if rows_all is None:
        for i in live:
            if orig_rows[i] >= 0:
                new_row[i] = new_slot[i]
        rec_index = [0] + live_slots   # compact row j <- original row
    else:
        k = 0
        for i in live:
            if orig_rows[i] >= 0:
                new_row[i] = k
                k += 1
        rec_index = row_src

    dev = L.state.device
    idx = torch.tensor([0] + live_slots, device=dev)
    ridx = torch.tensor(rec_index if rec_index else [0], device=dev)
    tok_all = [t for ts in tok for t in ts]
    tidx = torch.tensor(tok_all, device=dev, dtype=torch.long)
    state = f64(L.state.index_select(0, idx))
    state[0] = 0.0
    conv = f64(wl.conv_state_dim_first(layer).index_select(0, idx))
    corr = f64(L.correction.index_select(0, ridx))
    kg = f64(L.key_gate.index_select(0, ridx))
    if not rec_index:
        corr, kg = corr[:0], kg[:0]
    # (no index_select at all when there are no tokens: the activation
    # tensors may then have no rows)
    take = (lambda t: f64(t.index_select(0, tidx)) if tok_all else
            np.zeros((0,) + tuple(t.shape[1:])))
    new_qsl = np.concatenate([[0], np.cumsum([len(ts) for ts in tok])])
    inputs = dict(
        mixed_qkv=take(L.mixed_qkv), raw_gate=take(L.raw_gate),
        raw_beta=take(L.raw_beta), A_log=f64(L.A_log),
        dt_bias=f64(L.dt_bias), state=state, correction=corr,
        key_gate=kg, out=np.zeros((len(tok_all), wl.H * wl.D)),
        conv_state=conv, conv_weight=f64(L.conv_weight),
        query_start_loc=new_qsl, state_indices=new_slot,
        num_accepted_tokens=acc_all[reqs], spec_query_len=Q,
        null_block_id=0, use_lower_bound=L.use_lower_bound,
        lower_bound=L.lower_bound,
        record_rows=None if rows_all is None else new_row,
        key_gate_dtype=wl.kg_dtype)
    return Sample(reqs=reqs, valid=valid, slots=np.array(orig_slots),
                  rows=np.array(orig_rows), tok=tok, inputs=inputs,
                  new_slot=new_slot, new_row=new_row)
