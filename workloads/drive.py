"""Runs a seeded Workload through the HIP library's Python binding.

Argument plumbing only (which tensor goes to which parameter); used by the
GPU tests and bench.py.  Not imported by `workloads/__init__` so that the
oracle tests never load the HIP library.
"""
from __future__ import annotations

from typing import Optional

import torch

import linear_attention_speculative_amd as kda

from .gen import Workload


def counter(wl: Workload, device="cuda") -> torch.Tensor:
    """A zeroed work-counter array for any verify schedule of `wl`: the
    ticket counter plus one arrival counter per (request, head)."""
    return torch.zeros(1 + wl.B * wl.H, dtype=torch.int32, device=device)


def verify_kwargs(wl: Workload, layer: int, counter: torch.Tensor,
                  max_workgroups: int = 0, items_per_ticket: int = 0,
                  schedule: int = 0, pending_lens=None,
                  v_tiles: int = 0) -> dict:
    L = wl.layers[layer]
    return dict(
        mixed_qkv=L.mixed_qkv, raw_gate=L.raw_gate, raw_beta=L.raw_beta,
        A_log=L.A_log, dt_bias=L.dt_bias,
        lower_bound=L.lower_bound if L.use_lower_bound else None,
        state=L.state, correction=L.correction, key_gate=L.key_gate,
        out=L.out, conv_state=L.conv_state, conv_weight=L.conv_weight,
        query_start_loc=wl.query_start_loc, state_indices=wl.state_indices,
        num_accepted_tokens=wl.num_accepted_tokens,
        spec_query_len=wl.Q, conv_dim_first=wl.conv_dim_first,
        work_counter=counter, record_rows=wl.record_rows,
        null_block_id=wl.null_block_id, max_workgroups=max_workgroups,
        items_per_ticket=items_per_ticket, schedule=schedule,
        pending_lens=pending_lens, v_tiles=v_tiles)


def verify(wl: Workload, layer: int, counter: torch.Tensor,
           max_workgroups: int = 0, items_per_ticket: int = 0,
           stream=None, schedule: int = 0, pending_lens=None,
           v_tiles: int = 0) -> None:
    kda.conv_update_verify(stream=stream,
                           **verify_kwargs(wl, layer, counter,
                                           max_workgroups, items_per_ticket,
                                           schedule, pending_lens, v_tiles))


def verify_qkv_kwargs(wl: Workload, layer: int, mixed_qkv: torch.Tensor,
                      counter=None, **kw) -> dict:
    """Arguments of the unfused verify: `mixed_qkv` holds the convolved
    q | k | v of every token; the conv state, taps and accepted counts are
    left out."""
    d = verify_kwargs(wl, layer, counter, **kw)
    for k in ("conv_state", "conv_weight", "num_accepted_tokens",
              "conv_dim_first"):
        del d[k]
    d["mixed_qkv"] = mixed_qkv
    return d


def verify_qkv(wl: Workload, layer: int, counter=None, mixed_qkv=None,
               stream=None, **kw) -> None:
    """The unfused verify of `layer`; `mixed_qkv` (default: the layer's
    activation tensor) is taken as the convolved q | k | v."""
    L = wl.layers[layer]
    kda.verify_qkv(stream=stream, **verify_qkv_kwargs(
        wl, layer, L.mixed_qkv if mixed_qkv is None else mixed_qkv,
        counter, **kw))


def commit_context(wl: Workload, layers: Optional[list] = None,
                   conv: bool = False) -> kda.CommitContext:
    """The layers' commit context; `conv` adds their conv states (for the
    compaction)."""
    idx = range(len(wl.layers)) if layers is None else layers
    return kda.CommitContext(
        [dict(state=wl.layers[i].state, correction=wl.layers[i].correction,
              key_gate=wl.layers[i].key_gate, A_log=wl.layers[i].A_log,
              dt_bias=wl.layers[i].dt_bias,
              lower_bound=wl.layers[i].lower_bound
              if wl.layers[i].use_lower_bound else None,
              **({"conv_state": wl.conv_state_dim_first(i)} if conv else {}))
         for i in idx],
        spec_query_len=wl.Q, null_block_id=wl.null_block_id)


def commit(wl: Workload, ctx: kda.CommitContext,
           commit_lens: Optional[torch.Tensor] = None,
           final_state_indices: Optional[torch.Tensor] = None,
           stream=None) -> None:
    ctx.commit(wl.state_indices,
               wl.commit_lens if commit_lens is None else commit_lens,
               final_state_indices=final_state_indices,
               record_rows=wl.record_rows, stream=stream)
