"""Helpers of the GPU parity tests: capture the oracle inputs of a sample of
requests before a launch, run the fp64 oracle on a compact copy of them, and
compare what the HIP path wrote.

Comparison rule (one number per tensor): err = max|gpu - ref| / max|ref|
over the written region, at most 2e-3 for bf16 activations and 1e-4 for
fp32 inputs (a bf16 `out` adds its own rounding, 2^-8).  Copies (conv-state roll, raw-gate record half), null outputs
and every byte that must not change are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads.sample import Sample, f64, snapshot  # noqa: F401

TOL = {"f32": 1e-4, "bf16": 2e-3}


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    diff = float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)))
    return diff / scale if scale > 0 else diff


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns (for bitwise comparisons, NaN-safe)."""
    t = t.detach().contiguous().to("cpu")
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy()


def run_oracle_verify(sample: Sample, inputs: dict = None) -> dict:
    return oracle.conv_update_verify(**(inputs or sample.inputs))


def run_oracle_verify_qkv(sample: Sample) -> dict:
    """The oracle's unfused verify on the sample, whose `mixed_qkv` is taken
    as the convolved q | k | v."""
    return oracle.verify_qkv(**{
        k: v for k, v in sample.inputs.items()
        if k not in ("conv_state", "conv_weight", "num_accepted_tokens")})


def check_verify(wl, layer: int, sample: Sample, ref: dict,
                 kg_k_tol: float = None, rec_before=None,
                 extra_tol: float = 0.0) -> dict:
    """Compare the GPU tensors of `layer` (after the verify launch) with the
    oracle results `ref` for the sample.  Returns the measured errors.

    Record positions the launch does not write must keep their bytes: by
    default the oracle's inputs hold them; `rec_before` = (correction,
    key_gate) GPU tensors cloned before the launch is used instead when an
    earlier launch wrote them.  `extra_tol` widens every float bound (one
    bf16 step when the key record is stored in the activation dtype)."""
    L = wl.layers[layer]
    tol = TOL[wl.act] + extra_tol
    errs = {}
    dev = L.state.device
    tok_all = [t for ts in sample.tok for t in ts]
    Q, D = wl.Q, wl.D

    # outputs
    if tok_all:
        out = L.out.index_select(0, torch.tensor(tok_all, device=dev))
        out_gpu = f64(out)
        out_bits = bits(out)
        m = ref["out_written"]
        live_rows, null_rows = [], []
        k = 0
        for i, ts in enumerate(sample.tok):
            q = min(len(ts), Q)
            rows = list(range(k, k + q))
            (live_rows if sample.valid[i] else null_rows).extend(rows)
            k += len(ts)
        if live_rows:
            lr = np.array(live_rows)
            assert m[lr].all()
            errs["out"] = rel_err(out_gpu[lr], ref["out"][lr])
            # A bf16 `out` adds its own rounding: up to half a bf16 ulp of
            # the largest output, i.e. 2^-8 of its leading power of two.
            tol_out = tol + (2.0 ** -8 if out.dtype == torch.bfloat16 else 0)
            assert errs["out"] <= tol_out, ("out", errs["out"])
        if null_rows:
            nb = out_bits[np.array(null_rows)]
            assert np.all(nb == 0), "null outputs must be +0.0"

    # conv state roll: bitwise (the unfused verify has none)
    live = [i for i, ok in enumerate(sample.valid) if ok]
    if live and "conv_state" in ref:
        oslots = torch.tensor([int(sample.slots[i]) for i in live], device=dev)
        conv_gpu = f64(wl.conv_state_dim_first(layer).index_select(0, oslots))
        conv_ref = ref["conv_state"][[int(sample.new_slot[i]) for i in live]]
        assert np.array_equal(conv_gpu, conv_ref), "conv state roll mismatch"

    # records
    rec = [(i, int(sample.rows[i]), int(sample.new_row[i])) for i in live
           if sample.rows[i] >= 0]
    if rec:
        ridx = torch.tensor([r for _, r, _ in rec], device=dev)
        corr_gpu = f64(L.correction.index_select(0, ridx))
        kg_t = L.key_gate.index_select(0, ridx)
        kg_gpu = f64(kg_t)
        nr = [n for _, _, n in rec]
        corr_ref = ref["correction"][nr]
        kg_ref = ref["key_gate"][nr]
        if rec_before is not None:
            kept_c = f64(rec_before[0].index_select(0, ridx))
            kept_k = f64(rec_before[1].index_select(0, ridx))
        else:
            kept_c, kept_k = corr_ref, kg_ref
        w = ref["rec_written"][nr]                      # [n, H, Q]
        wc = np.broadcast_to(w[..., None], corr_ref.shape)
        errs["correction"] = rel_err(corr_gpu[wc], corr_ref[wc])
        assert errs["correction"] <= tol, ("correction", errs["correction"])
        # unwritten positions keep their bytes
        assert np.array_equal(corr_gpu[~wc], kept_c[~wc])
        wk = np.broadcast_to(w[..., None], kg_ref[..., :D].shape)
        kt = kg_k_tol if kg_k_tol is not None else tol
        errs["key"] = rel_err(kg_gpu[..., :D][wk], kg_ref[..., :D][wk])
        assert errs["key"] <= kt, ("key record", errs["key"])
        assert np.array_equal(kg_gpu[..., D:][wk], kg_ref[..., D:][wk]), \
            "raw gate record half must be an exact copy"
        assert np.array_equal(kg_gpu[~w], kept_k[~w])
    return errs


def commit_layer_inputs(sample: Sample, ref: dict, L) -> dict:
    """Oracle commit inputs of one layer: the checkpoint the sample was
    taken from and the records the oracle's verify produced."""
    return dict(state=sample.inputs["state"], correction=ref["correction"],
                key_gate=ref["key_gate"], A_log=sample.inputs["A_log"],
                dt_bias=sample.inputs["dt_bias"],
                use_lower_bound=L.use_lower_bound,
                lower_bound=L.lower_bound)


def check_commit(wl, layer: int, sample: Sample, new_state: np.ndarray,
                 written: np.ndarray, final_slots=None,
                 extra_tol: float = 0.0) -> float:
    """Compare the GPU checkpoint of `layer` after the commit with the
    oracle's committed states of the sample (compact pool).  `extra_tol`
    widens the bound (one bf16 step for a key record stored in the
    activation dtype: the two sides may round a key element to neighbouring
    bf16 values)."""
    L = wl.layers[layer]
    dev = L.state.device
    idx, cidx = [], []
    for i, ok in enumerate(sample.valid):
        ns = int(sample.new_slot[i])
        if ok and written[ns].any():
            dst = int(sample.slots[i]) if final_slots is None \
                else int(final_slots[sample.reqs[i]])
            idx.append(dst)
            cidx.append(ns)
    if not idx:
        return 0.0
    gpu = f64(L.state.index_select(0, torch.tensor(idx, device=dev)))
    err = rel_err(gpu, new_state[cidx])
    assert err <= TOL[wl.act] + extra_tol, ("committed state", err)
    return err


def kg_extra_tol(wl) -> float:
    """Widening of the float bounds downstream of an activation-dtype key
    record: GPU (fp32 k, then RNE) and oracle (fp64 k, then RNE) may round a
    key element to neighbouring bf16 values, one bf16 step (2^-8 of the
    element) apart."""
    return 2.0 ** -8 if wl.kg_dtype == "bf16" else 0.0


def full_inputs(wl, layer: int) -> dict:
    """Oracle keyword arguments for every request of `layer` over the whole
    (uncompacted) pool, copied from the seeded tensors as they are now: take
    it before any launch writes them, so that no value the HIP path produced
    becomes an oracle input."""
    L = wl.layers[layer]
    return dict(
        mixed_qkv=f64(L.mixed_qkv), raw_gate=f64(L.raw_gate),
        raw_beta=f64(L.raw_beta), A_log=f64(L.A_log), dt_bias=f64(L.dt_bias),
        state=f64(L.state), correction=f64(L.correction),
        key_gate=f64(L.key_gate), out=np.zeros((wl.T, wl.H * wl.D)),
        conv_state=f64(wl.conv_state_dim_first(layer)),
        conv_weight=f64(L.conv_weight),
        query_start_loc=wl.query_start_loc.cpu().numpy().astype(np.int64),
        state_indices=wl.state_indices.cpu().numpy().astype(np.int64),
        num_accepted_tokens=wl.num_accepted_tokens.cpu().numpy()
        .astype(np.int64),
        spec_query_len=wl.Q, null_block_id=wl.null_block_id,
        use_lower_bound=L.use_lower_bound, lower_bound=L.lower_bound,
        record_rows=None if wl.record_rows is None
        else wl.record_rows.cpu().numpy().astype(np.int64),
        key_gate_dtype=wl.kg_dtype)
