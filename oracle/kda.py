"""fp64 reference for the KDA RecoverSSM verify (with the fused short
convolution) and the multi-layer commit.  TEST INFRASTRUCTURE ONLY (see the
package docstring): the product path never imports this module.

Everything is computed in numpy float64 from the exact widenings of the
inputs.  Values that the GPU stores in a narrower type and that a later
stage reads back (records, committed states) are rounded to that storage type
with round-to-nearest-even, as the storage itself would do.

Readings taken where the pages are silent:
  * The null block id is an argument; a slot <= it, or past the pool, is null.
  * The convolution history sits at offset (accepted - 1) of a conv state of
    length Q + W - 2; the roll writes the W - 2 newest history entries
    followed by the q new raw inputs at the front, leaving the tail as is.
  * Conv taps: weight[:, W-1] multiplies the newest input; no bias; SiLU.
  * Records go to `record_rows[b]` when given, else to the request's state
    slot; a negative or out-of-range row means "write no records" (verify)
    and "skip" (commit).
  * q_b is clamped to [0, Q], accepted to [1, Q], commit length to [0, Q];
    token rows outside [0, T) are never touched; negative slots are null.
"""
from __future__ import annotations

import numpy as np

# The 1e-6 sits inside the square root of both normalisations (ops page,
# `_kda_recurrent_step` for keys, `_kda_recoverssm_verify_kernel` for
# queries); softplus switches to the identity above 20 (ops page `_kda_gate`).
EPS = 1e-6
SOFTPLUS_THRESHOLD = 20.0


def sigmoid(x):
    """Logistic function 1 / (1 + e^-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(y):
    """SiLU activation y * sigmoid(y) applied after the short convolution
    (state page, `deferred_recoverssm_verify`: the conv update runs with the
    silu activation)."""
    return y * sigmoid(y)


def kda_gate(raw_g, dt_bias, A, use_lower_bound, lower_bound):
    """Per-channel log-decay g of one position (ops page, `_kda_gate`).

    x = raw_g + dt_bias.  Bounded form: g = lower_bound * sigmoid(A x).
    Softplus form: g = -A * softplus(x) with softplus(x) = x for x > 20 and
    ln(1 + e^x) otherwise.  A = exp(A_log[h]) is passed in.
    """
    x = np.asarray(raw_g, dtype=np.float64) + np.asarray(dt_bias,
                                                        dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    if use_lower_bound:
        return lower_bound * sigmoid(A * x)
    small = np.minimum(x, SOFTPLUS_THRESHOLD)
    sp = np.where(x > SOFTPLUS_THRESHOLD, x, np.log1p(np.exp(small)))
    return -A * sp


def l2_normalize(x):
    """x / sqrt(sum x^2 + 1e-6) along the last axis (ops page,
    `_kda_recurrent_step`)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def normalize_query(q):
    """Query scaling of the verify (ops page, `_kda_recoverssm_verify_kernel`):
    L2-normalise as the keys, then multiply by K^-1/2."""
    q = np.asarray(q, dtype=np.float64)
    return l2_normalize(q) * (q.shape[-1] ** -0.5)


def delta_step(S, k, v, g, raw_beta):
    """One gated delta-rule step (ops page, `_kda_recurrent_step`).

    S [..., V, K] is decayed along K by exp(g), the correction is
    c = sigmoid(raw_beta) * (v - S_decayed k_hat), and the state becomes
    S_decayed + c k_hat^T.  Returns (new S, c).
    """
    khat = l2_normalize(k)
    S = np.asarray(S, dtype=np.float64) * np.exp(g)[..., None, :]
    u = np.einsum("...vk,...k->...v", S, khat)
    c = sigmoid(raw_beta)[..., None] * (np.asarray(v, np.float64) - u)
    S = S + c[..., :, None] * khat[..., None, :]
    return S, c


def round_to(x, dtype: str):
    """Round float64 values to the storage type ("f32" or "bf16") with
    round-to-nearest-even; bf16 goes through fp32 as a GPU store does."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = x32.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def conv_update(conv_state_slot, x, weight, accepted):
    """Depthwise causal short convolution over one request's new raw inputs,
    with the conv state rolled (kernels page, `CuteRecoverSSMVerify`: the
    verify fuses the conv update; state page, `deferred_recoverssm_verify`:
    history offset from the accepted count, SiLU, no bias).

    conv_state_slot [C, Lc] (dim-first logical view), x [q, C], weight [C, W].
    Returns (y [q, C] after SiLU, rolled conv state [C, Lc]).
    """
    cs = np.asarray(conv_state_slot)
    C, Lc = cs.shape
    W = weight.shape[1]
    Q = Lc - W + 2
    q = x.shape[0]
    a = min(max(int(accepted), 1), Q)
    history = cs[:, a - 1:a - 1 + W - 1]                # W-1 oldest..newest
    seq = np.concatenate([history, np.asarray(x).T], axis=1)  # [C, W-1+q]
    y = np.empty((q, C), dtype=np.float64)
    for t in range(q):
        y[t] = np.sum(weight * seq[:, t:t + W], axis=1)
    new = cs.copy()
    new[:, :W - 2 + q] = seq[:, 1:W - 1 + q]
    return silu(y), new


def conv_update_verify(*, mixed_qkv, raw_gate, raw_beta, A_log, dt_bias,
                       state, correction, key_gate, out, conv_state,
                       conv_weight, query_start_loc, state_indices,
                       num_accepted_tokens, spec_query_len, null_block_id=0,
                       use_lower_bound=False, lower_bound=0.0,
                       record_rows=None, key_gate_dtype="f32", heads=None,
                       requests=None):
    """Speculative verify of one KDA layer with the short conv fused in.

    Follows the ops page's `_kda_recoverssm_verify_kernel` (per request and
    head, from the checkpoint: gate, normalisations, delta step, readout with
    the updated state, records of the correction and of [raw k | raw gate])
    preceded by the conv update of the kernels page.  The checkpoint `state`
    is only read.

    Array arguments are float64 (exact widenings); `conv_state` is the
    dim-first logical view [N, 3HK, Lc].  Returns a dict of updated copies
    `out`, `correction`, `key_gate`, `conv_state` and masks `out_written`
    [T, HV] and `rec_written` [R, H, Q].  `heads` / `requests` restrict the
    work to a sample (for checking large workloads); requests are
    independent, so a sample's results equal the full run's.
    """
    return _verify(
        mixed_qkv=mixed_qkv, raw_gate=raw_gate, raw_beta=raw_beta,
        A_log=A_log, dt_bias=dt_bias, state=state, correction=correction,
        key_gate=key_gate, out=out, conv_state=conv_state,
        conv_weight=conv_weight, query_start_loc=query_start_loc,
        state_indices=state_indices, num_accepted_tokens=num_accepted_tokens,
        spec_query_len=spec_query_len, null_block_id=null_block_id,
        use_lower_bound=use_lower_bound, lower_bound=lower_bound,
        record_rows=record_rows, key_gate_dtype=key_gate_dtype, heads=heads,
        requests=requests)


def verify_qkv(*, mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state,
               correction, key_gate, out, query_start_loc, state_indices,
               spec_query_len, null_block_id=0, use_lower_bound=False,
               lower_bound=0.0, record_rows=None, key_gate_dtype="f32",
               heads=None, requests=None):
    """The unfused verify (ops page, `kda_recoverssm_verify` with
    `_kda_recoverssm_verify_kernel`): `mixed_qkv` [T, 3HK] already holds
    the convolved q | k | v; there is no conv state.  Same per-head steps
    and records as `conv_update_verify` (the key record is that k).
    Returns the same dict without `conv_state`."""
    r = _verify(
        mixed_qkv=mixed_qkv, raw_gate=raw_gate, raw_beta=raw_beta,
        A_log=A_log, dt_bias=dt_bias, state=state, correction=correction,
        key_gate=key_gate, out=out, conv_state=None, conv_weight=None,
        query_start_loc=query_start_loc, state_indices=state_indices,
        num_accepted_tokens=None, spec_query_len=spec_query_len,
        null_block_id=null_block_id, use_lower_bound=use_lower_bound,
        lower_bound=lower_bound, record_rows=record_rows,
        key_gate_dtype=key_gate_dtype, heads=heads, requests=requests)
    del r["conv_state"]
    return r


def _verify(*, mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state,
            correction, key_gate, out, conv_state, conv_weight,
            query_start_loc, state_indices, num_accepted_tokens,
            spec_query_len, null_block_id, use_lower_bound, lower_bound,
            record_rows, key_gate_dtype, heads, requests):
    """Both verifies; `conv_state` None means q | k | v come convolved."""
    Q = int(spec_query_len)
    N, H, V, K = state.shape
    R = correction.shape[0]
    HK = H * K
    dt_bias = np.asarray(dt_bias, np.float64).reshape(H, K)
    out = np.array(out, dtype=np.float64, copy=True)
    correction = np.array(correction, dtype=np.float64, copy=True)
    key_gate = np.array(key_gate, dtype=np.float64, copy=True)
    if conv_state is not None:
        conv_state = np.array(conv_state, copy=True)
    out_written = np.zeros(out.shape, dtype=bool)
    rec_written = np.zeros(correction.shape[:3], dtype=bool)
    hs = np.arange(H) if heads is None else np.asarray(heads)
    qsl = np.asarray(query_start_loc)
    bs = range(len(state_indices)) if requests is None else requests
    T = out.shape[0]
    for b in bs:
        bos = int(qsl[b])
        q = 0 if (bos < 0 or bos >= T) else \
            min(max(int(qsl[b + 1]) - bos, 0), Q, T - bos)
        if q == 0:
            continue
        slot = int(state_indices[b])
        if slot <= null_block_id or slot < 0 or slot >= N:
            out[bos:bos + q, :] = 0.0
            out_written[bos:bos + q, :] = True
            continue
        r = int(record_rows[b]) if record_rows is not None else slot
        rec_ok = 0 <= r < R
        if conv_state is not None:
            y, conv_state[slot] = conv_update(conv_state[slot],
                                              mixed_qkv[bos:bos + q],
                                              conv_weight,
                                              num_accepted_tokens[b])
        else:
            y = np.asarray(mixed_qkv[bos:bos + q], np.float64)
        qm = y[:, :HK].reshape(q, H, K)[:, hs]
        km = y[:, HK:2 * HK].reshape(q, H, K)[:, hs]
        vm = y[:, 2 * HK:].reshape(q, H, V)[:, hs]
        S = state[slot][hs].astype(np.float64)
        A = np.exp(np.asarray(A_log, np.float64)[hs])
        for t in range(q):
            graw = raw_gate[bos + t].reshape(H, K)[hs]
            g = kda_gate(graw, dt_bias[hs], A[:, None], use_lower_bound,
                         lower_bound)
            S, c = delta_step(S, km[t], vm[t], g, raw_beta[bos + t][hs])
            o = np.einsum("hvk,hk->hv", S, normalize_query(qm[t]))
            rows = out[bos + t].reshape(H, V)
            rows[hs] = o
            out[bos + t] = rows.reshape(-1)
            ow = out_written[bos + t].reshape(H, V)
            ow[hs] = True
            out_written[bos + t] = ow.reshape(-1)
            if rec_ok:
                correction[r, hs, t] = round_to(c, "f32")
                key_gate[r, hs, t, :K] = round_to(km[t], key_gate_dtype)
                key_gate[r, hs, t, K:] = round_to(graw, key_gate_dtype)
                rec_written[r, hs, t] = True
    return dict(out=out, correction=correction, key_gate=key_gate,
                conv_state=conv_state, out_written=out_written,
                rec_written=rec_written)


def commit(*, layers, state_indices, commit_lens, spec_query_len,
           null_block_id=0, final_state_indices=None, record_rows=None,
           boundary_state_indices=None, boundary_recovery_lens=None,
           heads=None, requests=None):
    """Fold each request's first n accepted positions into its checkpoint,
    for every layer (ops page, `_commit_kda_state_kernel` and
    `KDARecoverSSMCommitContext.commit`; kernels page,
    `cute_recoverssm_commit`).

    Written here in the forward order of the recurrence: for t < n,
    S <- S * exp(g_t)[None, :] + c_t k_hat_t^T, with k from the key record,
    g from the recorded raw gate with the layer's own dt_bias, A and gate
    kind, and c_t the recorded correction.  The result is stored (rounded
    to fp32) at the final slot, which defaults to the source slot.

    `layers` is a list of dicts with float64 `state` [N,H,V,K], `correction`
    [R,H,Q,V], `key_gate` [R,H,Q,2K], `A_log` [H], `dt_bias` [H,K] and
    `use_lower_bound`, `lower_bound`.  Returns a list of (new state, written
    mask [N, H]).  `heads` / `requests` restrict the work to a sample.

    Align mode (ops page, `_commit_kda_state_kernel` with ALIGN_MODE):
    when `boundary_state_indices` is given, a request that commits also
    stores the state after its first m = boundary_recovery_lens[b] (clamped
    to [0, n]) positions at its boundary slot, if that slot is live.  Every
    state is computed from the source checkpoint as it was before the
    launch; the boundary is stored before the final state.
    """
    Q = int(spec_query_len)
    results = []
    for layer in layers:
        state = layer["state"]
        N, H, V, K = state.shape
        R = layer["correction"].shape[0]
        dt_bias = np.asarray(layer["dt_bias"], np.float64).reshape(H, K)
        A = np.exp(np.asarray(layer["A_log"], np.float64))
        new = np.array(state, dtype=np.float64, copy=True)
        written = np.zeros((N, H), dtype=bool)
        hs = np.arange(H) if heads is None else np.asarray(heads)
        bs = range(len(state_indices)) if requests is None else requests
        for b in bs:
            slot = int(state_indices[b])
            if slot <= null_block_id or slot < 0 or slot >= N:
                continue
            n = min(max(int(commit_lens[b]), 0), Q)
            if n == 0:
                continue
            f = slot if final_state_indices is None \
                else int(final_state_indices[b])
            if f <= null_block_id or f < 0 or f >= N:
                continue
            r = int(record_rows[b]) if record_rows is not None else slot
            if not 0 <= r < R:
                continue
            bslot, m = null_block_id, 0
            if boundary_state_indices is not None:
                bslot = int(boundary_state_indices[b])
                m = min(max(int(boundary_recovery_lens[b]), 0), n)
            S = np.asarray(state[slot][hs], dtype=np.float64)
            at_boundary = S
            for t in range(n):
                kg = layer["key_gate"][r, hs, t]
                khat = l2_normalize(kg[:, :K])
                g = kda_gate(kg[:, K:], dt_bias[hs], A[hs][:, None],
                             layer["use_lower_bound"], layer["lower_bound"])
                c = layer["correction"][r, hs, t]
                S = S * np.exp(g)[:, None, :] + c[:, :, None] * khat[:, None, :]
                if t + 1 == m:
                    at_boundary = S
            if null_block_id < bslot < N:
                new[bslot, hs] = round_to(at_boundary, "f32")
                written[bslot, hs] = True
            new[f, hs] = round_to(S, "f32")
            written[f, hs] = True
        results.append((new, written))
    return results


def commit_fold_reverse(S0, corrections, keys, raw_gates, dt_bias, A,
                        use_lower_bound, lower_bound):
    """The pages' form of the fold for one head (ops page,
    `_commit_kda_state_kernel`): walk the committed positions from newest
    to oldest, adding each position's c k_hat^T scaled by the product of the
    decays of the positions after it, while accumulating the total decay;
    the result is S0 scaled by the total decay plus that sum.

    S0 [V, K], corrections [n, V], keys [n, K], raw_gates [n, K].
    """
    S0 = np.asarray(S0, dtype=np.float64)
    V, K = S0.shape
    later_decay = np.ones(K)
    acc = np.zeros((V, K))
    for t in range(len(corrections) - 1, -1, -1):
        khat = l2_normalize(keys[t])
        d = np.exp(kda_gate(raw_gates[t], dt_bias, A, use_lower_bound,
                            lower_bound))
        acc += np.outer(corrections[t], khat) * later_decay[None, :]
        later_decay = later_decay * d
    return S0 * later_decay[None, :] + acc


def commit_plan(*, num_accepted_tokens, state_indices, query_start_loc,
                spec_query_len, null_block_id=0, request_indices=None,
                block_table=None, num_computed_tokens=None,
                mamba_block_size=None):
    """Per-request commit plan (ops page, `_prepare_commit_plan_kernel` as
    launched by `KDARecoverSSMCommitContext.commit`; its body is not on the
    pages, so this is the reading stated here).

    Row b of the batch reads its per-request values (accepted count, block
    table row, computed-token count) at row request_indices[b] (default b);
    its state slot and window at b.  A row outside those arrays plans no
    commit (n = 0, final = source, no boundary).  Then
      n = accepted count clamped to [0, q_b]   (0 for a null slot);
    without a block table: final = source slot, no boundary;
    with one (prefix caching, one state block per `mamba_block_size` = bs
    tokens), for c = computed tokens before the window and end = c + n:
      final = block_table[row, end // bs], the block of the next token to
              compute, which holds the running checkpoint (null if past the
              table);
      if that block starts at P with c < P <= end, the committed tokens
      completed the block before it: boundary = block_table[row, P/bs - 1]
      receives the state after its last token, i.e. after P - c positions
      (all n of them when P = end: then both blocks get the same state);
      a boundary block past the table's width is null (length 0).
    Since bs >= Q, one window completes at most one block.  The running
    block is always the incomplete one, so the verify's in-place conv roll
    (at the source, the block of token c) never touches a completed block.
    Returns int arrays (commit_lens, final, boundary, boundary_lens).
    """
    Q = int(spec_query_len)
    B = len(state_indices)
    qsl = np.asarray(query_start_loc)
    # rows of the per-request arrays; a row outside them commits nothing
    rows = len(num_accepted_tokens)
    if block_table is not None:
        rows = min(rows, len(block_table), len(num_computed_tokens))
    if request_indices is None:
        rows = max(rows, B)
    lens = np.zeros(B, dtype=np.int64)
    final = np.array(state_indices, dtype=np.int64, copy=True)
    boundary = np.full(B, null_block_id, dtype=np.int64)
    blens = np.zeros(B, dtype=np.int64)
    for b in range(B):
        row = b if request_indices is None else int(request_indices[b])
        if not 0 <= row < rows:
            continue
        q = min(max(int(qsl[b + 1]) - int(qsl[b]), 0), Q)
        n = min(max(int(num_accepted_tokens[row]), 0), q)
        if int(state_indices[b]) <= null_block_id:
            n = 0
        lens[b] = n
        if block_table is None or n == 0:
            continue
        bs = int(mamba_block_size)
        c = max(int(num_computed_tokens[row]), 0)
        last = (c + n) // bs
        width = np.asarray(block_table).shape[1]
        final[b] = int(block_table[row][last]) if last < width \
            else null_block_id
        start = last * bs
        if c < start and last - 1 < width:
            boundary[b] = int(block_table[row][last - 1])
            blens[b] = start - c
    return lens, final, boundary, blens


def compact_conv_state(*, conv_states, state_indices, commit_lens,
                       final_state_indices, null_block_id=0,
                       boundary_state_indices=None,
                       boundary_recovery_lens=None):
    """Conv-state compaction at commit (ops page, `_compact_conv_state_kernel`
    as launched by `KDARecoverSSMCommitContext.commit`; body not on the
    pages, reading stated here).

    With the verify's rolled layout (entry 2 + t holds the window's input t,
    entries 0 and 1 the two inputs before it), the history after the first
    n committed positions is entries [n - 1, n - 1 + W - 1).  It is copied
    to entries [0, W - 1) of the final slot, so that the next verify reads
    it with accepted count 1; in align mode, the history after m boundary
    positions (m >= 1) goes to the boundary slot the same way.  Other
    entries are left as they are; everything is read before anything is
    written; the boundary is written before the final slot.

    conv_states: per layer, the dim-first logical view [N, C, Lc] (any
    dtype: values are moved, not computed).  Returns updated copies.
    """
    out = []
    for cs in conv_states:
        cs = np.asarray(cs)
        N, _, Lc = cs.shape
        new = cs.copy()
        for b in range(len(state_indices)):
            slot = int(state_indices[b])
            if slot <= null_block_id or slot >= N:
                continue
            Qm = Lc - 2
            n = min(max(int(commit_lens[b]), 0), Qm)
            if n == 0:
                continue
            f = int(final_state_indices[b])
            if f <= null_block_id or f >= N:
                continue
            hist_n = cs[slot][:, n - 1:n + 2].copy()
            if boundary_state_indices is not None:
                bslot = int(boundary_state_indices[b])
                m = min(max(int(boundary_recovery_lens[b]), 0), n)
                if null_block_id < bslot < N and m >= 1:
                    new[bslot][:, 0:3] = cs[slot][:, m - 1:m + 2]
            new[f][:, 0:3] = hist_n
        out.append(new)
    return out
