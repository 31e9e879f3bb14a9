"""Pins of the oracle's verify (with the fused conv) and commit against a
library convolution, a brute-force scalar implementation, the algebraic
identity commit(n) == n recurrence steps, the pages' reverse-accumulation
fold and the slot / null / record-row rules (no GPU)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from workloads import make_workload, to_f64

RNG = np.random.default_rng(99)


def _library_conv(stream, weight):
    """Causal depthwise conv by torch's conv1d over an explicit stream:
    stream [C, L], weight [C, W] -> [L - W + 1, C] (pre-activation)."""
    x = torch.from_numpy(stream)[None]
    w = torch.from_numpy(weight)[:, None, :]
    return torch.nn.functional.conv1d(x, w, groups=stream.shape[0])[0].T \
        .numpy()


# ---- the fused short convolution -------------------------------------------

def test_conv_matches_library_conv1d():
    C, W, Q = 10, 4, 5
    Lc = Q + W - 2
    for a in range(1, Q + 1):
        for q in range(1, Q + 1):
            cs = RNG.normal(size=(C, Lc))
            x = RNG.normal(size=(q, C))
            w = RNG.normal(size=(C, W))
            y, new = oracle.conv_update(cs, x, w, a)
            stream = np.concatenate([cs[:, a - 1:a - 1 + W - 1], x.T], axis=1)
            ref = _library_conv(stream, w)
            np.testing.assert_allclose(y, oracle.silu(ref), rtol=1e-13,
                                       atol=1e-14)
            # roll: the W-2 newest history entries then x, tail untouched
            assert np.array_equal(new[:, :W - 2], cs[:, a:a + W - 2])
            assert np.array_equal(new[:, W - 2:W - 2 + q], x.T)
            assert np.array_equal(new[:, W - 2 + q:], cs[:, W - 2 + q:])


def test_conv_multi_step_self_consistency():
    # Simulate a request through many speculative steps with ragged draft
    # counts and acceptance.  Each step's conv output must equal the library
    # convolution over the truly accepted token stream followed by the new
    # drafts.  This fixes the history offset and the roll together.
    C, W, Q = 6, 4, 4
    Lc = Q + W - 2
    w = RNG.normal(size=(C, W))
    accepted_stream = [RNG.normal(size=C) for _ in range(W - 1)]
    cs = RNG.normal(size=(C, Lc))          # garbage beyond the history
    cs[:, :W - 1] = np.array(accepted_stream).T
    a = 1                                  # a prefilled request starts at 1
    for step in range(40):
        q = int(RNG.integers(1, Q + 1))
        x = RNG.normal(size=(q, C))
        y, cs = oracle.conv_update(cs, x, w, a)
        hist = np.array(accepted_stream[-(W - 1):]).T
        ref = _library_conv(np.concatenate([hist, x.T], axis=1), w)
        np.testing.assert_allclose(y, oracle.silu(ref), rtol=1e-13,
                                   atol=1e-14)
        a = int(RNG.integers(1, q + 1))    # tokens accepted from this step
        accepted_stream.extend(x[:a])


# ---- brute force ------------------------------------------------------------

def _oracle_inputs(wl, layer=0):
    L = wl.layers[layer]
    return dict(
        mixed_qkv=to_f64(L.mixed_qkv), raw_gate=to_f64(L.raw_gate),
        raw_beta=to_f64(L.raw_beta), A_log=to_f64(L.A_log),
        dt_bias=to_f64(L.dt_bias), state=to_f64(L.state),
        correction=to_f64(L.correction), key_gate=to_f64(L.key_gate),
        out=np.zeros((wl.T, wl.H * wl.D)),
        conv_state=to_f64(wl.conv_state_dim_first(layer)),
        conv_weight=to_f64(L.conv_weight),
        query_start_loc=wl.query_start_loc.numpy(),
        state_indices=wl.state_indices.numpy(),
        num_accepted_tokens=wl.num_accepted_tokens.numpy(),
        spec_query_len=wl.Q, null_block_id=wl.null_block_id,
        use_lower_bound=L.use_lower_bound, lower_bound=L.lower_bound,
        record_rows=None if wl.record_rows is None else wl.record_rows.numpy(),
        key_gate_dtype=wl.kg_dtype)


@pytest.mark.parametrize("gate", [None, -5.0])
@pytest.mark.parametrize("dim_first", [True, False])
def test_tiny_verify_and_commit_match_brute_force(gate, dim_first):
    wl = make_workload("tiny", gates=[gate], conv_dim_first=dim_first)
    inp = _oracle_inputs(wl)
    res = oracle.conv_update_verify(**inp)
    H, K, W = wl.H, wl.D, wl.W
    qsl = inp["query_start_loc"]
    for b in range(wl.B):
        slot = int(inp["state_indices"][b])
        a = int(inp["num_accepted_tokens"][b])
        bos, eos = int(qsl[b]), int(qsl[b + 1])
        cs = inp["conv_state"][slot]
        outs, corr, keys = brute.verify_one(
            S0=inp["state"][slot].tolist(), xs=inp["mixed_qkv"][bos:eos].tolist(),
            history=cs[:, a - 1:a - 1 + W - 1].tolist(),
            weight=inp["conv_weight"].tolist(),
            raw_gates=inp["raw_gate"][bos:eos].tolist(),
            raw_betas=inp["raw_beta"][bos:eos].tolist(),
            dt_bias=inp["dt_bias"].tolist(), A_log=inp["A_log"].tolist(),
            use_lb=gate is not None, lb=gate or 0.0, H=H, K=K)
        np.testing.assert_allclose(res["out"][bos:eos], np.array(outs),
                                   rtol=0, atol=1e-12)
        q = eos - bos
        for h in range(H):
            np.testing.assert_allclose(res["correction"][slot, h, :q],
                                       np.array(corr[h]), rtol=1e-6, atol=1e-7)
            np.testing.assert_allclose(res["key_gate"][slot, h, :q, :K],
                                       np.array(keys[h]), rtol=1e-6, atol=1e-7)
    # commit, one head at a time against the brute-force fold
    layer = dict(state=inp["state"], correction=res["correction"],
                 key_gate=res["key_gate"], A_log=inp["A_log"],
                 dt_bias=inp["dt_bias"], use_lower_bound=gate is not None,
                 lower_bound=gate or 0.0)
    (new, written), = oracle.commit(
        layers=[layer], state_indices=inp["state_indices"],
        commit_lens=wl.commit_lens.numpy(), spec_query_len=wl.Q)
    for b in range(wl.B):
        slot = int(inp["state_indices"][b])
        n = int(wl.commit_lens[b])
        for h in range(H):
            S = brute.fold_one(
                S0=inp["state"][slot, h].tolist(),
                corr=res["correction"][slot, h, :n].tolist(),
                keys=res["key_gate"][slot, h, :n, :K].tolist(),
                raw_gates=res["key_gate"][slot, h, :n, K:].tolist(),
                dt_bias=inp["dt_bias"][h].tolist(), A_log=inp["A_log"][h],
                use_lb=gate is not None, lb=gate or 0.0)
            np.testing.assert_allclose(new[slot, h], np.array(S), rtol=1e-6,
                                       atol=1e-8)
            assert written[slot, h]


# ---- the unfused verify -------------------------------------------------------

def _library_qkv(inp, wl):
    """Each request's q | k | v from the library convolution (torch conv1d +
    SiLU) over its accepted history and drafts; zero rows for nulls."""
    y = np.zeros_like(inp["mixed_qkv"])
    qsl, W = inp["query_start_loc"], wl.W
    for b in range(wl.B):
        slot = int(inp["state_indices"][b])
        bos, eos = int(qsl[b]), int(qsl[b + 1])
        if eos == bos or slot <= 0 or slot >= wl.N:
            continue
        a = int(inp["num_accepted_tokens"][b])
        cs = inp["conv_state"][slot]
        stream = np.concatenate([cs[:, a - 1:a + W - 2],
                                 inp["mixed_qkv"][bos:eos].T], axis=1)
        y[bos:eos] = oracle.silu(_library_conv(stream, inp["conv_weight"]))
    return y


@pytest.mark.parametrize("cfg,gate", [("ragged", None), ("ragged", -5.0),
                                      ("deferred", None)])
def test_unfused_verify_on_convolved_input_equals_fused(cfg, gate):
    # The unfused verify takes q | k | v already convolved.  Fed the library
    # convolution of each request's stream, it must reproduce the fused
    # verify (itself pinned to brute force above) output for output, write
    # the same masks, and record that k as the key.
    wl = make_workload(cfg, B=8, H=2, D=8, Q=4, N=12, act="f32",
                       weight="f32", gates=[gate], null_frac=0.25)
    inp = _oracle_inputs(wl)
    fused = oracle.conv_update_verify(**inp)
    y = _library_qkv(inp, wl)
    kw = {k: v for k, v in inp.items()
          if k not in ("conv_state", "conv_weight", "num_accepted_tokens")}
    kw["mixed_qkv"] = y
    res = oracle.verify_qkv(**kw)
    assert "conv_state" not in res
    for k in ("out_written", "rec_written"):
        assert np.array_equal(res[k], fused[k]), k
    np.testing.assert_allclose(res["out"], fused["out"], rtol=1e-10,
                               atol=1e-12)
    np.testing.assert_allclose(res["correction"], fused["correction"],
                               rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(res["key_gate"], fused["key_gate"],
                               rtol=1e-6, atol=1e-7)
    # the key record is the given k, rounded to the record dtype only
    K, H = wl.D, wl.H
    qsl = inp["query_start_loc"]
    rows = inp["record_rows"]
    for b in range(wl.B):
        slot = int(inp["state_indices"][b])
        if slot <= 0:
            continue
        r = slot if rows is None else int(rows[b])
        bos, eos = int(qsl[b]), int(qsl[b + 1])
        for t in range(eos - bos):
            k = y[bos + t, H * K:2 * H * K].reshape(H, K)
            assert np.array_equal(res["key_gate"][r, :, t, :K],
                                  oracle.round_to(k, "f32"))


def test_unfused_verify_with_identity_taps_is_silu_of_input():
    # A conv whose only tap is the newest input (weight [0, 0, 0, 1]) turns
    # the fused verify into the unfused one applied to SiLU(x).
    wl = make_workload("ragged", B=6, H=2, D=8, Q=4, N=10, act="f32",
                       weight="f32", null_frac=0.0)
    inp = _oracle_inputs(wl)
    inp["conv_weight"] = np.zeros_like(inp["conv_weight"])
    inp["conv_weight"][:, -1] = 1.0
    fused = oracle.conv_update_verify(**inp)
    kw = {k: v for k, v in inp.items()
          if k not in ("conv_state", "conv_weight", "num_accepted_tokens")}
    kw["mixed_qkv"] = oracle.silu(inp["mixed_qkv"])
    res = oracle.verify_qkv(**kw)
    for k in ("out", "correction", "key_gate", "out_written", "rec_written"):
        assert np.array_equal(res[k], fused[k]), k


# ---- commit fold identities --------------------------------------------------

@pytest.mark.parametrize("gate", [None, -5.0])
def test_verify_then_commit_equals_fresh_recurrence(gate):
    # For every n <= q: commit(n) of the verify's records == n steps of the
    # delta rule from the checkpoint, with q/k/v from the library conv.
    wl = make_workload("ragged", B=6, H=3, D=8, Q=4, N=10, act="f32",
                       weight="f32", gates=[gate], null_frac=0.0)
    inp = _oracle_inputs(wl)
    res = oracle.conv_update_verify(**inp)
    H, K, W, Q = wl.H, wl.D, wl.W, wl.Q
    qsl = inp["query_start_loc"]
    for b in range(wl.B):
        slot = int(inp["state_indices"][b])
        a = int(inp["num_accepted_tokens"][b])
        bos, eos = int(qsl[b]), int(qsl[b + 1])
        q = eos - bos
        cs = inp["conv_state"][slot]
        stream = np.concatenate([cs[:, a - 1:a + W - 2],
                                 inp["mixed_qkv"][bos:eos].T], axis=1)
        y = oracle.silu(_library_conv(stream, inp["conv_weight"]))
        for n in range(0, q + 1):
            layer = dict(state=inp["state"], correction=res["correction"],
                         key_gate=res["key_gate"], A_log=inp["A_log"],
                         dt_bias=inp["dt_bias"], use_lower_bound=gate is not None,
                         lower_bound=gate or 0.0)
            lens = np.zeros(wl.B, dtype=np.int64)
            lens[b] = n
            (new, written), = oracle.commit(
                layers=[layer], state_indices=inp["state_indices"],
                commit_lens=lens, spec_query_len=Q)
            if n == 0:
                assert not written.any()
                assert np.array_equal(new, inp["state"])
                continue
            for h in range(H):
                S = inp["state"][slot, h].copy()
                A = np.exp(inp["A_log"][h])
                for t in range(n):
                    g = oracle.kda_gate(inp["raw_gate"][bos + t, h * K:(h + 1) * K],
                                        inp["dt_bias"][h], A, gate is not None,
                                        gate or 0.0)
                    S, _ = oracle.delta_step(
                        S, y[t, H * K + h * K:H * K + (h + 1) * K],
                        y[t, 2 * H * K + h * K:2 * H * K + (h + 1) * K], g,
                        inp["raw_beta"][bos + t, h])
                np.testing.assert_allclose(new[slot, h], S, rtol=1e-6,
                                           atol=1e-8)
            # only that slot was written
            others = np.ones(wl.N, bool)
            others[slot] = False
            assert np.array_equal(new[others], inp["state"][others])


def test_reverse_fold_equals_forward_fold():
    K, V = 9, 7
    for gate in (None, -5.0):
        for n in range(0, 6):
            S0 = RNG.normal(size=(V, K))
            corr = RNG.normal(size=(n, V))
            keys = RNG.normal(size=(n, K))
            graw = RNG.normal(size=(n, K))
            bias = RNG.normal(size=K) * 0.1
            A = 3.0
            S = S0.copy()
            for t in range(n):
                g = oracle.kda_gate(graw[t], bias, A, gate is not None, gate or 0)
                S = S * np.exp(g)[None, :] + np.outer(corr[t],
                                                      oracle.l2_normalize(keys[t]))
            R = oracle.commit_fold_reverse(S0, corr, keys, graw, bias, A,
                                           gate is not None, gate or 0.0)
            np.testing.assert_allclose(R, S, rtol=1e-12, atol=1e-13)


# ---- slots, nulls, record rows -----------------------------------------------

def test_null_slots_zero_outputs_and_touch_nothing():
    wl = make_workload("ragged", B=10, H=2, D=8, Q=4, N=16, act="f32",
                       weight="f32", null_frac=0.3)
    inp = _oracle_inputs(wl)
    inp["out"] = RNG.normal(size=inp["out"].shape)
    # make one more request point past the pool: treated as null
    si = inp["state_indices"].copy()
    live = np.nonzero(si > 0)[0]
    si[live[0]] = wl.N + 3
    inp["state_indices"] = si
    res = oracle.conv_update_verify(**inp)
    qsl = inp["query_start_loc"]
    nulls = [b for b in range(wl.B) if si[b] <= 0 or si[b] >= wl.N]
    assert len(nulls) == 4
    for b in nulls:
        rows = slice(int(qsl[b]), int(qsl[b + 1]))
        assert np.all(res["out"][rows] == 0.0)
        assert np.all(res["out_written"][rows])
    touched = {int(s) for s in si if 0 < s < wl.N}
    for s in range(wl.N):
        if s not in touched:
            assert np.array_equal(res["conv_state"][s], inp["conv_state"][s])
            assert np.array_equal(res["correction"][s], inp["correction"][s])
            assert np.array_equal(res["key_gate"][s], inp["key_gate"][s])
    # rows of live requests were written, positions past q were not
    for b in range(wl.B):
        if b in nulls:
            continue
        q = int(qsl[b + 1] - qsl[b])
        s = int(si[b])
        assert res["rec_written"][s, :, :q].all()
        assert not res["rec_written"][s, :, q:].any()
        assert np.array_equal(res["correction"][s, :, q:],
                              inp["correction"][s, :, q:])


def test_zero_length_request_is_a_no_op():
    wl = make_workload("tiny")
    inp = _oracle_inputs(wl)
    inp["query_start_loc"] = np.array([0, 0, 3])
    inp["mixed_qkv"] = inp["mixed_qkv"][:3]
    inp["raw_gate"] = inp["raw_gate"][:3]
    inp["raw_beta"] = inp["raw_beta"][:3]
    inp["out"] = inp["out"][:3]
    res = oracle.conv_update_verify(**inp)
    s0 = int(inp["state_indices"][0])
    assert np.array_equal(res["conv_state"][s0], inp["conv_state"][s0])
    assert not res["rec_written"][s0].any()


def test_record_rows_redirect_and_negative_rows_skip():
    wl = make_workload("deferred", B=6, H=2, D=8, Q=4, N=12, act="f32",
                       weight="f32")
    inp = _oracle_inputs(wl)
    rows = inp["record_rows"].copy()
    rows[2] = -1
    inp["record_rows"] = rows
    res = oracle.conv_update_verify(**inp)
    for b in range(wl.B):
        r = int(rows[b])
        if r < 0:
            continue
        assert res["rec_written"][r].all()
    assert res["rec_written"].sum() == 5 * 2 * 4
    # request 2 still produced outputs
    qsl = inp["query_start_loc"]
    assert res["out_written"][int(qsl[2]):int(qsl[3])].all()
    # the commit skips a negative row, and folds the others from their rows
    layers = [dict(state=inp["state"], correction=res["correction"],
                   key_gate=res["key_gate"], A_log=inp["A_log"],
                   dt_bias=inp["dt_bias"], use_lower_bound=False,
                   lower_bound=0.0)]
    (new, written), = oracle.commit(
        layers=layers, state_indices=inp["state_indices"],
        commit_lens=np.full(wl.B, 2), spec_query_len=wl.Q, record_rows=rows)
    s2 = int(inp["state_indices"][2])
    assert not written[s2].any()
    assert written.sum() == 5 * 2


def test_commit_final_slot_and_clamps():
    wl = make_workload("tiny")
    inp = _oracle_inputs(wl)
    res = oracle.conv_update_verify(**inp)
    layer = dict(state=inp["state"], correction=res["correction"],
                 key_gate=res["key_gate"], A_log=inp["A_log"],
                 dt_bias=inp["dt_bias"], use_lower_bound=False, lower_bound=0.)
    si = inp["state_indices"]
    free = [s for s in range(1, wl.N) if s not in set(si.tolist())]
    final = np.array([free[0], 0])        # second request: null final, skip
    (new, written), = oracle.commit(
        layers=[layer], state_indices=si, commit_lens=np.array([99, 3]),
        spec_query_len=wl.Q, final_state_indices=final)
    assert written[free[0]].all() and written.sum() == wl.H
    # n = 99 is clamped to Q: same as n = Q in place
    (ref, _), = oracle.commit(layers=[layer], state_indices=si,
                              commit_lens=np.array([wl.Q, 0]),
                              spec_query_len=wl.Q)
    assert np.array_equal(new[free[0]], ref[int(si[0])])
    # the source slot is untouched when the result goes elsewhere
    assert np.array_equal(new[int(si[0])], inp["state"][int(si[0])])


def test_verify_does_not_modify_its_inputs():
    wl = make_workload("tiny")
    inp = _oracle_inputs(wl)
    before = {k: np.array(v, copy=True) for k, v in inp.items()
              if isinstance(v, np.ndarray)}
    oracle.conv_update_verify(**inp)
    for k, v in before.items():
        assert np.array_equal(inp[k], v), k
