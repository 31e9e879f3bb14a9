"""Pins of the oracle's commit plan, align-mode (boundary) commit and conv
compaction (no GPU).

The plan kernel and the compaction kernel have no body on the pages; what
pins them is the property prefix caching needs and that the pages state:
after every commit, the block holding a request's last committed token holds
the state (and the conv history) after exactly that many tokens, and every
block the sequence has completed holds the state after its own last token.
The simulations below run many speculative steps with random drafts and
acceptance through verify -> plan -> compaction -> commit and compare, at
every step, with a fresh recurrence over the accepted token stream whose q/k/v
come from torch's conv1d."""
import numpy as np
import pytest
import torch

import oracle

H, K, Q, W = 2, 8, 4, 4
C = 3 * H * K


class TrueModel:
    """The accepted token stream and the states after each prefix, by the
    plain recurrence with q/k/v from torch's conv1d."""

    def __init__(self, rng, gate):
        self.w = rng.normal(size=(C, W)) * 0.5
        self.A_log = np.log(rng.uniform(1, 16, size=H))
        self.dt_bias = rng.normal(size=(H, K)) * 0.1
        self.gate = gate
        self.xs = [rng.normal(size=C) for _ in range(W - 1)]   # pre-history
        self.gs, self.bs = [], []
        self.S = [rng.normal(size=(H, K, K)) * 0.2]            # after 0 tokens
        self.outs = []

    def y(self, i):
        """Conv output of token i (inputs i-3 .. i of the stream)."""
        win = np.array(self.xs[i:i + W]).T                     # [C, W]
        x = torch.from_numpy(win)[None]
        w = torch.from_numpy(self.w)[:, None, :]
        pre = torch.nn.functional.conv1d(x, w, groups=C)[0, :, 0].numpy()
        return oracle.silu(pre)

    def append(self, x, g, beta):
        i = len(self.gs)
        self.xs.append(x)
        self.gs.append(g)
        self.bs.append(beta)
        y = self.y(i)
        S = self.S[-1].copy()
        A = np.exp(self.A_log)
        for h in range(H):
            gate = oracle.kda_gate(g[h * K:(h + 1) * K], self.dt_bias[h], A[h],
                                   self.gate is not None, self.gate or 0.0)
            S[h], _ = oracle.delta_step(
                S[h], y[H * K + h * K:H * K + (h + 1) * K],
                y[2 * H * K + h * K:2 * H * K + (h + 1) * K], gate, beta[h])
        self.S.append(S)
        qh = oracle.normalize_query(y[:H * K].reshape(H, K))
        self.outs.append(np.einsum("hvk,hk->hv", S, qh).reshape(-1))

    def history(self, c):
        """The W-1 raw inputs before token c, as conv-state columns."""
        return np.array(self.xs[c:c + W - 1]).T


def _simulate(rng, gate, bs, steps, c0, align=True):
    tm = TrueModel(rng, gate)
    for _ in range(c0):
        tm.append(rng.normal(size=C), rng.normal(size=H * K),
                  rng.normal(size=H))
    N, width = 80, 40
    table = rng.permutation(np.arange(1, N))[:width]
    state = np.zeros((N, H, K, K))
    conv = rng.normal(size=(N, C, Q + W - 2))
    corr = rng.normal(size=(N, H, Q, K))
    kg = rng.normal(size=(N, H, Q, 2 * K))
    fixed = int(table[0])

    def home(c):
        """The running block: the one that will hold token c."""
        return int(table[c // bs]) if align else fixed

    c = c0
    state[home(c)] = oracle.round_to(tm.S[c], "f32")
    conv[home(c)][:, :W - 1] = tm.history(c)
    layer = dict(A_log=tm.A_log, dt_bias=tm.dt_bias,
                 use_lower_bound=gate is not None, lower_bound=gate or 0.0)
    crossings = 0
    for _ in range(steps):
        q = int(rng.integers(1, Q + 1))
        X = rng.normal(size=(q, C))
        G = rng.normal(size=(q, H * K))
        Bt = rng.normal(size=(q, H))
        a = int(rng.integers(1, q + 1))
        src = home(c)
        res = oracle.conv_update_verify(
            mixed_qkv=X, raw_gate=G, raw_beta=Bt, A_log=tm.A_log,
            dt_bias=tm.dt_bias, state=state, correction=corr, key_gate=kg,
            out=np.zeros((q, H * K)), conv_state=conv, conv_weight=tm.w,
            query_start_loc=np.array([0, q]), state_indices=np.array([src]),
            num_accepted_tokens=np.array([1]), spec_query_len=Q,
            use_lower_bound=gate is not None, lower_bound=gate or 0.0)
        conv, corr, kg = res["conv_state"], res["correction"], res["key_gate"]
        lens, final, bnd, blens = oracle.commit_plan(
            num_accepted_tokens=np.array([a]), state_indices=np.array([src]),
            query_start_loc=np.array([0, q]), spec_query_len=Q,
            block_table=table[None] if align else None,
            num_computed_tokens=np.array([c]) if align else None,
            mamba_block_size=bs if align else None)
        assert lens[0] == a
        crossings += int(bnd[0] > 0)
        conv, = oracle.compact_conv_state(
            conv_states=[conv], state_indices=np.array([src]),
            commit_lens=lens, final_state_indices=final,
            boundary_state_indices=bnd if align else None,
            boundary_recovery_lens=blens if align else None)
        (state, _), = oracle.commit(
            layers=[dict(layer, state=state, correction=corr, key_gate=kg)],
            state_indices=np.array([src]), commit_lens=lens,
            spec_query_len=Q, final_state_indices=final,
            boundary_state_indices=bnd if align else None,
            boundary_recovery_lens=blens if align else None)
        for t in range(a):
            tm.append(X[t], G[t], Bt[t])
        # the verify's accepted outputs are the model's outputs there
        np.testing.assert_allclose(res["out"][:a], np.array(tm.outs[c:c + a]),
                                   rtol=1e-5, atol=1e-6)
        c += a
        # the block of the last committed token: state and history after c
        np.testing.assert_allclose(state[home(c)], tm.S[c], rtol=1e-5,
                                   atol=1e-6)
        assert np.array_equal(conv[home(c)][:, :W - 1], tm.history(c))
        # every block completed since the start: state after its last token
        if align:
            for j in range(c // bs):
                end = (j + 1) * bs
                if end <= c0:
                    continue
                blk = int(table[j])
                np.testing.assert_allclose(state[blk], tm.S[end], rtol=1e-5,
                                           atol=1e-6)
                assert np.array_equal(conv[blk][:, :W - 1], tm.history(end))
    return c, crossings


@pytest.mark.parametrize("gate,bs", [(None, 4), (-5.0, 6), (None, 7)])
def test_align_sequence_keeps_prefix_states(gate, bs):
    rng = np.random.default_rng(bs * 11 + (gate is None))
    c, crossings = _simulate(rng, gate, bs, steps=30, c0=5)
    assert c > 5 + 30 and crossings >= 5     # boundaries were exercised


def test_non_align_sequence_with_compaction():
    rng = np.random.default_rng(5)
    _simulate(rng, -5.0, 4, steps=25, c0=3, align=False)


def test_compaction_equals_accepted_offset():
    # Compacting after the commit and then verifying with accepted count 1
    # gives the same conv outputs (and outputs) as verifying without the
    # compaction, with the accepted count as offset.
    rng = np.random.default_rng(8)
    N, Lc = 6, Q + W - 2
    w = rng.normal(size=(C, W))
    conv = rng.normal(size=(N, C, Lc))
    args = dict(raw_gate=rng.normal(size=(3, H * K)),
                raw_beta=rng.normal(size=(3, H)), A_log=np.zeros(H),
                dt_bias=np.zeros((H, K)),
                state=rng.normal(size=(N, H, K, K)),
                correction=np.zeros((N, H, Q, K)),
                key_gate=np.zeros((N, H, Q, 2 * K)), out=np.zeros((3, H * K)),
                conv_weight=w, query_start_loc=np.array([0, 3]),
                state_indices=np.array([2]), spec_query_len=Q)
    X = rng.normal(size=(3, C))
    for n in range(1, Q + 1):
        comp, = oracle.compact_conv_state(
            conv_states=[conv], state_indices=np.array([2]),
            commit_lens=np.array([n]), final_state_indices=np.array([2]))
        a = oracle.conv_update_verify(mixed_qkv=X, conv_state=comp,
                                      num_accepted_tokens=np.array([1]),
                                      **args)
        b = oracle.conv_update_verify(mixed_qkv=X, conv_state=conv,
                                      num_accepted_tokens=np.array([n]),
                                      **args)
        assert np.array_equal(a["out"], b["out"])
        assert np.array_equal(a["key_gate"], b["key_gate"])


def test_boundary_state_is_the_partial_fold():
    rng = np.random.default_rng(3)
    N, R = 8, 8
    layer = dict(state=rng.normal(size=(N, H, K, K)),
                 correction=rng.normal(size=(R, H, Q, K)),
                 key_gate=rng.normal(size=(R, H, Q, 2 * K)),
                 A_log=np.log(rng.uniform(1, 16, size=H)),
                 dt_bias=rng.normal(size=(H, K)) * 0.1,
                 use_lower_bound=False, lower_bound=0.0)
    for n in range(1, Q + 1):
        for m in range(-1, n + 2):
            (new, written), = oracle.commit(
                layers=[layer], state_indices=np.array([2]),
                commit_lens=np.array([n]), spec_query_len=Q,
                final_state_indices=np.array([5]),
                boundary_state_indices=np.array([6]),
                boundary_recovery_lens=np.array([m]), record_rows=None)
            mm = min(max(m, 0), n)
            # the boundary holds commit(mm) of the same records; commit(0)
            # is the checkpoint itself
            if mm == 0:
                ref = oracle.round_to(layer["state"][2], "f32")
            else:
                (r, _), = oracle.commit(
                    layers=[layer], state_indices=np.array([2]),
                    commit_lens=np.array([mm]), spec_query_len=Q,
                    final_state_indices=np.array([6]))
                ref = r[6]
            assert np.array_equal(new[6], ref)
            (r, _), = oracle.commit(
                layers=[layer], state_indices=np.array([2]),
                commit_lens=np.array([n]), spec_query_len=Q,
                final_state_indices=np.array([5]))
            assert np.array_equal(new[5], r[5])
            assert written[[5, 6]].all() and written.sum() == 2 * H
    # a null boundary slot stores nothing
    (new, written), = oracle.commit(
        layers=[layer], state_indices=np.array([2]), commit_lens=np.array([3]),
        spec_query_len=Q, final_state_indices=np.array([5]),
        boundary_state_indices=np.array([0]),
        boundary_recovery_lens=np.array([2]))
    assert written.sum() == H


def test_plan_worked_cases():
    # Block size 8, window 4, computed tokens c, accepted a: the tokens
    # c .. c+a-1 are committed; the final block is the one that will hold
    # token c+a; a boundary exists when that block starts after c.
    table = np.array([[11, 12, 13, 14]])
    qsl = np.array([0, 4])
    cases = [  # c, a -> final, boundary, boundary len
        (5, 2, 11, 0, 0),      # tokens 5, 6: inside block 0
        (6, 2, 12, 11, 2),     # tokens 6, 7 complete block 0
        (6, 3, 12, 11, 2),     # tokens 6, 7 | 8: crosses after 2
        (7, 4, 12, 11, 1),     # tokens 7 | 8, 9, 10
        (8, 1, 12, 0, 0),      # starts a block: nothing to recover
        (15, 4, 13, 12, 1),
        (29, 3, 0, 14, 3),     # past the table: null final
    ]
    for c, a, f, bnd, bl in cases:
        lens, final, boundary, blens = oracle.commit_plan(
            num_accepted_tokens=np.array([a]), state_indices=np.array([9]),
            query_start_loc=qsl, spec_query_len=4, block_table=table,
            num_computed_tokens=np.array([c]), mamba_block_size=8)
        assert (lens[0], final[0], boundary[0], blens[0]) == (a, f, bnd, bl), \
            (c, a)


def test_plan_clamps_nulls_and_request_map():
    qsl = np.array([0, 2, 2, 6, 9])
    acc = np.array([7, 3, 1, 4, 9, 2])          # by request row
    rows = np.array([3, 0, 5, 1])
    slots = np.array([4, 5, 0, 6])
    lens, final, boundary, blens = oracle.commit_plan(
        num_accepted_tokens=acc, state_indices=slots, query_start_loc=qsl,
        spec_query_len=4, request_indices=rows)
    # accepted of rows 3, 0, 5, 1 clamped to q = 2, 0, 4, 3; null slot -> 0
    assert lens.tolist() == [2, 0, 0, 3]
    assert final.tolist() == slots.tolist()
    assert boundary.tolist() == [0, 0, 0, 0] and blens.tolist() == [0] * 4
