"""Pins of the fp64 oracle's building blocks against closed forms and special
cases that the mathematics fixes (no GPU).

Each test states the fact it checks.  The facts are chosen so that a dropped
term, a wrong sign or a transposed operand in the oracle fails at least one.
"""
import math

import numpy as np
import pytest

from oracle import (EPS, delta_step, kda_gate, l2_normalize,
                    normalize_query, round_to, sigmoid, silu)

RNG = np.random.default_rng(1234)


# ---- gate (ops page, `_kda_gate`) -------------------------------------------

def test_softplus_gate_at_zero_is_minus_A_ln2():
    for A in (1.0, 3.7, 16.0):
        g = kda_gate(np.zeros(5), np.zeros(5), A, False, 0.0)
        np.testing.assert_allclose(g, -A * math.log(2.0), rtol=0, atol=1e-15)


def test_softplus_gate_is_identity_above_threshold():
    x = np.array([20.5, 25.0, 100.0])
    g = kda_gate(x, np.zeros(3), 2.5, False, 0.0)
    np.testing.assert_array_equal(g, -2.5 * x)


def test_softplus_gate_below_threshold_and_bias_is_added():
    raw = np.array([-3.0, 0.5, 19.0])
    bias = np.array([1.0, -0.25, 0.5])
    x = raw + bias
    expect = -1.5 * np.array([math.log(1 + math.exp(v)) for v in x])
    np.testing.assert_allclose(kda_gate(raw, bias, 1.5, False, 0.0), expect,
                               rtol=1e-15)


def test_softplus_gate_far_negative_is_minus_A_exp():
    x = np.array([-30.0, -50.0])
    g = kda_gate(x, np.zeros(2), 4.0, False, 0.0)
    np.testing.assert_allclose(g, -4.0 * np.exp(x), rtol=1e-12)


def test_lower_bound_gate_limits():
    lb = -5.0
    big = kda_gate(np.array([1e3]), np.zeros(1), 2.0, True, lb)
    small = kda_gate(np.array([-1e3]), np.zeros(1), 2.0, True, lb)
    mid = kda_gate(np.array([0.0]), np.zeros(1), 2.0, True, lb)
    assert big[0] == lb
    assert small[0] == 0.0
    assert mid[0] == lb / 2
    # lb = 0: the gate vanishes whatever the input ("gate 0").
    g0 = kda_gate(RNG.normal(size=8), RNG.normal(size=8), 3.0, True, 0.0)
    assert np.all(g0 == 0.0)


def test_lower_bound_gate_uses_A_times_x():
    raw, bias, A, lb = 0.3, 0.2, 4.0, -5.0
    expect = lb / (1 + math.exp(-A * (raw + bias)))
    got = kda_gate(np.array([raw]), np.array([bias]), A, True, lb)[0]
    assert abs(got - expect) < 1e-15


@pytest.mark.parametrize("use_lb", [False, True])
def test_decay_in_unit_interval(use_lb):
    raw = RNG.normal(size=1000) * 3
    bias = RNG.normal(size=1000) * 0.1
    d = np.exp(kda_gate(raw, bias, 7.0, use_lb, -5.0))
    assert np.all(d > 0) and np.all(d <= 1)


def test_sigmoid_and_silu():
    assert sigmoid(0.0) == 0.5
    assert sigmoid(800.0) == 1.0 and sigmoid(-800.0) == 0.0
    np.testing.assert_allclose(sigmoid(np.array([1.0])), 1 / (1 + math.e ** -1))
    np.testing.assert_allclose(silu(np.array([2.0])), 2 / (1 + math.e ** -2))


# ---- normalisation -----------------------------------------------------------

def test_key_normalisation_norm_identity():
    k = RNG.normal(size=(6, 16))
    n2 = np.sum(k * k, axis=-1)
    got = np.sum(l2_normalize(k) ** 2, axis=-1)
    np.testing.assert_allclose(got, n2 / (n2 + EPS), rtol=1e-14)
    # direction unchanged
    cos = np.sum(l2_normalize(k) * k, -1) / np.sqrt(n2) / np.sqrt(got)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)


def test_query_normalisation_carries_inverse_sqrt_K():
    q = RNG.normal(size=(3, 32))
    n2 = np.sum(q * q, axis=-1)
    qh = normalize_query(q)
    np.testing.assert_allclose(np.sum(qh * qh, -1), n2 / (32 * (n2 + EPS)),
                               rtol=1e-14)


def test_zero_vector_normalises_to_zero():
    assert np.all(l2_normalize(np.zeros(8)) == 0.0)


# ---- one delta-rule step (ops page, `_kda_recurrent_step`) -------------------

def _rand_step(V=8, K=8):
    S = RNG.normal(size=(V, K)) * 0.3
    k = RNG.normal(size=K)
    v = RNG.normal(size=V)
    return S, k, v


def test_gate_zero_saturated_beta_writes_value():
    # With no decay and sigmoid(beta) = 1, S' k_hat = v up to the epsilon:
    # S' k_hat = v - (v - S k_hat) * eps / (|k|^2 + eps).
    S, k, v = _rand_step()
    S1, c = delta_step(S, k, v, np.zeros(8), 50.0)
    kh = l2_normalize(k)
    n2 = np.sum(k * k)
    expect = v - (v - S @ kh) * EPS / (n2 + EPS)
    np.testing.assert_allclose(S1 @ kh, expect, rtol=0, atol=1e-13)
    assert np.max(np.abs(S1 @ kh - v)) < 1e-6 * np.max(np.abs(v - S @ kh)) + 1e-15


def test_beta_minus_infinity_gate_zero_keeps_state_bitwise():
    S, k, v = _rand_step()
    S1, c = delta_step(S, k, v, np.zeros(8), -800.0)
    assert np.array_equal(S1, S)
    assert np.all(c == 0.0)


def test_decay_acts_along_K_columns():
    # With beta -> -inf the step is a pure decay: S'[v,k] = S[v,k] exp(g[k]).
    S, k, v = _rand_step(V=5, K=7)
    g = -RNG.uniform(0, 2, size=7)
    S1, _ = delta_step(S, k, v, g, -800.0)
    np.testing.assert_allclose(S1, S * np.exp(g)[None, :], rtol=1e-15)


def test_single_position_closed_form():
    # Q = 1: S' = S D + s (v - S D k_hat) k_hat^T and
    # o = S' q_hat = S D q_hat + s (v - S D k_hat)(k_hat . q_hat).
    S, k, v = _rand_step(V=6, K=10)
    q = RNG.normal(size=10)
    g = -RNG.uniform(0, 1, size=10)
    rb = 0.37
    s = 1 / (1 + math.exp(-rb))
    S1, c = delta_step(S, k, v, g, rb)
    D = np.diag(np.exp(g))
    kh = k / math.sqrt(k @ k + EPS)
    qh = q / math.sqrt(q @ q + EPS) / math.sqrt(10)
    corr = s * (v - S @ D @ kh)
    np.testing.assert_allclose(c, corr, rtol=1e-13)
    np.testing.assert_allclose(S1, S @ D + np.outer(corr, kh), rtol=1e-13)
    o = S1 @ normalize_query(q)
    np.testing.assert_allclose(o, S @ D @ qh + corr * (kh @ qh), rtol=1e-12,
                               atol=1e-15)


def test_textbook_delta_rule_orthonormal_keys():
    # No decay, beta = 1, orthonormal keys: after writing (k_i, v_i) in order,
    # S k_i = v_i for every i (the delta rule stores each association exactly
    # and orthogonal later writes do not disturb it), up to the epsilon.
    K, n = 12, 5
    Qm, _ = np.linalg.qr(RNG.normal(size=(K, K)))
    keys = Qm[:, :n].T
    vals = RNG.normal(size=(n, K))
    S = RNG.normal(size=(K, K))
    for i in range(n):
        S, _ = delta_step(S, keys[i], vals[i], np.zeros(K), 60.0)
    for i in range(n):
        np.testing.assert_allclose(S @ keys[i], vals[i], atol=1e-5)


def test_batched_step_matches_per_head():
    S = RNG.normal(size=(3, 4, 5))
    k = RNG.normal(size=(3, 5))
    v = RNG.normal(size=(3, 4))
    g = -RNG.uniform(size=(3, 5))
    rb = RNG.normal(size=3)
    Sb, cb = delta_step(S, k, v, g, rb)
    for h in range(3):
        Sh, ch = delta_step(S[h], k[h], v[h], g[h], rb[h])
        np.testing.assert_allclose(Sb[h], Sh, rtol=1e-15)
        np.testing.assert_allclose(cb[h], ch, rtol=1e-15)


# ---- storage rounding ---------------------------------------------------------

def test_round_to_bf16_is_rne_on_fp32_bits():
    import torch
    x = RNG.normal(size=2000) * 10
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) \
        .to(torch.float64).numpy()
    assert np.array_equal(round_to(x, "bf16"), ref)
    assert np.array_equal(round_to(x, "f32"), x.astype(np.float32))
    # ties go to even: 1 + 2^-8 is halfway between two bf16 values
    assert round_to(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0
    assert round_to(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6
