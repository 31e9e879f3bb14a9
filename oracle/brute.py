"""Scalar brute-force KDA verify/commit for tiny cases.  TEST INFRASTRUCTURE
ONLY.

Written separately from `kda.py` (no shared helpers) with plain Python
loops and the `math` module, following the ops page's `_kda_gate`,
`_kda_recurrent_step`, `_kda_recoverssm_verify_kernel` and
`_commit_kda_state_kernel` and the conv update of the kernels page.  Used to
cross-check the vectorised oracle on tiny shapes; it is far too slow for
anything else.
"""
from __future__ import annotations

import math


def _sig(x):
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def _gate(raw, bias, A, use_lb, lb):
    x = raw + bias
    if use_lb:
        return lb * _sig(A * x)
    if x > 20.0:
        return -A * x
    return -A * math.log1p(math.exp(x))


def verify_one(*, S0, xs, history, weight, raw_gates, raw_betas, dt_bias,
               A_log, use_lb, lb, H, K):
    """One request.

    S0[h][v][k]: checkpoint.  xs[t][c]: raw projections, c < 3HK.
    history[c][j]: the W-1 conv inputs before xs[0] (oldest first).
    weight[c][j]: taps, j = W-1 multiplies the newest input.
    raw_gates[t][h*K+k], raw_betas[t][h].

    Returns (outs[t][h*K+v], corr[h][t][v], keys[h][t][k]) where keys are the
    post-conv raw keys.
    """
    W = len(weight[0])
    C = 3 * H * K
    q = len(xs)
    # conv + silu per channel and position
    y = [[0.0] * C for _ in range(q)]
    for c in range(C):
        stream = list(history[c]) + [xs[t][c] for t in range(q)]
        for t in range(q):
            acc = 0.0
            for j in range(W):
                acc += weight[c][j] * stream[t + j]
            y[t][c] = acc * _sig(acc)
    outs = [[0.0] * (H * K) for _ in range(q)]
    corr = [[[0.0] * K for _ in range(q)] for _ in range(H)]
    keys = [[[0.0] * K for _ in range(q)] for _ in range(H)]
    for h in range(H):
        S = [[S0[h][v][k] for k in range(K)] for v in range(K)]
        A = math.exp(A_log[h])
        for t in range(q):
            qv = [y[t][h * K + i] for i in range(K)]
            kv = [y[t][H * K + h * K + i] for i in range(K)]
            vv = [y[t][2 * H * K + h * K + i] for i in range(K)]
            kn = math.sqrt(sum(x * x for x in kv) + 1e-6)
            khat = [x / kn for x in kv]
            qn = math.sqrt(sum(x * x for x in qv) + 1e-6)
            qhat = [x / qn / math.sqrt(K) for x in qv]
            d = [math.exp(_gate(raw_gates[t][h * K + i], dt_bias[h][i], A,
                                use_lb, lb)) for i in range(K)]
            beta = _sig(raw_betas[t][h])
            for v in range(K):
                for k in range(K):
                    S[v][k] *= d[k]
            c = []
            for v in range(K):
                u = 0.0
                for k in range(K):
                    u += S[v][k] * khat[k]
                c.append(beta * (vv[v] - u))
            for v in range(K):
                for k in range(K):
                    S[v][k] += c[v] * khat[k]
            for v in range(K):
                o = 0.0
                for k in range(K):
                    o += S[v][k] * qhat[k]
                outs[t][h * K + v] = o
            corr[h][t] = c
            keys[h][t] = kv
    return outs, corr, keys


def fold_one(*, S0, corr, keys, raw_gates, dt_bias, A_log, use_lb, lb):
    """Commit of one head: apply n recorded positions in order to S0[v][k].
    corr[t][v], keys[t][k], raw_gates[t][k]."""
    K = len(S0[0])
    S = [row[:] for row in S0]
    A = math.exp(A_log)
    for t in range(len(corr)):
        kn = math.sqrt(sum(x * x for x in keys[t]) + 1e-6)
        khat = [x / kn for x in keys[t]]
        for v in range(len(S)):
            for k in range(K):
                d = math.exp(_gate(raw_gates[t][k], dt_bias[k], A, use_lb, lb))
                S[v][k] = S[v][k] * d + corr[t][v] * khat[k]
    return S
