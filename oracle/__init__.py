"""Plain fp64 CPU oracle for the KDA RecoverSSM speculative verify and commit.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check of
`__graft_entry__` and the CPU-baseline leg of `bench.py` use it.  It shares
no code with the HIP library (no kernels, headers, helpers or constants).

Sources (the vLLM Kimi-K3 pages):
  * ops page   -- `vLLM/vllm/models/kimi_k3/nvidia/ops/recoverssm.py` source;
  * kernels page -- `vllm.models.kimi_k3.nvidia.recoverssm.kernels` API page;
  * state page -- `vllm.models.kimi_k3.nvidia.specialized_decode.recoverssm.
    state` API page.

Parity status: every function below is pinned by the `-m "not gpu"` tests in
tests/test_oracle_*.py (closed forms, special cases, a library convolution,
a brute-force scalar implementation, an exact rational-arithmetic case and
the algebraic identity between the verify recurrence and the commit fold).
The commit plan, the boundary fold and the conv compaction are pinned by
multi-step simulations against a fresh recurrence over the accepted stream.
"""
from .kda import (  # noqa: F401
    EPS,
    SOFTPLUS_THRESHOLD,
    commit,
    commit_fold_reverse,
    commit_plan,
    compact_conv_state,
    conv_update,
    conv_update_verify,
    delta_step,
    kda_gate,
    l2_normalize,
    normalize_query,
    round_to,
    sigmoid,
    silu,
    verify_qkv,
)
