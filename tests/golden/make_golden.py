"""Writes tests/golden/tiny_oracle.json: the oracle's verify and commit
results on the seeded tiny workload (two requests, two heads, head dim 16,
three draft tokens, fp32), for both gate kinds.

The pages print no worked numeric example, so this fixture is a regression
pin of the oracle itself: it is produced by this script, which calls only
the `oracle` package and the seeded input generators, never the HIP library.
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(
    __file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from workloads import make_workload, to_f64  # noqa: E402


def run(gate):
    wl = make_workload("tiny", gates=[gate])
    L = wl.layers[0]
    res = oracle.conv_update_verify(
        mixed_qkv=to_f64(L.mixed_qkv), raw_gate=to_f64(L.raw_gate),
        raw_beta=to_f64(L.raw_beta), A_log=to_f64(L.A_log),
        dt_bias=to_f64(L.dt_bias), state=to_f64(L.state),
        correction=to_f64(L.correction), key_gate=to_f64(L.key_gate),
        out=np.zeros((wl.T, wl.H * wl.D)),
        conv_state=to_f64(wl.conv_state_dim_first(0)),
        conv_weight=to_f64(L.conv_weight),
        query_start_loc=wl.query_start_loc.numpy(),
        state_indices=wl.state_indices.numpy(),
        num_accepted_tokens=wl.num_accepted_tokens.numpy(),
        spec_query_len=wl.Q, use_lower_bound=gate is not None,
        lower_bound=gate or 0.0)
    (new, _), = oracle.commit(
        layers=[dict(state=to_f64(L.state), correction=res["correction"],
                     key_gate=res["key_gate"], A_log=to_f64(L.A_log),
                     dt_bias=to_f64(L.dt_bias),
                     use_lower_bound=gate is not None,
                     lower_bound=gate or 0.0)],
        state_indices=wl.state_indices.numpy(),
        commit_lens=wl.commit_lens.numpy(), spec_query_len=wl.Q)
    slots = [int(s) for s in wl.state_indices]
    return {
        "out": res["out"].tolist(),
        "committed": {str(s): new[s].tolist() for s in slots},
        "correction": {str(s): res["correction"][s].tolist() for s in slots},
    }


if __name__ == "__main__":
    data = {"workload": "tiny", "softplus": run(None), "lower_bound_-5": run(-5.0)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(data, f)
    print("wrote", path)
