"""The oracle still reproduces its stored tiny-workload results
(tests/golden/tiny_oracle.json, written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

from tests.golden.make_golden import run

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_stored_tiny_results():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        data = json.load(f)
    for key, gate in (("softplus", None), ("lower_bound_-5", -5.0)):
        now = run(gate)
        np.testing.assert_allclose(np.array(now["out"]),
                                   np.array(data[key]["out"]), rtol=0,
                                   atol=1e-12)
        for s, v in data[key]["committed"].items():
            np.testing.assert_allclose(np.array(now["committed"][s]),
                                       np.array(v), rtol=0, atol=1e-12)
