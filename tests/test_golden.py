"""The oracle still reproduces its stored small-case outputs (CPU only)."""
import json
import os

import numpy as np

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_small.json")


def test_oracle_matches_stored_fixture():
    with open(HERE) as fh:
        data = json.load(fh)
    assert len(data["cases"]) == len(make_golden.CASES)
    for stored in data["cases"]:
        res = make_golden.compute(stored["case"])
        for key in ("o", "lse", "dq", "dk", "dv"):
            assert np.allclose(np.array(stored[key]), res[key], atol=1e-13, rtol=0), (stored["case"]["name"], key)
