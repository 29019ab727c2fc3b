"""Regression pin: the oracle still reproduces tests/golden/small_pack_oracle.json."""
import json
import os

import numpy as np

from tests.golden import make_golden


def test_oracle_matches_stored_values():
    path = os.path.join(os.path.dirname(make_golden.__file__), "small_pack_oracle.json")
    stored = json.load(open(path))["values"]
    now = make_golden.compute()
    for name in ("o", "lse", "dq", "dk", "dv"):
        a = np.array([np.nan if x is None else x for x in stored[name]])
        b = np.array([np.nan if x is None else x for x in now[name]])
        assert np.array_equal(np.isnan(a), np.isnan(b)), name
        m = ~np.isnan(a)
        assert np.max(np.abs(a[m] - b[m])) <= 1e-12, name
