"""The oracle against its stored regression fixture (CPU).

The fixture was written by tests/golden/make_golden.py from the oracle itself;
it guards the oracle against unintended changes, while the independent pins
live in test_oracle_pins.py."""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_golden  # noqa: E402


def test_oracle_matches_stored_fixture():
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small_seed11.json")
    with open(path) as f:
        stored = json.load(f)
    live = make_golden.build()
    assert live["kv_len"] == stored["kv_len"]
    for a, b in zip(live["rows"], stored["rows"]):
        assert a["indices"] == b["indices"]
        assert a["score_sum"] == b["score_sum"]
        np.testing.assert_array_equal(np.float32(a["out_sample"]), np.float32(b["out_sample"]))
        assert abs(a["out_abs_sum"] - b["out_abs_sum"]) <= 1e-9 * max(1.0, b["out_abs_sum"])
