"""The oracle's frozen output on the 1K-Gaussian workload (see
tests/golden/make_golden.py): any change to its arithmetic shows here."""
import json
import os

import pytest

from tests.golden.make_golden import tiny_forward_record

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_forward_matches_frozen_oracle_record():
    with open(os.path.join(HERE, "golden", "tiny_1k_forward.json")) as f:
        stored = json.load(f)
    now = tiny_forward_record()
    for k, v in stored.items():
        if isinstance(v, float):
            assert now[k] == pytest.approx(v, rel=1e-12), k
        else:
            assert now[k] == v, k
