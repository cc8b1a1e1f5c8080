"""The oracle still reproduces its frozen tiny-chain output (tests/golden/tiny_chain.json).

The fixture is written by tests/golden/make_golden.py, which calls only the
oracle and the seeded input generator.
"""
import json
import os

import numpy as np

from tests.golden.make_golden import tiny_chain_record


def test_tiny_chain_matches_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_chain.json")
    with open(path) as f:
        want = json.load(f)
    got = tiny_chain_record()
    assert got["sha256"] == want["sha256"]
    assert got["z_sf_words_row0"] == want["z_sf_words_row0"]
    assert np.array_equal(np.array(got["out64_row0_first8"]), np.array(want["out64_row0_first8"]))
