"""The oracle's outputs on the tiny workload match the digests stored by
tests/golden/make_golden.py (a regression guard on the oracle itself: any later
change to its arithmetic must regenerate them and say why)."""
import json
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_golden  # noqa: E402


def test_tiny_digests_unchanged():
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_512x256.json")) as f:
        want = json.load(f)
    got = make_golden.tiny_outputs()
    for key, value in got.items():
        assert want[key] == value, key
