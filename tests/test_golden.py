"""The oracle's tiny-workload outputs against the stored digest (regression anchor)."""
import json
import os

from tests.golden.make_golden import compute


def test_tiny_oracle_digest_unchanged():
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_digest.json")) as f:
        stored = json.load(f)
    assert compute() == stored
