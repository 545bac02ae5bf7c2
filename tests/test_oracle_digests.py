"""The oracle's outputs on the seeded tiny workloads must not drift silently."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

from make_oracle_digests import digests  # noqa: E402


def test_oracle_digests_unchanged():
    stored = {}
    with open(os.path.join(HERE, "golden", "oracle_digests.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                stored[k] = v
    now = digests()
    assert set(now) == set(stored)
    changed = [k for k in now if now[k] != stored[k]]
    assert not changed, changed
