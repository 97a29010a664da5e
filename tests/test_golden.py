"""The oracle still produces the recorded outputs on the small cells
(tests/golden/oracle_digests.json, written by tests/golden/make_golden.py).
A deliberate change to the oracle's arithmetic regenerates that file."""
import json
import os

from golden import make_golden


def test_oracle_matches_recorded_digests():
    with open(make_golden.OUT) as f:
        recorded = json.load(f)
    now = make_golden.compute()
    assert set(now) == set(recorded)
    changed = sorted(k for k in now if now[k] != recorded[k])
    assert not changed, f"oracle output changed on: {changed}"
