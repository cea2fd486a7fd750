"""The oracle still reproduces the digests its generator script stored."""
import json
import os

import golden.make_golden as mg


def test_oracle_matches_stored_digests():
    with open(mg.OUT) as f:
        stored = json.load(f)
    assert mg.digests() == stored
