"""The oracle still reproduces its stored tiny-workload record (written by
tests/golden/make_golden.py, which calls only the oracle)."""
import json
import os

from tests.golden.make_golden import record

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_golden_record():
    with open(os.path.join(HERE, "golden", "tiny_seed0.json")) as f:
        want = json.load(f)
    got = json.loads(json.dumps(record()))
    assert got["z32"] == want["z32"]
    for a, b in zip(got["heads"], want["heads"]):
        assert a["counts"] == b["counts"] and a["stats"] == b["stats"]
        assert a["idx_sha1"] == b["idx_sha1"]
        assert abs(a["lse"] - b["lse"]) < 1e-12 and abs(a["out_l2"] - b["out_l2"]) < 1e-12
