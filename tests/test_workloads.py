"""The seeded workloads are what the parity tests and the bench were run on: each named workload's
canonical inputs hash to the values stored in tests/golden/workload_fingerprints.json (written by
make_workload_fingerprints.py beside it from the generator alone). A changed generator, seed or
shape fails here before it can shift any measured or compared number."""
import json
import os

import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_fingerprints.json")


def test_every_workload_has_a_fingerprint():
    assert set(json.load(open(GOLDEN))) == set(workloads.WORKLOADS)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_fingerprint(name):
    assert workloads.fingerprint(workloads.get(name)) == json.load(open(GOLDEN))[name]


def test_fingerprint_sees_a_changed_seed():
    import dataclasses
    wl = workloads.get("tiny")
    assert workloads.fingerprint(dataclasses.replace(wl, seed=wl.seed + 1))["x"] != workloads.fingerprint(wl)["x"]
