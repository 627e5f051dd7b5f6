"""Writes tests/golden/workload_fingerprints.json: the sha256 of every named workload's canonical
inputs (workloads.fingerprint), from the seeded generator alone. Run after a deliberate change of the
generator or of a workload's definition:  python tests/golden/make_workload_fingerprints.py"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import workloads  # noqa: E402


def main():
    out = {name: workloads.fingerprint(wl) for name, wl in sorted(workloads.WORKLOADS.items())}
    path = os.path.join(ROOT, "tests", "golden", "workload_fingerprints.json")
    json.dump(out, open(path, "w"), indent=1, sort_keys=True)
    print(f"{len(out)} workloads -> {path}")


if __name__ == "__main__":
    main()
