"""Write workload_digests.json: sha256 of every array of the seeded synthetic
workloads (configurations 1-5 at a small bag count, and the 4- and 5-core
workloads), so that any change to the input generator is detected.  Calls the
input generator only.  Run from the repository root:
    python tests/golden/make_workload_digests.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from tensor_train_compressed_gather_amd import workloads as W  # noqa: E402

CASES = [("config", 1, None), ("config", 2, 64), ("config", 3, 64), ("config", 4, 8), ("config", 5, 8),
         ("kcore", "k4", 16), ("kcore", "k5", 16)]


def digests():
    out = {}
    for kind, which, bags in CASES:
        w = W.make_workload(which, bags=bags) if kind == "config" else W.make_kcore_workload(which, bags=bags)
        out[f"{kind}:{which}:{bags}"] = {"name": w.name, "nnz": int(w.nnz), "sha256": w.digest()}
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "workload_digests.json"), "w") as f:
        json.dump(digests(), f, indent=1, sort_keys=True)
        f.write("\n")
