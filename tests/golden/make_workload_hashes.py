"""Record SHA-256 digests of the small synthetic workloads' bytes.

Calls only the shared input generator (workloads/); writes
tests/golden/workload_sha256.json.  Run from the repository root:
    python tests/golden/make_workload_hashes.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402


def main():
    rec = {}
    for name in ("tiny_n32_fp32", "crop_n256"):
        w = W.make_inputs(name)
        rec[name] = {t: hashlib.sha256(np.ascontiguousarray(getattr(w, t)).tobytes()).hexdigest()
                     for t in ("q", "k", "v", "bias")}
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_sha256.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
