"""Writes tests/golden/input_hashes.json: content hashes of the seeded workloads.

These pin the input generator's reproducibility (same seed -> same bytes); they
are not expected outputs of the method.  Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import moe_synth as ms  # noqa: E402

hashes = {name: ms.make_workload(name).content_hash() for name in ("tiny", "mid")}
with open(os.path.join(HERE, "input_hashes.json"), "w") as f:
    json.dump({"_about": "sha256[:16] of x, router W, records and shared record per config (seed 0)",
               "hashes": hashes}, f, indent=2)
print(hashes)
