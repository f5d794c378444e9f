"""Writes worklist_digests.json: SHA-256 of the work list of every workload and
edge case, computed with the Python twin in oracle/worklist.py only."""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

from oracle import worklist as twin  # noqa: E402
from worklist_cases import CASES, hp_dict  # noqa: E402

if __name__ == "__main__":
    out = {k: hashlib.sha256(twin.build(d, hp_dict(hp))).hexdigest() for k, (d, hp) in CASES.items()}
    with open(os.path.join(HERE, "worklist_digests.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(f"wrote {len(out)} digests")
