"""Writes generator_hashes.json: SHA-256 of the bytes the seeded workload
generator (workloads/) produces on the CPU for two small workloads, one
contiguous and planted, one paged.  It calls only the generator; no value
comes from the HIP library or the oracle.

    python tests/golden/make_generator_hashes.py
"""

import hashlib
import json
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from workloads import make_custom  # noqa: E402

CASES = {
    "contiguous_planted": dict(seq_lens=[3000, 1200, 70000], seed=11, plant=True),
    "paged_prefill": dict(seq_lens=[500, 130], seed=12, paged=True, prefill=True),
}
FIELDS = ("q_idx", "w", "k_idx", "q_mla", "kv", "q_seq", "q_nvis", "row0", "block_table")


def digests(wl):
    out = {}
    for f in FIELDS:
        t = getattr(wl, f)
        if t is not None:
            out[f] = hashlib.sha256(t.contiguous().view(-1).view(torch.uint8).numpy().tobytes()).hexdigest()
    return out


def compute():
    return {name: digests(make_custom(device="cpu", **kw)) for name, kw in CASES.items()}


if __name__ == "__main__":
    data = {"generator": "workloads.make_custom on the CPU (torch CPU generator, one seed per 65536-row chunk)",
            "torch": torch.__version__, "cases": {k: {"args": v} for k, v in CASES.items()}}
    for name, d in compute().items():
        data["cases"][name]["sha256"] = d
    with open(os.path.join(HERE, "generator_hashes.json"), "w") as f:
        json.dump(data, f, indent=1)
    print("written")
