"""Writes the stored expected values under tests/golden/ that come from the oracle.

Calls only ``oracle/`` (and the seeded input builders); nothing here touches
the GPU path.  Re-run after a deliberate change to the oracle or the input
recipe, and say in the commit which passage justifies the change.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def tiny_fp32_expected():
    b = workloads.tiny_fp32()
    k_pool, v_pool = oracle.ref_reshape_and_cache(b.k_new, b.v_new, b.slot_mapping, b.k_pool, b.v_pool)
    out = oracle.ref_paged_attention_decode(b.q, k_pool, v_pool, b.block_tables, b.context_lens, b.scale, b.dtype)
    return {
        "about": "Oracle output (float64) of the tiny fp32 workload (seed 3721) after its cache write; "
                 "regression guard for the oracle and the input recipe, written by make_golden.py.",
        "seed": b.seed,
        "context_lens": b.context_lens.tolist(),
        "expected": [[[float(repr_v) for repr_v in row] for row in head] for head in out.tolist()],
    }


if __name__ == "__main__":
    path = os.path.join(HERE, "oracle_tiny_fp32.json")
    with open(path, "w") as f:
        json.dump(tiny_fp32_expected(), f, indent=0)
    print("wrote", path)
