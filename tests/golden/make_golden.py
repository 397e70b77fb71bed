"""Writes tests/golden/tiny_oracle_digest.json from the CPU oracle only.

The digest anchors the oracle's outputs on the tiny workload (8 experts,
top-2, hidden 256, intermediate 128, 16 tokens, seed 0) so that any later
change to the oracle's arithmetic shows up as a test failure and has to be
justified.  It is produced by this script alone; nothing from the HIP path
enters it.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def compute() -> dict:
    d = synth.make_workload("tiny", seed=0)
    wl = d["wl"]
    inputs = {k: digest(d[k]) for k in ("X", "topk_ids", "topk_weights", "codes13", "scales13",
                                         "codes2", "scales2")}
    r = oracle.moe_forward(d["X"], d["topk_ids"], d["topk_weights"], wl.E_global,
                           d["expert_map"], d["codes13"], d["scales13"], d["codes2"],
                           d["scales2"], intermediates=True)
    al = oracle.moe_align(d["topk_ids"], wl.E_global, wl.E_local, 16, d["expert_map"])
    outs = {k: digest(r[k]) for k in ("Y13", "Z", "Y2", "out")}
    outs["sorted_ids"] = digest(al["sorted_ids"])
    outs["expert_ids"] = digest(al["expert_ids"])
    outs["num_tokens_padded"] = al["num_tokens_padded"]
    first = [int(v) for v in r["out"][0, :8]]
    return {"workload": "tiny seed 0", "inputs": inputs, "outputs": outs,
            "out_row0_first8_bf16_bits": first}


if __name__ == "__main__":
    path = os.path.join(HERE, "tiny_oracle_digest.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1, sort_keys=True)
    print("wrote", path)
