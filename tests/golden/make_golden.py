"""Writes tiny_oracle_samples.json from the fp64 oracle (no GPU, no HIP code)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from exact_attention_state_amd import synth  # noqa: E402

ROWS = [0, 5, 63, 80, 87, 95, 96, 127]


def build():
    wl = synth.WORKLOADS["tiny"]
    p = synth.params(wl)
    cfg = oracle.Layer0Config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.rope_theta, wl.rms_eps)
    ids = synth.initial_ids(wl)
    ref = oracle.refresh(p, cfg, ids, wl.table())
    ids1, blk = synth.step_ids(wl, ids, 1)
    step = oracle.cached_step(p, cfg, ref, blk, wl.table())
    return {
        "workload": "tiny", "rows": ROWS,
        "ids_sum": int(np.sum(ids)), "ids1_sum": int(np.sum(ids1)),
        "refresh_out_row_head0_first4": [ref["out"][r, 0, :4].tolist() for r in ROWS],
        "refresh_lse": [ref["lse"][r].tolist() for r in ROWS],
        "step1_out_row_head1_first4": [step["out"][r, 1, :4].tolist() for r in ROWS],
        "step1_lse": [step["lse"][r].tolist() for r in ROWS],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle_samples.json"), "w") as f:
        json.dump(build(), f, indent=1)
