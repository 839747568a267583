"""Writes graph_hashes.json: the FNV-1a hash of the task graph each workload's decoder runs, built on
the host for 256 compute units (an MI355X) with the cache sized exactly as the benchmark and the
parity tests size it (every workload's full decode: prompt or pre-filled context plus all its steps).

These hashes pin that the builder is deterministic across processes and machines and that a change
to it is deliberate (the script is re-run and the new file committed with it). They are not parity
values: what the graph computes is checked by the validator, the simulator and the GPU parity tests.

Run from the repository root:  python tests/golden/make_graph_hashes.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import persistent_megakernel_03_amd as mk  # noqa: E402
import seeded_inputs as si  # noqa: E402

N_CUS = 256
NAMES = ["tiny", "qwen0.5b", "llama8b", "llama8b_long", "llama8b_b16", "tiny_b4", "mid_b16"]


def workload_config(wl):
    """The decoder config of a workload's full decode: one sequence with a prompt uses an identity table of
    ceil((prompt + steps) / 16) blocks; pre-filled workloads use their block tables for context + steps."""
    m = wl.model
    if wl.prompt_len > 0:
        nb = (wl.prompt_len + wl.steps + 15) // 16
        return mk.make_config(m, max_seqs=1, max_blocks_per_seq=nb, num_blocks=nb)
    cap = si.context_lengths(wl).astype(np.int64) + wl.steps
    table, nblocks = si.block_tables(wl, cap)
    return mk.make_config(m, max_seqs=wl.n_seqs, max_blocks_per_seq=table.shape[1], num_blocks=nblocks)


def graph_entry(name, n_cus=N_CUS):
    cfg = workload_config(si.WORKLOADS[name])
    ctx = mk.mk_create_host(cfg, n_cus)
    try:
        info = mk.mk_graph_stats(ctx)
        return {"n_cus": n_cus, "hash": "0x%016x" % info.hash, "n_tasks": int(info.n_tasks),
                "attn_tasks": int(info.attn_tasks), "max_blocks_per_seq": int(cfg.max_blocks_per_seq),
                "num_blocks": int(cfg.num_blocks)}
    finally:
        mk.mk_destroy(ctx)


def main():
    os.environ.pop("MK_BATCHED_MAX_KSPLIT", None)
    out = {"what": "task-graph hashes per workload (mk_graph_stats.hash), host-built for %d CUs" % N_CUS,
           "graphs": {name: graph_entry(name) for name in NAMES}}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "graph_hashes.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
