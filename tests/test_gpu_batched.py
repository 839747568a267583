"""GPU parity of batched decode: several sequences per step, the GEMVs as 16-wide MFMA tiles.

Each sequence starts from its own pre-filled, randomly paged KV cache (N(0, 1) bf16 K/V at
positions < its context length) and a seeded first token. After every step, each active
sequence's logits are compared with the oracle stepping that sequence alone (teacher-forced:
the oracle's greedy token feeds both sides). Bars: logits within 5e-3 relative L2; the device
token equals the argmax of the device's own logits (exact); the device token equals the
oracle's on >= 99% of (sequence, step) pairs, every disagreement a near-tie; context lengths
of the active sequences advance by one per step and those of inactive ones do not move.
"""
import sys

import numpy as np
import pytest

import seeded_inputs as si
from parity_util import REL_L2_BAR, cached_weights, prefilled_case, rel_l2

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_batched(wl, n_decode, n_active=None, attn_splits=0, weights=None, capacity=None):
    import torch
    n = wl.n_seqs
    na = n if n_active is None else n_active
    dec, om, ctx, table, w = prefilled_case(wl, n_decode, attn_splits=attn_splits, weights=weights, capacity=capacity)
    toks = si.first_tokens(wl).astype(np.int64).copy()
    rels, agree, gaps_bad = [], [], []
    out = torch.zeros(n, dtype=torch.int32, device=dec.dev)
    for i in range(n_decode):
        dec.tokens[:n] = torch.as_tensor(toks, dtype=torch.int32)
        dec.step(dec.tokens, na, out)
        dev_tok = out.cpu().numpy()
        for s in range(na):
            o_tok, o_logits = om.step(s, int(toks[s]), int(ctx[s]) + i)
            d_logits = dec.read_logits(s)
            rels.append(rel_l2(d_logits, o_logits))
            assert int(dev_tok[s]) == int(np.argmax(d_logits)), "seq %d step %d: token is not the logits' argmax" % (s, i)
            agree.append(int(dev_tok[s]) == o_tok)
            if int(dev_tok[s]) != o_tok:
                srt = np.sort(o_logits)
                gaps_bad.append(float(srt[-1] - srt[-2]))
            toks[s] = o_tok
    dec.sync_check()
    lens = dec.ctx_lens.cpu().numpy()
    assert (lens[:na] == ctx[:na] + n_decode).all()
    assert (lens[na:] == ctx[na:]).all()
    rels = np.array(rels)
    log("%s: %d active of %d, %d steps: max rel L2 %.3e mean %.3e, token agreement %.3f" %
        (wl.name, na, n, n_decode, rels.max(), rels.mean(), np.mean(agree)))
    assert rels.max() <= REL_L2_BAR
    assert np.mean(agree) >= 0.99
    assert all(g < 1e-3 for g in gaps_bad)
    dec.close()
    om.close()
    return rels


def test_tiny_four_sequences():
    log("case: tiny_b4, 4 sequences, 6 steps")
    run_batched(si.WORKLOADS["tiny_b4"], 6)


def test_tiny_inactive_sequences():
    # 4 sequences configured, 3 run: the fourth keeps its context length
    log("case: tiny_b4, 3 of 4 sequences active, 3 steps")
    run_batched(si.WORKLOADS["tiny_b4"], 3, n_active=3)


def test_mid_sixteen_sequences_column_splits():
    # 256 CUs: the GEMVs split their columns over 4..16 CUs and exchange partial sums
    log("case: mid_b16, 16 sequences, 3 steps, column-split tiles")
    run_batched(si.WORKLOADS["mid_b16"], 3)


def test_mid_sixteen_sequences_row_tiles(monkeypatch):
    # one column split per tile: every task streams its columns in 512-column blocks
    monkeypatch.setenv("MK_BATCHED_MAX_KSPLIT", "1")
    log("case: mid_b16, 16 sequences, 2 steps, row tiles only")
    run_batched(si.WORKLOADS["mid_b16"], 2)


def test_mid_long_contexts_several_pieces_per_task():
    # one split per KV head (64 attention tasks) over contexts 300..1847: the cut by cost gives tasks
    # two whole segments, or the end of a segment (merged last) plus whole segments plus a partial
    log("case: mid_b16_long, 16 sequences, 2 steps, 64 attention tasks")
    run_batched(si.WORKLOADS["mid_b16_long"], 2, attn_splits=1)


@pytest.mark.timeout(900)
def test_llama8b_sixteen_sequences():
    # the 8B shape at full size, 16 sequences with contexts in [512, 8192], on the cache and graph the
    # benchmark times (each cache sized for the workload's 128 steps)
    wl = si.WORKLOADS["llama8b_b16"]
    n = 4
    log("case: llama8b_b16 full size, 16 sequences, %d steps" % n)
    run_batched(wl, n, weights=cached_weights(wl.model), capacity=si.context_lengths(wl) + wl.steps)


def test_mid_staged_launch_matches_fused():
    # batched: one dispatch per dependency stage gives the same logits and tokens, bit for bit
    import torch
    wl = si.WORKLOADS["mid_b16"]
    log("case: mid_b16 staged launch vs one launch")
    a, om, ctx, table, w = prefilled_case(wl, 2)
    om.close()
    b, om2, _, _, _ = prefilled_case(wl, 2)
    om2.close()
    n = wl.n_seqs
    toks = torch.as_tensor(si.first_tokens(wl), dtype=torch.int32)
    for i in range(2):
        a.tokens[:n] = toks
        b.tokens[:n] = toks
        oa = torch.zeros(n, dtype=torch.int32, device=a.dev)
        ob = torch.zeros(n, dtype=torch.int32, device=b.dev)
        a.step(a.tokens, n, oa)
        b.step_staged(b.tokens, n, ob)
        for s in range(n):
            assert np.array_equal(a.read_logits(s), b.read_logits(s)), "step %d seq %d" % (i, s)
        assert torch.equal(oa, ob)
        toks = oa.cpu()
    a.close()
    b.close()
