"""GPU: chunked prefill (mk_prefill through the batched graph, R positions of one sequence per step)
against the oracle run over the same prompt one position at a time.

Bars: every cached key and value within one bf16 ulp of the oracle's (plus 1e-5 of the head row's
scale), equal on > 99% of elements; the last prompt token's logits within 5e-3 relative L2 and no
further from the fp64 oracle than twice the oracle's fp32 build (floor 1e-5); the returned token is
the argmax of the device's logits and the oracle's token unless that is a near-tie; the context
length grows by the prompt length exactly; decode steps that follow meet the same bars.
"""
import sys

import numpy as np
import pytest

import oracle as orc
import persistent_megakernel_03_amd as mk
import seeded_inputs as si
from parity_util import (BUG_FLOOR, REL_L2_BAR, cached_weights, capacity_blocks, check_kv, gpu_step, prefilled_case,
                         rel_l2)

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_chunked(shape, weights, n_positions, rows, paging="permuted"):
    nb = capacity_blocks(n_positions)
    cfg = mk.make_config(shape, max_seqs=1, max_blocks_per_seq=nb, num_blocks=nb, prefill_rows=rows)
    dec = mk.Decoder(cfg, 0)
    dec.load_weights(weights)
    if paging == "permuted":
        table = si.permutation(si.tensor_seed(shape.name, "prefill-pages"), nb).reshape(1, nb)
    else:
        table = np.arange(nb, dtype=np.int32).reshape(1, nb)
    dec.set_page_table(table)
    dec.set_ctx_lens([0])
    return dec, table


def oracle_prompt(om, seq, prompt, start, o32=None):
    """The oracle over the prompt from position `start`; returns (token, logits, fp32 build's rel L2)."""
    tok = logits = None
    r32 = 0.0
    for i, t in enumerate(prompt):
        tok, logits = om.step(seq, int(t), start + i)
        if o32 is not None:
            r32 = max(r32, rel_l2(o32.step(seq, int(t), start + i)[1], logits))
    return tok, logits, r32


def check_last(dec, d_tok, o_tok, o_logits, r32, seq=0, what=""):
    logits = dec.read_logits(seq)
    rel = rel_l2(logits, o_logits)
    bar = max(BUG_FLOOR, 2.0 * r32) if r32 > 0 else REL_L2_BAR
    log("  %s last-token logits rel L2 %.3e (fp32 oracle %.3e), token %d / oracle %d" % (what, rel, r32, d_tok, o_tok))
    assert rel <= REL_L2_BAR and rel <= bar
    assert d_tok == int(np.argmax(logits))
    if d_tok != o_tok:
        srt = np.sort(o_logits)
        assert srt[-1] - srt[-2] < 1e-3, "token disagreement is not a near-tie"


def prefill(dec, prompt, seq=0):
    import torch
    out = torch.full((1,), -1, dtype=torch.int32, device=dec.dev)
    dec.prefill(list(prompt), out, seq=seq)
    return int(out.item())


@pytest.fixture(scope="module")
def tiny():
    return si.gen_weights(si.TINY), si.prompt_tokens(si.WORKLOADS["tiny"])


@pytest.mark.parametrize("rows", [16, 4])
def test_tiny_chunked_prefill(tiny, rows):
    # 16 prompt tokens in chunks of 16 or 4 positions, then decode steps on the cache it built
    w, prompt = tiny
    m = si.TINY
    n_pos = 48
    log("case: tiny, prompt %d, prefill_rows %d, permuted pages" % (len(prompt), rows))
    dec, table = make_chunked(m, w, n_pos, rows)
    om = orc.OracleModel(m, w, 1, n_pos)
    o32 = orc.OracleModel(m, w, 1, n_pos, precision="f32")
    d_tok = prefill(dec, prompt)
    o_tok, o_logits, r32 = oracle_prompt(om, 0, prompt, 0, o32)
    assert int(dec.ctx_lens.item()) == len(prompt)
    check_last(dec, d_tok, o_tok, o_logits, r32, what="prefill")
    check_kv(dec, table[0], om, 0, m, 0, len(prompt))
    tok = o_tok
    for i in range(6):
        d_tok, d_logits = gpu_step(dec, tok)
        o_tok, o_logits = om.step(0, tok, len(prompt) + i)
        assert rel_l2(d_logits, o_logits) <= REL_L2_BAR and d_tok == int(np.argmax(d_logits))
        tok = o_tok
    check_kv(dec, table[0], om, 0, m, 0, len(prompt) + 6)
    dec.close(); om.close(); o32.close()


def test_tiny_prefill_in_pieces_and_ragged(tiny):
    # a 35-token prompt in three calls (5, 19 and 11 tokens; chunks of 16 start mid-block and end ragged),
    # each continuing from the length the one before left
    w, _ = tiny
    m = si.TINY
    prompt = si.uniform_int(si.tensor_seed("tiny", "prefill-pieces"), 35, 0, m.vocab - 1)
    log("case: tiny, prompt 35 in pieces 5 + 19 + 11, prefill_rows 16")
    dec, table = make_chunked(m, w, 48, 16)
    om = orc.OracleModel(m, w, 1, 48)
    at = 0
    for n in (5, 19, 11):
        piece = prompt[at:at + n]
        d_tok = prefill(dec, piece)
        o_tok, o_logits, _ = oracle_prompt(om, 0, piece, at)
        at += n
        assert int(dec.ctx_lens.item()) == at
        check_last(dec, d_tok, o_tok, o_logits, 0.0, what="piece of %d" % n)
    check_kv(dec, table[0], om, 0, m, 0, at)
    dec.close(); om.close()


def test_tiny_prefill_errors(tiny):
    w, prompt = tiny
    log("case: tiny, prefill argument checks")
    dec, _ = make_chunked(si.TINY, w, 48, 16)
    dec.set_ctx_lens([40])
    with pytest.raises(mk.MKError) as e:       # 40 + 16 positions do not fit a 48-position cache
        dec.prefill(list(prompt))
    assert e.value.status == -1
    with pytest.raises(mk.MKError) as e:
        dec.prefill([0, si.TINY.vocab])
    assert e.value.status == -1
    with pytest.raises(mk.MKError) as e:
        dec.prefill([1, 2], seq=1)
    assert e.value.status == -1
    assert int(dec.ctx_lens.item()) == 40       # nothing ran
    dec.set_ctx_lens([0])
    prefill(dec, prompt[:3])
    assert int(dec.ctx_lens.item()) == 3
    dec.close()


def test_batched_context_prefill_leaves_other_sequences():
    # four sequences with pre-filled caches; sequence 2 takes an 11-token prompt in chunks of 4 positions.
    # Its cache and logits match the oracle; the other sequences' caches, lengths and logits are untouched.
    import torch
    wl = si.WORKLOADS["tiny_b4"]
    m = wl.model
    log("case: tiny_b4, prefill of sequence 2 (11 tokens, chunks of 4)")
    dec, om, ctx, table, w = prefilled_case(wl, 12)
    first = torch.as_tensor(si.first_tokens(wl), dtype=torch.int32, device=dec.dev)
    dec.tokens[:4].copy_(first)
    dec.step(dec.tokens, 4, dec.tokens)          # one step of all four: every logits row is written
    toks0 = si.first_tokens(wl)
    for s in range(4):
        om.step(s, int(toks0[s]), int(ctx[s]))
    logits_before = [dec.read_logits(s) for s in range(4)]
    lens_before = dec.ctx_lens.cpu().numpy().copy()
    pools_before = [p.cpu().numpy().copy() for p in dec.k_pools + dec.v_pools]
    prompt = si.uniform_int(si.tensor_seed("tiny_b4", "prefill"), 11, 0, m.vocab - 1)
    d_tok = prefill(dec, prompt, seq=2)
    o_tok, o_logits, _ = oracle_prompt(om, 2, prompt, int(lens_before[2]))
    lens = dec.ctx_lens.cpu().numpy()
    assert lens[2] == lens_before[2] + 11
    assert (np.delete(lens, 2) == np.delete(lens_before, 2)).all()
    check_last(dec, d_tok, o_tok, o_logits, 0.0, seq=2, what="sequence 2")
    for s in (0, 1, 3):
        assert np.array_equal(dec.read_logits(s), logits_before[s])
    check_kv(dec, table[2], om, 2, m, int(lens_before[2]), int(lens[2]))
    # outside sequence 2's blocks, nothing in the pools changed
    nb = (int(lens[2]) + 15) // 16
    mine = set(int(b) for b in table[2, :nb])
    for before, pool in zip(pools_before, dec.k_pools + dec.v_pools):
        a = before.reshape(-1, m.n_kv_heads * 16 * m.head_dim)
        b = pool.cpu().numpy().reshape(-1, m.n_kv_heads * 16 * m.head_dim)
        others = [i for i in range(a.shape[0]) if i not in mine]
        assert np.array_equal(a[others], b[others])
    dec.close(); om.close()


def test_qwen_shape_chunked_prefill():
    # QKV bias and the tied LM head, 39-token prompt (16 + 16 + 7), then 4 decode steps
    wl = si.WORKLOADS["qwen0.5b"]
    m = wl.model
    w = si.gen_weights(m)
    prompt = si.prompt_tokens(wl)
    n_pos = wl.prompt_len + 8
    log("case: qwen0.5b shape, prompt %d, prefill_rows 16" % len(prompt))
    dec, table = make_chunked(m, w, n_pos, 16)
    om = orc.OracleModel(m, w, 1, n_pos)
    o32 = orc.OracleModel(m, w, 1, n_pos, precision="f32")
    d_tok = prefill(dec, prompt)
    o_tok, o_logits, r32 = oracle_prompt(om, 0, prompt, 0, o32)
    check_last(dec, d_tok, o_tok, o_logits, r32, what="qwen prefill")
    check_kv(dec, table[0], om, 0, m, 0, len(prompt), layers=[0, m.n_layers // 2, m.n_layers - 1], o32=o32)
    tok = o_tok
    for i in range(4):
        d_tok, d_logits = gpu_step(dec, tok)
        o_tok, o_logits = om.step(0, tok, len(prompt) + i)
        assert rel_l2(d_logits, o_logits) <= REL_L2_BAR and d_tok == int(np.argmax(d_logits))
        tok = o_tok
    dec.close(); om.close(); o32.close()


def test_llama8b_chunked_prefill():
    # the 8B shape with the cache the decode benchmark uses (35 blocks): the 39-token prompt in three
    # steps of the 16-row graph, then 4 decode steps on the batch-1 graph
    wl = si.WORKLOADS["llama8b"]
    m = wl.model
    w = cached_weights(m)
    prompt = si.prompt_tokens(wl)
    n_pos = wl.prompt_len + wl.steps
    log("case: llama8b shape, prompt %d, prefill_rows 16, cache %d positions" % (len(prompt), n_pos))
    dec, table = make_chunked(m, w, n_pos, 16)
    om = orc.OracleModel(m, w, 1, n_pos)
    d_tok = prefill(dec, prompt)
    o_tok, o_logits, _ = oracle_prompt(om, 0, prompt, 0)
    check_last(dec, d_tok, o_tok, o_logits, 0.0, what="8B prefill")
    check_kv(dec, table[0], om, 0, m, 0, len(prompt), layers=[0, m.n_layers - 1])
    tok = o_tok
    for i in range(4):
        d_tok, d_logits = gpu_step(dec, tok)
        o_tok, o_logits = om.step(0, tok, len(prompt) + i)
        rel = rel_l2(d_logits, o_logits)
        log("  decode step %d: rel L2 %.3e" % (i, rel))
        assert rel <= REL_L2_BAR and d_tok == int(np.argmax(d_logits))
        tok = o_tok
    dec.close(); om.close()
