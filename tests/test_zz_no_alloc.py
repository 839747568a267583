"""GPU: mk_decode_step_static, the decode step for callers that cannot allocate, against
mk_decode_step on the same inputs.

Two calls in a row through the C ABI, the second with a smaller input: first a 4-sequence batched
step (the larger graph and working memory), then a one-sequence step of a smaller model, whose
call finds the static array holding the first call's leftovers. Each call's logits, tokens and
context lengths must equal, bit for bit, those of mk_decode_step on a context bound to its own
scratch buffer, given the same state (the same kernel and graph run in both). A graph whose
scratch exceeds the static array is refused with MK_ERR_SHAPE before anything runs.
"""
import sys

import numpy as np
import pytest

import persistent_megakernel_03_amd as mk
import seeded_inputs as si
from parity_util import make_gpu, prefilled_case

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def same_state(a, b, n_seqs, what):
    import torch
    for s in range(n_seqs):
        assert np.array_equal(a.read_logits(s), b.read_logits(s)), "%s: logits of sequence %d differ" % (what, s)
    assert torch.equal(a.ctx_lens, b.ctx_lens), "%s: context lengths differ" % what


def test_static_scratch_step_equals_the_bound_one():
    import torch
    # call 1: four sequences, batched tiles (the larger working memory)
    wl = si.WORKLOADS["tiny_b4"]
    log("case: mk_decode_step_static, tiny_b4 (4 sequences) then tiny (1 sequence)")
    a, om, ctx, table, w = prefilled_case(wl, 2)
    om.close()
    b, om2, _, _, _ = prefilled_case(wl, 2)
    om2.close()
    first = torch.as_tensor(si.first_tokens(wl), dtype=torch.int32, device=a.dev)
    oa = torch.zeros(4, dtype=torch.int32, device=a.dev)
    ob = torch.zeros(4, dtype=torch.int32, device=b.dev)
    big = mk.mk_workspace_size(b.ctx)[2]
    mk.mk_decode_step(a.ctx, first, 4, oa, a.stream_ptr())
    mk.mk_decode_step_static(b.ctx, first, 4, ob, b.stream_ptr())
    b.sync_check()
    assert torch.equal(oa, ob)
    same_state(a, b, 4, "4 sequences")
    a.close(); b.close()
    # call 2: a smaller input, one sequence of the tiny model after a 6-token prompt
    wt = si.gen_weights(si.TINY)
    prompt = si.prompt_tokens(si.WORKLOADS["tiny"])[:6]
    c, _ = make_gpu(si.TINY, wt, 16)
    d, _ = make_gpu(si.TINY, wt, 16)
    assert mk.mk_workspace_size(d.ctx)[2] < big
    for dec in (c, d):
        dec.prefill(list(prompt))
    tok = torch.full((1,), 7, dtype=torch.int32, device=c.dev)
    oc = torch.zeros(1, dtype=torch.int32, device=c.dev)
    od = torch.zeros(1, dtype=torch.int32, device=d.dev)
    mk.mk_decode_step(c.ctx, tok, 1, oc, c.stream_ptr())
    mk.mk_decode_step_static(d.ctx, tok, 1, od, d.stream_ptr())
    d.sync_check()
    assert torch.equal(oc, od)
    same_state(c, d, 1, "1 sequence")
    # and again from the static path's own output, to check the flags restart cleanly
    mk.mk_decode_step(c.ctx, oc, 1, oc, c.stream_ptr())
    mk.mk_decode_step_static(d.ctx, od, 1, od, d.stream_ptr())
    d.sync_check()
    assert torch.equal(oc, od)
    same_state(c, d, 1, "1 sequence, second step")
    c.close(); d.close()


def test_static_scratch_refuses_a_graph_too_large():
    # a cache of 16384 blocks per sequence makes the rotary table alone larger than the 64 MiB array
    import torch
    wt = si.gen_weights(si.TINY)
    cfg = mk.make_config(si.TINY, max_seqs=1, max_blocks_per_seq=16384, num_blocks=4)
    dec = mk.Decoder(cfg, 0)
    assert mk.mk_workspace_size(dec.ctx)[2] > 64 << 20
    dec.load_weights(wt)
    dec.set_page_table(np.arange(16384, dtype=np.int32).reshape(1, -1) % 4)
    dec.set_ctx_lens([0])
    out = torch.zeros(1, dtype=torch.int32, device=dec.dev)
    dec.tokens[0] = 3
    with pytest.raises(mk.MKError) as e:
        mk.mk_decode_step_static(dec.ctx, dec.tokens, 1, out, dec.stream_ptr())
    assert e.value.status == -2 and "static scratch" in str(e.value)
    dec.close()
