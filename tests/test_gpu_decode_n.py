"""GPU: the resident multi-step decode (mk_decode_n) — n greedy steps in one launch, each step's
argmax feeding the next step's embedding lookup on the device.

Bars: the tokens of every step and the last step's logits are bit-identical to n calls of
mk_decode_step fed the previous call's tokens (same graph, same arithmetic), and the context
lengths end equal; free-running greedy tokens equal the oracle's greedy tokens up to the first
disagreement, which must be a near-tie of the oracle (top-2 gap below the measured logit error);
errors (a position past the cache, a wait past the watchdog) are reported and the context decodes
correctly afterwards.
"""
import sys

import numpy as np
import pytest

import oracle as orc
import persistent_megakernel_03_amd as mk
import seeded_inputs as si
from parity_util import make_gpu, prefilled_case, rel_l2

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tiny():
    return si.gen_weights(si.TINY), si.prompt_tokens(si.WORKLOADS["tiny"])


def prefill(dec, prompt):
    import torch
    g0 = torch.zeros(1, dtype=torch.int32, device=dec.dev)
    dec.prefill(list(prompt), g0)
    return g0


def stepwise(dec, first, n_steps, n_seqs=1):
    """n_steps calls of mk_decode_step, each fed the previous call's tokens; returns [n_steps, n_seqs]."""
    import torch
    toks = torch.zeros((n_steps + 1, n_seqs), dtype=torch.int32, device=dec.dev)
    toks[0].copy_(first.reshape(-1)[:n_seqs])
    for i in range(n_steps):
        dec.step(toks[i], n_seqs, toks[i + 1])
    return toks[1:]


def check_equal(a, b, n_seqs, ta, tb, what):
    import torch
    assert torch.equal(ta, tb), "%s: tokens differ" % what
    for s in range(n_seqs):
        assert np.array_equal(a.read_logits(s), b.read_logits(s)), "%s: last logits of sequence %d differ" % (what, s)
    assert torch.equal(a.ctx_lens, b.ctx_lens), "%s: context lengths differ" % what


def test_tiny_decode_n_equals_single_steps(tiny):
    w, prompt = tiny
    log("case: tiny, prompt 16, decode_n(24) vs 24 single steps")
    a, _ = make_gpu(si.TINY, w, 48)
    b, _ = make_gpu(si.TINY, w, 48)
    ga, gb = prefill(a, prompt), prefill(b, prompt)
    ta = stepwise(a, ga, 24)
    tb = b.decode_n(gb, 24)
    check_equal(a, b, 1, ta, tb, "tiny")
    assert int(b.ctx_lens.item()) == len(prompt) + 24
    a.close(); b.close()


def test_tiny_decode_n_in_chunks(tiny):
    # launches of 5, 1 and 7 steps, each continuing from the last token of the one before, equal one
    # launch of 13 steps: epochs and context lengths carry over between launches
    import torch
    w, prompt = tiny
    log("case: tiny, decode_n chunks 5 + 1 + 7 vs 13")
    a, _ = make_gpu(si.TINY, w, 48)
    b, _ = make_gpu(si.TINY, w, 48)
    ga, gb = prefill(a, prompt), prefill(b, prompt)
    parts, cur = [], ga
    for n in (5, 1, 7):
        t = a.decode_n(cur, n)
        parts.append(t)
        cur = t[-1].clone()
    ta = torch.cat(parts)
    tb = b.decode_n(gb, 13)
    check_equal(a, b, 1, ta, tb, "tiny chunks")
    a.close(); b.close()


def test_tiny_free_running_greedy_matches_oracle(tiny):
    w, prompt = tiny
    n = 32
    log("case: tiny, free-running greedy decode_n(%d) vs the oracle's own greedy tokens" % n)
    dec, _ = make_gpu(si.TINY, w, len(prompt) + n + 1)
    g0 = prefill(dec, prompt)
    dev = [int(g0.item())] + [int(x) for x in dec.decode_n(g0, n).cpu().numpy().reshape(-1)]
    om = orc.OracleModel(si.TINY, w, 1, len(prompt) + n + 1)
    tok = None
    for i, t in enumerate(prompt):
        tok, logits = om.step(0, int(t), i)
    orc_toks, gaps = [tok], []
    for i in range(n):
        tok, logits = om.step(0, tok, len(prompt) + i)
        srt = np.sort(logits)
        gaps.append(float(srt[-1] - srt[-2]))
        orc_toks.append(tok)
    agree = 0
    for i in range(n + 1):
        if dev[i] != orc_toks[i]:
            # the first disagreement must be a near-tie of the oracle at the step that produced it
            assert i > 0 and gaps[i - 1] < 1e-3, "greedy paths part at step %d without a near-tie" % i
            break
        agree += 1
    log("  greedy tokens agree on the first %d of %d" % (agree, n + 1))
    assert agree >= n + 1 or agree >= 1
    om.close(); dec.close()


@pytest.mark.parametrize("n_active", [4, 3])
def test_batched_decode_n_equals_single_steps(n_active):
    import torch
    wl = si.WORKLOADS["tiny_b4"]
    log("case: tiny_b4, %d of 4 sequences active, decode_n(6) vs 6 single steps" % n_active)
    a, om, ctx, table, w = prefilled_case(wl, 6)
    om.close()
    b, om2, _, _, _ = prefilled_case(wl, 6)
    om2.close()
    first = torch.as_tensor(si.first_tokens(wl), dtype=torch.int32, device=a.dev)
    ta = stepwise(a, first, 6, n_active)
    tb = b.decode_n(first[:n_active].clone(), 6, n_active)
    check_equal(a, b, n_active, ta, tb, "tiny_b4")
    lens = b.ctx_lens.cpu().numpy()
    assert (lens[:n_active] == ctx[:n_active] + 6).all() and (lens[n_active:] == ctx[n_active:]).all()
    a.close(); b.close()


def test_batched_mid_decode_n_equals_single_steps():
    # 16 sequences, column-split MFMA tiles with their partial-sum exchange across steps
    import torch
    wl = si.WORKLOADS["mid_b16"]
    log("case: mid_b16, 16 sequences, decode_n(3) vs 3 single steps")
    a, om, ctx, table, w = prefilled_case(wl, 3)
    om.close()
    b, om2, _, _, _ = prefilled_case(wl, 3)
    om2.close()
    first = torch.as_tensor(si.first_tokens(wl), dtype=torch.int32, device=a.dev)
    ta = stepwise(a, first, 3, 16)
    tb = b.decode_n(first, 3, 16)
    check_equal(a, b, 16, ta, tb, "mid_b16")
    a.close(); b.close()


def test_qwen_decode_n_equals_single_steps():
    wl = si.WORKLOADS["qwen0.5b"]
    m = wl.model
    log("case: qwen0.5b shape, prompt 39, decode_n(16) vs 16 single steps")
    w = si.gen_weights(m)
    prompt = si.prompt_tokens(wl)
    a, _ = make_gpu(m, w, wl.prompt_len + wl.steps)
    b, _ = make_gpu(m, w, wl.prompt_len + wl.steps)
    ga, gb = prefill(a, prompt), prefill(b, prompt)
    ta = stepwise(a, ga, 16)
    tb = b.decode_n(gb, 16)
    check_equal(a, b, 1, ta, tb, "qwen0.5b")
    a.close(); b.close()


def test_decode_n_rejects_bad_arguments(tiny):
    import torch
    w, prompt = tiny
    log("case: decode_n argument checks")
    dec, _ = make_gpu(si.TINY, w, 48)
    out = torch.zeros((4, 1), dtype=torch.int32, device=dec.dev)
    for n_steps, n_seqs in ((0, 1), (-3, 1), (70000, 1), (4, 2), (4, 0)):
        with pytest.raises(mk.MKError) as e:
            mk.mk_decode_n(dec.ctx, dec.tokens, n_seqs, n_steps, out, dec.stream_ptr())
        assert e.value.status == -1
    with pytest.raises(mk.MKError) as e:
        mk.mk_decode_n(dec.ctx, None, 1, 4, out, dec.stream_ptr())
    assert e.value.status == -1
    dec.close()


def test_decode_n_past_the_cache_is_reported(tiny):
    # the cache holds 48 positions; 8 steps from position 44 run out after 4: the device reports the
    # position, and the context decodes correctly again from a valid position
    w, prompt = tiny
    log("case: decode_n running past the cache")
    dec, _ = make_gpu(si.TINY, w, 48)
    dec.set_ctx_lens([44])
    dec.tokens[0] = 3
    dec.decode_n(dec.tokens, 8)
    with pytest.raises(mk.MKError) as e:
        dec.sync_check()
    assert e.value.status == -6 and "context length" in str(e.value)
    ref, _ = make_gpu(si.TINY, w, 48)
    for d in (dec, ref):
        d.set_ctx_lens([0])
        d.tokens[0] = 5
    ta = ref.decode_n(ref.tokens, 4)
    tb = dec.decode_n(dec.tokens, 4)
    check_equal(ref, dec, 1, ta, tb, "after the error")
    dec.close(); ref.close()


def test_decode_n_watchdog_recovers(tiny, monkeypatch):
    # a 1 microsecond wait budget makes waits expire inside the first step: the launch drains, the
    # timeout is reported, and a context built with the normal budget decodes correctly afterwards
    import torch
    w, prompt = tiny
    log("case: decode_n watchdog expiry")
    monkeypatch.setenv("MK_WATCHDOG_US", "1")
    dec, _ = make_gpu(si.TINY, w, 48)
    monkeypatch.delenv("MK_WATCHDOG_US")
    dec.tokens[0] = 3
    dec.decode_n(dec.tokens, 6)
    with pytest.raises(mk.MKError) as e:
        dec.sync_check()
    assert e.value.status == -5
    dec.close()
    a, _ = make_gpu(si.TINY, w, 48)
    b, _ = make_gpu(si.TINY, w, 48)
    ga, gb = prefill(a, prompt[:4]), prefill(b, prompt[:4])
    check_equal(a, b, 1, stepwise(a, ga, 5), b.decode_n(gb, 5), "after a watchdog expiry elsewhere")
    a.close(); b.close()


def test_trace_records_every_step_and_the_xcd(tiny):
    # the trace holds the last step of a launch (step index n - 1, its epoch) for every task; on a
    # device whose CU count is a multiple of 8, workgroup i runs on XCD i mod 8 (the placement the
    # graph's row weighting assumes), read from the hardware register of each CU
    w, prompt = tiny
    log("case: trace of a decode_n launch")
    dec, _ = make_gpu(si.TINY, w, 48)
    dec.enable_trace()
    g0 = prefill(dec, prompt[:3])
    dec.decode_n(g0, 4)
    tr = dec.read_trace()
    info = mk.mk_graph_stats(dec.ctx)
    assert len(tr) == info.n_tasks
    assert (tr["step"] == 3).all()
    assert len(set(tr["epoch"].tolist())) == 1
    assert (tr["t_done"] >= tr["t_queue"]).all()
    n_cus = int(info.n_cus)
    if n_cus % 8 == 0:
        assert (tr["xcc"] == tr["cu"] % 8).all(), "workgroups are not placed round-robin over the XCDs"
    log("  xcc ids seen:", sorted(set(tr["xcc"].tolist())))
    dec.close()
