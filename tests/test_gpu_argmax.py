"""GPU: the argmax is integer work and must be exact — ties go to the lowest index, and a NaN among
the logits is reported instead of being ranked.

The tiny model's LM head is rebuilt so that the outcome is known exactly: every row is zero except
rows i1 < j1, which are the same vector v, and rows i2 < j2, which are -v. The logits are then
exactly 0 except v.h at i1 and j1 and -v.h at i2 and j2, bit-identical within each pair (the same
row arithmetic on the same input). Whatever the hidden state h, the greedy token is the lowest
index of a tied maximum: i1 when v.h > 0, i2 when v.h < 0, and 0 when v.h == 0. An all-zero head
ties every index, so the token is 0.
"""
import sys

import numpy as np
import pytest

import oracle as orc
import persistent_megakernel_03_amd as mk
import seeded_inputs as si
from parity_util import gpu_step, make_gpu

pytestmark = pytest.mark.gpu

I1, J1, I2, J2 = 1000, 3071, 517, 4000


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tie_weights(zero_head=False):
    w = si.gen_weights(si.TINY)
    head = np.zeros_like(w["lm_head"])
    if not zero_head:
        v = si.normal_bf16(si.tensor_seed("tiny", "tie-row"), si.TINY.d_model, 0.0, 0.5)
        head[I1] = head[J1] = v
        head[I2] = head[J2] = v ^ np.uint16(0x8000)   # -v: the sign bit flipped
    w["lm_head"] = head
    return w


def expected_token(logits):
    top = logits.max()
    return int(np.nonzero(logits == top)[0][0])


@pytest.mark.parametrize("zero_head", [False, True])
def test_ties_go_to_the_lowest_index(zero_head):
    w = tie_weights(zero_head)
    prompt = si.prompt_tokens(si.WORKLOADS["tiny"])
    log("case: tied LM-head rows (zero head: %s)" % zero_head)
    dec, _ = make_gpu(si.TINY, w, 48)
    om = orc.OracleModel(si.TINY, w, 1, 48)
    seen = set()
    for i, t in enumerate(prompt[:12]):
        d_tok, logits = gpu_step(dec, int(t))
        o_tok, o_logits = om.step(0, int(t), i)
        if zero_head:
            assert (logits == 0).all() and d_tok == 0
        else:
            assert logits[I1] == logits[J1] and logits[I2] == logits[J2], "tied rows gave different bits"
            assert logits[I1] == -logits[I2]
            rest = np.delete(logits, [I1, J1, I2, J2])
            assert (rest == 0).all()
        assert d_tok == expected_token(logits), "step %d: device token %d is not the lowest tied maximum" % (i, d_tok)
        assert d_tok == o_tok, "step %d: device %d, oracle %d" % (i, d_tok, o_tok)
        seen.add(d_tok)
    log("  tokens seen:", sorted(seen))
    if not zero_head:
        assert seen <= {0, I1, I2} and seen & {I1, I2}
    dec.close(); om.close()


@pytest.mark.parametrize("nan_bits", [0x7FC0, 0xFFC0])
def test_nan_logit_is_reported(nan_bits):
    # a NaN weight in one LM-head row makes that logit NaN; the step reports it as a device fault
    # (either sign of NaN), and the context decodes again once the weights are good
    w = si.gen_weights(si.TINY)
    bad = dict(w)
    head = w["lm_head"].copy()
    head[777, 5] = nan_bits
    bad["lm_head"] = head
    log("case: NaN in LM-head row 777 (bits 0x%04x)" % nan_bits)
    dec, _ = make_gpu(si.TINY, bad, 48)
    dec.tokens[0] = 3
    dec.step(dec.tokens, 1, dec.tokens.clone())
    with pytest.raises(mk.MKError) as e:
        dec.sync_check()
    assert e.value.status == -6 and "NaN" in str(e.value)
    dec.load_weights(w)
    dec.set_ctx_lens([0])
    tok, logits = gpu_step(dec, 3)
    assert np.isfinite(logits).all() and tok == int(np.argmax(logits))
    dec.close()


def test_batched_ties_go_to_the_lowest_index():
    # four sequences through the batched (MFMA) path with the tied head: each sequence's token is the
    # lowest index of the maximum of its own logits (exact), and the oracle's token wherever the tied
    # pair came out bit-equal (a batched tile may sum a row group split between two waves in two
    # parts, so identical rows need not give identical bits there)
    import torch
    from parity_util import prefilled_case
    wl = si.WORKLOADS["tiny_b4"]
    log("case: tiny_b4 with the tied LM head")
    w = tie_weights()
    dec, om, ctx, table, _ = prefilled_case(wl, 3, weights=w)
    out = torch.zeros(4, dtype=torch.int32, device=dec.dev)
    toks = si.first_tokens(wl).astype(np.int64)
    for i in range(3):
        dec.tokens[:4] = torch.as_tensor(toks, dtype=torch.int32)
        dec.step(dec.tokens, 4, out)
        dev = out.cpu().numpy()
        for s in range(4):
            logits = dec.read_logits(s)
            assert int(dev[s]) == expected_token(logits)
            o_tok, _ = om.step(s, int(toks[s]), int(ctx[s]) + i)
            if logits[I1] == logits[J1] and logits[I2] == logits[J2]:
                assert int(dev[s]) == o_tok
            toks[s] = o_tok
    dec.close(); om.close()
