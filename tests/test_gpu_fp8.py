"""GPU: FP8 weights (weight_format = MK_WEIGHTS_FP8_E4M3) against the oracle's FP8 model.

Bars: the codes and row exponents the device quantiser writes equal the oracle's quantiser bit for
bit (integer work); a crafted LM head whose rows hold every finite E4M3 code gives logits equal to
16 * decode(code) * 2^-12 exactly (the streamed decode of every code, subnormals and signs included);
teacher-forced logits within 5e-3 relative L2 of the fp64 oracle run with the exact dequantised
weights, and no further than twice the oracle's fp32 build (floor 4e-5, see FP8_BUG_FLOOR); the device
token is the argmax of its own logits, and every disagreement with the oracle's token is one the
device's own logit error can cause (oracle top-2 gap at most twice the largest logit error); a resident
multi-step launch bit-identical to single steps.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle as orc
import persistent_megakernel_03_amd as mk
import seeded_inputs as si
from parity_util import BUG_FLOOR, REL_L2_BAR, cached_weights, capacity_blocks, check_kv, gpu_step, rel_l2

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# The derived bar's floor for FP8 runs. On weights FP8 represents exactly, the FP8 path and the bf16 path
# multiply the same values; the FP8 path groups each row's sums differently (16 codes per lane, half the
# lanes per row) and lands 2.1e-5 from the fp64 oracle on the tiny model where the bf16 path lands 7.5e-6,
# with every cached key and value of both within one bf16 ulp (the representable-weights test below
# pins that relation). The floor is the bf16 one (1e-5) times four, the factor that test allows.
FP8_BUG_FLOOR = 4 * BUG_FLOOR


def make_fp8(shape, weights, n_positions):
    nb = capacity_blocks(n_positions)
    cfg = mk.make_config(shape, max_seqs=1, max_blocks_per_seq=nb, num_blocks=nb, weight_format=1)
    dec = mk.Decoder(cfg, 0)
    dec.load_weights(weights)
    dec.set_page_table(si.permutation(si.tensor_seed(shape.name, "fp8-pages"), nb).reshape(1, nb))
    dec.set_ctx_lens([0])
    return dec


def matrix_rows(shape, t):
    d, qd = shape.d_model, shape.n_q_heads * shape.head_dim
    return {"wq": (qd, d), "wk": (shape.n_kv_heads * shape.head_dim, d), "wv": (shape.n_kv_heads * shape.head_dim, d),
            "wo": (d, qd), "wg": (shape.d_ffn, d), "wu": (shape.d_ffn, d), "wd": (d, shape.d_ffn)}[t]


def check_codes(dec, shape, weights, names):
    for name in names:
        if name in ("lm_head", "embed"):
            rows, cols = shape.vocab, shape.d_model
            src = weights["embed" if shape.tied_embeddings else "lm_head"]
        else:
            rows, cols = matrix_rows(shape, name.split(".")[-1])
            src = weights[name]
        codes, exps = mk.mk_read_fp8_weights(dec.ctx, name, rows, cols, dec.stream_ptr())
        rc, re_ = orc.fp8_quantize(np.asarray(src).reshape(rows, cols))
        assert np.array_equal(exps, re_), "%s: row exponents differ" % name
        bad = np.nonzero(codes != rc)
        assert bad[0].size == 0, "%s: %d codes differ, first at %s (device %d, oracle %d)" % (
            name, bad[0].size, (bad[0][0], bad[1][0]), codes[bad[0][0], bad[1][0]], rc[bad[0][0], bad[1][0]])


def teacher_forced_fp8(shape, weights, prompt, n_decode, f32=True, min_agree=0.99):
    m8, w8 = orc.fp8_model(shape, weights)
    total = len(prompt) + n_decode
    om = orc.OracleModel(m8, w8, 1, total)
    o32 = orc.OracleModel(m8, w8, 1, total, precision="f32") if f32 else None
    dec = make_fp8(shape, weights, total)
    rels, r32, agree, gaps, linf = [], [], [], [], []
    tok = int(prompt[0])
    for i in range(total):
        if i < len(prompt):
            tok = int(prompt[i])
        o_tok, o_logits = om.step(0, tok, i)
        if o32 is not None:
            r32.append(rel_l2(o32.step(0, tok, i)[1], o_logits))
        d_tok, d_logits = gpu_step(dec, tok)
        rels.append(rel_l2(d_logits, o_logits))
        assert d_tok == int(np.argmax(d_logits))
        srt = np.sort(o_logits)
        gaps.append(srt[-1] - srt[-2])
        linf.append(float(np.abs(d_logits - o_logits).max()))
        agree.append(d_tok == o_tok)
        if d_tok != o_tok:
            log("  step %d: device %d, oracle %d, oracle top-2 gap %.3e, largest logit error %.3e" % (
                i, d_tok, o_tok, gaps[-1], linf[-1]))
        tok = o_tok
    log("  steps %d, max rel L2 %.3e (fp32 oracle %.3e), token agreement %.3f" % (
        total, max(rels), max(r32) if r32 else float("nan"), np.mean(agree)))
    assert max(rels) <= REL_L2_BAR
    if r32:
        assert max(rels) <= max(FP8_BUG_FLOOR, 2 * max(r32))
    # a disagreement is allowed only where the device's own logit error could flip the oracle's top two:
    # with |d - o| < gap / 2 everywhere, the argmax cannot move
    for a, g, e in zip(agree, gaps, linf):
        if not a:
            assert g <= 2 * e, "token disagreement with a top-2 gap (%.3e) above twice the logit error" % g
    assert np.mean(agree) >= min_agree
    om.close()
    if o32 is not None:
        o32.close()
    return dec


@pytest.fixture(scope="module")
def tiny():
    return si.gen_weights(si.TINY), si.prompt_tokens(si.WORKLOADS["tiny"])


def test_tiny_codes_match_the_oracle_quantiser(tiny):
    w, _ = tiny
    log("case: tiny FP8, device codes vs the oracle's quantiser, every matrix")
    dec = make_fp8(si.TINY, w, 48)
    names = ["layers.%d.%s" % (l, t) for l in range(si.TINY.n_layers) for t in orc.FP8_MATRICES] + ["lm_head"]
    check_codes(dec, si.TINY, w, names)
    dec.close()


def test_every_code_streams_exactly():
    # eps = 0, zero O and down projections: the residual stream stays the token's embedding row, here the
    # unit vector e_j, so the LM head's input is exactly 16 e_j (d = 256: 1 / sqrt(1/256) = 16). Every
    # LM-head row holds 448 * 2^-12 in column j2 (its scale exponent is then -12) and, in column j, the
    # value of one finite E4M3 code times 2^-12, cycling through all 254 of them: logit i is exactly
    # 16 * decode(code_i) * 2^-12.
    shape = dataclasses.replace(si.TINY, name="tiny-codes", rms_eps=0.0)
    assert shape.d_model == 256
    w = si.gen_weights(si.TINY)
    for l in range(shape.n_layers):
        w["layers.%d.wo" % l] = np.zeros_like(w["layers.%d.wo" % l])
        w["layers.%d.wd" % l] = np.zeros_like(w["layers.%d.wd" % l])
    j, j2, tok = 77, 200, 5
    emb = w["embed"].copy()
    emb[tok] = 0
    emb[tok, j] = orc.bf16(1.0)
    w["embed"] = emb
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    codes = np.array([finite[i % len(finite)] for i in range(shape.vocab)], dtype=np.int64)
    head = np.zeros((shape.vocab, shape.d_model), dtype=np.uint16)
    head[:, j2] = orc.bf16(448.0 * 2.0 ** -12)
    vals = np.array([orc.fp8_decode(int(c)) for c in codes]) * 2.0 ** -12
    head[:, j] = [orc.bf16(float(v)) for v in vals]
    assert all(orc.from_bf16(int(b)) == v for b, v in zip(head[:300, j], vals[:300]))
    w["lm_head"] = head.reshape(w["lm_head"].shape)
    log("case: tiny, every finite E4M3 code through the LM head")
    dec = make_fp8(shape, w, 48)
    c, e = mk.mk_read_fp8_weights(dec.ctx, "lm_head", shape.vocab, shape.d_model, dec.stream_ptr())
    assert (e == -12).all() and np.array_equal(c[:, j], codes.astype(np.uint8))
    d_tok, logits = gpu_step(dec, tok)
    expect = (16.0 * vals).astype(np.float32)
    bad = np.nonzero(logits != expect)[0]
    assert bad.size == 0, "%d logits differ, first row %d: code 0x%02x gave %r, expected %r" % (
        bad.size, bad[0], codes[bad[0]], logits[bad[0]], expect[bad[0]])
    assert d_tok == int(np.argmax(expect))
    dec.close()


def test_tiny_teacher_forced_fp8(tiny):
    w, prompt = tiny
    log("case: tiny FP8, prompt %d + 16 decode steps, teacher-forced" % len(prompt))
    dec = teacher_forced_fp8(si.TINY, w, prompt, 16)
    dec.close()


def test_fp8_path_tracks_bf16_path_on_representable_weights(tiny):
    # weights that FP8 represents exactly (the oracle's dequantised set): the bf16 path and the FP8 path
    # then multiply the same values, and differ only in summation order and row grouping
    w, prompt = tiny
    m8, w8 = orc.fp8_model(si.TINY, w)
    om = orc.OracleModel(m8, w8, 1, 48)
    a = make_fp8(si.TINY, w8, 48)
    from parity_util import make_gpu
    b, _ = make_gpu(m8, w8, 48)
    worst = [0.0, 0.0, 0.0]
    tok = int(prompt[0])
    for i in range(24):
        if i < len(prompt):
            tok = int(prompt[i])
        o_tok, o_logits = om.step(0, tok, i)
        _, la = gpu_step(a, tok)
        _, lb = gpu_step(b, tok)
        worst = [max(worst[0], rel_l2(la, o_logits)), max(worst[1], rel_l2(lb, o_logits)), max(worst[2], rel_l2(la, lb))]
        tok = o_tok
    log("  FP8 path vs oracle %.3e, bf16 path vs oracle %.3e, FP8 vs bf16 path %.3e" % tuple(worst))
    # every cached key and value of both paths within one bf16 ulp of the oracle's (their QKV GEMVs
    # multiply the same values), > 99% equal
    for dec in (a, b):
        check_kv(dec, np.asarray(dec.page_table.cpu().numpy())[0], om, 0, m8, 0, 24)
    assert worst[0] <= 4 * max(worst[1], BUG_FLOOR) and worst[2] <= 4 * max(worst[1], BUG_FLOOR)
    a.close(); b.close(); om.close()


def test_tiny_fp8_decode_n_equals_single_steps(tiny):
    import torch
    w, prompt = tiny
    log("case: tiny FP8, decode_n(12) vs 12 single steps")
    a = make_fp8(si.TINY, w, 48)
    b = make_fp8(si.TINY, w, 48)
    ga = torch.zeros(1, dtype=torch.int32, device=a.dev)
    gb = torch.zeros(1, dtype=torch.int32, device=b.dev)
    a.prefill(list(prompt), ga)
    b.prefill(list(prompt), gb)
    toks = torch.zeros((13, 1), dtype=torch.int32, device=a.dev)
    toks[0].copy_(ga)
    for i in range(12):
        a.step(toks[i], 1, toks[i + 1])
    tb = b.decode_n(gb, 12)
    assert torch.equal(toks[1:], tb)
    assert np.array_equal(a.read_logits(0), b.read_logits(0))
    a.close(); b.close()


def test_qwen_shape_fp8():
    # QKV bias, odd row and lane counts (K = 896: 16 lanes per row, units padded to an even count), the
    # tied LM head quantised while the embedding lookup stays bf16
    wl = si.WORKLOADS["qwen0.5b"]
    m = wl.model
    w = si.gen_weights(m)
    prompt = si.prompt_tokens(wl)
    log("case: qwen0.5b shape FP8, codes of three matrices, prompt %d + 4 steps" % len(prompt))
    dec = teacher_forced_fp8(m, w, prompt, 4)
    check_codes(dec, m, w, ["layers.0.wq", "layers.%d.wd" % (m.n_layers - 1), "embed"])
    dec.close()


def test_llama8b_fp8():
    wl = si.WORKLOADS["llama8b"]
    m = wl.model
    w = cached_weights(m)
    prompt = si.prompt_tokens(wl)
    log("case: llama8b shape FP8, codes of three matrices, prompt %d + 24 steps" % len(prompt))
    dec = teacher_forced_fp8(m, w, prompt, 24, f32=False, min_agree=0.9)
    check_codes(dec, m, w, ["layers.0.wk", "layers.31.wd", "lm_head"])
    dec.close()
