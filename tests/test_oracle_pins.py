"""Pins of the oracle to facts outside itself: closed forms, special cases, invariants,
library routines on tiny inputs, and the generator's published definition.

Each test names the plausible mistake it would catch.  None of them re-types the
oracle's formula: they check values the mathematics fixes.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle as orc
import seeded_inputs as si

pytestmark = pytest.mark.usefixtures("oracle_lib", "inputs_lib")

RNG = np.random.default_rng(1234)


def rand_bf16(shape, std=1.0):
    x = RNG.normal(0.0, std, size=shape).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64); b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------- generator
def test_generator_matches_published_definition():
    # SplitMix64 output for seed 0 is a published test vector (first output 0xE220A8397B1DCDAF).
    assert si.lib().si_splitmix_out(0, 0) == 0xE220A8397B1DCDAF
    assert si.py_splitmix_out(0, 0) == 0xE220A8397B1DCDAF
    s = si.tensor_seed("tiny", "layers.0.wq")
    a = si.normal_bf16(s, 2000, 0.0, 0.02, offset=123)
    b = np.array([si.py_bf16_from_double(0.02 * si.py_normal_at(s, 123 + i)) for i in range(2000)], np.uint16)
    assert (a == b).all()
    # any slice can be drawn alone
    full = si.normal_bf16(s, 5000, 0.0, 0.02)
    assert (full[123:2123] == a).all()


def test_generator_distribution():
    x = orc.bf16_to_f64(si.normal_bf16(77, 1_000_000, 0.0, 0.02))
    assert abs(x.mean()) < 1e-4 and abs(x.std() - 0.02) < 1e-4
    p = si.permutation(5, 1000)
    assert sorted(p.tolist()) == list(range(1000)) and (p != np.arange(1000)).any()
    t = si.uniform_int(9, 100000, 512, 8192)
    assert t.min() >= 512 and t.max() <= 8192 and abs(t.mean() - 4352) < 40


# --------------------------------------------------------------------------- bf16
def test_bf16_round_to_nearest_even():
    assert orc.bf16(1.0) == 0x3F80 and orc.bf16(-2.0) == 0xC000
    assert orc.bf16(1.0 + 2 ** -8) == 0x3F80            # tie -> even mantissa (down)
    assert orc.bf16(1.0 + 3 * 2 ** -8) == 0x3F82        # tie -> even mantissa (up)
    assert orc.bf16(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81  # above the tie -> up
    for b in [0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000]:
        assert orc.bf16(orc.from_bf16(b)) == b           # exact round trip


# --------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    # constant vector c with unit gain -> c / sqrt(c^2 + eps)  (catches sum-vs-mean, missing eps or sqrt)
    d, c, eps = 256, 0.37, 1e-5
    g = np.full(d, 0x3F80, np.uint16)
    out = orc.rmsnorm(np.full(d, c), g, eps)
    assert np.allclose(out, c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)   # d equal squares: a few ulps
    # (3, 4) with eps 0 -> (3, 4) / sqrt(12.5)
    out = orc.rmsnorm(np.array([3.0, 4.0]), np.array([0x3F80, 0x3F80], np.uint16), 0.0)
    assert np.allclose(out, np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=2e-16, atol=0)
    # the gain multiplies element-wise (catches a dropped or transposed gain)
    gb = np.array([0x4000, 0x3F00], np.uint16)    # 2.0, 0.5
    out = orc.rmsnorm(np.array([3.0, 4.0]), gb, 0.0)
    assert np.allclose(out, np.array([6.0, 2.0]) / math.sqrt(12.5), rtol=2e-16, atol=0)


# --------------------------------------------------------------------------- GEMV
def test_gemv_one_hot_and_bias_and_library():
    n, k = 37, 100
    w = rand_bf16((n, k))
    wf = orc.bf16_to_f64(w)
    for j in [0, 17, k - 1]:
        x = np.zeros(k); x[j] = 1.0
        assert (orc.gemv(w, x) == wf[:, j]).all()            # one-hot picks column j (catches transposition)
    b = rand_bf16((n,))
    assert (orc.gemv(np.zeros((n, k), np.uint16), RNG.normal(size=k), b) == orc.bf16_to_f64(b)).all()
    x = RNG.normal(size=k)
    assert rel(orc.gemv(w, x), wf @ x) < 1e-14                # matrix-vector product (library routine)


# --------------------------------------------------------------------------- RoPE
def test_rope_closed_forms():
    dh, theta = 64, 10000.0
    u = RNG.normal(size=dh)
    assert (orc.rope(u, 0, theta) == u).all()                  # position 0 is the identity
    for p in [1, 7, 1000, 32767]:
        r = orc.rope(u, p, theta)
        h = dh // 2
        assert np.allclose(r[:h] ** 2 + r[h:] ** 2, u[:h] ** 2 + u[h:] ** 2, rtol=1e-13)   # each pair keeps its norm
    # e_0 rotates by angle p into coordinate dh/2 (frequency theta^0 = 1); pairs are (i, i + dh/2)
    e0 = np.zeros(dh); e0[0] = 1.0
    r = orc.rope(e0, 3, theta)
    assert abs(r[0] - math.cos(3)) < 1e-15 and abs(r[dh // 2] - math.sin(3)) < 1e-15
    assert np.count_nonzero(np.abs(r) > 1e-300) == 2
    # e_1 rotates with frequency theta^(-2/dh), toward coordinate 1 + dh/2 (positive direction)
    e1 = np.zeros(dh); e1[1] = 1.0
    r = orc.rope(e1, 5, theta)
    a = 5 * theta ** (-2.0 / dh)
    assert abs(r[1] - math.cos(a)) < 1e-15 and abs(r[1 + dh // 2] - math.sin(a)) < 1e-15
    # e_{dh/2} rotates toward -e_0
    eh = np.zeros(dh); eh[dh // 2] = 1.0
    r = orc.rope(eh, 3, theta)
    assert abs(r[0] + math.sin(3)) < 1e-15 and abs(r[dh // 2] - math.cos(3)) < 1e-15


def test_rope_relative_position():
    dh, theta = 128, 500000.0
    q, k = RNG.normal(size=dh), RNG.normal(size=dh)
    for m_, n_, c in [(5, 2, 100), (40, 39, 32000), (0, 0, 7)]:
        a = orc.rope(q, m_, theta) @ orc.rope(k, n_, theta)
        b = orc.rope(q, m_ + c, theta) @ orc.rope(k, n_ + c, theta)
        assert abs(a - b) < 1e-11 * (1 + abs(a))


# --------------------------------------------------------------------------- softmax / attention
def test_softmax():
    s = RNG.normal(size=50) * 10
    p = orc.softmax(s)
    assert abs(p.sum() - 1.0) < 1e-15 and (p > 0).all()
    assert np.allclose(orc.softmax(s + 1234.5), p, rtol=1e-12)   # shift invariance (max subtraction)
    assert np.allclose(orc.softmax(np.array([0.0, math.log(3.0)])), [0.25, 0.75], rtol=1e-15)


def test_attention_special_cases():
    hq, hk, dh = 4, 2, 16
    q = RNG.normal(size=hq * dh)
    k1, v1 = rand_bf16((1, hk, dh)), rand_bf16((1, hk, dh))
    out = orc.attention(q, k1, v1, hq, hk, dh)
    for h in range(hq):                                          # one key: output is that value, exactly
        assert (out[h * dh:(h + 1) * dh] == orc.bf16_to_f64(v1[0, h // 2])).all()
    kk = np.repeat(rand_bf16((1, hk, dh)), 9, axis=0)            # equal keys: mean of the values
    vv = rand_bf16((9, hk, dh))
    out = orc.attention(q, kk, vv, hq, hk, dh)
    for h in range(hq):
        assert np.allclose(out[h * dh:(h + 1) * dh], orc.bf16_to_f64(vv[:, h // 2]).mean(0), rtol=1e-14, atol=1e-15)
    # two keys: o = v1 + (v2 - v1) * logistic((s2 - s1)), s = q.k / sqrt(dh)  (catches a missing scale)
    k2, v2 = rand_bf16((2, 1, dh)), rand_bf16((2, 1, dh))
    q1 = RNG.normal(size=dh)
    kf, vf = orc.bf16_to_f64(k2[:, 0]), orc.bf16_to_f64(v2[:, 0])
    s1, s2 = q1 @ kf[0] / math.sqrt(dh), q1 @ kf[1] / math.sqrt(dh)
    expect = vf[0] + (vf[1] - vf[0]) / (1.0 + math.exp(-(s2 - s1)))
    assert np.allclose(orc.attention(q1, k2, v2, 1, 1, dh), expect, rtol=1e-13, atol=1e-15)


def test_attention_brute_force_and_gqa_mapping():
    hq, hk, dh, npos = 8, 2, 32, 23
    q = RNG.normal(size=hq * dh)
    kc, vc = rand_bf16((npos, hk, dh)), rand_bf16((npos, hk, dh))
    out = orc.attention(q, kc, vc, hq, hk, dh)
    kf, vf = orc.bf16_to_f64(kc), orc.bf16_to_f64(vc)
    G = hq // hk
    for h in range(hq):                      # materialised scores for head h against KV head h // G
        s = kf[:, h // G] @ q[h * dh:(h + 1) * dh] / math.sqrt(dh)
        w = np.exp(s - s.max()); w /= w.sum()
        assert rel(out[h * dh:(h + 1) * dh], w @ vf[:, h // G]) < 1e-14
        # the same head computed alone with only its KV head (catches h % hk instead of h // G)
        solo = orc.attention(q[h * dh:(h + 1) * dh], kc[:, h // G:h // G + 1], vc[:, h // G:h // G + 1], 1, 1, dh)
        assert rel(out[h * dh:(h + 1) * dh], solo) < 1e-15


# --------------------------------------------------------------------------- SiLU / argmax
def test_silu_and_swiglu():
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 4e-16
    assert abs(orc.silu(40.0) - 40.0) < 1e-14 and abs(orc.silu(-40.0)) < 1e-15
    h = orc.swiglu(np.array([math.log(3.0), 2.0]), np.array([2.0, math.log(3.0)]))
    assert abs(h[0] - 1.5 * math.log(3.0)) < 1e-15             # silu applies to the gate, not to up
    assert abs(h[1] - 2.0 / (1 + math.exp(-2.0)) * math.log(3.0)) < 1e-15


def test_argmax_ties_lowest_index():
    v = np.array([1.0, 5.0, 3.0, 5.0, 5.0])
    assert orc.argmax(v) == 1
    for _ in range(20):
        x = np.round(RNG.normal(size=300), 1)
        assert orc.argmax(x) == int(np.argmax(x))               # numpy returns the first maximum


# --------------------------------------------------------------------------- whole step
SMALL = si.shrink(si.TINY, "pin-small", n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, d_ffn=96,
                  vocab=300)


def _model(shape, gain_std=0.1, w_std=0.08, seed_ns=None, n_seqs=1, max_pos=32, **over):
    w = si.gen_weights(shape, seed_ns=seed_ns, gain_std=gain_std, w_std=w_std)
    w.update(over)
    return orc.OracleModel(shape, w, n_seqs=n_seqs, max_pos=max_pos), w


def test_cached_decode_equals_no_cache_recompute():
    m, _ = _model(SMALL)
    toks = si.uniform_int(3, 12, 0, SMALL.vocab - 1)
    for p, t in enumerate(toks):
        tok, logits = m.step(0, t, p)
        ref_tok, ref = m.forward_nocache(toks[:p + 1])
        assert tok == ref_tok
        assert rel(logits, ref) < 1e-12


def test_zero_blocks_leave_the_embedding():
    # with Wo = Wd = 0 the residual stream stays E[t] -> logits = W_lm RMSNorm(E[t], g_final)
    # (catches a dropped or doubled residual and a wrong final norm)
    zeros = {}
    for l in range(SMALL.n_layers):
        zeros["layers.%d.wo" % l] = np.zeros((SMALL.d_model, SMALL.n_q_heads * SMALL.head_dim), np.uint16)
        zeros["layers.%d.wd" % l] = np.zeros((SMALL.d_model, SMALL.d_ffn), np.uint16)
    m, w = _model(SMALL, **zeros)
    for p, t in enumerate([5, 77, 299]):
        _, logits = m.step(0, t, p)
        e = orc.bf16_to_f64(w["embed"][t])
        expect = orc.gemv(w["lm_head"], orc.rmsnorm(e, w["final_norm"], SMALL.rms_eps))
        assert rel(logits, expect) < 1e-15


def test_position_shift_invariance():
    # attention scores depend on relative positions only (rotary embedding).  The cache stores the
    # *rotated* key in bf16, so a shifted run differs by that rounding (~2^-9 relative per key
    # element, ~1e-3 in the logits); rotating one side only, or with the wrong angle, moves the
    # logits by O(1).  The exact invariance is pinned per vector in test_rope_relative_position.
    m1, _ = _model(SMALL)
    m2, _ = _model(SMALL)
    toks = si.uniform_int(4, 8, 0, SMALL.vocab - 1)
    for p, t in enumerate(toks):
        _, a = m1.step(0, t, p)
        _, b = m2.step(0, t, p, rope_pos=p + 1000)
        assert rel(a, b) < 1e-2


def test_first_position_attends_to_itself():
    # at position 0 the only key is the token's own: attention output = its value row, so the
    # step equals the no-cache forward of one token (covered) and is independent of cache contents
    m, _ = _model(SMALL)
    m.set_kv(0, 0, 1, si.normal_bf16(1, 5 * 2 * 16).reshape(5, 2, 16), si.normal_bf16(2, 5 * 2 * 16).reshape(5, 2, 16))
    _, a = m.step(0, 42, 0)
    _, b = m.forward_nocache([42])
    assert rel(a, b) < 1e-12


def test_gqa_equals_mha_with_repeated_kv_heads():
    g = SMALL
    mha = dataclasses.replace(g, name="pin-mha", n_kv_heads=g.n_q_heads)
    mg, w = _model(g)
    wm = dict(w)
    G = g.n_q_heads // g.n_kv_heads
    for l in range(g.n_layers):
        for t in ("wk", "wv"):
            a = w["layers.%d.%s" % (l, t)].reshape(g.n_kv_heads, g.head_dim, g.d_model)
            wm["layers.%d.%s" % (l, t)] = np.repeat(a, G, axis=0).reshape(-1, g.d_model)
    mm = orc.OracleModel(mha, wm, 1, 32)
    for p, t in enumerate([3, 9, 27, 81]):
        _, a = mg.step(0, t, p)
        _, b = mm.step(0, t, p)
        assert rel(a, b) < 1e-15


def test_tied_head_equals_untied_copy_and_zero_bias():
    tied = dataclasses.replace(SMALL, name="pin-tied", tied_embeddings=True, qkv_bias=True)
    untied = dataclasses.replace(SMALL, name="pin-tied", tied_embeddings=False, qkv_bias=False)
    wt = si.gen_weights(tied, gain_std=0.1, w_std=0.08)
    for l in range(SMALL.n_layers):
        for b in ("bq", "bk", "bv"):
            wt["layers.%d.%s" % (l, b)] = np.zeros_like(wt["layers.%d.%s" % (l, b)])
    wu = {k: v for k, v in wt.items()}
    wu["lm_head"] = wt["embed"].copy()
    a = orc.OracleModel(tied, wt, 1, 16)
    b = orc.OracleModel(untied, wu, 1, 16)
    for p, t in enumerate([1, 2, 3]):
        assert (a.step(0, t, p)[1] == b.step(0, t, p)[1]).all()


def test_qkv_bias_enters():
    biased = dataclasses.replace(SMALL, name="pin-bias", qkv_bias=True)
    w = si.gen_weights(biased, gain_std=0.1, w_std=0.08)
    m1 = orc.OracleModel(biased, w, 1, 8)
    w0 = dict(w)
    w0["layers.0.bv"] = np.zeros_like(w["layers.0.bv"])
    m0 = orc.OracleModel(biased, w0, 1, 8)
    # at position 0 attention returns v = Wv xn + bv; removing bv changes layer 0's output
    assert rel(m1.step(0, 5, 0)[1], m0.step(0, 5, 0)[1]) > 1e-6


def test_sequences_are_independent_and_thread_count_free():
    m2, _ = _model(SMALL, n_seqs=2)
    ma, _ = _model(SMALL)
    mb, _ = _model(SMALL)
    ta = si.uniform_int(11, 6, 0, SMALL.vocab - 1)
    tb = si.uniform_int(12, 6, 0, SMALL.vocab - 1)
    for p in range(6):
        x1 = m2.step(0, ta[p], p)[1]
        y1 = m2.step(1, tb[p], p)[1]
        assert (x1 == ma.step(0, ta[p], p)[1]).all() and (y1 == mb.step(0, tb[p], p)[1]).all()
    n0 = orc.threads()
    try:
        m1, _ = _model(SMALL)
        orc.set_threads(1)
        a = [m1.step(0, t, p)[1] for p, t in enumerate(ta)]
        m8, _ = _model(SMALL)
        orc.set_threads(8)
        b = [m8.step(0, t, p)[1] for p, t in enumerate(ta)]
        assert all((x == y).all() for x, y in zip(a, b))
    finally:
        orc.set_threads(n0)


def test_kv_append_stores_bf16_of_rotated_key():
    # after a step at position p, cache row p holds bf16(k') for layer 0, where k' = RoPE(Wk xn, p)
    m, w = _model(SMALL)
    t, p = 17, 0
    m.step(0, t, p)
    k, v = m.get_kv(0, 0, 0, 1)
    e = orc.bf16_to_f64(w["embed"][t])
    xn = orc.rmsnorm(e, w["layers.0.attn_norm"], SMALL.rms_eps)
    kk = orc.gemv(w["layers.0.wk"], xn).reshape(SMALL.n_kv_heads, SMALL.head_dim)
    vv = orc.gemv(w["layers.0.wv"], xn).reshape(SMALL.n_kv_heads, SMALL.head_dim)
    for h in range(SMALL.n_kv_heads):
        kr = orc.rope(kk[h], p, SMALL.rope_theta)
        assert [orc.bf16(x) for x in kr] == k[0, h].tolist()
        assert [orc.bf16(x) for x in vv[h]] == v[0, h].tolist()
