"""Pins of the oracle's fp32 build (liboracle_f32.so): the same definition computed in fp32, which
the parity tests use to size how far plain fp32 rounding alone moves the logits, and which the
benchmark times as its CPU baseline.

The checks are the closed forms, special cases and library comparisons that pin the fp64 build,
with tolerances set by fp32 rounding (unit roundoff u = 2^-24, error bounds of the order of n*u
for sums of n terms), plus a direct comparison of whole decode steps with the fp64 build. A
plausible mistake in the fp32 path (a dropped term, a wrong index, a double-precision-only branch)
moves a result by far more than these bounds.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle as orc
import seeded_inputs as si

pytestmark = pytest.mark.usefixtures("oracle_lib", "inputs_lib")

U = 2.0 ** -24          # fp32 unit roundoff
RNG = np.random.default_rng(4321)


@pytest.fixture(autouse=True)
def fp32_build():
    old = orc.set_default_precision("f32")
    yield
    orc.set_default_precision(old)


def rand_bf16(shape, std=1.0):
    x = RNG.normal(0.0, std, size=shape).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64); b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def test_results_are_fp32_values():
    # every value the fp32 build returns is representable in fp32 (catches a build that kept doubles)
    x = RNG.normal(size=64)
    g = np.full(64, 0x3F80, np.uint16)
    out = orc.rmsnorm(x, g, 1e-5)
    assert (out.astype(np.float32).astype(np.float64) == out).all()
    w = rand_bf16((9, 64))
    y = orc.gemv(w, x)
    assert (y.astype(np.float32).astype(np.float64) == y).all()
    # and it differs from the fp64 build's result on random input (fp32 rounding is visible)
    old = orc.set_default_precision("f64")
    try:
        y64 = orc.gemv(w, x)
    finally:
        orc.set_default_precision(old)
    assert not (y == y64).all()
    assert rel(y, y64) < 64 * U


def test_rmsnorm_closed_forms():
    d, c, eps = 256, 0.37, 1e-5
    g = np.full(d, 0x3F80, np.uint16)
    out = orc.rmsnorm(np.full(d, c), g, eps)
    assert np.allclose(out, c / math.sqrt(c * c + eps), rtol=8 * U * math.log2(d), atol=0)
    out = orc.rmsnorm(np.array([3.0, 4.0]), np.array([0x3F80, 0x3F80], np.uint16), 0.0)
    assert np.allclose(out, np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=8 * U, atol=0)
    out = orc.rmsnorm(np.array([3.0, 4.0]), np.array([0x4000, 0x3F00], np.uint16), 0.0)
    assert np.allclose(out, np.array([6.0, 2.0]) / math.sqrt(12.5), rtol=8 * U, atol=0)


def test_gemv_one_hot_bias_and_library():
    n, k = 37, 100
    w = rand_bf16((n, k))
    wf = orc.bf16_to_f64(w)
    for j in [0, 17, k - 1]:
        x = np.zeros(k); x[j] = 1.0
        assert (orc.gemv(w, x) == wf[:, j]).all()          # one product, exact in fp32
    b = rand_bf16((n,))
    assert (orc.gemv(np.zeros((n, k), np.uint16), RNG.normal(size=k), b) == orc.bf16_to_f64(b)).all()
    x = RNG.normal(size=k).astype(np.float32).astype(np.float64)
    y = orc.gemv(w, x)
    # |fp32 sum - exact| <= k u sum |w x| per row (the standard bound for recursive summation)
    bound = k * U * (np.abs(wf) @ np.abs(x))
    assert (np.abs(y - wf @ x) <= bound + 1e-30).all()


def test_rope_closed_forms():
    dh, theta = 64, 10000.0
    u = RNG.normal(size=dh).astype(np.float32).astype(np.float64)
    assert (orc.rope(u, 0, theta) == u).all()
    for p in [1, 7, 1000, 32767]:
        r = orc.rope(u, p, theta)
        h = dh // 2
        assert np.allclose(r[:h] ** 2 + r[h:] ** 2, u[:h] ** 2 + u[h:] ** 2, rtol=16 * U, atol=16 * U)
    e0 = np.zeros(dh); e0[0] = 1.0
    r = orc.rope(e0, 3, theta)
    assert abs(r[0] - math.cos(3)) < 2 * U and abs(r[dh // 2] - math.sin(3)) < 2 * U
    e1 = np.zeros(dh); e1[1] = 1.0
    r = orc.rope(e1, 5, theta)
    a = 5 * theta ** (-2.0 / dh)
    assert abs(r[1] - math.cos(a)) < 2 * U and abs(r[1 + dh // 2] - math.sin(a)) < 2 * U
    eh = np.zeros(dh); eh[dh // 2] = 1.0
    r = orc.rope(eh, 3, theta)
    assert abs(r[0] + math.sin(3)) < 2 * U and abs(r[dh // 2] - math.cos(3)) < 2 * U


def test_softmax():
    s = RNG.normal(size=50) * 10
    p = orc.softmax(s)
    assert abs(p.sum() - 1.0) < 64 * U and (p > 0).all()
    assert np.allclose(orc.softmax(np.array([0.0, math.log(3.0)])), [0.25, 0.75], rtol=8 * U)


def test_attention_special_cases():
    hq, hk, dh = 4, 2, 16
    q = RNG.normal(size=hq * dh)
    k1, v1 = rand_bf16((1, hk, dh)), rand_bf16((1, hk, dh))
    out = orc.attention(q, k1, v1, hq, hk, dh)
    for h in range(hq):                                      # one key: weight exactly 1, output = v
        assert (out[h * dh:(h + 1) * dh] == orc.bf16_to_f64(v1[0, h // 2])).all()
    kk = np.repeat(rand_bf16((1, hk, dh)), 9, axis=0)
    vv = rand_bf16((9, hk, dh))
    out = orc.attention(q, kk, vv, hq, hk, dh)
    for h in range(hq):
        ref = orc.bf16_to_f64(vv[:, h // 2]).mean(0)
        assert np.allclose(out[h * dh:(h + 1) * dh], ref, rtol=0, atol=32 * U * np.abs(orc.bf16_to_f64(vv)).max())


def test_attention_brute_force_and_gqa_mapping():
    hq, hk, dh, npos = 8, 2, 32, 23
    q = RNG.normal(size=hq * dh)
    kc, vc = rand_bf16((npos, hk, dh)), rand_bf16((npos, hk, dh))
    out = orc.attention(q, kc, vc, hq, hk, dh)
    kf, vf = orc.bf16_to_f64(kc), orc.bf16_to_f64(vc)
    G = hq // hk
    for h in range(hq):
        s = kf[:, h // G] @ q[h * dh:(h + 1) * dh] / math.sqrt(dh)
        w = np.exp(s - s.max()); w /= w.sum()
        assert rel(out[h * dh:(h + 1) * dh], w @ vf[:, h // G]) < 1e-5


def test_silu_swiglu_argmax():
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 4 * U
    assert abs(orc.silu(40.0) - 40.0) < 40 * 2 * U and abs(orc.silu(-40.0)) < 1e-15
    h = orc.swiglu(np.array([math.log(3.0), 2.0]), np.array([2.0, math.log(3.0)]))
    assert abs(h[0] - 1.5 * math.log(3.0)) < 8 * U
    assert orc.argmax(np.array([1.0, 5.0, 3.0, 5.0, 5.0])) == 1


SMALL = si.shrink(si.TINY, "pin-small", n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, d_ffn=96,
                  vocab=300)


def test_cached_decode_equals_no_cache_recompute_fp32():
    w = si.gen_weights(SMALL, gain_std=0.1, w_std=0.08)
    m = orc.OracleModel(SMALL, w, 1, 32, precision="f32")
    toks = si.uniform_int(3, 12, 0, SMALL.vocab - 1)
    for p, t in enumerate(toks):
        tok, logits = m.step(0, t, p)
        ref_tok, ref = m.forward_nocache(toks[:p + 1])
        assert tok == ref_tok
        assert rel(logits, ref) < 1e-6
    m.close()


def test_gqa_equals_mha_fp32():
    g = SMALL
    mha = dataclasses.replace(g, name="pin-mha", n_kv_heads=g.n_q_heads)
    w = si.gen_weights(g, gain_std=0.1, w_std=0.08)
    wm = dict(w)
    G = g.n_q_heads // g.n_kv_heads
    for l in range(g.n_layers):
        for t in ("wk", "wv"):
            a = w["layers.%d.%s" % (l, t)].reshape(g.n_kv_heads, g.head_dim, g.d_model)
            wm["layers.%d.%s" % (l, t)] = np.repeat(a, G, axis=0).reshape(-1, g.d_model)
    mg = orc.OracleModel(g, w, 1, 16, precision="f32")
    mm = orc.OracleModel(mha, wm, 1, 16, precision="f32")
    for p, t in enumerate([3, 9, 27, 81]):
        assert (mg.step(0, t, p)[1] == mm.step(0, t, p)[1]).all()    # same fp32 operations, same order
    mg.close(); mm.close()


def test_fp32_step_tracks_fp64_step():
    # whole decode steps of the two builds on the same model: fp32 rounding alone separates them, by
    # a relative amount far below 1e-3 on this 2-layer model (a dropped term would be O(1))
    w = si.gen_weights(SMALL, gain_std=0.1, w_std=0.08)
    a = orc.OracleModel(SMALL, w, 1, 32, precision="f32")
    b = orc.OracleModel(SMALL, w, 1, 32, precision="f64")
    toks = si.uniform_int(8, 16, 0, SMALL.vocab - 1)
    worst = 0.0
    for p, t in enumerate(toks):
        ta, la = a.step(0, t, p)
        tb, lb = b.step(0, t, p)
        worst = max(worst, rel(la, lb))
        assert ta == tb or abs(np.sort(lb)[-1] - np.sort(lb)[-2]) < 1e-4
    assert 0.0 < worst < 1e-5
    a.close(); b.close()
