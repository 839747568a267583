"""Pins of the oracle's FP8 weight format: OCP E4M3 codes with one power-of-two scale per output row.

Checked against what the format's definition fixes (values of named codes, the full code table built
independently from the bit fields, round-to-nearest with ties to an even mantissa at every midpoint),
against the scale rule's boundary cases, and against exactness (dequantised weights are bf16 values,
and quantising them again returns the same values). The model-level helper is pinned by a GEMV with
one-hot inputs, which must return the dequantised columns exactly.
"""
import math

import numpy as np
import pytest

import oracle as orc
import seeded_inputs as si

pytestmark = pytest.mark.usefixtures("oracle_lib")


def table_from_fields():
    """E4M3 values written out from the bit layout: 1 sign, 4 exponent (bias 7), 3 mantissa bits."""
    vals = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue                               # NaN
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals[c] = -v if s else v
    return vals


def test_named_codes():
    assert orc.fp8_decode(0x00) == 0.0 and math.copysign(1, orc.fp8_decode(0x80)) == -1
    assert orc.fp8_decode(0x01) == 2.0 ** -9           # smallest subnormal
    assert orc.fp8_decode(0x07) == 7 * 2.0 ** -9       # largest subnormal
    assert orc.fp8_decode(0x08) == 2.0 ** -6           # smallest normal
    assert orc.fp8_decode(0x38) == 1.0
    assert orc.fp8_decode(0x7E) == 448.0               # largest finite
    assert orc.fp8_decode(0xFE) == -448.0
    assert math.isnan(orc.fp8_decode(0x7F)) and math.isnan(orc.fp8_decode(0xFF))


def test_full_table_and_exact_roundtrip():
    vals = table_from_fields()
    assert len(vals) == 254
    for c, v in vals.items():
        assert orc.fp8_decode(c) == v
        if v != 0.0 or c == 0x00:
            assert orc.fp8_encode(v) == c                # every finite value encodes to itself
    assert orc.fp8_encode(-0.0) == 0x80
    pos = sorted(set(v for v in vals.values() if v >= 0))
    assert len(pos) == 127 and pos == sorted(pos)


def test_round_to_nearest_ties_to_even():
    vals = table_from_fields()
    pos = [(vals[c], c) for c in range(0x7F)]
    for (a, ca), (b, cb) in zip(pos, pos[1:]):
        mid = (a + b) / 2
        even = ca if ca % 2 == 0 else cb
        assert orc.fp8_encode(mid) == even, (a, b)
        assert orc.fp8_encode(-mid) == even | 0x80
        q = (b - a) / 4
        assert orc.fp8_encode(a + q) == ca and orc.fp8_encode(b - q) == cb
    assert orc.fp8_encode(1.0625) == 0x38 and orc.fp8_encode(1.1875) == 0x3A
    assert orc.fp8_encode(2.0 ** -11) == 0x00            # a quarter of the smallest subnormal


def bf16_of(x):
    return orc.bf16(float(x))


def test_row_exponent_boundaries():
    def exp_of(m):
        row = np.array([bf16_of(m), bf16_of(-m / 3), 0], dtype=np.uint16)
        return orc.fp8_row_exp(row)
    assert exp_of(448.0) == 0 and exp_of(224.0) == -1 and exp_of(448.0 * 2 ** -12) == -12
    assert exp_of(450.0) == 1                          # just above 448: the next power
    assert exp_of(1.0) == -8                           # 1 <= 448 / 256 = 1.75, 1 > 448 / 512
    assert exp_of(1.75) == -8 and exp_of(1.765625) == -7
    assert orc.fp8_row_exp(np.zeros(5, np.uint16)) == 0
    rng = np.random.default_rng(7)
    for _ in range(50):
        m = float(np.abs(rng.normal(0, 10)) + 1e-3)
        b = orc.from_bf16(bf16_of(m))
        e = exp_of(b)
        assert b <= 448 * 2.0 ** e and b > 448 * 2.0 ** (e - 1)


def test_quantize_dequantize_exact_and_idempotent():
    w = si.normal_bf16(si.tensor_seed("fp8", "pins"), 37 * 300, 0.0, 0.02).reshape(37, 300)
    w[3] = 0
    codes, exps = orc.fp8_quantize(w)
    assert exps[3] == 0 and (codes[3] == 0).all()
    dq = orc.fp8_dequantize(codes, exps)
    vals = table_from_fields()
    for i in (0, 5, 36):
        for j in (0, 17, 299):
            assert orc.from_bf16(dq[i, j]) == vals[int(codes[i, j])] * 2.0 ** int(exps[i])
            # the code is the nearest one to the scaled weight
            x = orc.from_bf16(w[i, j]) * 2.0 ** -int(exps[i])
            best = min(abs(x - v) for c, v in vals.items())
            assert abs(x - vals[int(codes[i, j])]) == best
    # quantising the dequantised weights again changes no value (a row whose maximum rounded down to
    # exactly 448 * 2^(e-1) takes the smaller exponent and codes one binade higher: same values)
    c2, e2 = orc.fp8_quantize(dq)
    assert np.array_equal(orc.fp8_dequantize(c2, e2), dq)
    same = e2 == exps
    assert same.mean() > 0.5 and (c2[same] == codes[same]).all()
    rel = np.linalg.norm(orc.bf16_to_f64(dq) - orc.bf16_to_f64(w)) / np.linalg.norm(orc.bf16_to_f64(w))
    assert 0.005 < rel < 0.05                          # 3 mantissa bits: a few percent, not zero


def test_fp8_model_gemv_columns():
    # the dequantised model's matrices are what a GEMV with one-hot inputs returns, column by column
    shape = si.shrink(si.TINY, "fp8-pin", n_layers=1, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                      d_ffn=96, vocab=50)
    w = si.gen_weights(shape)
    m8, w8 = orc.fp8_model(shape, w)
    assert not m8.tied_embeddings
    wq = w8["layers.0.wq"].reshape(-1, shape.d_model)
    codes, exps = orc.fp8_quantize(np.asarray(w["layers.0.wq"]).reshape(-1, shape.d_model))
    for j in (0, 9, 63):
        x = np.zeros(shape.d_model)
        x[j] = 1.0
        y = orc.gemv(wq, x)
        ref = np.array([orc.fp8_decode(int(c)) for c in codes[:, j]]) * 2.0 ** exps.astype(np.float64)
        assert (y == ref).all()
    assert np.array_equal(w8["embed"], w["embed"]) and np.array_equal(w8["layers.0.attn_norm"], w["layers.0.attn_norm"])
