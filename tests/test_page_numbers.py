"""Pins the bytes-moved accounting (persistent_megakernel_03_amd.roofline) to numbers the
pages print. No GPU needed."""
import json
import os

from persistent_megakernel_03_amd import roofline as rf

HERE = os.path.dirname(os.path.abspath(__file__))
G = json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))


def test_kv_cache_size_worked_example():
    c = G["kv_cache_size"]
    b = rf.kv_bytes(c["batch"], c["layers"], c["seq"], c["head_dim"], c["heads"], c["elem_bytes"])
    assert b == c["expected_gib"] * 2 ** 30


def test_decode_lower_bound():
    c = G["decode_lower_bound"]
    assert abs(rf.roofline_ms(c["weight_bytes"], c["bandwidth_gbs"]) - c["expected_ms"]) < 1e-12


def test_8b_shape_bytes_per_token():
    # the 8B shape's weight stream: every GEMV matrix once, one embedding row, the gains
    import seeded_inputs as si
    m = si.LLAMA8B
    per_layer = (32 + 16) * 128 * 4096 + 4096 * 4096 + 3 * 14336 * 4096
    assert rf.gemv_weight_bytes(m) == 2 * (32 * per_layer + 128256 * 4096)
    assert rf.weight_bytes_per_token(m) == rf.gemv_weight_bytes(m) + 2 * 4096 + 2 * 65 * 4096
    # a step at context c also reads 2 (K, V) x layers x c x head_dim x kv heads x 2 bytes
    assert rf.step_bytes(m, [100]) - rf.weight_bytes_per_token(m) == 2 * 32 * 100 * 128 * 8 * 2
