"""Host-only checks of the C-ABI library and its task-graph builder (no GPU needed).

The library must load and export every symbol include/mk.h declares. The graph it builds
for each workload shape must validate:
  - each queue follows one global topological order;
  - every consumer comes after its producers;
  - each flag slot has one writer;
  - each tile is contiguous.
Random interleavings of the per-CU queues, simulated against symbolic buffers, must find
neither a read before its producer finished nor an overwrite while a reader still needs
the old value.
"""
import ctypes
import dataclasses
import os
import re

import pytest

import persistent_megakernel_03_amd as mk
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mk.LIB_PATH):
        mk.build(force=True)
    return mk.lib()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    return sorted(set(re.findall(r"^(?:mk_status|void|const char\*)\s+(mk_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_symbols()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mk.EXPORTS)


def cfg_for(shape, max_blocks=64, num_blocks=64, splits=0):
    return mk.make_config(shape, max_seqs=1, max_blocks_per_seq=max_blocks, num_blocks=num_blocks, attn_splits=splits)


@pytest.mark.parametrize("shape,blocks", [(si.TINY, 3), (si.QWEN05B, 35), (si.LLAMA8B, 35), (si.LLAMA8B, 2053)])
def test_graph_validates(L, shape, blocks):
    ctx = mk.mk_create_host(cfg_for(shape, blocks, blocks), 256)
    try:
        mk.mk_graph_validate(ctx)
        info = mk.mk_graph_stats(ctx)
        assert info.n_tasks > 0 and info.lds_bytes <= 160 * 1024
        # the packed tiles hold every GEMV weight once (plus zero padding of partial groups)
        m = shape
        gemv = (m.n_layers * ((m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim * m.d_model
                              + m.d_model * m.n_q_heads * m.head_dim + 3 * m.d_ffn * m.d_model)
                + m.vocab * m.d_model) * 2
        assert gemv <= info.weight_bytes <= gemv * 1.07
    finally:
        mk.mk_destroy(ctx)


@pytest.mark.parametrize("blocks,attn_tasks", [(35, 64), (512, 64), (2052, 256)])
def test_one_sequence_attention_split_rule(L, blocks, attn_tasks):
    # one sequence at the 8B shape: 8 attention tasks per KV head for a short cache, growing with a long
    # one (blocks / 64 per KV head, at most 32): 256 tasks, one per CU, at 32K positions
    ctx = mk.mk_create_host(cfg_for(si.LLAMA8B, blocks, blocks), 256)
    try:
        info = mk.mk_graph_stats(ctx)
        m = si.LLAMA8B
        other = m.n_layers * 256 * 2 + 256 + 1  # gate/up and down on every CU, the LM head, the argmax
        # QKV and O skip the attention CUs when those are few
        qo_tasks = 256 - attn_tasks if attn_tasks * 4 <= 256 else 256
        assert info.n_tasks == other + m.n_layers * (attn_tasks + 2 * qo_tasks)
    finally:
        mk.mk_destroy(ctx)


def test_8b_tiles_have_no_padding(L):
    ctx = mk.mk_create_host(cfg_for(si.LLAMA8B, 35, 35), 256)
    try:
        info = mk.mk_graph_stats(ctx)
        m = si.LLAMA8B
        gemv = (m.n_layers * (6144 * 4096 + 4096 * 4096 + 3 * 14336 * 4096) + m.vocab * 4096) * 2
        assert info.weight_bytes == gemv
    finally:
        mk.mk_destroy(ctx)


def test_graph_is_deterministic(L):
    hs = []
    for _ in range(2):
        ctx = mk.mk_create_host(cfg_for(si.QWEN05B, 35, 35), 256)
        hs.append(mk.mk_graph_stats(ctx).hash)
        mk.mk_destroy(ctx)
    assert hs[0] == hs[1]
    ctx = mk.mk_create_host(cfg_for(si.QWEN05B, 35, 35), 128)   # different CU count, different graph
    assert mk.mk_graph_stats(ctx).hash != hs[0]
    mk.mk_destroy(ctx)


@pytest.mark.parametrize("n_cus,splits", [(256, 0), (7, 2), (3, 1), (64, 3)])
def test_random_interleavings(L, n_cus, splits):
    ctx = mk.mk_create_host(cfg_for(si.TINY, 3, 3, splits), n_cus)
    try:
        for seed in range(12):
            mk.mk_graph_simulate(ctx, seed, 3)
    finally:
        mk.mk_destroy(ctx)


def test_interleavings_small_qwen_shape(L):
    shape = si.shrink(si.QWEN05B, "q-small", n_layers=2, vocab=4096)
    ctx = mk.mk_create_host(cfg_for(shape, 8, 8), 32)
    try:
        for seed in range(4):
            mk.mk_graph_simulate(ctx, seed, 2)
    finally:
        mk.mk_destroy(ctx)


def test_rejects_bad_configs(L):
    bad = [
        dataclasses.replace(si.TINY, n_q_heads=3),       # not a multiple of kv heads
        dataclasses.replace(si.TINY, head_dim=96),       # unsupported head dim
        dataclasses.replace(si.TINY, d_model=250),       # not a multiple of 8
        dataclasses.replace(si.TINY, n_q_heads=32, n_kv_heads=2),  # 16 q heads per kv head
    ]
    for shape in bad:
        with pytest.raises(mk.MKError) as e:
            mk.mk_create_host(cfg_for(shape, 4, 4), 256)
        assert e.value.status == -2
    c = cfg_for(si.TINY, 4, 4)
    c.block_size = 32
    with pytest.raises(mk.MKError):
        mk.mk_create_host(c, 256)
    with pytest.raises(mk.MKError) as e:
        mk.mk_create_host(cfg_for(si.TINY, 4, 4), 0)
    assert e.value.status == -2
    c = cfg_for(si.TINY, 4, 4)
    c.attn_min_blocks = -1
    with pytest.raises(mk.MKError) as e:
        mk.mk_create_host(c, 256)
    assert e.value.status == -2


def test_prefill_rows_config(L):
    # prefill_rows > 1 adds the batched graph's re-laid-out weights (every GEMV matrix once more) and its
    # working memory to the buffers mk_workspace_size asks for; 0 and 1 add nothing
    base = mk.mk_create_host(cfg_for(si.TINY, 3, 3), 64)
    w0, kv0, s0 = mk.mk_workspace_size(base)
    mk.mk_destroy(base)
    for rows in (0, 1):
        c = cfg_for(si.TINY, 3, 3)
        c.prefill_rows = rows
        ctx = mk.mk_create_host(c, 64)
        assert mk.mk_workspace_size(ctx) == (w0, kv0, s0)
        mk.mk_destroy(ctx)
    m = si.TINY
    gemv = 2 * (m.n_layers * ((m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim * m.d_model
                              + m.d_model * m.n_q_heads * m.head_dim + 3 * m.d_ffn * m.d_model) + m.vocab * m.d_model)
    for rows in (2, 16):
        c = cfg_for(si.TINY, 3, 3)
        c.prefill_rows = rows
        ctx = mk.mk_create_host(c, 64)
        w, kv, s = mk.mk_workspace_size(ctx)
        assert kv == kv0 and s > s0 and w >= w0 + gemv
        mk.mk_graph_validate(ctx)
        mk.mk_destroy(ctx)
    for rows, n_seqs in ((17, 1), (-1, 1), (4, 4)):     # out of range; a batched context prefills through its own rows
        c = mk.make_config(si.TINY, max_seqs=n_seqs, max_blocks_per_seq=3, num_blocks=3 * n_seqs)
        c.prefill_rows = rows
        with pytest.raises(mk.MKError) as e:
            mk.mk_create_host(c, 64)
        assert e.value.status == -2


@pytest.mark.parametrize("shape,blocks", [(si.TINY, 3), (si.QWEN05B, 35), (si.LLAMA8B, 35)])
def test_fp8_weights_graph(L, shape, blocks):
    # FP8 weights: half-size tiles (16 codes per lane per unit, units per row group
    # padded to even), one fp32 scale per packed GEMV row; the graph validates and simulates
    c = cfg_for(shape, blocks, blocks)
    c.weight_format = 1
    ctx = mk.mk_create_host(c, 256)
    base = mk.mk_create_host(cfg_for(shape, blocks, blocks), 256)
    try:
        mk.mk_graph_validate(ctx)
        mk.mk_graph_simulate(ctx, 3, 1)
        i8, i16 = mk.mk_graph_stats(ctx), mk.mk_graph_stats(base)
        assert i8.hash != i16.hash
        m = shape
        rows = m.n_layers * ((m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim + m.d_model + 2 * m.d_ffn + m.d_model) + m.vocab
        assert i8.weight_bytes * 2 == i16.weight_bytes    # these shapes need no extra padding
        w8, _, _ = mk.mk_workspace_size(ctx)
        w16, _, _ = mk.mk_workspace_size(base)
        assert w8 - i8.weight_bytes >= (w16 - i16.weight_bytes) + 4 * rows   # the row scales
    finally:
        mk.mk_destroy(ctx)
        mk.mk_destroy(base)
    for n_seqs, rows_pf in ((4, 0), (1, 16)):     # batched contexts and chunked prefill keep bf16
        c = mk.make_config(si.TINY, max_seqs=n_seqs, max_blocks_per_seq=3, num_blocks=3 * n_seqs,
                           prefill_rows=rows_pf, weight_format=1)
        with pytest.raises(mk.MKError) as e:
            mk.mk_create_host(c, 64)
        assert e.value.status == -2
    c = cfg_for(si.TINY, 3, 3)
    c.weight_format = 2
    with pytest.raises(mk.MKError):
        mk.mk_create_host(c, 64)


def test_host_context_refuses_device_calls(L):
    ctx = mk.mk_create_host(cfg_for(si.TINY, 3, 3), 16)
    try:
        w, kv, s = mk.mk_workspace_size(ctx)
        assert w > 0 and kv == 3 * 2 * 16 * 64 * 2 and s > 0
        one = ctypes.c_void_p(256)
        arr = (ctypes.c_void_p * 2)(256, 256)
        st = L.mk_bind_memory(ctx, one, arr, arr, one, one, one, one)
        assert st == -3   # MK_ERR_STATE
        assert "host-only" in mk.mk_last_error()
        st = L.mk_decode_step(ctx, one, 1, one, None)
        assert st == -3
        assert L.mk_decode_step(ctx, None, 1, one, None) == -1
        assert L.mk_graph_validate(None) == -1
        assert mk.mk_status_str(-5) == "MK_ERR_DEVICE_TIMEOUT"
    finally:
        mk.mk_destroy(ctx)


# --------------------------------------------------------------------------- batched graphs
def batched_cfg(shape, n_seqs, blocks_per_seq, splits=0):
    return mk.make_config(shape, max_seqs=n_seqs, max_blocks_per_seq=blocks_per_seq,
                          num_blocks=n_seqs * blocks_per_seq, attn_splits=splits)


@pytest.fixture
def ksplit_cap(monkeypatch):
    """Sets MK_BATCHED_MAX_KSPLIT (read when a graph is built) for the test's duration."""
    def set_cap(v):
        if v is None:
            monkeypatch.delenv("MK_BATCHED_MAX_KSPLIT", raising=False)
        else:
            monkeypatch.setenv("MK_BATCHED_MAX_KSPLIT", str(v))
    return set_cap


@pytest.mark.parametrize("shape,n_seqs,n_cus,cap", [
    (si.TINY, 4, 256, None), (si.TINY, 4, 7, None), (si.TINY, 16, 64, None), (si.TINY, 2, 3, None),
    (si.MID, 16, 256, None), (si.MID, 16, 256, 1), (si.MID, 3, 40, 2)])
def test_batched_graph_interleavings(L, ksplit_cap, shape, n_seqs, n_cus, cap):
    ksplit_cap(cap)
    ctx = mk.mk_create_host(batched_cfg(shape, n_seqs, 4), n_cus)
    try:
        mk.mk_graph_validate(ctx)
        assert mk.mk_graph_stats(ctx).lds_bytes <= 160 * 1024
        for seed in range(3):
            mk.mk_graph_simulate(ctx, seed, 2)
    finally:
        mk.mk_destroy(ctx)


def test_batched_8b_graph(L, ksplit_cap):
    # the 16-sequence 8B decode: contexts up to 8192 + 128 steps, 16-token blocks
    ksplit_cap(None)
    nb = (8192 + 128 + 15) // 16
    ctx = mk.mk_create_host(batched_cfg(si.LLAMA8B, 16, nb), 256)
    try:
        mk.mk_graph_validate(ctx)
        info = mk.mk_graph_stats(ctx)
        assert info.lds_bytes <= 160 * 1024
        m = si.LLAMA8B
        gemv = (m.n_layers * (6144 * 4096 + 4096 * 4096 + 3 * 14336 * 4096) + m.vocab * 4096) * 2
        assert info.weight_bytes == gemv   # every row tile is whole 16-row groups of whole 32-column units
        # the batched graph differs from the one-sequence graph of the same shape
        one = mk.mk_create_host(cfg_for(m, nb, nb), 256)
        assert mk.mk_graph_stats(one).hash != info.hash
        mk.mk_destroy(one)
    finally:
        mk.mk_destroy(ctx)


def test_batched_weights_cover_every_column_once(L, ksplit_cap):
    # the packed size equals rows x columns, each padded to its tile: no column is streamed twice
    for cap in (None, 1, 3):
        ksplit_cap(cap)
        ctx = mk.mk_create_host(batched_cfg(si.MID, 16, 4), 256)
        m = si.MID
        gemv = (m.n_layers * ((m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim * m.d_model
                              + m.d_model * m.n_q_heads * m.head_dim + 3 * m.d_ffn * m.d_model)
                + m.vocab * m.d_model) * 2
        w = mk.mk_graph_stats(ctx).weight_bytes
        assert gemv <= w <= gemv * 1.1, (cap, w, gemv)
        mk.mk_destroy(ctx)


# --------------------------------------------------------------------------- the checks reject broken graphs
# Each case breaks a freshly built graph in one way (mk_graph_corrupt, host-only) and names the message
# the validator must give. A validator that accepted everything would fail every case.
@pytest.mark.parametrize("kind,message", [
    (1, "queue not in global order"),
    (2, "waits on a later producer"),
    (3, "has two writers"),
    (4, "has no writer"),
    (5, "twice"),
    (7, "does not end at row"),
])
@pytest.mark.parametrize("shape,n_seqs,n_cus", [(si.TINY, 1, 256), (si.TINY, 1, 7), (si.MID, 16, 256)])
def test_validator_rejects_broken_graphs(L, ksplit_cap, kind, message, shape, n_seqs, n_cus):
    ksplit_cap(None)
    cfg = batched_cfg(shape, n_seqs, 4) if n_seqs > 1 else cfg_for(shape, 3, 3)
    ctx = mk.mk_create_host(cfg, n_cus)
    try:
        mk.mk_graph_validate(ctx)
        mk.mk_graph_corrupt(ctx, kind)
        with pytest.raises(mk.MKError) as e:
            mk.mk_graph_validate(ctx)
        assert e.value.status == -2 and message in str(e.value), str(e.value)
    finally:
        mk.mk_destroy(ctx)


@pytest.mark.parametrize("n_cus", [256, 16])
def test_simulator_catches_a_consumer_that_does_not_wait(L, n_cus):
    # an attention task whose wait on the QKV stage is removed: the graph still validates (nothing in
    # it is out of order), but some interleaving runs the task before its queries exist
    ctx = mk.mk_create_host(cfg_for(si.TINY, 3, 3, 2), n_cus)
    try:
        mk.mk_graph_corrupt(ctx, 6)
        mk.mk_graph_validate(ctx)
        failures = []
        for seed in range(16):
            try:
                mk.mk_graph_simulate(ctx, seed, 1)
            except mk.MKError as e:
                failures.append(str(e))
        assert failures and all("before its producer finished" in f for f in failures), failures[:2]
    finally:
        mk.mk_destroy(ctx)


@pytest.mark.parametrize("kind", [8, 9])
@pytest.mark.parametrize("n_cus", [256, 7])
def test_simulator_catches_broken_ready_queue_tables(L, kind, n_cus):
    # the run-time scheduling tables: a consumer that is never queued, or an event that never completes;
    # the static checks do not read these tables, the host run of the ready queue does
    ctx = mk.mk_create_host(cfg_for(si.TINY, 3, 3, 2), n_cus)
    try:
        mk.mk_graph_simulate(ctx, 1, 1)
        mk.mk_graph_corrupt(ctx, kind)
        mk.mk_graph_validate(ctx)
        with pytest.raises(mk.MKError) as e:
            mk.mk_graph_simulate(ctx, 1, 1)
        assert "dynamic schedule" in str(e.value), str(e.value)
    finally:
        mk.mk_destroy(ctx)


def test_simulator_catches_rows_written_twice(L):
    # overlapping down tiles: the validator names it; the simulator's data checks stay consistent
    # (the extra row's second writer is the later task)
    ctx = mk.mk_create_host(cfg_for(si.TINY, 3, 3), 256)
    try:
        mk.mk_graph_corrupt(ctx, 5)
        with pytest.raises(mk.MKError):
            mk.mk_graph_validate(ctx)
    finally:
        mk.mk_destroy(ctx)


def test_corruption_needs_a_host_context_and_a_known_kind(L):
    ctx = mk.mk_create_host(cfg_for(si.TINY, 3, 3), 256)
    try:
        with pytest.raises(mk.MKError) as e:
            mk.mk_graph_corrupt(ctx, 99)
        assert e.value.status == -1
    finally:
        mk.mk_destroy(ctx)


# --------------------------------------------------------------------------- determinism
def test_golden_graph_hashes(L, ksplit_cap):
    # every workload's graph, built as the benchmark and the parity tests build it, hashes to the
    # stored value (tests/golden/graph_hashes.json, written by tests/golden/make_graph_hashes.py)
    import importlib.util
    import json
    ksplit_cap(None)
    spec = importlib.util.spec_from_file_location("make_graph_hashes", os.path.join(ROOT, "tests", "golden", "make_graph_hashes.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    stored = json.load(open(os.path.join(ROOT, "tests", "golden", "graph_hashes.json")))["graphs"]
    assert set(stored) == set(mod.NAMES)
    for name in mod.NAMES:
        got = mod.graph_entry(name, stored[name]["n_cus"])
        assert got == stored[name], (name, got, stored[name])


def test_graph_hash_is_the_same_in_a_fresh_process(L):
    # the builder keeps no state between contexts and depends on no address: a new interpreter (other
    # heap addresses) builds the same graph
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import persistent_megakernel_03_amd as mk, seeded_inputs as si;"
            "c = mk.make_config(si.LLAMA8B, max_seqs=1, max_blocks_per_seq=35, num_blocks=35);"
            "x = mk.mk_create_host(c, 256); print(mk.mk_graph_stats(x).hash)" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True).stdout
    ctx = mk.mk_create_host(cfg_for(si.LLAMA8B, 35, 35), 256)
    try:
        assert int(out.strip()) == mk.mk_graph_stats(ctx).hash
    finally:
        mk.mk_destroy(ctx)
