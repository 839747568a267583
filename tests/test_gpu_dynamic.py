"""GPU: dynamic scheduling (mk_decode_step_dynamic): the decode step with its tasks taken from a
device-side ready queue at run time instead of the ahead-of-time per-CU queues.

Bars: the tasks and their arithmetic are the same, so tokens, logits, context lengths and the KV cache
are bit-identical to mk_decode_step step for step; the trace shows every task run exactly once, each
consumer stage starting only after its producer stage finished, and tasks on other CUs than the static
graph placed them; contexts the mode does not serve are refused; a wait past the watchdog drains the
launch and is reported.
"""
import sys

import numpy as np
import pytest

import persistent_megakernel_03_amd as mk
import seeded_inputs as si
from parity_util import cached_weights, make_gpu

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_pair(shape, weights, prompt, n_steps, n_positions):
    """Two contexts over the same prompt; then n_steps greedy steps, static on one and dynamic on the
    other, compared bit for bit after every step."""
    import torch
    a, table = make_gpu(shape, weights, n_positions, "permuted")
    b, _ = make_gpu(shape, weights, n_positions, "permuted")
    ga = torch.zeros(1, dtype=torch.int32, device=a.dev)
    gb = torch.zeros(1, dtype=torch.int32, device=b.dev)
    a.prefill(list(prompt), ga)
    b.prefill(list(prompt), gb)
    assert int(ga.item()) == int(gb.item())
    for i in range(n_steps):
        a.step(ga, 1, ga)
        b.step_dynamic(gb, 1, gb)
        b.sync_check()
        assert int(ga.item()) == int(gb.item()), "step %d: tokens differ" % i
        assert np.array_equal(a.read_logits(0), b.read_logits(0)), "step %d: logits differ" % i
    assert torch.equal(a.ctx_lens, b.ctx_lens)
    for pa, pb in zip(a.k_pools + a.v_pools, b.k_pools + b.v_pools):
        assert torch.equal(pa, pb)
    return a, b


@pytest.fixture(scope="module")
def tiny():
    return si.gen_weights(si.TINY), si.prompt_tokens(si.WORKLOADS["tiny"])


def test_tiny_dynamic_equals_static(tiny):
    w, prompt = tiny
    log("case: tiny, prompt 16 + 12 steps, dynamic vs static")
    a, b = run_pair(si.TINY, w, prompt, 12, 48)
    a.close(); b.close()


def test_tiny_dynamic_trace(tiny):
    # every task once, with the step's epoch; a stage's tasks start only after the stage they wait on
    # has finished (the queue holds them until then); and the placement is not the static one
    import torch
    w, prompt = tiny
    log("case: tiny, trace of a dynamic step")
    dec, _ = make_gpu(si.TINY, w, 48)
    g0 = torch.zeros(1, dtype=torch.int32, device=dec.dev)
    dec.prefill(list(prompt[:5]), g0)
    dec.enable_trace()
    dec.step(g0, 1, g0)
    static = dec.read_trace().copy()
    dec.step_dynamic(g0, 1, g0)
    dec.sync_check()
    tr = dec.read_trace()
    n = mk.mk_graph_stats(dec.ctx).n_tasks
    assert len(tr) == n and len(set(tr["epoch"].tolist())) == 1 and tr["epoch"][0] == static["epoch"][0] + 1
    assert (tr["t_done"] >= tr["t_ready"]).all() and (tr["t_ready"] >= tr["t_queue"]).all()
    # stage order: in the global order, each (type, layer) run starts after the previous run's last end
    ty, ly = tr["type"], tr["layer"]
    starts = 0
    prev_end = None
    for i in range(n):
        if i == 0 or ty[i] != ty[i - 1] or ly[i] != ly[i - 1]:
            if i > 0:
                prev_end = tr["t_done"][starts:i].max()
            starts = i
        if prev_end is not None:
            assert tr["t_queue"][i] >= prev_end, "task %d left the queue before its producers finished" % i
    moved = float((tr["cu"] != static["cu"]).mean())
    log("  tasks on another CU than the static graph placed them: %.2f" % moved)
    assert moved > 0.1
    dec.close()


def test_qwen_shape_dynamic_equals_static():
    wl = si.WORKLOADS["qwen0.5b"]
    m = wl.model
    log("case: qwen0.5b shape, prompt 8 + 6 steps, dynamic vs static")
    a, b = run_pair(m, si.gen_weights(m), si.prompt_tokens(wl)[:8], 6, 64)
    a.close(); b.close()


def test_llama8b_dynamic_equals_static():
    wl = si.WORKLOADS["llama8b"]
    m = wl.model
    log("case: llama8b shape, prompt 4 + 4 steps, dynamic vs static, the benchmark's cache")
    a, b = run_pair(m, cached_weights(m), si.prompt_tokens(wl)[:4], 4, wl.prompt_len + wl.steps)
    a.close(); b.close()


def test_dynamic_refuses_other_contexts(tiny):
    import torch
    w, _ = tiny
    log("case: dynamic scheduling argument checks")
    wl = si.WORKLOADS["tiny_b4"]
    cfg = mk.make_config(si.TINY, max_seqs=4, max_blocks_per_seq=3, num_blocks=12)
    dec = mk.Decoder(cfg, 0)
    dec.load_weights(w)
    t = torch.zeros(4, dtype=torch.int32, device=dec.dev)
    with pytest.raises(mk.MKError) as e:
        mk.mk_decode_step_dynamic(dec.ctx, t, 1, t, dec.stream_ptr())
    assert e.value.status == -7
    dec.close()
    cfg = mk.make_config(si.TINY, max_seqs=1, max_blocks_per_seq=3, num_blocks=3, weight_format=1)
    dec = mk.Decoder(cfg, 0)
    dec.load_weights(w)
    with pytest.raises(mk.MKError) as e:
        mk.mk_decode_step_dynamic(dec.ctx, dec.tokens, 1, dec.tokens, dec.stream_ptr())
    assert e.value.status == -7
    dec.close()
    dec, _ = make_gpu(si.TINY, w, 48)
    with pytest.raises(mk.MKError) as e:
        mk.mk_decode_step_dynamic(dec.ctx, dec.tokens, 2, dec.tokens, dec.stream_ptr())
    assert e.value.status == -1
    dec.close()


def test_dynamic_watchdog_recovers(tiny, monkeypatch):
    # a 1 microsecond wait budget: waits expire inside the step (queue slots and inputs alike), the launch
    # drains and the timeout is reported; a context with the normal budget then matches the static step
    import torch
    w, prompt = tiny
    log("case: dynamic step under a 1 us watchdog")
    monkeypatch.setenv("MK_WATCHDOG_US", "1")
    dec, _ = make_gpu(si.TINY, w, 48)
    monkeypatch.delenv("MK_WATCHDOG_US")
    dec.tokens[0] = 3
    dec.step_dynamic(dec.tokens, 1, dec.tokens)
    with pytest.raises(mk.MKError) as e:
        dec.sync_check()
    assert e.value.status == -5
    dec.close()
    a, b = run_pair(si.TINY, w, prompt[:3], 3, 48)
    a.close(); b.close()
