"""Host logic: the per-stage summary of an in-kernel trace, on a synthetic trace whose figures are
known by construction."""
import numpy as np

import persistent_megakernel_03_amd as mk
from persistent_megakernel_03_amd import trace as tz


def synthetic_trace(n_layers=5, tasks=4):
    # every stage of every layer: its tasks reach the queue 1 us after the previous stage ends, see
    # their input 2 us (task 0) to 5 us (task 3) after it, stream 10 us and publish 1 us later; the
    # last task of each stage ends last. Times in 100 MHz ticks from an arbitrary origin.
    recs, t = [], 123456789
    stages = [(l, ty) for l in range(n_layers) for ty in (1, 2, 3, 4, 5)] + [(n_layers - 1, 6), (n_layers - 1, 7)]
    for l, ty in stages:
        prev_end = t
        for i in range(tasks):
            q = prev_end - 100          # the CU was already waiting: handoff measured from prev_end
            r = prev_end + 200 + 100 * i
            s = r + 1000
            d = s + 100
            recs.append((q, r, s, d, i, ty, l, 7, i % 8, 0))
        t = prev_end + 200 + 100 * (tasks - 1) + 1100
    return np.array(recs, dtype=mk.trace_dtype())


def test_stage_summary_figures():
    tr = synthetic_trace()
    summ, total = tz.stage_summary(tr)
    names = [x["stage"] for x in summ]
    assert names == ["qkv", "attention", "o_proj", "gate_up", "down", "lm_head", "argmax"]
    for x in summ:
        assert x["n"] == 4
        assert abs(x["span_us"] - (2.0 + 3.0 + 11.0)) < 1e-9     # last task ready 5 us in, + 10 + 1
        assert abs(x["handoff_med_us"] - 3.5) < 1e-9            # median of 2, 3, 4, 5
        # 90th percentile of the middle layers' 2, 3, 4, 5 us (the last and the LM head's one layer)
        assert abs(x["handoff_p90_us"] - (5.0 if x["layers"] > 3 else 4.7)) < 1e-9
        assert abs(x["stream_med_us"] - 10.0) < 1e-9
        assert abs(x["epilogue_med_us"] - 1.0) < 1e-9
    assert [x["layers"] for x in summ[:5]] == [5] * 5 and summ[5]["layers"] == 1
    assert abs(total - (27 * 16.0 + 1.0)) < 1e-9                # 27 stages of 16 us, + the 1 us queue lead
    text = tz.format_summary(summ, total, "synthetic")
    assert text.splitlines()[0].startswith("synthetic: step span") and len(text.splitlines()) == 2 + len(summ)


def test_handoff_counts_from_queue_arrival_when_late():
    # a task whose CU reaches it after the previous stage ended: its handoff runs from its own arrival
    tr = synthetic_trace(n_layers=1, tasks=1)
    first_down = np.nonzero(tr["type"] == 5)[0][0]
    prev_end = tr["t_done"][first_down - 1]
    tr["t_queue"][first_down] = prev_end + 150
    tr["t_ready"][first_down] = prev_end + 170
    rows = tz.stage_rows(tr)
    down = [x for x in rows if x["type"] == 5][0]
    assert abs(down["handoff"][0] - 0.2) < 1e-9
