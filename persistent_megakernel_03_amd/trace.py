"""Per-stage summary of the megakernel's in-kernel task trace.

With tracing on (mk_set_trace), every task of a step leaves four timestamps from the 100 MHz
constant-rate counter (s_memrealtime): t_queue (its CU reached it in its queue), t_ready (all of its
inputs were present), t_streamed (its own streaming ended) and t_done (its outputs were published).
This module turns one step's records into the per-stage figures that show where a decode step loses
time against the bytes it moves:

- span: from the end of the previous stage to the end of this one (the stage's share of the step);
- handoff: per task, t_ready - max(t_queue, end of the previous stage). For the stages whose every
  task reads the whole output of the stage before (QKV, O projection, gate/up, down and the LM head
  all start with a norm or a full-width input; the argmax reads every LM-head task's key), this is the
  time from the last producer's publication to the consumer seeing it: the event-to-start latency
  that the pages ("LLMs in einen MegaKernel kompilieren", section on event-driven execution) put at
  1-2 microseconds per task switch. Attention tasks read only their KV head's QKV rows, so theirs is
  measured from the same point and can be negative;
- stream: t_streamed - t_ready, the task's own weight (or KV) streaming;
- epilogue: t_done - t_streamed (reduction, activation, stores and the publication).
"""
import numpy as np

TICKS_PER_US = 100.0
STAGE_NAMES = {1: "qkv", 2: "attention", 3: "o_proj", 4: "gate_up", 5: "down", 6: "lm_head", 7: "argmax"}
ORDER = (1, 2, 3, 4, 5, 6, 7)


def stage_rows(tr):
    """One entry per (layer, stage) in execution order: dict(type, layer, n, span, handoff[], stream[],
    epilogue[]), times in microseconds from the step's first t_queue."""
    t0 = int(tr["t_queue"].min())
    us = lambda f: (tr[f].astype(np.int64) - t0) / TICKS_PER_US
    q, r, s, d = us("t_queue"), us("t_ready"), us("t_streamed"), us("t_done")
    ty, ly = tr["type"].astype(int), tr["layer"].astype(int)
    rows, prev_end = [], 0.0
    for l in range(int(ly.max()) + 1):
        for t in ORDER:
            m = (ty == t) & (ly == l)
            if not m.any():
                continue
            end = float(d[m].max())
            # a task with no stream of its own (the argmax) records t_streamed at its start: stream 0
            st = np.maximum(s[m], r[m])
            rows.append(dict(type=t, layer=l, n=int(m.sum()), span=end - prev_end,
                             handoff=r[m] - np.maximum(q[m], prev_end), stream=st - r[m], epilogue=d[m] - st))
            prev_end = end
    return rows


def stage_summary(tr):
    """Per stage type, averaged over the layers (the first and last layer left out when there are more
    than three, so that the step's ramp-up and the LM head's hand-off do not skew the per-layer view):
    n tasks, span, and the median and 90th percentile of handoff, the median of stream and epilogue.
    Also the step's total span (us)."""
    rows = stage_rows(tr)
    out = []
    for t in ORDER:
        rs = [x for x in rows if x["type"] == t]
        if not rs:
            continue
        keep = rs[1:-1] if len(rs) > 3 else rs
        cat = lambda k: np.concatenate([x[k] for x in keep])
        h = cat("handoff")
        out.append(dict(stage=STAGE_NAMES.get(t, str(t)), layers=len(rs), n=keep[0]["n"],
                        span_us=float(np.mean([x["span"] for x in keep])),
                        handoff_med_us=float(np.median(h)), handoff_p90_us=float(np.percentile(h, 90)),
                        stream_med_us=float(np.median(cat("stream"))), epilogue_med_us=float(np.median(cat("epilogue")))))
    total = float((tr["t_done"].astype(np.int64).max() - tr["t_queue"].astype(np.int64).min()) / TICKS_PER_US)
    return out, total


def format_summary(summary, total, label=""):
    lines = ["%sstep span %.1f us" % (label + ": " if label else "", total),
             "%-10s %6s %6s %9s %12s %12s %10s %11s" % ("stage", "layers", "tasks", "span_us", "handoff_med",
                                                       "handoff_p90", "stream_med", "epilog_med")]
    for x in summary:
        lines.append("%-10s %6d %6d %9.2f %12.2f %12.2f %10.2f %11.2f" % (
            x["stage"], x["layers"], x["n"], x["span_us"], x["handoff_med_us"], x["handoff_p90_us"],
            x["stream_med_us"], x["epilogue_med_us"]))
    return "\n".join(lines)
