"""Benchmark: per-token decode latency of the persistent megakernel on one MI355X.

Workload (default): the Llama-3-8B-shaped decoder at batch 1 with bf16 random weights
N(0, 0.02) (about 16 GB). A 39-token uniform-random prompt runs through the step, then
greedy decode steps follow at positions 39, 40, ... This is the latency workload shape
of the MegaKernel article (39-token prompt, 512 generated tokens). Weights and the KV
cache are resident in HBM before timing starts.

Prints ONE JSON line on stdout. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode ms/token (batch 1, 8B-shape bf16); achieved HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_info():
    """The host CPU as /proc/cpuinfo names it (model string, family/model/stepping) and the cores this
    process may use."""
    info = {"model": "unknown", "family": None, "model_id": None, "stepping": None}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "model name" and info["model"] == "unknown":
                info["model"] = v
            elif k == "cpu family" and info["family"] is None:
                info["family"] = v
            elif k == "model" and info["model_id"] is None:
                info["model_id"] = v
            elif k == "stepping" and info["stepping"] is None:
                info["stepping"] = v
    except OSError:
        pass
    info["cores"] = len(os.sched_getaffinity(0))
    return info


def timed_steps(torch, stream, step, K):
    """Runs step() K times between events recorded on `stream` before the first and after every step;
    returns (ms over all K steps, per-step ms)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(K):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return evs[0].elapsed_time(evs[K]), [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]


def timed_once(torch, stream, fn):
    """ms of one call of fn() between two events on `stream`."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def oracle_sample(wl, weights, positions, precision, seconds):
    """The oracle as it stands, on this host's cores: single-sequence decode steps of the workload's model
    at the given positions, with a cache holding the workload's seeded N(0, 1) K/V below each position
    (the values do not change the work). Stops after `seconds` (at least 2 steps).
    Returns (ms per step, steps run, threads)."""
    import oracle as orc
    si = si_mod()
    orc.set_threads(len(os.sched_getaffinity(0)))
    m = wl.model
    max_pos = max(positions) + 1
    om = orc.OracleModel(m, weights, 1, max_pos, precision=precision)
    for l in range(m.n_layers):
        om.set_kv(l, 0, 0, si.kv_fill(wl, l, 0, max_pos, "k"), si.kv_fill(wl, l, 0, max_pos, "v"))
    times = []
    t_all = time.perf_counter()
    for i, pos in enumerate(positions):
        t0 = time.perf_counter()
        om.step(0, (1 + 7919 * i) % m.vocab, pos)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > seconds and len(times) >= 2:
            break
    th = orc.threads()
    om.close()
    return 1e3 * sum(times) / len(times), len(times), th


def cpu_baseline(wl, weights, positions, seconds, what):
    """The plain fp32 oracle (the reported baseline) and its fp64 build beside it, each on a bounded
    sample of the timed workload's decode steps."""
    cpu = cpu_info()
    ms32, n32, th32 = oracle_sample(wl, weights, positions, "f32", seconds * 0.5)
    ms64, n64, _ = oracle_sample(wl, weights, positions, "f64", seconds * 0.5)
    return {"value": ms32, "unit": "ms/token", "tokens_per_s": 1e3 / ms32, "cores": th32, "kind": "oracle",
            "precision": "fp32 (plain C, OpenMP over rows and heads)",
            "cpu": cpu["model"], "cpu_family_model_stepping": [cpu["family"], cpu["model_id"], cpu["stepping"]],
            "sample": "%d single-sequence decode steps of the full model (%s) at positions %s; weights read "
                      "from host memory each step" % (n32, what, ", ".join(str(p) for p in positions[:n32])),
            "fp64": {"value": ms64, "unit": "ms/token", "steps": n64,
                     "what": "the fp64 build of the same oracle (the parity reference), same positions"},
            "note": "a reported baseline, not the optimisation target"}


def spread(lo, hi, n):
    """n integer points spread evenly over [lo, hi]."""
    if n <= 1 or hi <= lo:
        return [lo]
    return [lo + (hi - lo) * i // (n - 1) for i in range(n)]


def graph_info(mk, dec):
    """The task graph the timed decoder runs (what the parity tests pin by hash)."""
    info = mk.mk_graph_stats(dec.ctx)
    c = dec.cfg
    return {"n_cus": int(info.n_cus), "max_blocks_per_seq": int(c.max_blocks_per_seq), "num_blocks": int(c.num_blocks),
            "n_tasks": int(info.n_tasks), "attn_tasks_per_layer": int(info.attn_tasks),
            "n_stages": int(info.n_stages), "max_queue_len": int(info.max_queue_len),
            "hash": "0x%016x" % int(info.hash)}


def si_mod():
    import seeded_inputs as si
    return si


def decode_legs(torch, dec, n, K, first, reset, stream):
    """The timed decode of K greedy steps of n sequences from one starting state, two ways:
      - resident: mk_decode_n, all K steps in one launch (each step's argmax feeds the next on the device);
      - per launch: K calls of mk_decode_step, one launch each, events around every step.
    reset() restores the starting context lengths. Returns (resident ms, per-launch ms, per-step ms list,
    whether both produced the same tokens)."""
    toks = torch.zeros((K + 1, n), dtype=torch.int32, device=dec.dev)
    toks[0].copy_(first)
    reset()
    rows = iter(range(K))

    def one_step():  # step i reads row i and writes row i + 1
        i = next(rows)
        dec.step(toks[i], n, toks[i + 1])

    ms_launch, per_step = timed_steps(torch, stream, one_step, K)
    dec.sync_check()
    reset()
    out = torch.zeros((K, n), dtype=torch.int32, device=dec.dev)
    ms_res = timed_once(torch, stream, lambda: dec.decode_n(first, K, n, out))
    dec.sync_check()
    same = bool(torch.equal(out, toks[1:]))
    return ms_res, ms_launch, per_step, same


def trace_leg(dec, first, positions):
    """After the timed legs: one traced step at each of the given positions (a two-step resident launch
    whose second step is the one the trace keeps), summarised per stage. Returns {position: summary}."""
    from persistent_megakernel_03_amd import trace as tz
    dec.enable_trace()
    res = {}
    for pos in positions:
        dec.set_ctx_lens([pos - 1])
        dec.decode_n(first, 2, 1)
        dec.sync_check()
        summ, total = tz.stage_summary(dec.read_trace())
        log(tz.format_summary(summ, total, "traced step at position %d" % pos))
        res[str(pos)] = {"step_span_us": round(total, 2),
                         "stages": [{k: (round(v, 2) if isinstance(v, float) else v) for k, v in x.items()} for x in summ]}
    dec.disable_trace()
    return res


def dynamic_leg(torch, np, dec, g0, P, n, stream):
    """The same n steps from position P, one launch per step, with the tasks scheduled ahead of time
    (mk_decode_step) and at run time from the device's ready queue (mk_decode_step_dynamic); both must
    give the same tokens. Returns {ms per token each way, tokens equal}."""
    res = {}
    toks = {}
    for name, fn in (("static", dec.step), ("dynamic", dec.step_dynamic)):
        dec.set_ctx_lens([P])
        t = torch.zeros((n + 1, 1), dtype=torch.int32, device=dec.dev)
        t[0].copy_(g0)
        rows = iter(range(n))

        def one(fn=fn, t=t, rows=rows):
            i = next(rows)
            fn(t[i], 1, t[i + 1])

        res[name] = timed_once(torch, stream, lambda: [one() for _ in range(n)]) / n
        dec.sync_check()
        toks[name] = t
    same = bool(torch.equal(toks["static"], toks["dynamic"]))
    log("scheduling: ahead of time %.4f ms/token, at run time (ready queue) %.4f ms/token over %d steps; tokens "
        "equal: %s" % (res["static"], res["dynamic"], n, same))
    return {"static_ms_per_token": round(res["static"], 5), "dynamic_ms_per_token": round(res["dynamic"], 5),
            "steps": n, "tokens_equal": same,
            "what": "one launch per step both ways: per-CU queues built ahead of time, or a device-side ready "
                    "queue fed by event completion (mk_decode_step_dynamic)"}


def prefill_leg(mk, torch, np, m, weights, prompt, nb, dec, g0, rf):
    """Time to the first token for the workload's prompt, two ways: one decode step per prompt token
    (the context `dec`, one-sequence graph) and chunked through the 16-row batched graph (a second
    context with prefill_rows = 16). Each is timed on the host around one mk_prefill call after one
    untimed call, from an empty cache; both must give the same next token unless the logits tie."""
    P = len(prompt)
    g1 = torch.zeros(1, dtype=torch.int32, device=dec.dev)
    dec.set_ctx_lens([0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec.prefill(list(prompt), g1)
    torch.cuda.synchronize()
    ms_seq = 1e3 * (time.perf_counter() - t0)
    dec.sync_check()
    seq_logits = dec.read_logits(0)
    cfg = mk.make_config(m, max_seqs=1, max_blocks_per_seq=nb, num_blocks=nb, prefill_rows=16)
    d2 = mk.Decoder(cfg, 0)
    d2.load_weights(weights)
    d2.set_page_table(np.arange(nb, dtype=np.int32).reshape(1, nb))
    g2 = torch.zeros(1, dtype=torch.int32, device=d2.dev)
    times = []
    for _ in range(3):
        d2.set_ctx_lens([0])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        d2.prefill(list(prompt), g2)   # synchronises and checks the device error word itself
        times.append(1e3 * (time.perf_counter() - t0))
    ms_chunk = float(np.median(times[1:]))
    chunk_logits = d2.read_logits(0)
    rel = float(np.linalg.norm(chunk_logits - seq_logits) / np.linalg.norm(seq_logits))
    n_chunks = (P + 15) // 16
    chunk_bytes = n_chunks * rf.weight_bytes_per_token(m) + sum(rf.kv_read_bytes_per_token(m, i + 1) for i in range(P))
    finish(d2)
    same = int(g1.item()) == int(g2.item())
    log("prefill of %d tokens: one step per token %.2f ms, chunks of 16 %.2f ms (%d launches); next token "
        "equal: %s; logits rel L2 between the two %.2e" % (P, ms_seq, ms_chunk, n_chunks, same, rel))
    return {"prompt_tokens": P, "one_step_per_token_ms": round(ms_seq, 3), "chunked_16_rows_ms": round(ms_chunk, 3),
            "chunk_launches": n_chunks, "speedup": round(ms_seq / ms_chunk, 2),
            "chunked_hbm_gbs": round(chunk_bytes / (ms_chunk * 1e-3) / 1e9, 1),
            "next_token_equal": same, "logits_rel_l2_between": float("%.3e" % rel),
            "what": "host wall time of one mk_prefill call from an empty cache (the chunked call synchronises "
                    "itself); algorithmic bytes of the chunked run: the weights once per chunk plus each "
                    "position's KV rows"}


def roofline_obj(rf, achieved, traffic_per_step, bytes_avg, K, ms_launch, kernel):
    """The roofline object of the timed kernel. One launch runs all K steps: `achieved` is the launch's
    algorithmic bytes (K x bytes_per_step) over its event-timed duration; `traffic` is the launch's HBM
    bytes from the rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, copy-calibrated) recorded for these
    kernel sources, else null."""
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": rf.MI355X_HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / rf.MI355X_HBM_PEAK_GBS, 4),
            "traffic": None if traffic_per_step is None else int(traffic_per_step * K),
            "traffic_unit": "HBM bytes per launch of %d steps" % K,
            "traffic_per_step": traffic_per_step, "bytes_per_step": int(bytes_avg),
            "bytes_per_launch": int(bytes_avg * K), "launch_ms": round(ms_launch, 3), "steps_per_launch": K,
            "kernel": kernel}


def fp8_leg(mk, torch, np, m, weights, prompt, nb, K, W, rf, ms_bf16):
    """The same decode with FP8 weights (weight_format = 1: E4M3 codes, one power-of-two scale per row,
    quantised on the device at load): the prompt, W warm-up steps, then K greedy steps at positions
    P .. P+K-1 in one resident launch, timed with events. Its bytes per step count one byte per GEMV
    weight plus the row scales."""
    P = len(prompt)
    cfg = mk.make_config(m, max_seqs=1, max_blocks_per_seq=nb, num_blocks=nb, weight_format=1)
    d8 = mk.Decoder(cfg, 0)
    d8.load_weights(weights)
    d8.set_page_table(np.arange(nb, dtype=np.int32).reshape(1, nb))
    d8.set_ctx_lens([0])
    g0 = torch.zeros(1, dtype=torch.int32, device=d8.dev)
    d8.prefill(list(prompt), g0)
    d8.decode_n(g0, W, 1)
    d8.set_ctx_lens([P])
    d8.sync_check()
    stream = torch.cuda.current_stream(d8.dev)
    out = torch.zeros((K, 1), dtype=torch.int32, device=d8.dev)
    ms_launch = timed_once(torch, stream, lambda: d8.decode_n(g0, K, 1, out))
    d8.sync_check()
    ms = ms_launch / K
    bytes_avg = sum(rf.step_bytes(m, [P + i + 1], fp8=True) for i in range(K)) / K
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    info = mk.mk_graph_stats(d8.ctx)
    finish(d8)
    traffic = None
    if m.name == "llama8b":
        traffic = rf.profiled_traffic(os.path.join(ROOT, "profiles", "mk_megakernel_llama8b_b1_fp8_decode.md"))
    log("fp8 weights: resident %.4f ms/token (%.1f tok/s), %.1f GB/s (%.1f%% of %.0f GB/s); %.2fx the bf16 decode"
        % (ms, 1e3 / ms, achieved, 100 * achieved / rf.MI355X_HBM_PEAK_GBS, rf.MI355X_HBM_PEAK_GBS, ms_bf16 / ms))
    return {"ms_per_token": round(ms, 5), "tokens_per_s": round(1e3 / ms, 2), "steps": K,
            "weight_bytes_per_token": rf.weight_bytes_per_token_fp8(m), "graph_hash": "0x%016x" % info.hash,
            "roofline": roofline_obj(rf, achieved, traffic, bytes_avg, K, ms_launch, "mk_megakernel, FP8 weights"),
            "speedup_vs_bf16": round(ms_bf16 / ms, 3),
            "what": "E4M3 weight codes with one power-of-two scale per output row, decoded in the GEMV tile "
                    "(fp32 accumulation); the same prompt and positions as the bf16 decode"}


def finish(dec):
    """Release the decoder and its device buffers, with the device idle, before the process exits."""
    import torch
    torch.cuda.synchronize()
    dec.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bench_batched(args, wl):
    """Decode from pre-filled caches: all sequences of the workload in every step (one for the long-
    context workload, several for the batched ones), each from its own KV cache pre-filled to its
    context length, pages permuted. A step's algorithmic bytes are the weights once plus every
    sequence's KV rows."""
    import numpy as np
    import torch
    import persistent_megakernel_03_amd as mk
    from persistent_megakernel_03_amd import roofline as rf
    si = si_mod()
    m = wl.model
    n = wl.n_seqs
    K, W = args.steps if args.steps else wl.steps, args.warmup
    ctx = si.context_lengths(wl).astype(np.int64)
    # the cache (and so the task graph) holds the workload's full decode, whatever K is
    cap = ctx + max(wl.steps, K, W)
    table, nblocks = si.block_tables(wl, cap)
    t0 = time.time()
    weights = si.gen_weights(m)
    log("weights generated in %.1fs" % (time.time() - t0))
    cfg = mk.make_config(m, max_seqs=n, max_blocks_per_seq=table.shape[1], num_blocks=nblocks)
    dec = mk.Decoder(cfg, 0)
    dec.load_weights(weights)
    dec.set_page_table(table)
    graph = graph_info(mk, dec)
    # cache contents do not change the work; fill them on the device from a seeded generator
    g = torch.Generator(device=dec.dev)
    g.manual_seed(1234)
    for pool in dec.k_pools + dec.v_pools:
        pool.copy_(torch.randn(pool.numel(), generator=g, device=dec.dev).to(torch.bfloat16).view(torch.int16))
    first = torch.as_tensor(si.first_tokens(wl), dtype=torch.int32, device=dec.dev)
    dec.set_ctx_lens(ctx)
    dec.tokens[:n].copy_(first)
    for _ in range(W):
        dec.step(dec.tokens, n)
    # and one resident launch: the process's first cooperative launch of a kernel pays a one-time setup
    # (about 5 ms for the batched kernel), which is not a step's cost
    dec.decode_n(first, max(W, 1), n)
    dec.sync_check()
    stream = torch.cuda.current_stream(dec.dev)
    ms_res, ms_launch, per_step, same = decode_legs(torch, dec, n, K, first, lambda: dec.set_ctx_lens(ctx), stream)
    assert (dec.ctx_lens.cpu().numpy()[:n] == ctx + K).all()
    ms, ms1 = ms_res / K, ms_launch / K
    bytes_avg = sum(rf.step_bytes(m, list(ctx + i + 1)) for i in range(K)) / K
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    log("decode (%d sequences): resident %.4f ms/step, one launch per step %.4f ms/step; %.1f GB/s "
        "(%.1f%% of %.0f GB/s); tokens equal: %s" % (n, ms, ms1, achieved, 100 * achieved / rf.MI355X_HBM_PEAK_GBS,
                                                    rf.MI355X_HBM_PEAK_GBS, same))
    finish(dec)
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        c0 = int(ctx[0])
        cpu = cpu_baseline(wl, weights, spread(c0, c0 + K - 1, 8), args.cpu_seconds,
                           "%s, sequence 0 alone, cache pre-filled to its context" % wl.name)
        log("cpu baseline: %.1f ms/token on %d cores (%.1fs)" % (cpu["value"], cpu["cores"], time.time() - t0))
    traffic = None
    if wl.name == "llama8b_b16":
        traffic = rf.profiled_traffic(os.path.join(ROOT, "profiles", "mk_megakernel_llama8b_b16_decode.md"))
    if n == 1:
        metric = "decode ms/token (batch 1, %s-shape bf16, %d-position context); achieved HBM GB/s vs peak" % (
            m.name, int(ctx[0]))
        workload = "%s: one sequence, cache pre-filled to %d positions, %d steps" % (wl.name, int(ctx[0]), K)
    else:
        metric = "decode ms/step (%d sequences, %s-shape bf16); achieved HBM GB/s vs peak" % (n, m.name)
        workload = "%s: %d sequences, contexts %d..%d (seeded uniform in [%d, %d]), %d steps" % (
            wl.name, n, int(ctx.min()), int(ctx.max()), wl.ctx_range[0], wl.ctx_range[1], K)
    out = {
        "metric": metric,
        "value": round(ms, 5),
        "unit": "ms/token" if n == 1 else "ms/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(n * 1e3 / ms, 1),
        "achieved_hbm_gbs": round(achieved, 1),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "weights_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "batch": n, "decode_steps": K,
                   "weight_bytes_per_step": rf.weight_bytes_per_token(m),
                   "kv": "bf16, paged in 16-token blocks, permuted page tables", "graph": graph,
                   "timed": "mk_decode_n: all %d steps in one launch" % K},
        "one_launch_per_step": {"ms_per_step": round(ms1, 5),
                                "ms_per_step_median": round(float(np.median(per_step)), 5),
                                "tokens_equal_to_resident": same},
        "roofline": roofline_obj(rf, achieved, traffic, bytes_avg, K, ms_res,
                                 "mk_megakernel%s" % (", batched" if n > 1 else "")),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed decode steps (0: the workload's own count)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--staged-steps", type=int, default=64, help="steps of the stage-sliced comparison run (0: skip it)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the time-to-first-token comparison")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-weights decode")
    ap.add_argument("--dynamic-steps", type=int, default=64,
                    help="steps of the run-time scheduling comparison (0: skip it)")
    ap.add_argument("--trace-summary", action="store_true",
                    help="after the timed legs, trace one step at three positions and report per-stage times")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (to scale HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": 1 << 30, "dispatches": 5}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this decode path runs on one GPU and has no multi-GPU mode "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import persistent_megakernel_03_amd as mk
    from persistent_megakernel_03_amd import roofline as rf
    import seeded_inputs as si

    wl = si.WORKLOADS[args.workload]
    m = wl.model
    if wl.n_seqs > 1 or wl.prompt_len == 0:  # pre-filled caches: the batched and long-context workloads
        return bench_batched(args, wl)
    K, W = args.steps if args.steps else wl.steps, args.warmup
    P = wl.prompt_len
    # The cache, and so the task graph, is sized for the workload's whole decode (prompt + its steps),
    # whatever K is: the timed graph is the one the parity tests run.
    n_pos = P + max(wl.steps, K, W)
    t0 = time.time()
    weights = si.gen_weights(m)
    prompt = si.prompt_tokens(wl)
    log("weights generated in %.1fs" % (time.time() - t0))
    nb = (n_pos + 15) // 16
    cfg = mk.make_config(m, max_seqs=1, max_blocks_per_seq=nb, num_blocks=nb)
    dec = mk.Decoder(cfg, 0)
    t0 = time.time()
    dec.load_weights(weights)
    log("weights loaded in %.1fs" % (time.time() - t0))
    graph = graph_info(mk, dec)
    dec.set_page_table(np.arange(nb, dtype=np.int32).reshape(1, nb))
    dec.set_ctx_lens([0])
    g0 = torch.zeros(1, dtype=torch.int32, device=dec.dev)
    dec.prefill(list(prompt), g0)
    tokens = g0.clone()
    for _ in range(W):
        dec.step(tokens)
    dec.decode_n(g0, W, 1)
    dec.sync_check()
    stream = torch.cuda.current_stream(dec.dev)
    # timed: K greedy steps at positions P .. P+K-1 starting from the first generated token
    ms_res, ms_launch, per_step, same = decode_legs(torch, dec, 1, K, g0, lambda: dec.set_ctx_lens([P]), stream)
    assert int(dec.ctx_lens.item()) == P + K
    ms, ms1 = ms_res / K, ms_launch / K
    bytes_avg = sum(rf.step_bytes(m, [P + i + 1]) for i in range(K)) / K
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    log("decode: resident %.4f ms/token (%.1f tok/s), one launch per token %.4f ms/token; %.1f GB/s "
        "(%.1f%% of %.0f GB/s); tokens equal: %s" % (ms, 1e3 / ms, ms1, achieved,
                                                    100 * achieved / rf.MI355X_HBM_PEAK_GBS,
                                                    rf.MI355X_HBM_PEAK_GBS, same))
    # The same steps as one dispatch per dependency stage (same kernel and graph): the stop-and-go
    # execution the single launch replaces. Its extra time per token is the pass-to-pass cost removed.
    n_stages = graph["n_stages"]
    Ks = min(K, args.staged_steps)
    pass_to_pass = None
    if Ks > 0:
        dec.set_ctx_lens([P])
        tokens.copy_(g0)
        ms_staged = timed_once(torch, stream, lambda: [dec.step_staged(tokens) for _ in range(Ks)]) / Ks
        dec.sync_check()
        dec.set_ctx_lens([P])
        tokens.copy_(g0)
        ms_fused_same = timed_once(torch, stream, lambda: [dec.step(tokens) for _ in range(Ks)]) / Ks
        dec.set_ctx_lens([P])
        ms_res_same = timed_once(torch, stream, lambda: dec.decode_n(g0, Ks, 1)) / Ks
        dec.sync_check()
        log("staged: %.4f ms/token in %d dispatches; one launch per token %.4f, resident %.4f ms/token over the "
            "same %d steps" % (ms_staged, n_stages, ms_fused_same, ms_res_same, Ks))
        pass_to_pass = {"stage_sliced_ms_per_token": round(ms_staged, 5), "dispatches_per_token": n_stages,
                        "one_launch_per_token_ms": round(ms_fused_same, 5),
                        "resident_ms_per_token": round(ms_res_same, 5), "steps": Ks,
                        "removed_by_one_launch_ms_per_token": round(ms_staged - ms_fused_same, 5),
                        "removed_us_per_boundary": round(1e3 * (ms_staged - ms_fused_same) / max(1, n_stages - 1), 3),
                        "removed_by_resident_ms_per_token": round(ms_fused_same - ms_res_same, 5),
                        "what": "the same kernel and task graph launched once per dependency stage (stop-and-go), "
                                "once per token, and once for all the steps"}
    dynamic = dynamic_leg(torch, np, dec, g0, P, min(K, args.dynamic_steps), stream) if args.dynamic_steps > 0 else None
    task_trace = trace_leg(dec, g0, spread(P + 1, P + K - 1, 3)) if args.trace_summary else None
    prefill = None if args.no_prefill else prefill_leg(mk, torch, np, m, weights, prompt, nb, dec, g0, rf)
    finish(dec)
    fp8 = None if args.no_fp8 else fp8_leg(mk, torch, np, m, weights, prompt, nb, K, W, rf, ms)

    traffic = None
    if wl.name == "llama8b":
        traffic = rf.profiled_traffic(os.path.join(ROOT, "profiles", "mk_megakernel_llama8b_b1_decode.md"))

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(wl, weights, spread(P, P + K - 1, 8), args.cpu_seconds,
                           "%s, batch 1, the timed positions" % wl.name)
        log("cpu baseline: %.1f ms/token on %d cores (%.1fs)" % (cpu["value"], cpu["cores"], time.time() - t0))

    out = {
        "metric": METRIC if m.name == "llama8b" else METRIC.replace("8B-shape", "%s-shape" % m.name),
        "value": round(ms, 5),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(1e3 / ms, 2),
        "achieved_hbm_gbs": round(achieved, 1),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "weights_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s decode, batch 1, %d-token prompt, greedy steps at positions %d..%d"
                               % (wl.name, P, P, P + K - 1),
                   "batch": 1, "prompt_len": P, "decode_steps": K,
                   "weight_bytes_per_token": rf.weight_bytes_per_token(m),
                   "kv": "bf16, paged in 16-token blocks", "graph": graph,
                   "timed": "mk_decode_n: all %d steps in one launch" % K},
        "one_launch_per_step": {"ms_per_step": round(ms1, 5),
                                "ms_per_step_median": round(float(np.median(per_step)), 5),
                                "tokens_equal_to_resident": same},
        "roofline": roofline_obj(rf, achieved, traffic, bytes_avg, K, ms_res, "mk_megakernel"),
        "cpu_baseline": cpu,
        "pass_to_pass": pass_to_pass,
    }
    if dynamic is not None:
        out["dynamic_schedule"] = dynamic
    if prefill is not None:
        out["prefill"] = prefill
    if fp8 is not None:
        out["fp8_weights"] = fp8
    if task_trace is not None:
        out["task_trace"] = task_trace
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
