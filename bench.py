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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def cpu_baseline(shape, weights, prompt, seconds):
    """The oracle as it stands, on this host's cores: decode steps of the same model from
    position 0 (teacher-forced on the prompt tokens) until `seconds` have passed."""
    import oracle as orc
    cores = len(os.sched_getaffinity(0))
    orc.set_threads(cores)
    n_max = max(2, len(prompt))
    om = orc.OracleModel(shape, weights, 1, n_max)
    times = []
    t_all = time.perf_counter()
    for i in range(n_max):
        t0 = time.perf_counter()
        om.step(0, int(prompt[i]), i)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > seconds and len(times) >= 2:
            break
    om.close()
    ms = 1e3 * sum(times) / len(times)
    return {"value": ms, "unit": "ms/token", "tokens_per_s": 1e3 / ms, "cores": orc.threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": "%d decode steps of the full model at positions 0..%d (fp64 oracle, all weights streamed "
                      "from host memory each step)" % (len(times), len(times) - 1)}


def cpu_baseline_batched(wl, weights, seconds):
    """The oracle on this host's cores over a bounded sample of a batched workload: sequence 0 alone,
    its KV cache pre-filled as in the workload, decode steps at its context length."""
    import oracle as orc
    m = wl.model
    cores = len(os.sched_getaffinity(0))
    orc.set_threads(cores)
    ctx0 = int(si_mod().context_lengths(wl)[0])
    om = orc.OracleModel(m, weights, 1, ctx0 + 4)
    for l in range(m.n_layers):
        om.set_kv(l, 0, 0, si_mod().kv_fill(wl, l, 0, ctx0, "k"), si_mod().kv_fill(wl, l, 0, ctx0, "v"))
    tok = int(si_mod().first_tokens(wl)[0])
    times = []
    t_all = time.perf_counter()
    for i in range(4):
        t0 = time.perf_counter()
        tok, _ = om.step(0, tok, ctx0 + i)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > seconds and len(times) >= 2:
            break
    om.close()
    ms = 1e3 * sum(times) / len(times)
    return {"value": ms, "unit": "ms/token", "tokens_per_s": 1e3 / ms, "cores": orc.threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": "%d decode steps of sequence 0 alone (context %d, fp64 oracle, weights streamed from host "
                      "memory each step)" % (len(times), ctx0)}


def si_mod():
    import seeded_inputs as si
    return si


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
    K, W = min(args.steps, wl.steps), args.warmup
    ctx = si.context_lengths(wl).astype(np.int64)
    cap = ctx + max(K, W)
    table, nblocks = si.block_tables(wl, cap)
    t0 = time.time()
    weights = si.gen_weights(m)
    log("weights generated in %.1fs" % (time.time() - t0))
    cfg = mk.make_config(m, max_seqs=n, max_blocks_per_seq=table.shape[1], num_blocks=nblocks)
    dec = mk.Decoder(cfg, 0)
    dec.load_weights(weights)
    dec.set_page_table(table)
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
    dec.sync_check()
    dec.set_ctx_lens(ctx)
    dec.tokens[:n].copy_(first)
    stream = torch.cuda.current_stream(dec.dev)
    ms_total, per_step = timed_steps(torch, stream, lambda: dec.step(dec.tokens, n), K)
    ms = ms_total / K
    dec.sync_check()
    assert (dec.ctx_lens.cpu().numpy()[:n] == ctx + K).all()
    bytes_avg = sum(rf.step_bytes(m, list(ctx + i + 1)) for i in range(K)) / K
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    log("batched decode (%d sequences): %.4f ms/step, %.1f tok/s, %.1f GB/s (%.1f%% of %.0f GB/s)" %
        (n, ms, n * 1e3 / ms, achieved, 100 * achieved / rf.MI355X_HBM_PEAK_GBS, rf.MI355X_HBM_PEAK_GBS))
    dec.close()
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline_batched(wl, weights, args.cpu_seconds)
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
        "ms_per_step_median": round(float(np.median(per_step)), 5),
        "tokens_per_s": round(n * 1e3 / ms, 1),
        "achieved_hbm_gbs": round(achieved, 1),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "weights_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload,
                   "batch": n, "decode_steps": K, "weight_bytes_per_step": rf.weight_bytes_per_token(m),
                   "kv": "bf16, paged in 16-token blocks, permuted page tables"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": rf.MI355X_HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / rf.MI355X_HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes/launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "bytes_per_launch": int(bytes_avg),
                     "kernel": "mk_megakernel%s (one launch per step)" % (", batched" if n > 1 else "")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--staged-steps", type=int, default=64, help="steps of the stage-sliced comparison run (0: skip it)")
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
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
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
    K, W = args.steps, args.warmup
    P = wl.prompt_len
    n_pos = P + max(K, W)
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
    dec.set_page_table(np.arange(nb, dtype=np.int32).reshape(1, nb))
    dec.set_ctx_lens([0])
    g0 = torch.zeros(1, dtype=torch.int32, device=dec.dev)
    dec.prefill(list(prompt), g0)
    tokens = g0.clone()
    for _ in range(W):
        dec.step(tokens)
    dec.sync_check()
    # timed region: K greedy steps at positions P .. P+K-1 starting from the first generated token
    dec.set_ctx_lens([P])
    tokens.copy_(g0)
    stream = torch.cuda.current_stream(dec.dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms_total, per_step = timed_steps(torch, stream, lambda: dec.step(tokens), K)
    dec.sync_check()
    assert int(dec.ctx_lens.item()) == P + K
    ms = ms_total / K
    bytes_avg = sum(rf.step_bytes(m, [P + i + 1]) for i in range(K)) / K
    achieved = bytes_avg / (ms * 1e-3) / 1e9
    log("decode: %.4f ms/token, %.1f tok/s, %.1f GB/s (%.1f%% of %.0f GB/s)" %
        (ms, 1e3 / ms, achieved, 100 * achieved / rf.MI355X_HBM_PEAK_GBS, rf.MI355X_HBM_PEAK_GBS))
    # The same steps as one dispatch per dependency stage (same kernel and graph): the stop-and-go
    # execution the single launch replaces. Its extra time per token is the pass-to-pass cost removed.
    n_stages = int(mk.mk_graph_stats(dec.ctx).n_stages)
    Ks = min(K, args.staged_steps)
    pass_to_pass = None
    if Ks > 0:
        dec.set_ctx_lens([P])
        tokens.copy_(g0)
        torch.cuda.synchronize(dec.dev)
        ev0.record(stream)
        for _ in range(Ks):
            dec.step_staged(tokens)
        ev1.record(stream)
        torch.cuda.synchronize(dec.dev)
        ms_staged = ev0.elapsed_time(ev1) / Ks
        dec.sync_check()
        if Ks < K:  # the one-launch time over the same positions
            dec.set_ctx_lens([P])
            tokens.copy_(g0)
            torch.cuda.synchronize(dec.dev)
            ev0.record(stream)
            for _ in range(Ks):
                dec.step(tokens)
            ev1.record(stream)
            torch.cuda.synchronize(dec.dev)
            ms_fused_same = ev0.elapsed_time(ev1) / Ks
        else:
            ms_fused_same = ms
        log("staged: %.4f ms/token in %d dispatches (one launch: %.4f ms/token over the same %d steps)" %
            (ms_staged, n_stages, ms_fused_same, Ks))
        pass_to_pass = {"stage_sliced_ms_per_token": round(ms_staged, 5), "dispatches_per_token": n_stages,
                        "one_launch_ms_per_token": round(ms_fused_same, 5), "steps": Ks,
                        "removed_ms_per_token": round(ms_staged - ms_fused_same, 5),
                        "removed_us_per_boundary": round(1e3 * (ms_staged - ms_fused_same) / max(1, n_stages - 1), 3),
                        "what": "the same kernel and task graph launched once per dependency stage (stop-and-go) "
                                "vs once per step"}
    dec.close()

    traffic = None
    if wl.name == "llama8b":
        traffic = rf.profiled_traffic(os.path.join(ROOT, "profiles", "mk_megakernel_llama8b_b1_decode.md"))

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(m, weights, prompt, args.cpu_seconds)
        log("cpu baseline: %.1f ms/token on %d cores (%.1fs)" % (cpu["value"], cpu["cores"], time.time() - t0))

    out = {
        "metric": METRIC if m.name == "llama8b" else METRIC.replace("8B-shape", "%s-shape" % m.name),
        "value": round(ms, 5),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "ms_per_step_median": round(float(np.median(per_step)), 5),
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
                   "kv": "bf16, paged in 16-token blocks"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": rf.MI355X_HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / rf.MI355X_HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes/launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "bytes_per_launch": int(bytes_avg), "kernel": "mk_megakernel (one launch per decode step)"},
        "cpu_baseline": cpu,
        "pass_to_pass": pass_to_pass,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
