"""Decode benchmark: µs/token and achieved HBM bandwidth of the persistent
decode kernel on one MI355X.

    python bench.py [--gpus 1] [--steps 256] [--warmup 32] [--workload dense8b_ctx1024]

One "step" is one decode step (one token) through the whole hot path.  The
default workload is the 8B-shape dense decoder at batch 1: 32 layers, hidden
4096, 32 query / 8 KV heads of 128, SwiGLU 14336, vocabulary 128256, bf16
weights ~N(0, 0.02) from seed 0, the KV cache prefilled on the GPU from 1024
random tokens, then greedy decode.  The timed region is ONE engine call of
--steps steps (one persistent kernel launch), bracketed by device
synchronisation; it is repeated --repeats times from the same prefilled
position and the median is reported.  Inputs are resident in HBM.

Also reported: the roofline of the persistent kernel (algorithmic bytes per
launch over the launch time measured with HIP events on the launch stream,
against 8 TB/s), the one-kernel-per-operator baseline on the same workload,
the rate of a read-only streaming kernel measured on the same box, reported
beside the decode rate (stream_reference), the tiny-decoder persistent vs
baseline latency, and the CPU oracle timed on a bounded sample
(cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(workload, device="cuda", seed=0, prefill="engine", **eng_kw):
    """Weights, cache and engine of a workload.  prefill="engine" fills the
    cache by teacher-forced decode of the workload's random prompt (the
    workload as specified); "synthetic" writes seeded N(0,1) K/V rows instead
    and decodes from token 1 -- the same bytes and flops per step, without a
    prefill launch (used for profiler runs that must see only timed launches)."""
    import torch
    from persistent_resident_execution_amd import engine as E
    from persistent_resident_execution_amd import synth
    w = synth.WORKLOADS[workload]
    m = w.model
    t0 = time.time()
    W = synth.gen_weights(m, seed=seed, device=device)
    P = w.contexts[0]
    if m.batch > 1:
        # micro-batch: each sequence at its own context; the cache is the
        # seeded synthetic one (the prefill of unequal lengths is not a
        # lockstep decode), the first tokens seeded
        kc, vc = synth.gen_kv_cache(m, max(w.contexts), seed=seed + 1, device=device)
        eng = E.Engine(m, W, kc, vc, **eng_kw)
        g0 = synth.gen_tokens(m.vocab, m.batch, seed=seed + 2, device=device)
        log(f"[bench] {workload}: weights + synthetic cache of contexts {list(w.contexts)} "
            f"in {time.time() - t0:.1f}s")
        return w, m, W, kc, vc, eng, g0
    if prefill == "synthetic":
        kc, vc = synth.gen_kv_cache(m, P, seed=seed + 1, device=device)
    else:
        shape = (m.n_layers, m.batch, m.n_kv_heads, m.max_ctx, m.head_dim)
        kc = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        vc = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    eng = E.Engine(m, W, kc, vc, **eng_kw)
    if prefill == "synthetic":
        g0 = torch.ones(1, dtype=torch.int32, device=device)
    else:
        prompt = synth.gen_tokens(m.vocab, P, seed=seed, device=device)
        eng.set_positions([0])
        out = eng.decode(P, forced=prompt.view(P, 1))  # cache filled by the engine itself
        torch.cuda.synchronize()
        eng.status()
        g0 = out[-1].contiguous()
    log(f"[bench] {workload}: weights + {prefill} prefill of {P} tokens in {time.time() - t0:.1f}s")
    return w, m, W, kc, vc, eng, g0


def launches_per_token_per_op(m):
    """Kernels the one-kernel-per-operator path launches per step.  Batch 1:
    embedding; per layer two norms and one launch per task stage (5 dense, 6
    MoE); final norm, LM head, argmax.  Micro-batch: the embedding stage, six
    stages per layer, the LM head and the argmax."""
    if m.batch > 1:
        return 6 * m.n_layers + 3
    return (8 if m.is_moe else 7) * m.n_layers + 4


def time_calls(eng, fn, n_steps, g0, P, repeats, warmup_steps):
    """Seconds of each of `repeats` calls of n_steps from position(s) P (an
    int, or one per sequence); also returns the tokens of the last call."""
    import torch
    stream = torch.cuda.current_stream()
    pos = list(P) if isinstance(P, (list, tuple)) else [P]
    out = torch.empty((max(n_steps, warmup_steps, 1), len(pos)), dtype=torch.int32, device="cuda")
    if warmup_steps:
        eng.set_positions(pos)
        fn(warmup_steps, in_tokens=g0, out_tokens=out[:warmup_steps])
        torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        eng.set_positions(pos)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        fn(n_steps, in_tokens=g0, out_tokens=out[:n_steps])
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    eng.status()
    return times, out[:n_steps].cpu()


def cpu_baseline(m, W, P, budget_s=15.0, max_steps=64):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    decode steps of the same model (weights copied to the host; the cache is
    a seeded synthetic one -- its values do not change the work) at context P,
    or, for a micro-batch, whole steps = one decode of every sequence at its
    own context (the oracle decodes sequences one at a time)."""
    import numpy as np
    import oracle
    from persistent_resident_execution_amd import synth
    t0 = time.time()
    om = oracle.OracleModel(m, synth.weights_to_numpy(W))
    pos = list(P) if isinstance(P, (list, tuple)) else [P]
    kc_t, vc_t = synth.gen_kv_cache(m, max(pos), seed=1, device="cpu")
    kc_all, vc_all = synth.to_bits(kc_t), synth.to_bits(vc_t)
    caches = [(np.ascontiguousarray(kc_all[:, b]), np.ascontiguousarray(vc_all[:, b])) for b in range(len(pos))]
    log(f"[bench] oracle set-up {time.time() - t0:.1f}s ({oracle.num_threads()} threads)")
    toks, steps, t_start = [1] * len(pos), 0, time.time()
    while steps < max_steps:
        for b, (kc, vc) in enumerate(caches):
            toks[b], _, _ = om.decode_step(kc, vc, int(toks[b]), pos[b] + steps, want_logits=False,
                                           want_hidden=False)
        steps += 1
        if time.time() - t_start >= budget_s:
            break
    el = time.time() - t_start
    what = (f"context {pos[0]}, batch 1" if len(pos) == 1 else
            f"contexts {pos}, one step = every sequence")
    return {"value": round(el / steps * 1e6, 1), "unit": "us/step" if len(pos) > 1 else "us/token",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{steps} decode step(s) of the same {m.name} decoder at {what}, "
                      f"fp64 C oracle, {el:.1f}s wall"}


def tiny_comparison(repeats=5):
    """Persistent vs one-kernel-per-op on the tiny decoder (latency bound)."""
    import torch
    _, m, _, _, _, eng, g0 = setup("tiny")
    P, n = 128, 64
    tp, _ = time_calls(eng, eng.decode, n, g0, P, repeats, 8)
    tb, _ = time_calls(eng, eng.baseline_decode, n, g0, P, repeats, 8)
    res = {}
    for grid in (8, 16, 32, 64):
        e2 = __import__("persistent_resident_execution_amd.engine", fromlist=["Engine"]).Engine(
            m, eng._keep[0], eng._keep[1], eng._keep[2], grid_wgs=grid)
        t, _ = time_calls(e2, e2.decode, n, g0, P, repeats, 8)
        res[grid] = statistics.median(t) / n * 1e6
        e2.close()
    up = statistics.median(tp) / n * 1e6
    ub = statistics.median(tb) / n * 1e6
    best_grid = min(res, key=res.get)
    eng.close()
    torch.cuda.synchronize()
    return {"persistent_us_per_token": round(up, 2), "per_op_us_per_token": round(ub, 2),
            "speedup": round(ub / up, 2),
            "persistent_us_per_token_by_grid": {str(k): round(v, 2) for k, v in res.items()},
            "best_grid": best_grid, "best_speedup": round(ub / min(up, res[best_grid]), 2),
            "launches_per_token_per_op": launches_per_token_per_op(m), "launches_per_token_persistent": 1 / n}


def phases(args, w, m, eng, g0, P, K):
    """Busy and idle time per stage from the kernel's timestamp ring (one
    traced launch of K steps after a warm-up; the first traced step is
    skipped), written as a text summary."""
    import torch
    from persistent_resident_execution_amd import engine as E
    from persistent_resident_execution_amd import profiling
    info, _ = E.plan_describe(m, grid_wgs=args.grid)
    nsi, W = info.n_stage_inst, info.n_wgs
    tr = torch.zeros(K * nsi * W * 8, dtype=torch.int32, device="cuda")
    eng.set_trace(tr)
    t, _ = time_calls(eng, eng.decode, K, g0, P, 1, args.warmup)
    eng.set_trace(None)
    rec = tr.view(K, nsi, W, 8).cpu().numpy()
    if m.batch > 1:
        names, spl, first = ["embed", "qkv", "attn", "comb", "oproj", "gu", "down", "lm"], 6, 1
    elif m.is_moe:
        names, spl, first = ["qkv", "attn", "oproj", "router", "egu", "edown", "lm"], 6, 0
    else:
        names, spl, first = ["qkv", "attn", "oproj", "gu", "down", "lm"], 5, 0
    lines = [f"# per-stage wait / busy / phases (us) from the in-kernel timestamp ring, {w.note}",
             "command: python3 bench.py " + " ".join(sys.argv[1:]),
             f"traced: {K} steps in one launch ({t[0] / K * 1e6:.1f} us/step with the ring on), "
             f"{W} workgroups; means over steps 2..{K} and layers",
             "wait = task begin -> producers ready; busy = the rest of the task; span = first begin -> "
             "last end over the workgroups"]
    lines += profiling.phase_table(rec, names, m.n_layers, spl, first,
                                   profiling.PHASES_MB if m.batch > 1 else profiling.PHASES)
    with open(args.phases, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    eng.close()


def stream_reference(gbps, mib=2048, repeats=5):
    """The library's streamed GEMV alone (y = W x over a 2 GiB bf16 matrix,
    4096 columns, one workgroup per CU, streaming loads), best ring depth:
    a read-only streaming rate measured on this machine, reported beside the
    decode rate (not instead of the 8 TB/s peak)."""
    import torch
    from persistent_resident_execution_amd import engine as E
    K = 4096
    rows = (mib << 20) // (K * 2)
    W = torch.zeros((rows, K), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(K, dtype=torch.float32, device="cuda")
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    best = {}
    for variant, ring in ((3, 4), (5, 8), (7, 12)):
        E.debug_gemv(variant, W, x, y)
        torch.cuda.synchronize()
        ts = []
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            E.debug_gemv(variant, W, x, y)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        best[ring] = W.numel() * 2 / statistics.median(ts) / 1e9
    del W, x, y
    torch.cuda.empty_cache()
    ring, ref = max(best.items(), key=lambda kv: kv[1])
    return {"kernel": "pre_k_gemv_bench", "bytes": rows * K * 2, "gbps": round(ref, 1),
            "ring_units": ring, "gbps_by_ring": {str(k): round(v, 1) for k, v in best.items()},
            "decode_frac_of_stream": round(gbps / ref, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--workload", default="dense8b_ctx1024")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle sample")
    ap.add_argument("--no-baseline", action="store_true", help="skip the per-op baseline timing")
    ap.add_argument("--no-tiny", action="store_true", help="skip the tiny-decoder comparison")
    ap.add_argument("--no-stream", action="store_true", help="skip the read-only stream reference")
    ap.add_argument("--phases", default="",
                    help="instead of timing: trace --steps steps with the in-kernel timestamp ring and "
                         "write the per-stage wait/busy/phase summary to this file")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--prefill", choices=("engine", "synthetic"), default="engine")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first copy this many MiB with the library's copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from persistent_resident_execution_amd import engine as E
    from persistent_resident_execution_amd import profiling
    torch.cuda.set_device(0)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        E.debug_copy(a, b)
        torch.cuda.synchronize()
        del a, b
    w, m, W, kc, vc, eng, g0 = setup(args.workload, grid_wgs=args.grid, prefill=args.prefill)
    mb = m.batch > 1
    P, K = (list(w.contexts) if mb else w.contexts[0]), args.steps
    pos = P if mb else [P]
    if args.phases:
        phases(args, w, m, eng, g0, P, K)
        return
    log(f"[bench] timing {args.repeats} x {K} persistent steps from position(s) {P}")
    tp, toks = time_calls(eng, eng.decode, K, g0, P, args.repeats, args.warmup)
    kern = "pre_persistent_mb" if mb else "pre_persistent"
    t_med = statistics.median(tp)
    bytes_call = sum(E.step_bytes(m, [p + s for p in pos]) for s in range(K))
    us_tok = t_med / K * 1e6
    gbps = bytes_call / t_med / 1e9
    result = {
        "metric": ("decode us/step (micro-batch " + str(m.batch) + ") + achieved HBM GB/s as % of MI355X peak"
                   if mb else "decode us/token (batch 1) + achieved HBM GB/s as % of MI355X peak"),
        "value": round(us_tok, 2), "unit": "us/step" if mb else "us/token", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(us_tok / 1e3, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16 weights/KV, bf16 hi+lo activations on the matrix cores, fp32 accumulate" if mb
                  else "bf16 weights/KV, fp32 compute"),
        "data": ("synthetic (seeded N(0,0.02) bf16 weights, seeded N(0,1) K/V cache, seeded first tokens)"
                 if mb else "synthetic (seeded N(0,0.02) bf16 weights, random prompt tokens)"),
        "config": {"workload": w.note, "layers": m.n_layers, "hidden": m.hidden,
                   "heads": f"{m.n_q_heads}q/{m.n_kv_heads}kv x {m.head_dim}",
                   "ffn": m.ffn_dim, "vocab": m.vocab, "context": P, "batch": m.batch,
                   "parallelism": "single GPU, one workgroup per CU"},
        "tokens_per_s": round(K * m.batch / t_med, 1),
        "hbm_gbps_algorithmic": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "repeats_us_per_token": [round(t / K * 1e6, 2) for t in tp],
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": profiling.traffic_for(args.workload, K, kern),
                     "kernel": kern, "bytes_per_launch": bytes_call,
                     "launch_ms": round(t_med * 1e3, 3)},
    }
    if not args.no_baseline:
        log("[bench] timing the one-kernel-per-op baseline")
        tb, btoks = time_calls(eng, eng.baseline_decode, K, g0, P, max(1, args.repeats // 2), 0)
        ub = statistics.median(tb) / K * 1e6
        result["per_op_baseline"] = {("us_per_step" if mb else "us_per_token"): round(ub, 2),
                                     "launches_per_token": launches_per_token_per_op(m),
                                     "persistent_speedup": round(ub / us_tok, 3),
                                     "same_tokens": bool((btoks == toks).all())}
    eng.close()
    if not args.no_stream:
        log("[bench] read-only stream reference")
        result["stream_reference"] = stream_reference(gbps)
    if not args.no_tiny and not mb:
        log("[bench] tiny decoder persistent vs per-op")
        result["tiny"] = tiny_comparison()
    if not args.no_cpu:
        log("[bench] CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(m, W, P)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
