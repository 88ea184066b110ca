"""Decode benchmark: µs/token and achieved HBM bandwidth of the persistent
decode kernel on one MI355X, for every workload configuration.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense8b_ctx1024]
                    [--configs all|none|name,name,...]

One "step" is one decode step (one token per sequence) through the whole hot
path.  The headline workload is the 8B-shape dense decoder at batch 1: 32
layers, hidden 4096, 32 query / 8 KV heads of 128, SwiGLU 14336, vocabulary
128256, bf16 weights ~N(0, 0.02) from seed 0, the KV cache filled on the GPU
by the engine itself from 1024 random tokens, then greedy decode.  The timed
region is ONE engine call of K steps (one persistent kernel launch) starting
at the prefilled position, bracketed by device synchronisation and timed
with HIP events on the launch stream; it is repeated --repeats times from the
same position and the median is reported.  Inputs are resident in HBM.

The same run measures the other workloads the same way under "configs":
context 8192 (engine prefill of 8192 tokens), the MoE decoder (engine prefill
of 4096 tokens), the micro-batch of 8 (seeded synthetic caches at contexts
512..8192) and the tiny decoder (engine prefill of 128 tokens).  Each entry
carries its µs per step, its roofline (algorithmic bytes of the timed launch
over its HIP-event time, against 8 TB/s; HBM traffic from the committed
rocprofv3 counter summary when one matches the current kernel sources), the
one-kernel-per-operator path on the same call, and the CPU oracle timed on a
bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
CONFIG_ORDER = ["dense8b_ctx8192", "dense8b_ctx8192_kv8", "moe", "dense8b_mb8", "tiny"]
# what each path computes in (the "dtype" of its line)
DTYPE_B1 = ("bf16 weights and K/V cache; GEMV products and sums in fp32; attention scores and P.V on the "
            "matrix cores with q and p split into bf16 hi+lo parts (about 16 significant bits), fp32 accumulate")
DTYPE_MOE = DTYPE_B1.replace("bf16 weights", "bf16 attention/router weights, fp8 e4m3 experts with bf16 "
                             "128x128 block scales (decoded exactly to fp32)")
DTYPE_KV8 = DTYPE_B1.replace("bf16 weights and K/V cache", "bf16 weights, fp8 e4m3 K/V cache with an fp32 scale "
                             "per row (codes decoded exactly to bf16 for the matrix cores, scales applied to the "
                             "scores and to p)")
DTYPE_MB = ("bf16 weights and K/V cache; every GEMM and attention product on the matrix cores with the "
            "activations split into bf16 hi+lo parts (about 16 significant bits), fp32 accumulate")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(workload, W=None, device="cuda", seed=0, prefill="engine", **eng_kw):
    """Weights (reused if given: same shapes), cache, position array and engine
    of a workload.  prefill="engine" fills the cache by teacher-forced decode
    of the workload's random prompt (the workload as specified); "synthetic"
    writes seeded N(0,1) K/V rows instead and decodes from token 1 -- the same
    bytes and flops per step, without a prefill launch (used for profiler runs
    that must see only timed launches).  A micro-batch always uses the
    synthetic cache: a lockstep prefill cannot give eight different lengths."""
    import torch
    from persistent_resident_execution_amd import engine as E
    from persistent_resident_execution_amd import synth
    w = synth.WORKLOADS[workload]
    m = w.model
    t0 = time.time()
    if W is None:
        W = synth.gen_weights(m, seed=seed, device=device)
    pos = list(w.contexts)
    ctx = torch.zeros(m.batch, dtype=torch.int32, device=device)
    ks = vs = None
    if m.kv_fp8:  # the engine fills its own fp8 cache
        prefill = "engine"
        kc, vc, ks, vs = synth.empty_kv_cache(m, device=device)
    elif m.batch > 1 or prefill == "synthetic":
        kc, vc = synth.gen_kv_cache(m, max(pos), seed=seed + 1, device=device)
    else:
        kc, vc, _, _ = synth.empty_kv_cache(m, device=device)
    eng = E.Engine(m, W, kc, vc, ctx_len=ctx, k_scale=ks, v_scale=vs, **eng_kw)
    if m.batch > 1:
        g0 = synth.gen_tokens(m.vocab, m.batch, seed=seed + 2, device=device)
        how = f"synthetic caches of contexts {pos}"
    elif prefill == "synthetic":
        g0 = torch.ones(1, dtype=torch.int32, device=device)
        how = f"synthetic cache of {pos[0]} positions"
    else:
        prompt = synth.gen_tokens(m.vocab, pos[0], seed=seed, device=device)
        out = eng.decode(pos[0], forced=prompt.view(-1, 1))  # cache filled by the engine itself
        torch.cuda.synchronize()
        eng.status()
        g0 = out[-1].contiguous()
        how = f"engine prefill of {pos[0]} tokens"
    log(f"[bench] {workload}: weights + {how} in {time.time() - t0:.1f}s")
    return w, m, W, (kc, vc, ctx, ks, vs), eng, g0


def launches_per_step_per_op(m):
    """Kernels the one-kernel-per-operator path launches per step.  Batch 1:
    embedding; per layer two norms and one launch per task stage (5 dense, 6
    MoE); final norm, LM head, argmax.  Micro-batch: the embedding stage, six
    stages per layer, the LM head and the argmax.  (Plus one position-advance
    launch per call.)"""
    if m.batch > 1:
        return 6 * m.n_layers + 3
    return (8 if m.is_moe else 7) * m.n_layers + 4


def time_calls(eng, fn, n_steps, g0, pos, repeats, warmup_steps):
    """Seconds of each of `repeats` calls of n_steps from positions `pos`
    (HIP events on the launch stream); also the tokens of the last call."""
    import torch
    stream = torch.cuda.current_stream()
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
        del e0, e1
    eng.status()
    return times, out[:n_steps].cpu()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(m, W, pos, budget_s=12.0, single_thread_steps=0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    decode steps of the same model (weights copied to the host; the cache is a
    seeded synthetic one -- its values do not change the work) at the
    workload's context(s); for a micro-batch one step = one decode of every
    sequence at its own context (the oracle decodes sequences one at a time).
    With single_thread_steps > 0, that many steps are also timed on one
    thread."""
    import numpy as np
    import oracle
    from persistent_resident_execution_amd import synth
    t0 = time.time()
    om = oracle.OracleModel(m, synth.weights_to_numpy(W))
    if m.kv_fp8:  # (zero codes and scales: the work does not depend on the values)
        caches = [om.new_cache_fp8() for _ in pos]
    else:
        kc_t, vc_t = synth.gen_kv_cache(m, max(pos), seed=1, device="cpu")
        kc_all, vc_all = synth.to_bits(kc_t), synth.to_bits(vc_t)
        del kc_t, vc_t
        caches = [(np.ascontiguousarray(kc_all[:, b]), np.ascontiguousarray(vc_all[:, b])) for b in range(len(pos))]
        del kc_all, vc_all
    threads = oracle.num_threads()
    log(f"[bench] oracle set-up {time.time() - t0:.1f}s ({threads} threads)")

    def run(max_steps, budget):
        toks, steps, ts = [1] * len(pos), 0, time.time()
        while steps < max_steps:
            for b, c in enumerate(caches):
                step = om.decode_step_fp8 if m.kv_fp8 else om.decode_step
                toks[b], _, _ = step(*c, int(toks[b]), pos[b] + steps, want_logits=False, want_hidden=False)
            steps += 1
            if time.time() - ts >= budget:
                break
        return steps, time.time() - ts

    steps, el = run(64, budget_s)
    unit = "us/step" if len(pos) > 1 else "us/token"
    what = f"context {pos[0]}, batch 1" if len(pos) == 1 else f"contexts {pos}, one step = every sequence"
    res = {"value": round(el / steps * 1e6, 1), "unit": unit, "cores": threads, "kind": "oracle",
           "sample": f"{steps} decode step(s) of the same {m.name} decoder at {what}, fp64 C oracle, "
                     f"{el:.1f}s wall on {threads} threads", "cpu_model": cpu_model(),
           "host_cpus": len(os.sched_getaffinity(0))}
    if single_thread_steps:
        oracle.set_num_threads(1)
        try:
            s1, e1 = run(single_thread_steps, 0.0)
        finally:
            oracle.set_num_threads(threads)
        res["single_thread"] = {"value": round(e1 / s1 * 1e6, 1), "unit": unit, "steps": s1}
    del om, caches
    gc.collect()
    return res


def kernel_of(m, **kw):
    """The resident kernel the library launches for this model and options."""
    from persistent_resident_execution_amd import engine as E
    if m.batch > 1:
        return "pre_persistent_mb"
    if m.kv_fp8:
        return "pre_persistent_kv8"
    info, _ = E.plan_describe(m, **kw)
    return "pre_persistent_small" if (info.fold_ffn or info.fold_attn) else "pre_persistent"


def roofline(m, pos, K, t_med, kernel, workload):
    """Algorithmic bytes of one launch of K steps from positions pos over its
    HIP-event time, against the 8 TB/s peak; HBM traffic from the committed
    counter summary (per step, times K) while it matches the kernel sources."""
    from persistent_resident_execution_amd import engine as E
    from persistent_resident_execution_amd import profiling
    bytes_call = sum(E.step_bytes(m, [p + s for p in pos]) for s in range(K))
    gbps = bytes_call / t_med / 1e9
    tr = profiling.traffic_for(workload, K, kernel)
    return {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": tr["bytes_per_launch"] if tr else None,
            "traffic_basis": tr["basis"] if tr else "no counter summary for the current kernel sources",
            "kernel": kernel, "bytes_per_launch": bytes_call,
            "bytes_per_step_mean": round(bytes_call / K), "launch_ms": round(t_med * 1e3, 3)}


def measure(workload, args, W=None, baseline=True, cpu=True, single_thread_steps=0):
    """Everything reported for one workload; returns (entry, weights)."""
    import torch
    kw = dict(grid_wgs=args.grid, attn_splits=args.attn_splits, fold_ffn=args.fold_ffn, fold_attn=args.fold_attn)
    w, m, W, bufs, eng, g0 = setup(workload, W, prefill=args.prefill, **kw)
    mb = m.batch > 1
    pos = list(w.contexts)
    K = args.steps if args.steps > 0 else w.steps
    log(f"[bench] {workload}: timing {args.repeats} x {K} persistent steps from position(s) {pos}")
    tp, toks = time_calls(eng, eng.decode, K, g0, pos, args.repeats, args.warmup)
    kern = kernel_of(m, **kw)
    t_med = statistics.median(tp)
    us = t_med / K * 1e6
    unit = "us/step" if mb else "us/token"
    e = {"workload": w.note, "value": round(us, 2), "unit": unit,
         "window": {"steps": K, "start_positions": pos,
                    "note": f"one launch of {K} greedy steps from the prefilled position(s)"},
         "tokens_per_s": round(K * m.batch / t_med, 1),
         "repeats_us_per_step": [round(t / K * 1e6, 2) for t in tp],
         "dtype": DTYPE_MB if mb else (DTYPE_MOE if m.is_moe else (DTYPE_KV8 if m.kv_fp8 else DTYPE_B1)),
         "roofline": roofline(m, pos, K, t_med, kern, workload)}
    if baseline:
        log(f"[bench] {workload}: the one-kernel-per-operator path")
        tb, btoks = time_calls(eng, eng.baseline_decode, K, g0, pos, max(1, args.repeats // 2), 0)
        ub = statistics.median(tb) / K * 1e6
        e["per_op_baseline"] = {unit.replace("/", "_per_"): round(ub, 2),
                                "launches_per_step": launches_per_step_per_op(m),
                                "persistent_speedup": round(ub / us, 3),
                                "same_tokens": bool((btoks == toks).all())}
    eng.close()
    del eng, bufs, g0, toks
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu:
        log(f"[bench] {workload}: CPU oracle sample")
        e["cpu_baseline"] = cpu_baseline(m, W, pos, single_thread_steps=single_thread_steps)
    return e, W


def measure_chunk(args, W):
    """The chunk task set on the 8B shape: (1) prefill of the workload's 1024
    prompt tokens, 8 per step, one launch, against the same prompt fed
    through the decode path one token per step (teacher-forced, one launch);
    (2) speculative verify rounds of the current token plus 7 drafts that
    are the model's own greedy continuation (all accepted: 8 tokens
    committed per round), against greedy decode of the same tokens.  Each
    timed with HIP events on the launch stream, median of repeats."""
    import torch
    from persistent_resident_execution_amd import engine as E
    from persistent_resident_execution_amd import synth
    w = synth.WORKLOADS["dense8b_ctx1024"]
    m, P = w.model, w.contexts[0]
    shape = (m.n_layers, 1, m.n_kv_heads, m.max_ctx, m.head_dim)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng = E.Engine(m, W, kc, vc, ctx_len=ctx, chunk=8)
    prompt = synth.gen_tokens(m.vocab, P, seed=0, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            eng.set_positions([0])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            r = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        eng.status()
        return statistics.median(ts), r

    reps = max(3, args.repeats // 2)
    timed(lambda: eng.prefill(prompt), 1)  # warm-up
    t_chunk, out = timed(lambda: eng.prefill(prompt), reps)
    t_tok, out_tok = timed(lambda: eng.decode(P, forced=prompt.view(P, 1)), reps)
    import dataclasses
    m8 = dataclasses.replace(m, batch=8)
    nst = (P + 7) // 8
    bytes_pf = sum(E.step_bytes(m8, [min(s * 8 + j, P - 1) for j in range(8)]) for s in range(nst))
    g0 = int(out[-1].item())
    res = {"prefill": {
        "workload": f"{w.note.split(',')[0]}: prefill of the {P}-token prompt into an empty cache",
        "tokens": P, "chunk": 8, "us_per_token": round(t_chunk / P * 1e6, 2),
        "tokens_per_s": round(P / t_chunk, 1),
        "decode_path_us_per_token": round(t_tok / P * 1e6, 2),
        "speedup_vs_decode_path": round(t_tok / t_chunk, 2),
        "same_first_token": g0 == int(out_tok[-1, 0].item()),
        "roofline": {"bound": "hbm", "achieved": round(bytes_pf / t_chunk / 1e9, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(bytes_pf / t_chunk / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": None, "kernel": "pre_persistent_mb", "bytes_per_launch": bytes_pf,
                     "launch_ms": round(t_chunk * 1e3, 3)}}}
    # verify: the model's own greedy continuation as drafts (all accepted)
    rounds = 8
    eng.set_positions([P])
    g = eng.decode(rounds * 8, in_tokens=out[-1:].contiguous())
    torch.cuda.synchronize()
    seq = [g0] + g[:, 0].tolist()
    chunks = [torch.tensor(seq[8 * r:8 * r + 8], dtype=torch.int32, device="cuda") for r in range(rounds)]
    acc_all = []

    def verify_rounds():
        accs = []
        for c in chunks:
            _, a = eng.verify(c)
            accs.append(a)
        return accs

    def reset_to(p):
        eng.set_positions([p])

    ts = []
    for _ in range(reps + 1):
        reset_to(P)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        accs = verify_rounds()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
        acc_all = [int(a.item()) for a in accs]
    t_v = statistics.median(ts[1:])
    reset_to(P)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    eng.decode(rounds * 8, in_tokens=out[-1:].contiguous())
    e1.record(stream)
    torch.cuda.synchronize()
    t_d = e0.elapsed_time(e1) / 1e3
    committed = sum(a + 1 for a in acc_all)
    bytes_v = sum(E.step_bytes(m8, [P + 8 * r + j for j in range(8)]) for r in range(rounds))
    res["verify"] = {
        "workload": f"8B-shape dense decoder, context {P}: {rounds} verify rounds of the current token plus 7 "
                    "drafts (the model's own greedy continuation, so all are accepted), one launch per round",
        "accepted_per_round": acc_all, "tokens_committed": committed,
        "us_per_round": round(t_v / rounds * 1e6, 2), "us_per_committed_token": round(t_v / committed * 1e6, 2),
        "greedy_decode_us_per_token": round(t_d / (rounds * 8) * 1e6, 2),
        "speedup_vs_greedy_decode": round(t_d / t_v * committed / (rounds * 8), 2),
        "roofline": {"bound": "hbm", "achieved": round(bytes_v / t_v / 1e9, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(bytes_v / t_v / 1e9 / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "pre_persistent_mb", "bytes_per_launch": bytes_v // rounds,
                     "launch_ms": round(t_v / rounds * 1e3, 3)}}
    eng.close()
    del eng, kc, vc, ctx
    gc.collect()
    torch.cuda.empty_cache()
    return res


def tiny_grids(args, entry):
    """The tiny decoder's persistent µs/token at a few grid sizes (its
    default grid is one XCD's 32 CUs), and at the default grid with every
    stage run as a stage of its own (the default folds the down projection
    into the gate/up stage and the attention into the output projection)."""
    import torch
    from persistent_resident_execution_amd import engine as E
    w, m, W, bufs, eng, g0 = setup("tiny")
    eng.close()
    pos, K = list(w.contexts), (args.steps if args.steps > 0 else w.steps)
    res = {}
    for grid, fold in ((8, 0), (16, 0), (64, 0), (0, -1)):
        e2 = E.Engine(m, W, bufs[0], bufs[1], grid_wgs=grid, ctx_len=bufs[2], fold_ffn=fold, fold_attn=fold)
        t, _ = time_calls(e2, e2.decode, K, g0, pos, args.repeats, 8)
        res[str(grid) if grid else "32, no folded stages"] = round(statistics.median(t) / K * 1e6, 2)
        e2.close()
    res["32 (default)"] = entry["value"]
    del eng, bufs, W
    torch.cuda.empty_cache()
    return res


def phases(args):
    """Busy and idle time per stage from the kernel's timestamp ring (one
    traced launch of K steps after a warm-up; the first traced step is
    skipped), written as a text summary."""
    import torch
    from persistent_resident_execution_amd import engine as E
    from persistent_resident_execution_amd import profiling
    kw = dict(grid_wgs=args.grid, attn_splits=args.attn_splits, fold_ffn=args.fold_ffn, fold_attn=args.fold_attn)
    w, m, W, bufs, eng, g0 = setup(args.workload, prefill=args.prefill, **kw)
    pos, K = list(w.contexts), (args.steps if args.steps > 0 else w.steps)
    info, _ = E.plan_describe(m, **kw)
    nsi, nW = info.n_stage_inst, info.n_wgs
    tr = torch.zeros(K * nsi * nW * 8, dtype=torch.int32, device="cuda")
    eng.set_trace(tr)
    t, _ = time_calls(eng, eng.decode, K, g0, pos, 1, args.warmup)
    eng.set_trace(None)
    rec = tr.view(K, nsi, nW, 8).cpu().numpy()
    if m.batch > 1:
        names, spl, first = ["embed", "qkv", "attn", "comb", "oproj", "gu", "down", "lm"], 6, 1
    elif m.is_moe:
        names, spl, first = ["qkv", "attn", "oproj", "router", "egu", "edown", "lm"], 6, 0
    else:
        names, spl, first = ["qkv", "attn", "oproj", "gu", "down", "lm"], 5, 0
    lines = [f"# per-stage wait / busy / phases (us) from the in-kernel timestamp ring, {w.note}",
             "command: python3 bench.py " + " ".join(sys.argv[1:]),
             f"traced: {K} steps in one launch ({t[0] / K * 1e6:.1f} us/step with the ring on), "
             f"{nW} workgroups; means over steps 2..{K} and layers",
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
    ap.add_argument("--steps", type=int, default=0,
                    help="steps per timed launch (0: each workload's own step count)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--workload", default="dense8b_ctx1024", help="the headline workload")
    ap.add_argument("--configs", default="all",
                    help="other workloads measured in the same run: all, none, or a comma list")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle samples")
    ap.add_argument("--no-baseline", action="store_true", help="skip the per-op baseline timings")
    ap.add_argument("--no-stream", action="store_true", help="skip the read-only stream reference")
    ap.add_argument("--phases", default="",
                    help="instead of timing: trace --steps steps of --workload with the in-kernel timestamp "
                         "ring and write the per-stage wait/busy/phase summary to this file")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--attn-splits", type=int, default=0, help="attention chunks per KV head (0: default)")
    ap.add_argument("--fold-ffn", type=int, default=0,
                    help="0: fold the down projection into the gate/up stage where supported; -1: never")
    ap.add_argument("--fold-attn", type=int, default=0,
                    help="0: fold the attention into the output projection where supported; -1: never")
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
    torch.cuda.set_device(0)
    try:
        if args.calibrate_copy_mib:
            n = args.calibrate_copy_mib << 20
            a = torch.ones(n, dtype=torch.uint8, device="cuda")
            b = torch.empty_like(a)
            E.debug_copy(a, b)
            torch.cuda.synchronize()
            del a, b
        if args.phases:
            phases(args)
            return
        run_main(args)
    finally:
        # release every device allocation while the runtime (and a profiler
        # wrapped around this process) is still fully up
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        sys.stdout.flush()


def run_main(args):
    import torch
    from persistent_resident_execution_amd import synth
    head = args.workload
    cpu = not args.no_cpu
    e, W = measure(head, args, baseline=not args.no_baseline, cpu=cpu,
                   single_thread_steps=1 if head.startswith("dense8b") or head == "tiny" else 0)
    m = synth.WORKLOADS[head].model
    mb = m.batch > 1
    result = {
        "metric": ("decode us/step (micro-batch " + str(m.batch) + ") + achieved HBM GB/s as % of MI355X peak"
                   if mb else "decode us/token (batch 1) + achieved HBM GB/s as % of MI355X peak"),
        "value": e["value"], "unit": e["unit"], "n_gpus": 1, "steps": e["window"]["steps"],
        "warmup": args.warmup, "ms_per_step": round(e["value"] / 1e3, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": e["dtype"],
        "data": ("synthetic (seeded N(0,0.02) bf16 weights, seeded N(0,1) K/V cache, seeded first tokens)"
                 if mb else "synthetic (seeded N(0,0.02) bf16 weights, random prompt tokens prefilled by the "
                            "engine)"),
        "config": {"workload": e["workload"], "timed": e["window"]["note"],
                   "start_positions": e["window"]["start_positions"], "layers": m.n_layers,
                   "hidden": m.hidden, "heads": f"{m.n_q_heads}q/{m.n_kv_heads}kv x {m.head_dim}",
                   "ffn": m.ffn_dim, "vocab": m.vocab, "batch": m.batch,
                   "parallelism": "single GPU, one workgroup per CU"},
        "tokens_per_s": e["tokens_per_s"],
        "hbm_gbps_algorithmic": e["roofline"]["achieved"],
        "hbm_frac_of_peak": e["roofline"]["frac"],
        "repeats_us_per_step": e["repeats_us_per_step"],
        "roofline": e["roofline"],
    }
    for k in ("per_op_baseline", "cpu_baseline"):
        if k in e:
            result[k] = e[k]
    if not args.no_stream:
        log("[bench] read-only stream reference")
        result["stream_reference"] = stream_reference(e["roofline"]["achieved"])
    names = CONFIG_ORDER if args.configs == "all" else ([] if args.configs == "none" else args.configs.split(","))
    configs = {}
    if "chunk" in names or (args.configs == "all" and head == "dense8b_ctx1024"):
        log("[bench] chunk task set: prefill and speculative verify on the 8B shape")
        ch = measure_chunk(args, W)
        configs["dense8b_prefill"] = ch["prefill"]
        configs["dense8b_verify"] = ch["verify"]
    for name in names:
        if name == head or name == "chunk":
            continue
        mm = synth.WORKLOADS[name].model
        same = (mm.n_layers, mm.hidden, mm.vocab, mm.ffn_dim, mm.n_experts) == (
            m.n_layers, m.hidden, m.vocab, m.ffn_dim, m.n_experts)
        ce, W2 = measure(name, args, W=W if same else None, baseline=not args.no_baseline, cpu=cpu,
                         single_thread_steps=4 if name == "tiny" else 0)
        if name == "tiny":
            ce["by_grid_us_per_token"] = tiny_grids(args, ce)
        configs[name] = ce
        del W2
        gc.collect()
        torch.cuda.empty_cache()
    if configs:
        result["configs"] = configs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
