"""Full-size parity: the 8B shape at contexts 1024 and 8192, the MoE shape at
context 4096 and the micro-batch of 8, in the launch configuration the
benchmark times (default grid, split and threads), against the CPU oracle.

Batch 1 follows the benchmark's workload exactly: the engine fills the cache
itself by teacher-forced decode of the seeded random prompt, then decodes
greedily.  The oracle cannot prefill thousands of positions of these models
in a test's time, so it receives the engine's bf16 cache bytes for the
prompt's positions below the last one (the cache handover of the prefill /
decode split), recomputes the prompt's last position itself -- its greedy
token against the GPU's first token -- and then runs every decode step
teacher-forced on the GPU's tokens, comparing all logits and the hidden
state at every step (tests/parity.py).  The 8B shape at context 1024 runs the
64 steps the greedy rule names; context 8192 and MoE run 16.

The micro-batch starts from a seeded synthetic cache at the workload's eight
contexts (a lockstep prefill cannot give eight different lengths) and runs 8
steps; each sequence is checked against the oracle decoding it alone.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import parity  # noqa: E402

from persistent_resident_execution_amd import engine as E  # noqa: E402
from persistent_resident_execution_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dense8b(oracle_lib):
    """8B-shape weights on the GPU and their host bytes (shared by the
    context-1024, context-8192 and micro-batch workloads: same shapes)."""
    _say("[setup] 8B-shape weights on the GPU and host copies")
    t0 = time.time()
    W = synth.gen_weights(synth.DENSE8B, seed=0, device="cuda")
    Wnp = synth.weights_to_numpy(W)
    _say(f"  {time.time() - t0:.1f}s, oracle threads {oracle_lib.num_threads()}")
    yield W, Wnp
    del W
    torch.cuda.empty_cache()


def _batch1(oracle_lib, m, W, Wnp, P, steps):
    """Engine prefill of P seeded prompt tokens, `steps` greedy steps with
    check outputs, then the oracle from the engine's prompt cache."""
    shape = (m.n_layers, 1, m.n_kv_heads, m.max_ctx, m.head_dim)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng = E.Engine(m, W, kc, vc, ctx_len=ctx)
    prompt = synth.gen_tokens(m.vocab, P, seed=0, device="cuda")
    t0 = time.time()
    g0 = eng.decode(P, forced=prompt.view(P, 1))[-1].contiguous()
    lg = torch.zeros((steps, 1, m.vocab), dtype=torch.float32, device="cuda")
    hd = torch.zeros((steps, 1, m.hidden), dtype=torch.float32, device="cuda")
    out = eng.decode(steps, in_tokens=g0, logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    assert int(ctx.item()) == P + steps
    _say(f"  GPU prefill of {P} + {steps} steps in {time.time() - t0:.1f}s; tokens {out[:, 0].tolist()}")
    eng.close()
    toks, lgs, hds = out[:, 0].cpu().numpy(), lg[:, 0].cpu().numpy(), hd[:, 0].cpu().numpy()
    kc_h = np.ascontiguousarray(synth.to_bits(kc)[:, 0])
    vc_h = np.ascontiguousarray(synth.to_bits(vc)[:, 0])
    del kc, vc, lg, hd
    torch.cuda.empty_cache()
    om = oracle_lib.OracleModel(m, Wnp)
    t0 = time.time()
    g0_ref, lg0, _ = om.decode_step(kc_h, vc_h, int(prompt[-1]), P - 1)
    rec0 = {"step": "prompt end"}
    parity.check_token("prompt end", int(g0.item()), g0_ref, lg0, rec0)
    _say(f"  prompt end: GPU token {int(g0.item())}, oracle {g0_ref} {rec0}")
    recs = parity.check_forced(om, kc_h, vc_h, P, int(g0.item()), toks, lgs, hds, say=_say)
    _say(f"  oracle {steps + 1} steps in {time.time() - t0:.1f}s; max dlogit "
         f"{max(r['max_dlogit'] for r in recs):.2e}, max hidden rel {max(r['hidden_rel'] for r in recs):.2e}, "
         f"near-tie steps {[r['step'] for r in recs if r.get('near_tie')]}")
    assert len(recs) == steps


@pytest.mark.timeout(900)
def test_dense8b_ctx1024_64_steps_from_engine_prefill(oracle_lib, dense8b):
    w = synth.WORKLOADS["dense8b_ctx1024"]
    _say(f"[full-size] {w.note}: 64 steps")
    _batch1(oracle_lib, w.model, *dense8b, w.contexts[0], 64)


@pytest.mark.timeout(900)
def test_dense8b_ctx8192_16_steps_from_engine_prefill(oracle_lib, dense8b):
    w = synth.WORKLOADS["dense8b_ctx8192"]
    _say(f"[full-size] {w.note}: 16 steps")
    _batch1(oracle_lib, w.model, *dense8b, w.contexts[0], 16)


MB_STEPS = 8


@pytest.mark.timeout(900)
def test_full_size_microbatch_matches_oracle(oracle_lib, dense8b):
    """The micro-batch workload at full size (8B shape, 8 sequences at
    contexts 512..8192) in the benchmark's launch configuration: every
    sequence's logits and hidden state of 8 steps against the oracle decoding
    that sequence alone from the same cache bytes, teacher-forced on the
    GPU's tokens."""
    w = synth.WORKLOADS["dense8b_mb8"]
    m, ctx = w.model, list(w.contexts)
    W, Wnp = dense8b
    _say(f"[full-size] dense8b_mb8: caches of contexts {ctx}, {MB_STEPS} steps")
    kc, vc = synth.gen_kv_cache(m, max(ctx), seed=1, device="cuda")
    kc_h, vc_h = synth.to_bits(kc), synth.to_bits(vc)  # before the decode appends
    pos = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    eng = E.Engine(m, W, kc, vc, ctx_len=pos)
    tok0 = synth.gen_tokens(m.vocab, m.batch, seed=5, device="cuda")
    lg = torch.zeros((MB_STEPS, m.batch, m.vocab), dtype=torch.float32, device="cuda")
    hd = torch.zeros((MB_STEPS, m.batch, m.hidden), dtype=torch.float32, device="cuda")
    out = eng.decode(MB_STEPS, in_tokens=tok0, logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    assert pos.tolist() == [c + MB_STEPS for c in ctx]
    toks, lgs, hds = out.cpu().numpy(), lg.cpu().numpy(), hd.cpu().numpy()
    eng.close()
    del kc, vc, lg, hd
    torch.cuda.empty_cache()
    _say(f"  GPU tokens {toks.tolist()}; oracle per sequence follows")
    om = oracle_lib.OracleModel(m, Wnp)
    t0 = tok0.cpu().numpy()
    for b in range(m.batch):
        kb = np.ascontiguousarray(kc_h[:, b])
        vb = np.ascontiguousarray(vc_h[:, b])
        recs = parity.check_forced(om, kb, vb, ctx[b], int(t0[b]), toks[:, b], lgs[:, b], hds[:, b])
        _say(f"  sequence {b} (context {ctx[b]}): max dlogit {max(r['max_dlogit'] for r in recs):.2e}, "
             f"max hidden rel {max(r['hidden_rel'] for r in recs):.2e}, "
             f"near-tie steps {[r['step'] for r in recs if r.get('near_tie')]}")


@pytest.mark.timeout(900)
def test_moe_16_steps_from_engine_prefill(oracle_lib):
    w = synth.WORKLOADS["moe"]
    m = w.model
    _say(f"[full-size] {w.note}: weights on the GPU, host copies, 16 steps")
    t0 = time.time()
    W = synth.gen_weights(m, seed=0, device="cuda")
    Wnp = synth.weights_to_numpy(W)
    _say(f"  weights {time.time() - t0:.1f}s")
    _batch1(oracle_lib, m, W, Wnp, w.contexts[0], 16)
    del W
    torch.cuda.empty_cache()
