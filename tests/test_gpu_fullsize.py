"""Full-size parity: the 8B shape at contexts 1024 and 8192 and the MoE shape
at context 4096, in the launch configuration the benchmark times (default
grid, split and threads), against the CPU oracle on a few decode steps.

Both sides start from the same bytes: weights generated once on the GPU and
copied to the host, and a seeded synthetic K/V cache of the workload's
context (the oracle cannot prefill thousands of positions of these models in
a test's time).  The steps then run free on each side, greedy, under the
rules of tests/parity.py; the oracle computes every logit of every step.
"""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import parity  # noqa: E402

from persistent_resident_execution_amd import engine as E  # noqa: E402
from persistent_resident_execution_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu

STEPS = 3


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("workload", ["dense8b_ctx1024", "dense8b_ctx8192", "moe"])
def test_full_size_decode_matches_oracle(oracle_lib, workload):
    w = synth.WORKLOADS[workload]
    m, P = w.model, w.contexts[0]
    _say(f"[full-size] {workload}: weights on the GPU, host copies, cache of {P} positions")
    W = synth.gen_weights(m, seed=0, device="cuda")
    om = oracle_lib.OracleModel(m, synth.weights_to_numpy(W))
    kc, vc = synth.gen_kv_cache(m, P, seed=1, device="cuda")
    kc_h = np.ascontiguousarray(synth.to_bits(kc)[:, 0])
    vc_h = np.ascontiguousarray(synth.to_bits(vc)[:, 0])
    eng = E.Engine(m, W, kc, vc)
    eng.set_positions([P])
    tok0 = 7
    lg = torch.zeros((STEPS, 1, m.vocab), dtype=torch.float32, device="cuda")
    hd = torch.zeros((STEPS, 1, m.hidden), dtype=torch.float32, device="cuda")
    out = eng.decode(STEPS, in_tokens=torch.tensor([tok0], dtype=torch.int32, device="cuda"),
                     logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    toks, lgs, hds = out[:, 0].cpu().numpy(), lg[:, 0].cpu().numpy(), hd[:, 0].cpu().numpy()
    _say(f"  GPU tokens {toks.tolist()}; oracle steps follow")
    tok = tok0
    for s in range(STEPS):
        nxt, ref_lg, ref_hd = om.decode_step(kc_h, vc_h, tok, P + s)
        cont, rec = parity.compare_step(s, int(toks[s]), lgs[s], hds[s], nxt, ref_lg, ref_hd)
        _say(f"  step {s}: {rec}")
        if not cont:
            break
        tok = nxt
    eng.close()


MB_STEPS = 2


def test_full_size_microbatch_matches_oracle(oracle_lib):
    """The micro-batch workload at full size (8B shape, 8 sequences at
    contexts 512..8192) in the benchmark's launch configuration: every
    sequence's logits and hidden state of 2 free-running steps against the
    oracle decoding that sequence alone from the same cache bytes."""
    w = synth.WORKLOADS["dense8b_mb8"]
    m, ctx = w.model, list(w.contexts)
    _say(f"[full-size] dense8b_mb8: weights on the GPU, host copies, caches of contexts {ctx}")
    W = synth.gen_weights(m, seed=0, device="cuda")
    om = oracle_lib.OracleModel(m, synth.weights_to_numpy(W))
    kc, vc = synth.gen_kv_cache(m, max(ctx), seed=1, device="cuda")
    eng = E.Engine(m, W, kc, vc)
    eng.set_positions(ctx)
    tok0 = synth.gen_tokens(m.vocab, m.batch, seed=5, device="cuda")
    lg = torch.zeros((MB_STEPS, m.batch, m.vocab), dtype=torch.float32, device="cuda")
    hd = torch.zeros((MB_STEPS, m.batch, m.hidden), dtype=torch.float32, device="cuda")
    kc_h, vc_h = synth.to_bits(kc), synth.to_bits(vc)  # before the decode appends
    out = eng.decode(MB_STEPS, in_tokens=tok0, logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    toks, lgs, hds = out.cpu().numpy(), lg.cpu().numpy(), hd.cpu().numpy()
    eng.close()
    del W, kc, vc, lg, hd
    torch.cuda.empty_cache()
    _say(f"  GPU tokens {toks.tolist()}; oracle per sequence follows")
    t0 = tok0.cpu().numpy()
    for b in range(m.batch):
        kb = np.ascontiguousarray(kc_h[:, b])
        vb = np.ascontiguousarray(vc_h[:, b])
        tok = int(t0[b])
        for s in range(MB_STEPS):
            nxt, ref_lg, ref_hd = om.decode_step(kb, vb, tok, ctx[b] + s)
            cont, rec = parity.compare_step(s, int(toks[s, b]), lgs[s, b], hds[s, b], nxt, ref_lg, ref_hd)
            _say(f"  sequence {b} (context {ctx[b]}) step {s}: {rec}")
            if not cont:
                break
            tok = nxt
