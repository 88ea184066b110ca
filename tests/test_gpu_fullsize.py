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
