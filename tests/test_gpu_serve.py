"""The serving loop (pre_serve_*): one resident launch taking requests from a
ring in host memory, through the C ABI.

Requests are submitted from the host while the kernel stays resident; every
request's token stream is checked against the oracle (prompt prefilled,
then greedy steps teacher-forced on the GPU's tokens under the greedy rule of
tests/parity.py), the stop rules (budget, EOS) are checked, a request the
device must reject (its steps would pass max_ctx) is finished with that error
while the loop goes on, and after the loop ends the engine's positions and
ready-flag epochs continue into an ordinary decode call.  A loop nobody
submits to ends by itself after its idle limit.
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


def _oracle_request(om, kc, vc, pos, prompt, gpu_out):
    """The oracle on one request: the prompt decoded from position pos (its
    greedy successor is the first output), then every output teacher-forced
    (the greedy rule at each step).  kc, vc hold the sequence's positions <
    pos and are advanced in place; returns the oracle's tokens."""
    for i, t in enumerate(prompt[:-1]):
        om.decode_step(kc, vc, int(t), pos + i, want_logits=False, want_hidden=False)
    ref = []
    inputs = [int(prompt[-1])] + [int(t) for t in gpu_out[:-1]]
    for k, tok_in in enumerate(inputs):
        rt, rl, _ = om.decode_step(kc, vc, tok_in, pos + len(prompt) - 1 + k, want_hidden=False)
        parity.check_token(k, int(gpu_out[k]), rt, rl, {})
        ref.append(rt)
    return ref


@pytest.fixture(scope="module")
def tiny(oracle_lib):
    return parity.DenseSetup(oracle_lib, synth.TINY, seed=4)


def test_serving_loop_matches_oracle(tiny):
    S = tiny
    m = S.m
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng = E.Engine(m, S.Wd, S.kc, S.vc, ctx_len=ctx)
    pa = synth.gen_tokens(m.vocab, 24, seed=41).tolist()
    pb = synth.gen_tokens(m.vocab, 16, seed=42).tolist()
    pd = synth.gen_tokens(m.vocab, 20, seed=43).tolist()
    # the EOS request: stop at the oracle's fourth greedy token of prompt pd
    okc, ovc = S.om.new_cache()
    S.om.prefill(okc, ovc, pd[:-1])
    t, free = int(pd[-1]), []
    for k in range(6):
        t, _, _ = S.om.decode_step(okc, ovc, t, len(pd) - 1 + k, want_logits=False, want_hidden=False)
        free.append(t)
    eos = free[3]
    _say(f"[test] serving loop, tiny decoder; EOS request stops at token {eos} (oracle stream {free})")
    t_in = torch.zeros(1, dtype=torch.int32, device="cuda")  # (no GPU work is queued while the loop runs)
    torch.cuda.synchronize()
    srv = E.Server(eng, n_slots=4, max_prompt=64, max_out=m.max_ctx, idle_ms=20000)
    try:
        t0 = time.time()
        sa = srv.submit(pa, pos=0, budget=10)
        sb = srv.submit(pb, pos=0, budget=8)  # a new sequence over the same cache, after A (FIFO)
        with pytest.raises(E.PreError) as ei:  # the engine is held by the loop
            eng.decode(1, in_tokens=t_in)
        assert ei.value.code == -10
        out_a, err_a = srv.wait(sa)
        out_b, err_b = srv.wait(sb)
        sc = srv.submit([out_b[-1]], pos=-1, budget=6)  # continues B where it stands
        out_c, err_c = srv.wait(sc)
        sd = srv.submit(pd, pos=0, budget=20, eos=eos)
        out_d, err_d = srv.wait(sd)
        se = srv.submit([out_d[-1]], pos=-1, budget=m.max_ctx - 10)  # passes max_ctx: rejected on the device
        out_e, err_e = srv.wait(se)
        _say(f"  five requests in {time.time() - t0:.3f}s: A {out_a}, B {out_b}, C {out_c}, D {out_d}, "
             f"E error {err_e}")
    finally:
        stats = srv.stop()
    _say(f"  loop stats {stats}")
    assert (err_a, err_b, err_c, err_d, err_e) == (0, 0, 0, 0, 5) and out_e == []
    assert len(out_a) == 10 and len(out_b) == 8 and len(out_c) == 6
    assert out_d[-1] == eos and eos not in out_d[:-1] and len(out_d) <= 20
    steps = (24 + 10 - 1) + (16 + 8 - 1) + (1 + 6 - 1) + (20 + len(out_d) - 1)
    assert stats == {"steps": steps, "served": 4, "error": 0}
    pos_d = 20 + len(out_d) - 1
    assert eng.positions() == [pos_d] and int(ctx.item()) == pos_d
    # the oracle, request by request (B's cache continues into C)
    kc, vc = S.om.new_cache()
    _oracle_request(S.om, kc, vc, 0, pa, out_a)
    kc, vc = S.om.new_cache()
    _oracle_request(S.om, kc, vc, 0, pb, out_b)
    _oracle_request(S.om, kc, vc, 16 + 8 - 1, [out_b[-1]], out_c)
    kc, vc = S.om.new_cache()
    ref_d = _oracle_request(S.om, kc, vc, 0, pd, out_d)
    # after the loop: an ordinary decode call continues D (epochs and position carried over)
    lg = torch.zeros((5, 1, m.vocab), device="cuda")
    out = eng.decode(5, in_tokens=torch.tensor([out_d[-1]], dtype=torch.int32, device="cuda"), logits=lg)
    torch.cuda.synchronize()
    eng.status()
    toks = out[:, 0].cpu().numpy()
    recs = parity.check_forced(S.om, kc, vc, pos_d, out_d[-1], toks, lg[:, 0].cpu().numpy(), None)
    assert len(recs) == 5 and len(ref_d) == len(out_d)
    eng.close()


def test_serving_loop_ends_by_itself_when_idle(tiny):
    S = tiny
    eng = S.engine()
    _say("[test] serving loop with a 300 ms idle limit, nothing submitted")
    srv = E.Server(eng, n_slots=2, max_prompt=8, max_out=8, idle_ms=300)
    try:
        time.sleep(1.5)
        with pytest.raises(E.PreError) as ei:  # the loop has ended: nothing takes requests
            srv.submit([1, 2, 3], pos=0, budget=2)
        assert ei.value.code == -7
    finally:
        stats = srv.stop()
    assert stats == {"steps": 0, "served": 0, "error": 0}
    # the engine is free again
    out = eng.decode(2, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert eng.status()["error"] == 0 and out.shape == (2, 1)
    eng.close()
