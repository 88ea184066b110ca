"""Prefill and speculative verify through the chunk task set (the
micro-batch tiles over consecutive tokens of one sequence), through the C
ABI, against the oracle.

Prefill: every prompt position's logits and hidden state and its greedy
successor against the oracle decoding the prompt token by token; the cache
the chunked prefill wrote against the oracle's; ragged chunks; a prefill in
two calls continuing on the device; then greedy decode from the prefilled
cache (teacher-forced oracle, the greedy rule).

Verify: rounds of a current token plus k drafts at positions p..p+k; every
column's logits against the oracle fed the same tokens at the same
positions, every column's greedy successor under the greedy rule, the
device's acceptance count against the rule applied to the GPU's own greedy
tokens, the position advanced by accepted + 1; drafts that are the oracle's
greedy stream are all accepted, drafts that part from it are accepted up to
there, and the committed tokens reproduce the oracle's greedy stream.
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


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def tiny(oracle_lib):
    return parity.DenseSetup(oracle_lib, synth.TINY, seed=0)


def _engine(S, ctx, **kw):
    S.kc.zero_()
    S.vc.zero_()
    return E.Engine(S.m, S.Wd, S.kc, S.vc, ctx_len=ctx, chunk=8, **kw)


@pytest.mark.parametrize("grid", [0, 16])
def test_chunked_prefill_matches_oracle(tiny, grid):
    S = tiny
    m = S.m
    P = 61  # seven full chunks of 8 and a ragged one of 5
    prompt = synth.gen_tokens(m.vocab, P, seed=21)
    _say(f"[test] chunked prefill of {P} tokens, grid {grid}")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng = _engine(S, ctx, grid_wgs=grid)
    lg = torch.zeros((P, m.vocab), device="cuda")
    hd = torch.zeros((P, m.hidden), device="cuda")
    out = eng.prefill(prompt.cuda(), logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    assert int(ctx.item()) == P
    out, lg, hd = out.cpu().numpy(), lg.cpu().numpy(), hd.cpu().numpy()
    kc, vc = S.om.new_cache()
    worst = 0.0
    for i, t in enumerate(prompt.tolist()):
        rt, rl, rh = S.om.decode_step(kc, vc, t, i)
        rec = parity.compare_step(i, int(out[i]), lg[i], hd[i], rt, rl, rh)
        worst = max(worst, rec["max_dlogit"])
    _say(f"  {P} positions: max dlogit {worst:.2e}")
    for name, dev, host in (("K", S.kc, kc), ("V", S.vc, vc)):
        got = dev[:, 0, :, :P].float().cpu().numpy()
        want = (host[:, :, :P].astype(np.uint32) << 16).view(np.float32)
        diff = np.abs(got - want)
        rel, frac = diff.max() / np.abs(want).max(), float(np.mean(diff > 0))
        _say(f"  {name} cache: max rel diff {rel:.2e}, fraction of differing bf16 values {frac:.2e}")
        assert rel < 1e-2 and frac < 1e-2
    # greedy decode continues from the prefilled cache (ordinary decode path)
    n = 24
    lgd = torch.zeros((n, 1, m.vocab), device="cuda")
    hdd = torch.zeros((n, 1, m.hidden), device="cuda")
    toks = eng.decode(n, in_tokens=torch.tensor([int(out[-1])], dtype=torch.int32, device="cuda"), logits=lgd,
                      hidden=hdd)
    torch.cuda.synchronize()
    eng.status()
    parity.check_forced(S.om, kc, vc, P, int(out[-1]), toks[:, 0].cpu().numpy(), lgd[:, 0].cpu().numpy(),
                        hdd[:, 0].cpu().numpy())
    eng.close()


def test_prefill_in_two_calls_continues_on_the_device(tiny):
    S = tiny
    m = S.m
    prompt = synth.gen_tokens(m.vocab, 43, seed=22)
    _say("[test] prefill in two calls (13 + 30 tokens), then a third of 1")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng = _engine(S, ctx)
    lg = torch.zeros((44, m.vocab), device="cuda")
    o1 = eng.prefill(prompt[:13].cuda(), logits=lg[:13])
    o2 = eng.prefill(prompt[13:].cuda(), logits=lg[13:43])
    extra = torch.tensor([5], dtype=torch.int32)
    o3 = eng.prefill(extra.cuda(), logits=lg[43:])
    torch.cuda.synchronize()
    eng.status()
    assert int(ctx.item()) == 44
    out = torch.cat([o1, o2, o3]).cpu().numpy()
    lg = lg.cpu().numpy()
    kc, vc = S.om.new_cache()
    for i, t in enumerate(prompt.tolist() + [5]):
        rt, rl, _ = S.om.decode_step(kc, vc, t, i, want_hidden=False)
        parity.compare_step(i, int(out[i]), lg[i], None, rt, rl, None)
    eng.close()


def test_speculative_verify_matches_greedy_decoding(tiny):
    S = tiny
    m = S.m
    P = 40
    prompt = synth.gen_tokens(m.vocab, P, seed=23)
    # the oracle's greedy stream s_0 (after the prompt), s_1, ...
    okc, ovc = S.om.new_cache()
    S.om.prefill(okc, ovc, prompt[:-1].numpy())
    s0, _, _ = S.om.decode_step(okc, ovc, int(prompt[-1]), P - 1, want_logits=False, want_hidden=False)
    stream, t = [s0], s0
    for k in range(32):
        t, _, _ = S.om.decode_step(okc, ovc, t, P + k, want_logits=False, want_hidden=False)
        stream.append(t)
    bad = lambda tok: (tok + 1) % m.vocab  # noqa: E731  (a token that is not the greedy one)
    # rounds: (index of the current token in the stream, drafts, expected accepted)
    rounds = [(0, stream[1:8], 7), (8, [stream[9], stream[10], bad(stream[11]), stream[12]], 2),
              (11, [bad(stream[12])], 0), (12, stream[13:16], 3), (16, stream[17:24], 7)]
    _say(f"[test] speculative verify, oracle stream {stream}")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    eng = _engine(S, ctx)
    g0 = int(eng.prefill(prompt.cuda())[-1].item())
    assert g0 == s0, (g0, s0)  # (no near-tie expected on this seed)
    kc, vc = S.om.new_cache()
    S.om.prefill(kc, vc, prompt.numpy())
    pos, committed = P, []
    for cur_i, drafts, want in rounds:
        chunk = [stream[cur_i]] + list(drafts)
        k = len(drafts)
        lg = torch.zeros((k + 1, m.vocab), device="cuda")
        out, acc = eng.verify(torch.tensor(chunk, dtype=torch.int32, device="cuda"), logits=lg)
        torch.cuda.synchronize()
        eng.status()
        out, acc, lg = out.cpu().numpy(), int(acc.item()), lg.cpu().numpy()
        # every column against the oracle fed the same tokens at the same positions
        for b, tok in enumerate(chunk):
            rt, rl, _ = S.om.decode_step(kc, vc, tok, pos + b, want_hidden=False)
            parity.compare_step(b, int(out[b]), lg[b], None, rt, rl, None)
        a = 0
        while a < k and chunk[a + 1] == int(out[a]):
            a += 1
        _say(f"  at {pos}: tokens {chunk} -> greedy {out.tolist()}, accepted {acc}")
        assert acc == a == want
        assert int(ctx.item()) == pos + a + 1
        assert int(out[a]) == stream[cur_i + a + 1]
        committed += chunk[:a + 1]
        pos += a + 1
    assert committed == stream[:len(committed)]
    # ordinary decode continues after the last verify
    nxt = stream[rounds[-1][0] + rounds[-1][2] + 1]
    toks = eng.decode(4, in_tokens=torch.tensor([nxt], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    eng.status()
    i0 = len(committed)
    assert toks[:, 0].tolist() == stream[i0 + 1:i0 + 5]
    eng.close()


def test_chunk_task_set_refused_for_moe(oracle_lib):
    m = synth.SMALL_MOE
    W = synth.gen_weights(m, seed=0, device="cuda")
    kc = torch.zeros((m.n_layers, 1, m.n_kv_heads, m.max_ctx, m.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(E.PreError) as ei:
        E.Engine(m, W, kc, kc.clone(), chunk=8)
    assert ei.value.code == -6
