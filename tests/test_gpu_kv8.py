"""The fp8 e4m3 K/V cache (one fp32 scale per cached row) on the GPU against
the oracle's fp8 cache path, through the C ABI.

The engine fills the cache itself (teacher-forced prompt) -- the QKV stage
leaves each new row in fp32 and the attention task owning its position
quantizes and appends it -- then decodes greedily; the oracle prefills its
own fp8 cache from the same prompt and is teacher-forced on the GPU's tokens
(tests/parity.py).  Checked: every step's logits and hidden state, the
cached codes and scales against the oracle's, the per-operator path and the
XCD-local hand-offs, and the 8B shape at context 8192 from the engine's own
8192-token cache (its bytes handed to the oracle).
"""
import dataclasses
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


class Kv8Setup:
    def __init__(self, oracle_mod, m, seed):
        self.m = m
        W = synth.gen_weights(m, seed=seed, device="cpu")
        self.om = oracle_mod.OracleModel(m, synth.weights_to_numpy(W))
        self.Wd = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in W.items()}
        self.Wd["layers"] = [{k: t.cuda() for k, t in L.items()} for L in W["layers"]]

    def run(self, prompt, steps, baseline=False, **kw):
        m = self.m
        kc, vc, ks, vs = synth.empty_kv_cache(m, device="cuda")
        eng = E.Engine(m, self.Wd, kc, vc, k_scale=ks, v_scale=vs, **kw)
        g0, toks, lgs, hds = parity.gpu_run(eng, m, prompt, steps, baseline=baseline)
        eng.close()
        return g0, toks, lgs, hds, (kc, vc, ks, vs)

    def oracle_prompt(self, prompt):
        """The oracle's fp8 cache after the prompt but its last token, and
        (greedy, logits) of the last prompt position."""
        kc, vc, ks, vs = self.om.new_cache_fp8()
        for i, t in enumerate(prompt[:-1]):
            self.om.decode_step_fp8(kc, vc, ks, vs, int(t), i, want_logits=False, want_hidden=False)
        g0, lg0, _ = self.om.decode_step_fp8(kc, vc, ks, vs, int(prompt[-1]), len(prompt) - 1, want_hidden=False)
        return (kc, vc, ks, vs), g0, lg0

    def check(self, prompt, res):
        g0, toks, lgs, hds, dev_cache = res
        (kc, vc, ks, vs), g0_ref, lg0 = self.oracle_prompt(prompt)
        P = len(prompt)
        # the cache the engine wrote for the prompt against the oracle's
        for name, dev, host in (("K", dev_cache[0], kc), ("V", dev_cache[1], vc)):
            got = dev[:, 0, :, :P].cpu().numpy()
            frac = float(np.mean(got != host[:, :, :P]))
            _say(f"  {name} codes: fraction differing {frac:.2e}")
            if frac >= 1e-2:
                bad = np.argwhere(got != host[:, :, :P])[:6]
                _say(f"  first differences (layer, head, pos, dim): {bad.tolist()}")
                _say(f"  gpu {[int(got[tuple(i)]) for i in bad]} oracle {[int(host[:, :, :P][tuple(i)]) for i in bad]}")
                _say(f"  gpu row {got[0, 0, 5, :16].tolist()} oracle row {host[0, 0, 5, :16].tolist()}")
                _say(f"  scales gpu {dev_cache[2][0, 0, 0, :6].tolist()} oracle {ks[0, 0, :6].tolist()}")
            assert frac < 1e-2
        for name, dev, host in (("K", dev_cache[2], ks), ("V", dev_cache[3], vs)):
            got = dev[:, 0, :, :P].cpu().numpy()
            rel = float(np.max(np.abs(got - host[:, :, :P]) / host[:, :, :P]))
            _say(f"  {name} scales: max rel diff {rel:.2e}")
            assert rel < 1e-3
        rec0 = {}
        parity.check_token("prefill", g0, g0_ref, lg0, rec0)
        recs = parity.check_forced(self.om, kc, vc, P, g0, toks, lgs, hds, fp8=(ks, vs))
        _say(f"  {len(recs)} steps: max dlogit {max(r['max_dlogit'] for r in recs):.2e}, max hidden rel "
             f"{max(r['hidden_rel'] for r in recs):.2e}, near ties {[r['step'] for r in recs if r.get('near_tie')]}")
        return recs


@pytest.fixture(scope="module")
def tiny8(oracle_lib):
    return Kv8Setup(oracle_lib, dataclasses.replace(synth.TINY, kv_fp8=True), seed=0)


def test_fp8_encoder_matches_oracle_encoder(oracle_lib):
    """The device's e4m3 encoder against the oracle's on random values over
    the whole range, every code's value and every halfway point."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn(20000, generator=g) * torch.exp2(torch.randint(-14, 12, (20000,), generator=g).float())
    vals = oracle_lib.fp8_to_f64(np.arange(256, dtype=np.uint8))
    finite = np.sort(np.unique(vals[~np.isnan(vals)]))
    probe = np.concatenate([x.numpy(), finite, (finite[1:] + finite[:-1]) / 2, [447.0, 448.0, 464.0, 1e6]])
    probe = np.concatenate([probe, -probe]).astype(np.float32)
    got = E.fp8_encode(probe).numpy()
    want = oracle_lib.f32_to_fp8(probe)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(probe[i]), int(got[i]), int(want[i])) for i in bad[:8]]


def test_fp8_cache_tiny_persistent_matches_oracle(tiny8):
    prompt = synth.gen_tokens(tiny8.m.vocab, 128, seed=0).numpy()
    _say("[test] fp8 cache, tiny decoder, prompt 128, 64 steps, persistent")
    tiny8.check(prompt, tiny8.run(prompt, 64))


def test_fp8_cache_tiny_baseline_equals_persistent(tiny8):
    prompt = synth.gen_tokens(tiny8.m.vocab, 48, seed=1).numpy()
    _say("[test] fp8 cache, tiny decoder, per-operator path vs resident kernel")
    a = tiny8.run(prompt, 16)
    b = tiny8.run(prompt, 16, baseline=True)
    assert a[0] == b[0] and np.array_equal(a[1], b[1])
    assert np.abs(a[2] - b[2]).max() < 1e-3
    tiny8.check(prompt, b)


def test_fp8_cache_gqa8_xcd_local_matches_oracle(oracle_lib):
    S = Kv8Setup(oracle_lib, dataclasses.replace(synth.SMALL_GQA8, kv_fp8=True), seed=7)
    prompt = synth.gen_tokens(S.m.vocab, 48, seed=7).numpy()
    _say("[test] fp8 cache, 8 KV heads (XCD-local hand-offs), prompt 48, 24 steps")
    assert E.plan_describe(S.m)[0].xcd_local == 1
    S.check(prompt, S.run(prompt, 24))


@pytest.mark.timeout(900)
def test_fp8_cache_dense8b_ctx8192_16_steps(oracle_lib):
    w = synth.WORKLOADS["dense8b_ctx8192_kv8"]
    m, P = w.model, w.contexts[0]
    _say(f"[full-size] {w.note}: 16 steps from the engine's own prefill")
    t0 = time.time()
    W = synth.gen_weights(m, seed=0, device="cuda")
    Wnp = synth.weights_to_numpy(W)
    kc, vc, ks, vs = synth.empty_kv_cache(m, device="cuda")
    eng = E.Engine(m, W, kc, vc, k_scale=ks, v_scale=vs)
    prompt = synth.gen_tokens(m.vocab, P, seed=0, device="cuda")
    g0 = eng.decode(P, forced=prompt.view(P, 1))[-1].contiguous()
    steps = 16
    lg = torch.zeros((steps, 1, m.vocab), device="cuda")
    hd = torch.zeros((steps, 1, m.hidden), device="cuda")
    out = eng.decode(steps, in_tokens=g0, logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    eng.close()
    _say(f"  GPU {time.time() - t0:.1f}s; tokens {out[:, 0].tolist()}")
    host = [np.ascontiguousarray(x.cpu().numpy()[:, 0]) for x in (kc, vc, ks, vs)]
    toks, lgs, hds = out[:, 0].cpu().numpy(), lg[:, 0].cpu().numpy(), hd[:, 0].cpu().numpy()
    del W, kc, vc, ks, vs, lg, hd
    torch.cuda.empty_cache()
    om = oracle_lib.OracleModel(m, Wnp)
    g0_ref, lg0, _ = om.decode_step_fp8(host[0], host[1], host[2], host[3], int(prompt[-1]), P - 1,
                                        want_hidden=False)
    parity.check_token("prompt end", int(g0.item()), g0_ref, lg0, {})
    recs = parity.check_forced(om, host[0], host[1], P, int(g0.item()), toks, lgs, hds, fp8=(host[2], host[3]))
    _say(f"  max dlogit {max(r['max_dlogit'] for r in recs):.2e}, max hidden rel "
         f"{max(r['hidden_rel'] for r in recs):.2e}")
