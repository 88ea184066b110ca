"""GPU parity of the micro-batch decode path (2..8 sequences in lockstep, each
at its own context length) against the CPU oracle run sequence by sequence,
and the matrix-core lane layout the micro-batch GEMMs rely on.

Both sides start from the same bytes: seeded weights, a seeded synthetic K/V
cache (N(0, 1) at every position below the longest context) and seeded first
tokens.  Sequence b decodes from its own position; the oracle decodes each
sequence alone with its own copy of that sequence's cache.  The comparison
rules (logits, hidden state, tokens with near-tie divergence) are those of
tests/parity.py, applied to every sequence.
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


def test_mfma_lane_layout():
    """16x32 by 32x16 through the matrix-core instruction, with the operand
    and result lane mapping the micro-batch GEMMs assume: any transposed or
    permuted fragment gives a different matrix."""
    _say("[test] MFMA 16x16x32 bf16 lane layout")
    g = torch.Generator().manual_seed(3)
    A = torch.randn(16, 32, generator=g).bfloat16()
    B = torch.randn(32, 16, generator=g).bfloat16()
    got = E.debug_mfma(A, B).double().numpy()
    want = A.double().numpy() @ B.double().numpy()
    assert np.allclose(got, want, rtol=1e-5, atol=1e-5), np.abs(got - want).max()


class MbSetup:
    def __init__(self, oracle_mod, m, seed=0):
        self.m = m
        W = synth.gen_weights(m, seed=seed, device="cpu")
        self.om = oracle_mod.OracleModel(m, synth.weights_to_numpy(W))
        self.Wd = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in W.items()}
        self.Wd["layers"] = [{k: t.cuda() for k, t in L.items()} for L in W["layers"]]

    def run(self, ctx, steps, baseline=False, seed=1, forced=None, **kw):
        """GPU decode of `steps` steps from positions ctx; returns the
        outputs and the host cache the oracle starts from."""
        m = self.m
        kc, vc = synth.gen_kv_cache(m, max(max(ctx), 1), seed=seed, device="cuda")
        kc_h, vc_h = synth.to_bits(kc), synth.to_bits(vc)
        eng = E.Engine(m, self.Wd, kc, vc, **kw)
        eng.set_positions(ctx)
        tok0 = synth.gen_tokens(m.vocab, m.batch, seed=seed + 100).to(torch.int32).cuda()
        lg = torch.zeros((steps, m.batch, m.vocab), dtype=torch.float32, device="cuda")
        hd = torch.zeros((steps, m.batch, m.hidden), dtype=torch.float32, device="cuda")
        fn = eng.baseline_decode if baseline else eng.decode
        out = fn(steps, in_tokens=tok0, forced=forced, logits=lg, hidden=hd)
        torch.cuda.synchronize()
        eng.status()
        assert eng.positions() == [c + steps for c in ctx]
        res = (tok0.cpu().numpy(), out.cpu().numpy(), lg.cpu().numpy(), hd.cpu().numpy())
        eng.close()
        return res, kc_h, vc_h

    def check(self, ctx, res, kc_h, vc_h, forced=None):
        """Per sequence: the oracle decoding that sequence alone from the same
        cache, teacher-forced on the GPU's tokens (or on the forced tokens),
        every step compared."""
        tok0, toks, lgs, hds = res
        worst_l = worst_h = 0.0
        for b in range(self.m.batch):
            kb = np.ascontiguousarray(kc_h[:, b])
            vb = np.ascontiguousarray(vc_h[:, b])
            recs = parity.check_forced(self.om, kb, vb, ctx[b], int(tok0[b]), toks[:, b], lgs[:, b], hds[:, b],
                                       inputs=None if forced is None else forced[:, b])
            worst_l = max([worst_l] + [r["max_dlogit"] for r in recs])
            worst_h = max([worst_h] + [r["hidden_rel"] for r in recs])
            ties = [r["step"] for r in recs if r.get("near_tie")]
            if ties:
                _say(f"  sequence {b}: near-tie token differences at steps {ties}")
        return worst_l, worst_h


@pytest.fixture(scope="module")
def mb8(oracle_lib):
    _say("[setup] micro-batch 8 weights")
    return MbSetup(oracle_lib, synth.SMALL_MB)


CTX8 = [5, 40, 17, 100, 64, 0, 250, 31]


@pytest.mark.parametrize("grid", [0, 16, 40, 256])
def test_microbatch_matches_oracle(mb8, grid):
    """Eight sequences from contexts 0..250, several workgroup counts: the
    attention shares cross sequence boundaries, and at 256 workgroups a long
    sequence's records outnumber a combine lane group."""
    _say(f"[test] micro-batch 8, grid {grid}, contexts {CTX8}")
    res, kc_h, vc_h = mb8.run(CTX8, 4, grid_wgs=grid)
    wl, wh = mb8.check(CTX8, res, kc_h, vc_h)
    _say(f"  max dlogit {wl:.2e}, max hidden rel {wh:.2e}")


def test_microbatch_baseline_matches_oracle(mb8):
    _say("[test] micro-batch 8, one kernel per stage")
    res, kc_h, vc_h = mb8.run(CTX8, 3, baseline=True)
    wl, wh = mb8.check(CTX8, res, kc_h, vc_h)
    _say(f"  max dlogit {wl:.2e}, max hidden rel {wh:.2e}")


def test_microbatch_persistent_equals_baseline(mb8):
    _say("[test] micro-batch 8, resident kernel vs per-stage launches")
    a, _, _ = mb8.run(CTX8, 3)
    b, _, _ = mb8.run(CTX8, 3, baseline=True)
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(a[2], b[2])


def test_microbatch_forced_tokens(mb8):
    """Teacher forcing: every step consumes the given tokens of each sequence."""
    _say("[test] micro-batch 8, forced tokens")
    steps = 3
    forced = synth.gen_tokens(mb8.m.vocab, steps * mb8.m.batch, seed=77).to(torch.int32).view(steps, -1)
    res, kc_h, vc_h = mb8.run(CTX8, steps, forced=forced.cuda())
    mb8.check(CTX8, res, kc_h, vc_h, forced=forced.numpy())


def test_microbatch_of_three(oracle_lib):
    _say("[test] micro-batch 3")
    S = MbSetup(oracle_lib, synth.SMALL_MB3)
    ctx = [9, 77, 2]
    res, kc_h, vc_h = S.run(ctx, 4)
    wl, wh = S.check(ctx, res, kc_h, vc_h)
    _say(f"  max dlogit {wl:.2e}, max hidden rel {wh:.2e}")


def test_microbatch_seven_query_heads(oracle_lib):
    """Seven query heads per 128-dim KV head (q read from LDS in attention),
    five sequences, one of them at context 0."""
    _say("[test] micro-batch 5, seven query heads per KV head")
    S = MbSetup(oracle_lib, synth.SMALL_MB_G7)
    ctx = [3, 150, 60, 0, 201]
    res, kc_h, vc_h = S.run(ctx, 4)
    wl, wh = S.check(ctx, res, kc_h, vc_h)
    _say(f"  max dlogit {wl:.2e}, max hidden rel {wh:.2e}")
