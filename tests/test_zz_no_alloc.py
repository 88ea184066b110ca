"""The engine over the library's static workspace (pre_engine_create_static,
for callers that cannot allocate device memory) against the engine over a
caller workspace (pre_engine_create), through the C ABI.

Two creates in a row on one GPU, the second with a smaller model (a smaller
workspace, so whatever the first left in the static array past it must not
matter), each decoding a teacher-forced prompt and then greedy steps with
logits and hidden state.  The static engine runs the same kernels over the
same task table, so its tokens, logits and hidden states must equal the
ordinary engine's bit for bit; they also meet the oracle's tolerances (the
tiny case is checked against the oracle as well).  The first engine is
taken over by the second create and must refuse further calls.
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


def _decode(S, prompt, steps, static):
    S.kc.zero_()
    S.vc.zero_()
    eng = S.engine(static_workspace=static)
    g0, toks, lgs, hds = parity.gpu_run(eng, S.m, prompt, steps)
    return eng, (g0, toks, lgs, hds)


def test_static_workspace_engine_matches_workspace_engine(oracle_lib):
    first = None
    for m, P, steps, seed in ((synth.TINY, 96, 24, 0), (synth.SMALL_MHA, 40, 12, 9)):
        info, _ = E.plan_describe(m)
        assert info.workspace_bytes <= (32 << 20)
        _say(f"[test] static workspace, {m.name}: prompt {P}, {steps} steps, "
             f"workspace {info.workspace_bytes} bytes")
        S = parity.DenseSetup(oracle_lib, m, seed=seed)
        prompt = synth.gen_tokens(m.vocab, P, seed=seed).numpy()
        e_ref, ref = _decode(S, prompt, steps, static=False)
        e_ref.close()
        e_st, got = _decode(S, prompt, steps, static=True)
        assert got[0] == ref[0]
        for a, b in zip(got[1:], ref[1:]):
            assert np.array_equal(a, b)
        if m is synth.TINY:
            oref = parity.oracle_run(S.om, prompt, steps)
            parity.check_streams(S.om, P, got[0], oref, got[1:])
        if first is not None:
            # the earlier static engine's workspace now belongs to this one
            with pytest.raises(E.PreError) as ei:
                first.decode(1, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
            assert ei.value.code == -8
            first.close()
        first = e_st
    first.close()


def test_static_workspace_refuses_too_large_a_configuration():
    m = synth.WORKLOADS["dense8b_mb8"].model  # 227 MiB of workspace
    kc = torch.zeros((m.n_layers, m.batch, m.n_kv_heads, 8, m.head_dim), dtype=torch.bfloat16, device="cuda")
    cfg = E.make_config(m)
    import ctypes as C
    h = C.c_void_p()
    w = E.Weights(None, None, None, None)
    kv = E.KV(kc.data_ptr(), kc.data_ptr(), None)
    rc = E.lib().pre_engine_create_static(C.byref(cfg), C.byref(w), C.byref(kv), None, C.byref(h))
    assert rc == -4 and not h.value
