"""GPU parity of the HIP decode path against the CPU oracle (through the C ABI).

Both paths -- the persistent resident kernel and the one-kernel-per-operator
baseline -- fill the cache from the same seeded prompt (teacher-forced) and
then decode greedily; the oracle does the same on its own.  The rules are in
tests/parity.py.
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
    _say("[setup] tiny dense weights + oracle run (prompt 128, 64 steps)")
    S = parity.DenseSetup(oracle_lib, synth.TINY, seed=0)
    prompt = synth.gen_tokens(synth.TINY.vocab, 128, seed=0).numpy()
    ref = parity.oracle_run(S.om, prompt, 64)
    return S, prompt, ref


def _check_run(S, prompt, ref, baseline, **kw):
    eng = S.engine(**kw)
    g0, toks, lgs, hds = parity.gpu_run(eng, S.m, prompt, len(ref[2]), baseline=baseline)
    recs = parity.check_streams(S.om, len(prompt), g0, ref, (toks, lgs, hds))
    worst = max((r.get("max_dlogit", 0) for r in recs), default=0)
    ties = sum(1 for r in recs if r.get("near_tie"))
    _say(f"  {'baseline' if baseline else 'persistent'} {kw}: {len(recs) - 1} steps compared "
         f"({ties} near-tie token differences), "
         f"max dlogit {worst:.2e}, max hidden rel "
         f"{max((r.get('hidden_rel', 0) for r in recs), default=0):.2e}")
    return eng, toks, lgs


def test_fp8_unpacking_matches_oracle_decoder(oracle_lib):
    _say("[test] fp8 e4m3 unpacking, all 256 codes")
    got = E.fp8_decode_table().double().numpy()
    ref = oracle_lib.fp8_to_f64(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(ref)
    assert np.array_equal(got[finite], ref[finite])


def test_wavefront_lane_primitives():
    """The DPP / permlane reductions the tiles use, on known data."""
    _say("[test] wavefront lane primitives")
    x = torch.arange(64, dtype=torch.float32) * 1.5 - 17.0
    x[37] = 1000.0
    out = E.debug_lane_ops(x).numpy()
    xv = x.numpy()
    groups8 = xv.reshape(8, 8).sum(axis=1)
    rows16 = xv.reshape(4, 16).sum(axis=1)
    assert np.allclose(out[0:64], np.repeat(groups8, 8))
    assert np.allclose(out[64:128], np.repeat(rows16, 16))
    assert np.isclose(out[128], xv.sum()) and out[129] == xv.max()
    r = xv.reshape(4, 2, 8)
    assert np.allclose(out[192:256], np.repeat((r[:, 0] + r[:, 1])[:, None, :], 2, axis=1).ravel())
    assert np.allclose(out[256:320], np.tile(xv.reshape(4, 16).sum(axis=0), 4))


def test_tiny_persistent_matches_oracle(tiny):
    S, prompt, ref = tiny
    _say("[test] tiny persistent, 256 workgroups")
    _check_run(S, prompt, ref, baseline=False)


def test_tiny_persistent_cache_matches_oracle_prefill(tiny):
    S, prompt, ref = tiny
    _say("[test] tiny persistent prefill cache vs oracle cache")
    eng = S.engine()
    P = len(prompt)
    eng.set_positions([0])
    eng.decode(P, forced=torch.as_tensor(prompt.astype(np.int32), device="cuda").view(P, 1))
    torch.cuda.synchronize()
    eng.status()
    kc_ref, vc_ref = ref[5]
    for name, dev, host in (("K", S.kc, kc_ref), ("V", S.vc, vc_ref)):
        got = dev[:, 0, :, :P].float().cpu().numpy()
        want = host[:, :, :P].view(np.uint16).astype(np.uint32) << 16
        want = want.view(np.float32)
        diff = np.abs(got - want)
        rel = diff.max() / np.abs(want).max()
        frac = float(np.mean(diff > 0))
        _say(f"  {name}: max rel diff {rel:.2e}, fraction of differing bf16 values {frac:.2e}")
        assert rel < 1e-2 and frac < 1e-2


def test_tiny_baseline_matches_oracle(tiny):
    S, prompt, ref = tiny
    _say("[test] tiny one-kernel-per-op baseline")
    _check_run(S, prompt, ref, baseline=True)


@pytest.mark.parametrize("grid", [16, 64])
def test_tiny_persistent_fewer_workgroups(tiny, grid):
    S, prompt, ref = tiny
    _say(f"[test] tiny persistent, {grid} workgroups")
    _check_run(S, prompt, ref, baseline=False, grid_wgs=grid)


def test_persistent_deterministic_and_resumable(tiny):
    S, prompt, ref = tiny
    _say("[test] determinism and decode(n)+decode(m) == decode(n+m)")
    eng = S.engine()
    P = len(prompt)
    forced = torch.as_tensor(prompt.astype(np.int32), device="cuda").view(P, 1)
    runs = []
    for split in (None, 7):
        eng.set_positions([0])
        g0 = int(eng.decode(P, forced=forced)[-1, 0])
        lg = torch.zeros((20, 1, S.m.vocab), device="cuda")
        inp = torch.tensor([g0], dtype=torch.int32, device="cuda")
        if split is None:
            out = eng.decode(20, in_tokens=inp, logits=lg)
        else:
            a = eng.decode(split, in_tokens=inp, logits=lg[:split])
            b = eng.decode(20 - split, in_tokens=a[-1].contiguous(), logits=lg[split:])
            out = torch.cat([a, b])
        torch.cuda.synchronize()
        eng.status()
        runs.append((out.cpu().numpy(), lg.cpu().numpy()))
    assert np.array_equal(runs[0][0], runs[1][0])
    assert np.array_equal(runs[0][1], runs[1][1])


def test_persistent_equals_baseline_tokens(tiny):
    S, prompt, ref = tiny
    _say("[test] persistent vs baseline")
    _, t1, l1 = _check_run(S, prompt, ref, baseline=False)
    _, t2, l2 = _check_run(S, prompt, ref, baseline=True)
    assert np.array_equal(t1, t2)
    assert np.max(np.abs(l1 - l2)) < 1e-3


@pytest.mark.parametrize("fold_ffn,fold_attn", [(0, 0), (0, -1), (-1, 0)])
def test_tiny_folded_stages_match_unfolded(tiny, fold_ffn, fold_attn):
    """The tiny engine can fold the down projection into the gate/up stage
    (per-workgroup partials added by the next stage) and the attention into
    the output projection (every O-projection task attends its KV head over
    all positions).  Against the resident kernel with neither: both streams
    follow the oracle (64 steps, logits and hidden state), the tokens agree,
    and the logits differ only by the order of additions."""
    S, prompt, ref = tiny
    _say(f"[test] tiny folded stages fold_ffn={fold_ffn} fold_attn={fold_attn} vs neither")
    info, _ = E.plan_describe(S.m, fold_ffn=fold_ffn, fold_attn=fold_attn)
    assert (info.fold_ffn, info.fold_attn) == (int(fold_ffn == 0), int(fold_attn == 0))
    _, t1, l1 = _check_run(S, prompt, ref, baseline=False, fold_ffn=fold_ffn, fold_attn=fold_attn)
    _, t2, l2 = _check_run(S, prompt, ref, baseline=False, fold_ffn=-1, fold_attn=-1)
    assert np.array_equal(t1, t2)
    assert np.max(np.abs(l1 - l2)) < 1e-3


def test_bad_token_is_latched_and_reset_clears_it(tiny):
    S, _, _ = tiny
    _say("[test] out-of-range token -> device error, reset")
    eng = S.engine()
    eng.set_positions([0])
    eng.decode(1, in_tokens=torch.tensor([S.m.vocab + 5], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    st = eng.status(raise_on_error=False)
    assert st["error"] == 2 and st["observed"] == S.m.vocab + 5
    with pytest.raises(E.PreError):
        eng.decode(1, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
    eng.reset()
    eng.set_positions([0])
    eng.decode(1, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert eng.status()["error"] == 0


@pytest.mark.parametrize("persistent", [True, False])
def test_context_limit_is_checked_on_device(tiny, persistent):
    """Positions live on the device: a call whose steps would pass max_ctx
    latches PRE_DEV_CONTEXT (sequence, position, max_ctx), leaves the
    position unchanged and writes no cache row; reset clears it."""
    S, _, _ = tiny
    _say(f"[test] context limit on the device, {'persistent' if persistent else 'baseline'}")
    eng = S.engine()
    run = eng.decode if persistent else eng.baseline_decode
    P = S.m.max_ctx - 2
    eng.set_positions([P])
    before = S.kc[:, 0, :, P:].clone()
    run(3, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    st = eng.status(raise_on_error=False)
    assert st["error"] == 5 and st["slot"] == 0, st
    assert st["observed"] == P and st["expected"] == S.m.max_ctx, st
    assert eng.positions() == [P]
    assert torch.equal(S.kc[:, 0, :, P:], before)
    with pytest.raises(E.PreError) as ei:
        run(1, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
    assert ei.value.code == -8
    eng.reset()
    run(2, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert eng.status()["error"] == 0 and eng.positions() == [S.m.max_ctx]
    eng.close()


@pytest.mark.parametrize("persistent", [True, False])
def test_positions_advance_on_device(tiny, persistent):
    """A caller-owned device position array: each call reads it on the device
    and advances it there, so consecutive calls continue with no host
    bookkeeping; three calls (prefill, 9 steps, 11 steps) give the same
    tokens and logits as prefill + one call of 20 steps."""
    S, prompt, ref = tiny
    _say(f"[test] device positions across calls, {'persistent' if persistent else 'baseline'}")
    P = len(prompt)
    forced = torch.as_tensor(prompt.astype(np.int32), device="cuda").view(P, 1)
    runs = []
    for split in (None, 9):
        ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
        eng = E.Engine(S.m, S.Wd, S.kc, S.vc, ctx_len=ctx)
        run = eng.decode if persistent else eng.baseline_decode
        g0 = run(P, forced=forced)[-1].contiguous()
        lg = torch.zeros((20, 1, S.m.vocab), device="cuda")
        if split is None:
            out = run(20, in_tokens=g0, logits=lg)
        else:
            a = run(split, in_tokens=g0, logits=lg[:split])
            b = run(20 - split, in_tokens=a[-1].contiguous(), logits=lg[split:])
            out = torch.cat([a, b])
        torch.cuda.synchronize()
        eng.status()
        assert int(ctx.item()) == P + 20
        runs.append((int(g0.item()), out.cpu().numpy(), lg.cpu().numpy()))
        eng.close()
    assert runs[0][0] == runs[1][0]
    assert np.array_equal(runs[0][1], runs[1][1])
    assert np.array_equal(runs[0][2], runs[1][2])
    g0, toks, lgs = runs[0]
    recs = parity.check_streams(S.om, P, g0, ref, (toks[:, 0], lgs[:, 0], None))
    assert len(recs) == 21


@pytest.mark.parametrize("which", ["lm", "qkv"])
def test_watchdog_latches_timeout_and_every_workgroup_exits(tiny, which):
    """The watchdog path, forced from the host: the task that sets one ready
    flag skips its store (debug), so its consumers wait until the 1 ms
    watchdog fires.  Every workgroup must leave the resident kernel (the
    launch completes), the status names the timeout, and after a reset the
    engine decodes correctly again."""
    S, prompt, ref = tiny
    _say(f"[test] watchdog timeout on a dropped {which} flag")
    eng = S.engine()
    info, _ = E.plan_describe(S.m)
    W = info.n_wgs
    # the LM stage's flags are read by every workgroup's per-step reduction,
    # so the one missing flag is what any latching workgroup reports;
    # workgroup 3's flag of the second layer's QKV stage is read by that
    # head's attention chunks
    slot = (info.n_stage_inst - 1) * W + 3 if which == "lm" else 5 * W + 3
    eng.set_watchdog(1)
    eng.debug_drop_signal(slot)
    eng.set_positions([0])
    t0 = torch.tensor([1], dtype=torch.int32, device="cuda")
    eng.decode(4, in_tokens=t0)
    torch.cuda.synchronize()  # the launch ended: every workgroup left
    st = eng.status(raise_on_error=False)
    _say(f"  status {st}")
    assert st["error"] == 1, st
    assert st["step"] == 0 and st["expected"] == 1 and st["observed"] == 0, st
    if which == "lm":
        assert st["slot"] == slot, st
    else:
        assert st["slot"] >= slot, st
    eng.debug_drop_signal(-1)
    eng.set_watchdog(2000)
    eng.reset()
    g0, toks, lgs, hds = parity.gpu_run(eng, S.m, prompt, 8)
    parity.check_streams(S.om, len(prompt), g0, (ref[0], ref[1], ref[2][:8], ref[3][:8], ref[4][:8], ref[5]),
                         (toks, lgs, hds))
    eng.close()


@pytest.fixture(scope="module")
def small(oracle_lib):
    _say("[setup] small dense (ragged shapes) + oracle run (prompt 40, 24 steps)")
    S = parity.DenseSetup(oracle_lib, synth.SMALL_DENSE, seed=3)
    prompt = synth.gen_tokens(synth.SMALL_DENSE.vocab, 40, seed=3).numpy()
    ref = parity.oracle_run(S.om, prompt, 24)
    return S, prompt, ref


@pytest.mark.parametrize("grid,threads", [(0, 0), (16, 256), (37, 512)])
def test_small_dense_ragged_persistent(small, grid, threads):
    S, prompt, ref = small
    _say(f"[test] small dense persistent grid={grid} threads={threads}")
    _check_run(S, prompt, ref, baseline=False, grid_wgs=grid, wg_threads=threads)


def test_small_dense_ragged_baseline(small):
    S, prompt, ref = small
    _say("[test] small dense baseline")
    _check_run(S, prompt, ref, baseline=True)


@pytest.mark.parametrize("persistent", [True, False])
def test_layer0_intermediates_match_oracle_primitives(oracle_lib, persistent):
    """One decode step at position 0: each intermediate activation of layer 0
    (q, the per-KV-head output-projection partials, residual after attention,
    SwiGLU output, layer output) against the
    oracle's primitives applied step by step -- localises a faulty tile."""
    _say(f"[test] layer-0 intermediates, {'persistent' if persistent else 'baseline'}")
    m = synth.TINY
    S = parity.DenseSetup(oracle_lib, m, seed=0)
    W, L0, tok, d = S.Wnp, S.Wnp["layers"][0], 5, m.head_dim
    f = lambda b: oracle_lib.bf16_to_f64(b).reshape(b.shape)  # noqa: E731
    x = f(W["embed"][tok])
    a = oracle_lib.rmsnorm(x, L0["attn_norm"], m.rms_eps)
    q, v = oracle_lib.gemv_bf16(L0["wq"], a), oracle_lib.gemv_bf16(L0["wv"], a)
    vb = f(oracle_lib.f32_to_bf16(v.astype(np.float32)))  # single key: attention returns V
    grp = lambda h: h * m.n_kv_heads // m.n_q_heads  # noqa: E731
    o = np.concatenate([vb[grp(h) * d:(grp(h) + 1) * d] for h in range(m.n_q_heads)])
    xm = x + oracle_lib.gemv_bf16(L0["wo"], o)
    b = oracle_lib.rmsnorm(xm, L0["ffn_norm"], m.rms_eps)
    g, up = oracle_lib.gemv_bf16(L0["wg"], b), oracle_lib.gemv_bf16(L0["wu"], b)
    u = np.array([oracle_lib.silu(z) for z in g]) * up
    xo = xm + oracle_lib.gemv_bf16(L0["wd"], u)
    eng = S.engine(grid_wgs=16)
    eng.set_positions([0])
    run = eng.decode if persistent else eng.baseline_decode
    run(1, in_tokens=torch.tensor([tok], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    eng.status()
    sl = lambda n, c: eng.debug_slot(n, c).cpu().numpy().astype(np.float64)  # noqa: E731
    # the O projection is split by KV head: its partials plus the layer input
    # make the post-attention residual
    pb = sl("pbuf", m.n_kv_heads * m.hidden).reshape(m.n_kv_heads, m.hidden)
    got_xm = x + pb.sum(axis=0)
    o_proj_by_head = [oracle_lib.gemv_bf16(np.ascontiguousarray(
        L0["wo"][:, g * (m.n_q_heads // m.n_kv_heads) * d:(g + 1) * (m.n_q_heads // m.n_kv_heads) * d]),
        o[g * (m.n_q_heads // m.n_kv_heads) * d:(g + 1) * (m.n_q_heads // m.n_kv_heads) * d])
        for g in range(m.n_kv_heads)]
    for name, got, ref in (("q", sl("q", q.size), q), ("o-proj by head", pb, np.array(o_proj_by_head)),
                           ("xm", got_xm, xm), ("u", sl("u", m.ffn_dim), u),
                           ("x_out", sl("x_out", m.hidden), xo)):
        rel = np.abs(got - ref).max() / np.abs(ref).max()
        _say(f"  {name}: rel err {rel:.1e}")
        assert rel < 1e-5, name
    eng.close()


@pytest.fixture(scope="module")
def small_moe(oracle_lib):
    _say("[setup] small MoE (fp8 experts, odd scale-block count) + oracle run (prompt 24, 16 steps)")
    S = parity.DenseSetup(oracle_lib, synth.SMALL_MOE, seed=5)
    prompt = synth.gen_tokens(synth.SMALL_MOE.vocab, 24, seed=5).numpy()
    ref = parity.oracle_run(S.om, prompt, 16)
    return S, prompt, ref


@pytest.mark.parametrize("grid,threads", [(0, 0), (37, 256)])
def test_small_moe_persistent(small_moe, grid, threads):
    S, prompt, ref = small_moe
    _say(f"[test] small MoE persistent grid={grid} threads={threads}")
    _check_run(S, prompt, ref, baseline=False, grid_wgs=grid, wg_threads=threads)


def test_small_moe_baseline(small_moe):
    S, prompt, ref = small_moe
    _say("[test] small MoE baseline")
    _check_run(S, prompt, ref, baseline=True)


@pytest.fixture(scope="module")
def gqa8(oracle_lib):
    _say("[setup] small 8-KV-head decoder (XCD-local hand-offs) + oracle run (prompt 48, 24 steps)")
    S = parity.DenseSetup(oracle_lib, synth.SMALL_GQA8, seed=7)
    prompt = synth.gen_tokens(synth.SMALL_GQA8.vocab, 48, seed=7).numpy()
    ref = parity.oracle_run(S.om, prompt, 24)
    return S, prompt, ref


@pytest.mark.parametrize("grid", [0, 40])
def test_gqa8_xcd_local_matches_oracle(gqa8, grid):
    S, prompt, ref = gqa8
    _say(f"[test] 8-KV-head persistent, XCD-local hand-offs, grid={grid}")
    assert E.plan_describe(S.m, grid_wgs=grid)[0].xcd_local == 1
    _check_run(S, prompt, ref, baseline=False, grid_wgs=grid)


def test_gqa8_xcd_local_equals_device_scope(gqa8):
    """Only the cache scope of the hand-offs differs: identical results."""
    S, prompt, ref = gqa8
    _say("[test] 8-KV-head persistent, XCD-local vs device-scope hand-offs")
    _, t1, l1 = _check_run(S, prompt, ref, baseline=False)
    _, t2, l2 = _check_run(S, prompt, ref, baseline=False, xcd_local=-1)
    assert np.array_equal(t1, t2) and np.array_equal(l1, l2)


def test_zero_steps_launch_nothing(tiny):
    S, _, _ = tiny
    eng = S.engine()
    eng.set_positions([5])
    out = eng.decode(0, in_tokens=torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape[0] == 0 and eng.positions() == [5]
    assert eng.status()["error"] == 0


@pytest.mark.parametrize("persistent", [True, False])
def test_last_position_matches_oracle(oracle_lib, persistent):
    """One step at position max_ctx - 1 (the cache's last row) over a seeded
    synthetic cache handed to both sides."""
    m = synth.TINY
    _say(f"[test] last position, {'persistent' if persistent else 'baseline'}")
    S = parity.DenseSetup(oracle_lib, m, seed=11)
    P = m.max_ctx - 1
    kc, vc = synth.gen_kv_cache(m, P, seed=12, device="cuda")
    S.kc.copy_(kc)
    S.vc.copy_(vc)
    kc_h = np.ascontiguousarray(synth.to_bits(kc)[:, 0])
    vc_h = np.ascontiguousarray(synth.to_bits(vc)[:, 0])
    eng = S.engine()
    eng.set_positions([P])
    lg = torch.zeros((1, 1, m.vocab), device="cuda")
    hd = torch.zeros((1, 1, m.hidden), device="cuda")
    run = eng.decode if persistent else eng.baseline_decode
    out = run(1, in_tokens=torch.tensor([3], dtype=torch.int32, device="cuda"), logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    nxt, ref_lg, ref_hd = S.om.decode_step(kc_h, vc_h, 3, P)
    parity.compare_step(0, int(out[0, 0]), lg[0, 0].cpu().numpy(), hd[0, 0].cpu().numpy(), nxt, ref_lg, ref_hd)
    assert eng.positions() == [m.max_ctx]
    run(1, in_tokens=torch.tensor([3], dtype=torch.int32, device="cuda"))  # the cache is full now
    torch.cuda.synchronize()
    assert eng.status(raise_on_error=False)["error"] == 5
    eng.close()


@pytest.fixture(scope="module")
def mha(oracle_lib):
    _say("[setup] small multi-head decoder (one query head per KV head) + oracle run")
    S = parity.DenseSetup(oracle_lib, synth.SMALL_MHA, seed=9)
    prompt = synth.gen_tokens(synth.SMALL_MHA.vocab, 32, seed=9).numpy()
    ref = parity.oracle_run(S.om, prompt, 16)
    return S, prompt, ref


@pytest.mark.parametrize("baseline", [False, True])
def test_mha_matches_oracle(mha, baseline):
    S, prompt, ref = mha
    _say(f"[test] MHA (G = 1) {'baseline' if baseline else 'persistent'}")
    _check_run(S, prompt, ref, baseline=baseline)
