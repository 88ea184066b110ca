"""Shared parity rules for the GPU tests (GPU path vs the CPU oracle).

Tolerances (the decode engine's contract):
  * max |logit_gpu - logit_oracle| <= 2e-2 over the whole vocabulary, every step;
  * hidden state (residual stream before the final norm): max |delta| / max |ref|
    <= 1e-2, every step;
  * greedy tokens identical, except at a step where the oracle's top-1 minus
    top-2 logit gap is below 1e-3; there any token whose oracle logit is within
    1e-3 of the top passes.
The oracle is teacher-forced on the GPU's tokens: its step s consumes the
token the GPU emitted at step s - 1, so both sides always see the same input
and a permitted near-tie divergence does not end the comparison -- every
later step is still compared element by element.  (While the GPU's tokens
equal the oracle's own greedy tokens this is the same as running the oracle
free, so a precomputed free-running oracle stream is reused up to the first
difference.)  The GPU computes in fp32 over the same bf16/fp8 weights; the
oracle in fp64.  No oracle input or expected value comes from the GPU except
these fed-back tokens and, where a test says so, the bf16 cache bytes the
engine's own prefill wrote (handed over as the oracle's input cache).
"""
import numpy as np
import torch

from persistent_resident_execution_amd import engine as E
from persistent_resident_execution_amd import synth

LOGIT_TOL = 2e-2
HIDDEN_REL_TOL = 1e-2
TIE_GAP = 1e-3


def top2_gap(lg):
    s = np.sort(lg)
    return float(s[-1] - s[-2])


def check_token(step, gpu_tok, ref_tok, ref_logits, rec):
    """The greedy rule for one step (both sides consumed the same input)."""
    if gpu_tok == ref_tok:
        return
    gap = top2_gap(ref_logits)
    assert gap < TIE_GAP, f"step {step}: token {gpu_tok} != oracle {ref_tok} (top-2 gap {gap})"
    assert ref_logits[gpu_tok] >= ref_logits.max() - TIE_GAP, f"step {step}: token not near the top"
    rec["near_tie"] = True


def compare_step(step, gpu_tok, gpu_logits, gpu_hidden, ref_tok, ref_logits, ref_hidden):
    """One step with identical inputs on both sides.  Raises AssertionError on
    a violation; returns the step's record."""
    rec = {"step": step}
    if gpu_logits is not None:
        d = float(np.max(np.abs(gpu_logits.astype(np.float64) - ref_logits)))
        rec["max_dlogit"] = d
        assert d <= LOGIT_TOL, f"step {step}: max |dlogit| {d} > {LOGIT_TOL}"
    if gpu_hidden is not None:
        r = float(np.max(np.abs(gpu_hidden.astype(np.float64) - ref_hidden)) /
                  max(np.max(np.abs(ref_hidden)), 1e-30))
        rec["hidden_rel"] = r
        assert r <= HIDDEN_REL_TOL, f"step {step}: hidden rel err {r} > {HIDDEN_REL_TOL}"
    check_token(step, gpu_tok, ref_tok, ref_logits, rec)
    return rec


def check_forced(om, kc, vc, P, first_in, gpu_toks, gpu_lgs, gpu_hds, free=None, say=None, inputs=None,
                 fp8=None):
    """Teacher-forced comparison of len(gpu_toks) steps from position P.

    kc, vc: the oracle's cache [L][Hkv][max_ctx][d] holding positions < P (it
    is copied before the first oracle step that writes into it).  Step s
    consumes first_in (s = 0) or the GPU's token of step s - 1.  free:
    optional (toks, logits, hidden) of a free-running oracle run from the same
    cache state and first input; used while the inputs agree.  gpu_lgs /
    gpu_hds entries may be None (not compared).  inputs: when the GPU run was
    itself teacher-forced, the token step s consumed (replaces the feedback).
    fp8: (k_scale, v_scale) when kc, vc are an fp8 cache's codes.  Returns
    the records."""
    recs, copied = [], False
    tok_in = int(first_in)
    use_free = free is not None
    for s in range(len(gpu_toks)):
        if inputs is not None:
            tok_in = int(inputs[s])
        if use_free and s > 0 and int(gpu_toks[s - 1]) != int(free[0][s - 1]):
            use_free = False
        if use_free:
            rt, rl, rh = int(free[0][s]), free[1][s], free[2][s]
        else:
            if not copied:
                kc, vc, copied = kc.copy(), vc.copy(), True
                if fp8 is not None:
                    fp8 = (fp8[0].copy(), fp8[1].copy())
            if fp8 is None:
                rt, rl, rh = om.decode_step(kc, vc, tok_in, P + s)
            else:
                rt, rl, rh = om.decode_step_fp8(kc, vc, fp8[0], fp8[1], tok_in, P + s)
        rec = compare_step(s, int(gpu_toks[s]), None if gpu_lgs is None else gpu_lgs[s],
                           None if gpu_hds is None else gpu_hds[s], rt, rl, rh)
        recs.append(rec)
        if say is not None:
            say(f"  step {s}: {rec}")
        tok_in = int(gpu_toks[s])
    return recs


class DenseSetup:
    """Weights on the host (oracle) and on the device (engine), same bytes."""

    def __init__(self, oracle_mod, m: synth.ModelConfig, seed=0, device="cuda"):
        self.m = m
        W = synth.gen_weights(m, seed=seed, device="cpu")
        self.Wnp = synth.weights_to_numpy(W)
        self.om = oracle_mod.OracleModel(m, self.Wnp)
        self.Wd = {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in W.items()}
        self.Wd["layers"] = [{k: t.to(device) for k, t in L.items()} for L in W["layers"]]
        shape = (m.n_layers, m.batch, m.n_kv_heads, m.max_ctx, m.head_dim)
        self.kc = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.vc = torch.zeros(shape, dtype=torch.bfloat16, device=device)

    def engine(self, **kw):
        return E.Engine(self.m, self.Wd, self.kc, self.vc, **kw)


def oracle_run(om, prompt, n_steps):
    """Oracle prefill from the prompt, then n_steps free-running greedy steps.
    Returns (g0, logits at the last prompt position, toks[n], logits[n][V],
    hidden[n][h], caches holding the prompt's positions)."""
    kc, vc = om.new_cache()
    om.prefill(kc, vc, prompt[:-1])
    g0, lg0, _ = om.decode_step(kc, vc, int(prompt[-1]), len(prompt) - 1)
    cache = (kc.copy(), vc.copy())
    toks, lgs, hds = [], [], []
    tok = g0
    P = len(prompt)
    for s in range(n_steps):
        nxt, lg, hd = om.decode_step(kc, vc, tok, P + s)
        toks.append(nxt)
        lgs.append(lg)
        hds.append(hd)
        tok = nxt
    return g0, lg0, np.array(toks), np.array(lgs), np.array(hds), cache


def gpu_run(eng, m, prompt, n_steps, baseline=False, device="cuda"):
    """Engine prefill (teacher-forced prompt) then n_steps greedy steps with
    check outputs.  Returns (g0, toks, logits, hidden)."""
    P = len(prompt)
    forced = torch.as_tensor(np.asarray(prompt, np.int32), device=device).view(P, 1)
    run = eng.baseline_decode if baseline else eng.decode
    eng.set_positions([0])
    pre_out = run(P, forced=forced)
    torch.cuda.synchronize()
    eng.status()
    g0 = int(pre_out[-1, 0])
    lg = torch.zeros((n_steps, 1, m.vocab), dtype=torch.float32, device=device)
    hd = torch.zeros((n_steps, 1, m.hidden), dtype=torch.float32, device=device)
    inp = torch.tensor([g0], dtype=torch.int32, device=device)
    out = run(n_steps, in_tokens=inp, logits=lg, hidden=hd)
    torch.cuda.synchronize()
    eng.status()
    return g0, out[:, 0].cpu().numpy(), lg[:, 0].cpu().numpy(), hd[:, 0].cpu().numpy()


def check_streams(om, P, g0_gpu, ref, gpu):
    """The GPU's first token (from its prefill) under the greedy rule against
    the oracle's prefill logits, then every step teacher-forced (check_forced)
    from the oracle's prompt cache.  ref = oracle_run(...)."""
    g0_ref, lg0, rtoks, rlgs, rhds, (kc, vc) = ref
    rec0 = {"step": "prefill"}
    check_token("prefill", g0_gpu, g0_ref, lg0, rec0)
    free = (rtoks, rlgs, rhds) if g0_gpu == g0_ref else None
    toks, lgs, hds = gpu
    return [rec0] + check_forced(om, kc, vc, P, g0_gpu, toks, lgs, hds, free=free)
