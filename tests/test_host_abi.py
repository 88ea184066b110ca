"""Host-side checks that need no GPU: the C-ABI library loads and exports
every function include/pre.h declares; the task-table builder produces
tables its validator accepts for every workload; the validator rejects
tables with planted faults; and the per-step byte count agrees with an
independent count from the shapes."""
import os
import re

from dataclasses import replace

import numpy as np
import pytest

from persistent_resident_execution_amd import engine as E
from persistent_resident_execution_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(E.LIB_PATH):
        from persistent_resident_execution_amd import build
        build.build()
    return E.lib()


def test_library_exports_every_declared_function(lib):
    hdr = open(os.path.join(ROOT, "include", "pre.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"\b(pre_[a-z_0-9]+)\s*\(", hdr))
    assert len(names) >= 15
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in pre.h but not exported"
    assert names >= set(E.EXPORTS)


def test_strerror_and_argument_errors(lib):
    import ctypes as C
    assert lib.pre_strerror(0) == b"ok"
    for code in range(-1, -10, -1):
        assert lib.pre_strerror(code) != b"unknown error"
    chk = E.Check(None, None)
    assert lib.pre_engine_decode(None, 1, None, None, None, C.byref(chk), None) == -1
    assert lib.pre_baseline_decode(None, 1, None, None, None, C.byref(chk), None) == -1
    assert lib.pre_engine_destroy(None) == -1
    st = E.Status()
    assert lib.pre_engine_status(None, C.byref(st)) == -1


def _cdiv(a, b):
    return -(-a // b)


def _gemv_lds_bytes(m, W, threads=512):
    """LDS of the GEMV tasks: the staged input (padded to 1024 columns), two
    results per row pair per wavefront for the largest task of any stage,
    256 reduction words -- or, if larger, the output projection's padded
    input plus its KV head's attention chunk records (m, l, two unused
    words, o) and one weight each -- then the 80-entry segment table (12
    words each)."""
    nk = m.top_k + m.n_shared
    F = nk * m.expert_ffn if m.is_moe else m.ffn_dim
    kmax = _cdiv(max(m.hidden, m.n_q_heads * m.head_dim, F, m.n_experts,
                     ((nk - 1) * m.expert_ffn + _cdiv(m.expert_ffn, 1024) * 1024) if m.is_moe else 0),
                 1024) * 1024
    rows2 = lambda r: r + (r & 1)  # noqa: E731  (consecutive-row pairs)
    Tg = W // m.n_kv_heads
    pairs = m.n_kv_heads * (m.n_q_heads // m.n_kv_heads + 2) * m.head_dim // 2
    y = [2 * _cdiv(pairs, W), rows2(_cdiv(m.hidden, W)), rows2(_cdiv(m.vocab, W)), rows2(_cdiv(m.hidden, Tg))]
    if m.is_moe:
        y += [rows2(_cdiv(m.n_experts, W)), 2 * _cdiv(F, W), rows2(_cdiv(m.hidden, W)) * nk]
    else:
        y += [2 * _cdiv(m.ffn_dim, W)]
    ymax = _cdiv(max(y), 64) * 64
    return (_cdiv(kmax + ymax * (threads // 64) + 256, 4) * 4 + 80 * 12) * 4


ALL = [w.model for w in synth.WORKLOADS.values() if w.model.batch == 1] + [
    synth.TINY, synth.SMALL_DENSE, synth.SMALL_MOE, synth.SMALL_GQA8]


@pytest.mark.parametrize("m", ALL, ids=lambda m: f"{m.name}-{m.max_ctx}")
@pytest.mark.parametrize("grid", [0, 1, 7, 16, 37, 256])
def test_plans_validate(lib, m, grid):
    W = grid or 256
    if grid and grid < m.n_kv_heads:
        lds = None
    else:
        lds = _gemv_lds_bytes(m, W)
    if grid and (lds is None or lds > 160 * 1024):
        with pytest.raises(E.PreError) as ei:
            E.plan_describe(m, grid_wgs=grid)
        assert ei.value.code == -2
        return
    info, _ = E.plan_describe(m, grid_wgs=grid)
    assert info.validator == 0
    assert info.n_stage_inst == m.n_layers * (6 if m.is_moe else 5) + 1
    assert info.workspace_bytes > 0


MB = [synth.WORKLOADS["dense8b_mb8"].model, synth.SMALL_MB, synth.SMALL_MB3, synth.SMALL_MB_G7]


@pytest.mark.parametrize("m", MB, ids=lambda m: m.name)
@pytest.mark.parametrize("grid", [0, 8, 16, 40, 256])
def test_microbatch_plans_validate(lib, m, grid):
    """The micro-batch table: an embedding stage, six stages per layer, the LM
    head; every KV head's attention and combine on its own block of Tw
    workgroups; rows in whole groups of 8 where outputs are packed."""
    info, T = E.plan_describe(m, with_tasks=True, grid_wgs=grid)
    assert info.validator == 0
    W = info.n_wgs
    assert W % m.n_kv_heads == 0
    assert info.n_stage_inst == 6 * m.n_layers + 2
    Tw = W // m.n_kv_heads
    ops = [T[si * W][0] for si in range(info.n_stage_inst)]
    assert ops[0] == 10 and ops[-1] == 9 and ops[1:7] == [1, 2, 11, 3, 4, 5]
    attn, comb = T[2 * W:3 * W], T[3 * W:4 * W]
    for lam in range(W):
        assert attn[lam][4] == lam // Tw and attn[lam][2] == lam % Tw and attn[lam][3] == Tw
        assert comb[lam][4] == lam // Tw
        assert comb[lam][5] == 2 * W + (lam // Tw) * Tw and comb[lam][6] == comb[lam][5] + Tw
    for si in (0, 4, 5, 6):  # EMBED, OPROJ, GU, DOWN: row ranges in groups of 8
        for lam in range(W):
            assert T[si * W + lam][2] % 8 == 0 and T[si * W + lam][3] % 8 == 0


def test_microbatch_plan_validator_catches_mistakes(lib):
    m = synth.SMALL_MB
    info, T = E.plan_describe(m, with_tasks=True, grid_wgs=16)
    W = info.n_wgs
    bad = T.copy()
    bad[3 * W + 1][5] += 1  # a combine that no longer waits on all of its head's attention
    assert E.plan_validate(m, bad, grid_wgs=16) == 7
    bad = T.copy()
    bad[5 * W + 2][3] -= 8  # a gate/up row group nobody computes
    assert E.plan_validate(m, bad, grid_wgs=16) == 5
    bad = T.copy()
    bad[2 * W + 3][2] = 0  # two attention shares with the same index
    assert E.plan_validate(m, bad, grid_wgs=16) == 6


def test_microbatch_unsupported_and_bad_shapes(lib):
    from dataclasses import replace
    with pytest.raises(E.PreError) as ei:  # routed experts at batch > 1
        E.plan_describe(replace(synth.SMALL_MOE, batch=2))
    assert ei.value.code == -6
    with pytest.raises(E.PreError) as ei:  # ffn not in whole 32-column blocks
        E.plan_describe(replace(synth.SMALL_DENSE, batch=2))
    assert ei.value.code == -6
    with pytest.raises(E.PreError) as ei:  # KV heads' workgroup blocks must be equal
        E.plan_describe(synth.SMALL_MB3, grid_wgs=10)
    assert ei.value.code == -2


def test_attention_and_o_projection_are_xcd_local_on_the_8b_shape(lib):
    """Each KV head's attention chunks and its slice of the output projection
    sit on the XCD that computed the head's QKV rows, and wait only on tasks
    of that XCD (the head-to-XCD routing)."""
    m = synth.DENSE8B
    info, T = E.plan_describe(m, with_tasks=True)
    W = info.n_wgs
    per = W // 8  # workgroups per XCD (lambda is XCD-major)
    attn, oproj = T[1 * W:2 * W], T[2 * W:3 * W]
    n_attn = 0
    for lam in range(W):
        op, layer, r0, r1, aux, lo, hi, sig = attn[lam]
        if op == 0:
            continue
        n_attn += 1
        assert op == 2 and lam // per == aux % m.n_kv_heads
        assert lo == (aux % m.n_kv_heads) * per and hi == lo + per  # QKV slots of that XCD
        op, layer, r0, r1, aux, lo, hi, sig = oproj[lam]
    assert n_attn == m.n_kv_heads * info.attn_splits
    for lam in range(W):
        op, layer, r0, r1, aux, lo, hi, sig = oproj[lam]
        assert op == 3 and aux == lam // per
        assert lo == W + aux * per and hi == lo + info.attn_splits  # that head's chunk tasks


@pytest.mark.parametrize("wl,want", [("dense8b_ctx1024", 12), ("dense8b_ctx8192", 16), ("moe", 16),
                                     ("tiny", 2), ("dense8b_mb8", 1)])
def test_default_attention_split(lib, wl, want):
    """Default KV chunks per (sequence, KV head): about one per 128 positions
    of max_ctx, at most 16 and at most the workgroups per KV head; one for the
    micro-batch (its split follows the step's contexts)."""
    m = synth.WORKLOADS[wl].model
    info, _ = E.plan_describe(m)
    assert info.attn_splits == want
    info, _ = E.plan_describe(m, attn_splits=3) if m.batch == 1 else (info, None)
    assert info.attn_splits == (3 if m.batch == 1 else 1)


def _planted(m, mutate):
    info, T = E.plan_describe(m, with_tasks=True)
    T = T.copy()
    mutate(T, info.n_wgs)
    return E.plan_validate(m, T)


def test_validator_rejects_planted_faults(lib):
    m = synth.SMALL_DENSE
    W = E.plan_describe(m)[0].n_wgs
    info, T = E.plan_describe(m, with_tasks=True)
    assert E.plan_validate(m, T) == 0
    # a consumer that no longer waits for one producer
    assert _planted(m, lambda T, W: T.__setitem__((2 * W + 5, 6), T[2 * W + 5, 6] - 1)) == 7
    # two tasks computing the same rows (duplicate), one row range lost
    def dup(T, W):
        T[3 * W + 4, 2:4] = T[3 * W + 3, 2:4]
    assert _planted(m, dup) == 5
    # a wait on a slot of a later stage (would deadlock)
    assert _planted(m, lambda T, W: T.__setitem__((3 * W, 6), 9 * W)) == 3
    # a workgroup skipping a GEMV stage (breaks slot-reuse ordering)
    def skip(T, W):
        T[4 * W + 2] = [0, 0, 0, 0, 0, 0, 0, -1]
    assert _planted(m, skip) in (2, 8)
    # an attention chunk dropped (two tasks on the same chunk)
    def drop(T, W):
        T[1 * W + 1, 2] = T[1 * W + 0, 2]
    assert _planted(m, drop) == 6
    # a signal slot shared by two tasks
    assert _planted(m, lambda T, W: T.__setitem__((4 * W + 1, 7), 4 * W + 0)) == 4


def _independent_step_bytes(m, pos):
    wb = synth.weight_bytes(m)
    total = sum(v for k, v in wb.items())
    kv_row = m.n_kv_heads * m.head_dim * 2
    total += m.n_layers * 2 * kv_row * (pos + 1) + m.n_layers * 2 * kv_row
    return total


@pytest.mark.parametrize("m", [synth.TINY, synth.DENSE8B, synth.MOE], ids=lambda m: m.name)
def test_step_bytes_matches_shape_count(lib, m):
    for pos in (0, 1023, 4000):
        assert E.step_bytes(m, [pos]) == _independent_step_bytes(m, pos)


def test_step_bytes_8b_order_of_magnitude(lib):
    # 8B-shape: 32 x 436 MB of layer weights + 1.05 GB LM head ~ 15.0 GB of weights
    b = E.step_bytes(synth.DENSE8B, [1024])
    assert 15.0e9 < b < 15.3e9


@pytest.mark.parametrize("m,grid,flag,want", [
    (synth.DENSE8B, 0, 0, 1), (synth.DENSE8B, 64, 0, 1), (synth.DENSE8B, 0, -1, 0),
    (synth.DENSE8B, 100, 0, 0), (synth.MOE, 0, 0, 1), (synth.TINY, 0, 0, 2), (synth.TINY, 0, -1, 0),
    (synth.TINY, 64, 0, 0), (synth.TINY, 24, 0, 2), (synth.SMALL_DENSE, 40, 0, 0), (synth.SMALL_DENSE, 32, 0, 2),
    (synth.SMALL_GQA8, 40, 0, 1), (synth.SMALL_GQA8, 36, 0, 0), (synth.SMALL_GQA8, 12, 0, 2)],
    ids=lambda v: str(getattr(v, "name", v)))
def test_xcd_local_mode_only_where_each_head_fits_one_xcd(lib, m, grid, flag, want):
    """The per-head L2-local hand-offs (1) are used only with 8 KV heads on a
    grid that splits evenly over the 8 XCDs; there every QKV, attention and
    O-projection task of head g, and every slot it waits on, lies in XCD g's
    lambda range.  Otherwise a grid that fits one XCD's 32 CUs runs there
    entirely (2); the default grid of a small model is capped at 32."""
    info, T = E.plan_describe(m, with_tasks=True, grid_wgs=grid, xcd_local=flag)
    assert info.xcd_local == want
    if want == 2:
        assert info.n_wgs <= 32
    if want != 1:
        return
    W, per = info.n_wgs, info.n_wgs // 8
    spl = 6 if m.is_moe else 5
    for layer in range(m.n_layers):
        for k in range(3):  # QKV, ATTN, OPROJ
            for lam in range(W):
                op, _, r0, r1, aux, lo, hi, sig = T[(layer * spl + k) * W + lam]
                if op == 0 or lo >= hi or k == 0:
                    continue
                assert all((s % W) // per == lam // per for s in range(lo, hi)), (layer, k, lam)


@pytest.mark.parametrize("m,kw,want", [
    (synth.TINY, {}, 1), (synth.TINY, {"fold_ffn": -1}, 0), (synth.TINY, {"xcd_local": -1}, 0),
    (synth.TINY, {"grid_wgs": 64}, 0), (synth.TINY, {"grid_wgs": 16}, 0), (synth.TINY, {"grid_wgs": 24}, 1),
    (synth.DENSE8B, {}, 0), (synth.MOE, {}, 0), (synth.SMALL_MB, {}, 0), (synth.SMALL_GQA8, {"grid_wgs": 12}, 0)],
    ids=lambda v: str(getattr(v, "name", v)))
def test_ffn_fold_only_on_small_one_xcd_dense_engines(lib, m, kw, want):
    """The down projection is folded into the gate/up stage only for batch-1
    dense engines on one XCD whose hidden size fits the workgroup (one Wd row
    per thread) and whose gate/up tasks start at a multiple of 8 rows and hold
    at most 32 (tiny at its default 32 workgroups: 24; at 24 workgroups 32;
    at 16 workgroups 48 do not fit; hidden 640 does not fit 512 threads).
    The task table stays the unfolded one (the per-operator path runs it as
    it is), and the workspace gains the partials [L][W][hidden]."""
    info, _ = E.plan_describe(m, **kw)
    assert info.fold_ffn == want
    assert info.validator == 0
    if want:
        off, _ = E.plan_describe(m, **dict(kw, fold_ffn=-1))
        assert off.fold_ffn == 0 and off.n_tasks == info.n_tasks
        assert info.workspace_bytes - off.workspace_bytes >= m.n_layers * info.n_wgs * m.hidden * 4


@pytest.mark.parametrize("m,kw,want", [
    (synth.TINY, {}, 1), (synth.TINY, {"fold_attn": -1}, 0), (synth.TINY, {"xcd_local": -1}, 0),
    (synth.TINY, {"grid_wgs": 64}, 0), (synth.TINY, {"grid_wgs": 16}, 1), (synth.SMALL_DENSE, {}, 0),
    (synth.SMALL_DENSE, {"grid_wgs": 16, "wg_threads": 256}, 1), (synth.SMALL_MHA, {}, 1),
    (replace(synth.TINY, kv_fp8=True), {}, 0), (replace(synth.TINY, max_ctx=32768), {}, 0),
    (synth.DENSE8B, {}, 0), (synth.MOE, {}, 0), (synth.SMALL_MB, {}, 0)],
    ids=lambda v: str(getattr(v, "name", v)))
def test_attention_fold_only_on_small_one_xcd_bf16_engines(lib, m, kw, want):
    """Each output-projection task attends itself (the attention stage is
    skipped) only in batch-1 engines on one XCD with a bf16 cache whose whole
    context's scores fit the LDS; the table keeps its attention stage for
    the per-operator path."""
    info, T = E.plan_describe(m, with_tasks=True, **kw)
    assert info.fold_attn == want
    assert info.validator == 0
    if want:
        W = info.n_wgs
        assert (T[W:2 * W, 0] != 0).any()  # the attention stage is still in the table


def _folded_reading(T, W, Tg, fold, inl):
    """The table as the small-model kernel reads it (the device's fold_task):
    {(stage instance, workgroup): task} of the tasks it runs, waits re-pointed."""
    out = {}
    for si in range(len(T) // W):
        for lam in range(W):
            op, layer, r0, r1, aux, lo, hi, sig = (int(v) for v in T[si * W + lam])
            if op == 0:
                continue
            if inl and op == 2:
                continue
            if inl and op == 3:
                a = T[(si - 1) * W + aux * Tg]
                lo, hi = int(a[5]), int(a[6])
            if fold and op == 5:
                continue
            if fold and ((op == 1 and layer > 0) or op == 9):
                lo, hi = lo - W, hi - W
            out[(si, lam)] = (op, layer, r0, r1, aux, lo, hi, sig)
    return out


@pytest.mark.parametrize("m,kw", [(synth.TINY, {}), (synth.TINY, {"grid_wgs": 24}), (synth.SMALL_MHA, {}),
                                  (synth.SMALL_DENSE, {"grid_wgs": 16, "wg_threads": 256})],
                         ids=lambda v: str(getattr(v, "name", v)))
def test_folded_reading_keeps_every_dependency(lib, m, kw):
    """The folded stages skip the down and attention tasks and re-point their
    consumers' waits.  Read that way, the table must still order every hand-off:
    each wait names only slots that a task which still runs sets in an earlier
    stage; the next layer's QKV and the LM head wait for the whole gate/up
    stage (which now leaves the down partials); each output projection waits
    for every QKV task holding its KV head's pairs; and every QKV task is
    waited for by some output projection, so the residual shares it writes
    are ordered before the gate/up stage that reads them."""
    info, T = E.plan_describe(m, with_tasks=True, **kw)
    W, fold, inl = info.n_wgs, info.fold_ffn, info.fold_attn
    assert fold or inl
    Tg = W // (m.batch * m.n_kv_heads)
    R = _folded_reading(T, W, Tg, fold, inl)
    setters = {t[7]: si for (si, lam), t in R.items()}
    for (si, lam), t in R.items():
        for slot in range(t[5], t[6]):
            assert slot in setters and setters[slot] < si, (si, lam, slot)
    spl, pg = 5, m.head_dim // 2 * (m.n_q_heads // m.n_kv_heads + 2)  # RoPE pairs per KV head
    waited_qkv = set()
    for (si, lam), t in R.items():
        op, layer, lo, hi = t[0], t[1], t[5], t[6]
        if fold and ((op == 1 and layer > 0) or op == 9):
            gu = (layer - 1 if op == 1 else m.n_layers - 1) * spl + 3
            assert lo <= gu * W and hi >= (gu + 1) * W, (si, lam)
        if inl and op == 3:
            g, q = t[4] % m.n_kv_heads, layer * spl
            for w in range(W):
                r0, r1 = int(T[q * W + w][2]), int(T[q * W + w][3])
                if r0 < r1 and r0 < (g + 1) * pg and r1 > g * pg:
                    assert lo <= q * W + w < hi, (si, lam, w)
                    waited_qkv.add((layer, w))
    if fold and inl:
        assert waited_qkv == {(l, w) for l in range(m.n_layers) for w in range(W)}
    kept_ops = {t[0] for t in R.values()}
    assert (5 not in kept_ops) == bool(fold) and (2 not in kept_ops) == bool(inl)


def test_kv_descriptor_size_bound(lib):
    """The K/V append addresses a layer's whole cache with a 32-bit buffer
    size: a configuration whose layer cache reaches 4 GiB is refused, the
    largest one below passes.  (At batch 1 the attention chunk's LDS bounds
    max_ctx long before that.)"""
    import dataclasses
    m = synth.DENSE8B  # 8 KV heads x 128 dims: 4 KB per position and sequence
    per_pos = m.n_kv_heads * m.head_dim * 2
    for batch in (4, 8):
        limit = (1 << 32) // (per_pos * batch)  # first max_ctx whose layer cache is 4 GiB
        ok = dataclasses.replace(m, batch=batch, max_ctx=limit - 1)
        bad = dataclasses.replace(m, batch=batch, max_ctx=limit)
        assert E.plan_describe(ok)[0].validator == 0
        with pytest.raises(E.PreError) as ei:
            E.plan_describe(bad)
        assert ei.value.code == -2


def _host_weights(m):
    import torch
    W = synth.gen_weights(m, seed=0, device="cpu")
    shape = (m.n_layers, m.batch, m.n_kv_heads, m.max_ctx, m.head_dim)
    return W, torch.zeros(shape, dtype=torch.bfloat16), torch.zeros(shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("m", [synth.TINY, synth.SMALL_MOE], ids=lambda m: m.name)
def test_engine_arguments_are_checked_before_any_call(m):
    """The binding hands raw pointers to the C ABI, so it checks every tensor
    first: device, dtype, contiguity and shape/size.  Exercised here on host
    tensors with the device check set to the host (the binding uses 'cuda')."""
    import torch
    W, kc, vc = _host_weights(m)
    E.check_model_args(m, W, kc, vc, device_type="cpu")  # good arguments pass
    with pytest.raises(ValueError, match="expected a cuda tensor"):
        E.check_model_args(m, W, kc, vc)
    bad = [("k_cache", lambda: (W, kc[:, :, :, :-1], vc)),
           ("v_cache", lambda: (W, kc, vc.float())),
           ("k_cache", lambda: (W, kc.transpose(3, 4), vc)),
           ("embed", lambda: ({**W, "embed": W["embed"][:-1]}, kc, vc)),
           ("lm_head", lambda: ({**W, "lm_head": W["lm_head"].float()}, kc, vc)),
           ("layers[1].wq", lambda: ({**W, "layers": [W["layers"][0], {**W["layers"][1],
                                      "wq": W["layers"][1]["wq"].t()}]}, kc, vc)),
           ("weights", lambda: ({**W, "layers": W["layers"][:1]}, kc, vc))]
    if m.is_moe:
        bad.append(("layers[0].e_sd", lambda: ({**W, "layers": [{**W["layers"][0],
                                                 "e_sd": W["layers"][0]["e_sd"][:, :-1]}] + W["layers"][1:]},
                                               kc, vc)))
    for name, make in bad:
        with pytest.raises(ValueError, match=re.escape(name)):
            E.check_model_args(m, *make(), device_type="cpu")
    with pytest.raises(ValueError, match="ctx_len"):
        E.check_model_args(m, W, kc, vc, ctx_len=torch.zeros(m.batch, dtype=torch.int64), device_type="cpu")


def test_decode_arguments_are_checked_before_any_call():
    import torch
    m = synth.SMALL_MB3  # batch 3
    n, B, V, h = 4, m.batch, m.vocab, m.hidden
    i32 = lambda k: torch.zeros(k, dtype=torch.int32)  # noqa: E731
    good = dict(in_tokens=i32(B), forced=None, out_tokens=i32(n * B),
                logits=torch.zeros(n * B * V), hidden=torch.zeros(n * B * h))
    E.check_decode_args(m, n, device_type="cpu", **good)
    E.check_decode_args(m, 0, None, None, None, None, None, device_type="cpu")  # nothing is read
    with pytest.raises(ValueError, match="expected a cuda tensor"):
        E.check_decode_args(m, n, **good)
    cases = [("in_tokens", dict(in_tokens=torch.zeros(B, dtype=torch.int64))),
             ("in_tokens", dict(in_tokens=i32(B - 1))),
             ("forced", dict(forced=i32(n * B - 1))),
             ("out_tokens", dict(out_tokens=i32(n * B - 1))),
             ("logits", dict(logits=torch.zeros(n * B * V - 1))),
             ("hidden", dict(hidden=torch.zeros(n * B * h, dtype=torch.float64))),
             ("hidden", dict(hidden=torch.zeros(2 * n * B * h)[::2])),
             ("in_tokens or forced", dict(in_tokens=None)),
             ("n_steps", None)]
    for name, change in cases:
        with pytest.raises(ValueError, match=re.escape(name)):
            if change is None:
                E.check_decode_args(m, -1, device_type="cpu", **good)
            else:
                E.check_decode_args(m, n, device_type="cpu", **{**good, **change})
