"""Host logic of the profile summaries: the per-stage wait / busy / phase
table read from the in-kernel timestamp ring (synthetic records with known
gaps)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from persistent_resident_execution_amd import profiling as pf  # noqa: E402


def _records(steps, nsi, W, stride=300):
    rec = np.zeros((steps, nsi, W, 8), np.uint32)
    t = 1000
    for s in range(steps):
        for si in range(nsi):
            for w in range(W):
                rec[s, si, w, 0] = si | (w << 16)
                rec[s, si, w, 1] = t + w          # begin
                rec[s, si, w, 2] = t + 50 + w     # producers ready
                rec[s, si, w, 4] = t + 80         # phase marks
                rec[s, si, w, 5] = t + 150
                rec[s, si, w, 6] = t + 170
                rec[s, si, w, 3] = t + 200 + w    # end
            t += stride
    return rec


def test_phase_table_batch1():
    L, spl, W = 2, 5, 4
    lines = pf.phase_table(_records(3, L * spl + 1, W), ["qkv", "attn", "oproj", "gu", "down", "lm"], L, spl, 0)
    qkv = lines[0].split()
    assert qkv[:7] == ["qkv", "wait", "0.50", "busy", "1.50", "span", "2.03"]
    assert "stage 0.28  stream 0.70  epi 0.52" in lines[0]
    assert "pv 0.20  store 0.32" in lines[1]
    # stage ends 300 ticks apart: 3 us per stage on the critical path
    assert lines[-1].endswith("qkv 3.00  attn 3.00  oproj 3.00  gu 3.00  down 3.00")


def test_phase_table_microbatch_layout():
    # an embedding stage first, six stages per layer, the LM head last
    L, spl, W = 2, 6, 2
    names = ["embed", "qkv", "attn", "comb", "oproj", "gu", "down", "lm"]
    lines = pf.phase_table(_records(3, 1 + L * spl + 1, W, stride=100), names, L, spl, 1, pf.PHASES_MB)
    emb = lines[0].split()
    assert emb[:5] == ["embed", "wait", "0.00", "busy", "2.00"]  # no dependency wait: all of it is busy
    assert "stream 0.99  epi 0.51" in lines[1]  # ends at mark 1, then the task end
    assert lines[-1] == ("critical-path deltas per layer (us): qkv 1.00  attn 1.00  comb 1.00  oproj 1.00  "
                         "gu 1.00  down 1.00")


def test_phase_table_with_folded_stages():
    # the small-model kernel skips the attention and down stages: their
    # records stay zero; they report no line and a zero delta, and the stage
    # after each is measured from the stage before it
    L, spl, W = 2, 5, 4
    rec = _records(3, L * spl + 1, W)
    for l in range(L):
        rec[:, l * spl + 1] = 0  # attention
        rec[:, l * spl + 4] = 0  # down
    lines = pf.phase_table(rec, ["qkv", "attn", "oproj", "gu", "down", "lm"], L, spl, 0)
    kinds = [ln.split()[0] for ln in lines[:-1]]
    assert kinds == ["qkv", "oproj", "gu", "lm"]
    assert lines[-1].endswith("qkv 6.00  attn 0.00  oproj 6.00  gu 3.00  down 0.00")


def test_bench_names_the_kernel_each_engine_launches():
    import bench
    from persistent_resident_execution_amd import synth
    from dataclasses import replace
    assert bench.kernel_of(synth.TINY) == "pre_persistent_small"
    assert bench.kernel_of(synth.TINY, fold_ffn=-1, fold_attn=-1) == "pre_persistent"
    assert bench.kernel_of(synth.DENSE8B) == "pre_persistent"
    assert bench.kernel_of(synth.MOE) == "pre_persistent"
    assert bench.kernel_of(replace(synth.TINY, kv_fp8=True)) == "pre_persistent_kv8"
    assert bench.kernel_of(synth.SMALL_MB) == "pre_persistent_mb"
