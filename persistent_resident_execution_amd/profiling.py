"""Condense rocprofv3 output into the short text summaries kept under
profiles/, and read them back for the benchmark.

    python -m persistent_resident_execution_amd.profiling stats DIR --out FILE --command "..."
    python -m persistent_resident_execution_amd.profiling traffic FETCH_DIR WRITE_DIR --out FILE \\
        --command "..." --copy-bytes N --workload W --steps K
    python -m persistent_resident_execution_amd.profiling counters DIR --out FILE --command "..."
    python -m persistent_resident_execution_amd.profiling l2xcd DIR --out FILE --command "..."

`stats` condenses a `rocprofv3 --kernel-trace --stats` run: calls and
durations per kernel, plus every dispatch of the resident kernel from the
trace (--kernel: pre_persistent, or pre_persistent_mb for a micro-batch).

`traffic` takes two `--pmc` runs of the same command, one collecting
FETCH_SIZE and one WRITE_SIZE (both KiB per dispatch).  The command runs
the library's plain copy kernel (pre_k_copy) on a known number of bytes
before the decode launch; each counter of the decode launch (the last
pre_persistent dispatch) is scaled by copy bytes / the copy's reading of
that counter.  The summary records a hash of the kernel sources it was
measured with: the benchmark reports the traffic only while the sources
still hash the same.

`counters` lists any other counters of the last pre_persistent dispatch
(L2 hits and misses, GPU-active cycles).

`l2xcd` reads a `rocprofv3 --pmc TCC_HIT TCC_MISS --output-format json`
run, where each dispatch carries one record per counter instance (16 L2
channels x 8 XCDs, in the order the counter's instance list gives), and
writes the L2 hit rate of each XCD for the last dispatch of the kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL = "pre_persistent"
COPY_KERNEL = "pre_k_copy"


def source_hash() -> str:
    """sha256 over the kernel sources, the C ABI header and the build recipe."""
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*"))) + [
        os.path.join(ROOT, "include", "pre.h"), os.path.join(PKG, "build.py")]
    h = hashlib.sha256()
    for f in files:
        if os.path.isfile(f):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def _csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(hits[0], newline="") as fh:
        return list(csv.DictReader(fh))


def _short(name, n=60):
    return name if len(name) <= n else name[: n - 3] + "..."


def summarize_stats(d, out, command, kernel=KERNEL, index=None, workload=None):
    """index: the dispatch of `kernel` (in launch order) that ran `workload`
    when one profiled process ran several workloads; its duration is then the
    summary's mean_us."""
    rows = _csv(d, "kernel_stats.csv")
    trace = sorted(_csv(d, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
            if r["Kernel_Name"] == kernel]
    lines = [f"# rocprofv3 kernel trace + stats", f"command: {command}", f"source_sha256: {source_hash()}"]
    if workload is not None:
        lines.append(f"workload: {workload}")
    lines += ["",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>12s} {'min_us':>12s} {'max_us':>12s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{_short(r['Name']):60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:12.1f} "
                     f"{float(r['MinNs']) / 1e3:12.1f} {float(r['MaxNs']) / 1e3:12.1f} "
                     f"{float(r['Percentage']):6.2f}")
    lines += ["", f"{kernel} dispatches (us, in launch order): " + ", ".join(f"{x:.1f}" for x in durs)]
    if index is not None:
        lines.append(f"{kernel} dispatch {index} ran {workload}: {durs[index]:.1f} us")
        lines.append(f"{kernel} mean_us: {durs[index]:.1f}")
    elif durs:
        lines.append(f"{kernel} mean_us: {statistics.mean(durs):.1f}")
    _write(out, lines)


def _last_dispatch_value(rows, kernel, counter, index=-1):
    """The counter summed over its instances for one dispatch of kernel: the
    index-th in dispatch order (default the last); and how many there were."""
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and r["Kernel_Name"] == kernel:
            did = int(r["Dispatch_Id"])
            vals[did] = vals.get(did, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise ValueError(f"no {counter} rows for {kernel}")
    return vals[sorted(vals)[index]], len(vals)


def summarize_traffic(fetch_dir, write_dir, out, command, copy_bytes, workload, steps, kernel=KERNEL,
                      index=-1):
    fr, wr = _csv(fetch_dir, "counter_collection.csv"), _csv(write_dir, "counter_collection.csv")
    f_k, nf = _last_dispatch_value(fr, kernel, "FETCH_SIZE", index)
    w_k, nw = _last_dispatch_value(wr, kernel, "WRITE_SIZE", index)
    which = "last" if index == -1 else f"dispatch {index}"
    f_c, _ = _last_dispatch_value(fr, COPY_KERNEL, "FETCH_SIZE")
    w_c, _ = _last_dispatch_value(wr, COPY_KERNEL, "WRITE_SIZE")
    ff, fw = copy_bytes / (f_c * 1024.0), copy_bytes / (w_c * 1024.0)
    fetch_b, write_b = f_k * 1024.0 * ff, w_k * 1024.0 * fw
    lines = ["# HBM traffic of one decode launch from rocprofv3 --pmc (two runs)",
             f"command: {command}",
             f"workload: {workload}", f"steps: {steps}", f"source_sha256: {source_hash()}",
             f"copy_bytes: {copy_bytes}",
             f"copy_FETCH_SIZE_KiB: {f_c:.1f}", f"copy_WRITE_SIZE_KiB: {w_c:.1f}",
             f"fetch_scale: {ff:.4f}", f"write_scale: {fw:.4f}",
             f"kernel: {kernel}",
             f"kernel_FETCH_SIZE_KiB: {f_k:.1f}  ({which} of {nf} {kernel} dispatches)",
             f"kernel_WRITE_SIZE_KiB: {w_k:.1f}  ({which} of {nw} {kernel} dispatches)",
             f"fetch_bytes_per_launch: {fetch_b:.0f}", f"write_bytes_per_launch: {write_b:.0f}",
             f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
             f"traffic_bytes_per_step: {(fetch_b + write_b) / steps:.0f}"]
    _write(out, lines)


def summarize_counters(d, out, command, kernel=KERNEL):
    rows = _csv(d, "counter_collection.csv")
    names = sorted({r["Counter_Name"] for r in rows if r["Kernel_Name"] == kernel})
    lines = ["# rocprofv3 --pmc counters of the last decode launch", f"command: {command}",
             f"source_sha256: {source_hash()}"]
    vals = {}
    for n in names:
        v, cnt = _last_dispatch_value(rows, kernel, n)
        vals[n] = v
        lines.append(f"{n}: {v:.0f}  (last of {cnt} dispatches)")
    if "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals:
        tot = vals["TCC_HIT_sum"] + vals["TCC_MISS_sum"]
        lines.append(f"L2_hit_rate: {vals['TCC_HIT_sum'] / tot:.4f}" if tot else "L2_hit_rate: n/a")
    if "GRBM_GUI_ACTIVE" in vals and vals.get("GRBM_COUNT"):
        lines.append(f"gpu_active_frac: {vals['GRBM_GUI_ACTIVE'] / vals['GRBM_COUNT']:.4f}")
    _write(out, lines)


def summarize_l2_per_xcd(d, out, command, kernel=KERNEL):
    import json
    hits = sorted(glob.glob(os.path.join(d, "**", "*.json"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *.json under {d}")
    with open(hits[0]) as fh:
        doc = json.load(fh)
    top = doc["rocprofiler-sdk-tool"][0] if "rocprofiler-sdk-tool" in doc else doc
    # counter id -> (name, XCD index of each instance, in record order)
    ctr = {}
    for c in top["counters"]:
        xcd = []
        for inst in c.get("instances", []):
            dims = {x["dimension_name"]: x["index"] for x in inst["dimensions"]}
            xcd.append(dims.get("DIMENSION_XCC", 0))
        ctr[c["id"]["handle"]] = (c["name"], xcd)
    def is_kernel(sym):
        for key in ("formatted_kernel_name", "demangled_kernel_name", "truncated_kernel_name", "kernel_name"):
            nm = str(sym.get(key, ""))
            if nm == kernel or nm == kernel + ".kd" or nm.startswith(kernel + "("):
                return True
        return False
    ids = {k.get("kernel_id") for k in top.get("kernel_symbols", []) if is_kernel(k)}
    last = None
    for rec in top["callback_records"]["counter_collection"]:
        if rec["dispatch_data"]["dispatch_info"]["kernel_id"] in ids:
            last = rec
    if last is None:
        raise RuntimeError(f"no dispatch of {kernel}")
    per = {}  # name -> [per-XCD sum]
    seen = {}
    for r in last["records"]:
        cid = r["counter_id"]["handle"]
        name, xcd = ctr[cid]
        i = seen.get(cid, 0)
        seen[cid] = i + 1
        per.setdefault(name, [0.0] * 8)[xcd[i] if i < len(xcd) else 0] += float(r["value"])
    h, m = per.get("TCC_HIT", [0.0] * 8), per.get("TCC_MISS", [0.0] * 8)
    lines = ["# L2 hit rate per XCD of the last decode launch (rocprofv3 --pmc, per-instance records)",
             f"command: {command}", f"source_sha256: {source_hash()}", f"kernel: {kernel}"]
    for x in range(8):
        t = h[x] + m[x]
        lines.append(f"xcd{x}: hit {h[x]:.0f} miss {m[x]:.0f} hit_rate {h[x] / t if t else 0.0:.4f}")
    th, tm = sum(h), sum(m)
    lines.append(f"all: hit {th:.0f} miss {tm:.0f} hit_rate {th / (th + tm) if th + tm else 0.0:.4f}")
    _write(out, lines)


# Phases of each task kind in the trace ring: (name, mark index that ends
# it); the last phase ends with the task (END).
END = -1
PHASES = {"qkv": [("stage", 0), ("stream", 1), ("epi", END)],
          "attn": [("q+scores", 0), ("softmax", 1), ("pv", 2), ("store", END)],
          "oproj": [("combine", 0), ("stream", 1), ("epi", END)],
          "gu": [("stage", 0), ("stream", 1), ("epi", END)], "down": [("stage", 0), ("stream", 1), ("epi", END)],
          "router": [("stage", 0), ("stream", 1), ("epi", END)], "egu": [("stage", 0), ("stream", 1), ("epi", END)],
          "edown": [("stage", 0), ("stream", 1), ("epi", END)], "lm": [("stage", 0), ("stream", 1), ("epi", END)]}
# the micro-batch kernel marks only the end of its GEMM streams (input
# staging included); its attention and combine tasks set no marks
PHASES_MB = {k: [("stream", 1), ("epi", END)] for k in ("qkv", "oproj", "gu", "down", "lm")}


def phase_table(rec, stage_names, n_layers, stages_per_layer, first, phases=None):
    """Per task kind, means over the traced steps (the first one skipped) and
    layers, in µs: the wait for producers (begin -> wait end), the work after
    it (busy) split at the task's phase marks, and the span of the stage
    (earliest begin to latest end over the workgroups); plus the per-layer
    critical-path deltas (latest end of a stage minus latest end of the one
    before).  rec: uint32 trace records [steps][stage instances][W][8].
    stage_names: the per-layer kinds in order, optionally preceded by
    "embed" (stage instance 0) and followed by "lm" (the last one); kind k
    of layer l is stage instance first + l * stages_per_layer + k.  A stage
    without a dependency wait (embed) reports its whole task as busy."""
    import numpy as np
    phases = PHASES if phases is None else phases
    a = rec.astype(np.int64) & 0xffffffff
    steps, nsi = a.shape[0], a.shape[1]
    kinds = [n for n in stage_names if n not in ("embed", "lm")]
    lines = []
    for nm in stage_names:
        if nm == "lm":
            sis = [nsi - 1]
        elif nm == "embed":
            sis = [0]
        else:
            k = kinds.index(nm)
            sis = [first + l * stages_per_layer + k for l in range(n_layers)]
        wait, busy, span, ph = [], [], [], []
        for s in range(1, steps):
            for si in sis:
                r = a[s, si]
                r = r[r[:, 1] != 0]
                if len(r) == 0:
                    continue
                w0 = r[:, 1] if nm == "embed" else r[:, 2]
                wait.append(float(np.mean(w0 - r[:, 1])))
                busy.append(float(np.mean(r[:, 3] - w0)))
                span.append(float(r[:, 3].max() - r[:, 1].min()))
                spec = phases.get(nm, [])
                if spec:
                    pts = [w0] + [r[:, 3] if m == END else r[:, 4 + m] for _, m in spec]
                    ph.append([float(np.mean(pts[j + 1] - pts[j])) for j in range(len(spec))])
        if not busy:
            continue
        us = lambda v: round(float(np.mean(v)) / 100.0, 2)  # noqa: E731  (100 MHz ticks)
        line = f"{nm:7s} wait {us(wait):7.2f}  busy {us(busy):7.2f}  span {us(span):7.2f}"
        if ph:
            pm = np.mean(np.array(ph), axis=0) / 100.0
            line += "  | " + "  ".join(f"{n} {v:.2f}" for (n, _), v in zip(phases[nm], pm))
        lines.append(line)
    # d[j]: latest end of stage instance j + 1 minus that of instance j (a
    # stage that ran no task -- the down stage of a folded FFN -- ends where
    # the one before it did, so its delta is 0)
    ends = np.array([[a[s, si][:, 3].max() for si in range(nsi)] for s in range(1, steps)], dtype=np.float64)
    for j in range(1, nsi):
        empty = ends[:, j] == 0
        ends[empty, j] = ends[empty, j - 1]
    d = np.diff(ends, axis=1).mean(axis=0) / 100.0
    per = []
    for k in range(stages_per_layer):
        v = [d[first + l * stages_per_layer + k - 1] for l in range(n_layers)
             if first + l * stages_per_layer + k >= 1]
        per.append(float(np.mean(v)) if v else 0.0)
    lines.append("critical-path deltas per layer (us): " + "  ".join(f"{n} {v:.2f}" for n, v in zip(kinds, per)))
    return lines


def _write(out, lines):
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_summary(path) -> dict:
    """key: value lines of a summary file (values as strings)."""
    res = {}
    if not os.path.exists(path):
        return res
    with open(path) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                res[k.strip()] = v.strip().split()[0] if v.strip() else ""
    return res


def traffic_for(workload, steps, kernel=KERNEL):
    """HBM bytes of one launch of `steps` steps from the committed counter
    summary of this workload: its measured bytes per step (FETCH_SIZE +
    WRITE_SIZE of a profiled launch, scaled by the copy kernel's reading)
    times `steps`.  None when there is no summary or the kernel sources have
    changed since it was taken."""
    s = read_summary(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt"))
    if not s or s.get("workload") != workload:
        return None
    if s.get("source_sha256") != source_hash():
        return None
    per_step = float(s["traffic_bytes_per_step"])
    return {"bytes_per_launch": int(per_step * steps), "bytes_per_step": int(per_step),
            "basis": f"measured {int(per_step)} bytes/step over a profiled launch of {s.get('steps')} steps, "
                     f"times {steps} steps"}


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--out", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--kernel", default=KERNEL)
    a.add_argument("--index", type=int, default=None, help="the dispatch that ran --workload")
    a.add_argument("--workload", default=None)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--out", required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--steps", type=int, required=True)
    b.add_argument("--kernel", default=KERNEL)
    b.add_argument("--index", type=int, default=-1, help="the dispatch that ran --workload (default: last)")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--out", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--kernel", default=KERNEL)
    e = sub.add_parser("l2xcd")
    e.add_argument("dir")
    e.add_argument("--out", required=True)
    e.add_argument("--command", required=True)
    e.add_argument("--kernel", default=KERNEL)
    args = ap.parse_args()
    if args.cmd == "stats":
        summarize_stats(args.dir, args.out, args.command, args.kernel, args.index, args.workload)
    elif args.cmd == "traffic":
        summarize_traffic(args.fetch_dir, args.write_dir, args.out, args.command, args.copy_bytes,
                          args.workload, args.steps, args.kernel, args.index)
    elif args.cmd == "l2xcd":
        summarize_l2_per_xcd(args.dir, args.out, args.command, args.kernel)
    else:
        summarize_counters(args.dir, args.out, args.command, args.kernel)


if __name__ == "__main__":
    main()
