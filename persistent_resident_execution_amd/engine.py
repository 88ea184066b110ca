"""ctypes binding of the C ABI in include/pre.h (argument marshalling only).

Every step of the decode runs in the HIP kernels of libpre.so; this module
only turns torch tensors into device pointers and streams.  It raises if the
library has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from . import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpre.so")
_lib = None

PRE_OK = 0
ERRORS = {-1: "PRE_ERR_ARG", -2: "PRE_ERR_SHAPE", -3: "PRE_ERR_ALIGN", -4: "PRE_ERR_WORKSPACE",
          -5: "PRE_ERR_HIP", -6: "PRE_ERR_UNSUPPORTED", -7: "PRE_ERR_DEVICE", -8: "PRE_ERR_BROKEN",
          -9: "PRE_ERR_CONTEXT"}
DEV_ERRORS = {0: "ok", 1: "timeout", 2: "bad token", 3: "nan"}


class PreError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({lib().pre_strerror(code).decode()})")
        self.code = code


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
        "batch", "max_ctx")] + [("rope_theta", C.c_float), ("rms_eps", C.c_float)] + [
        (n, C.c_int32) for n in ("n_experts", "top_k", "n_shared", "expert_ffn", "expert_dtype",
                                 "grid_wgs", "wg_threads", "attn_splits", "xcd_local")]


LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd", "router",
                "e_wg", "e_wu", "e_wd", "e_sg", "e_su", "e_sd", "s_wg", "s_wu", "s_wd", "s_sg",
                "s_su", "s_sd"]


class LayerW(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in LAYER_FIELDS]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(LayerW))]


class KV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p)]


class Check(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("hidden", C.c_void_p)]


class Status(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("error", "step", "stage", "slot", "wg")] + [
        ("observed", C.c_uint32), ("expected", C.c_uint32), ("xcc_mismatch", C.c_int32)]


class PlanInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_stage_inst", "n_wgs", "n_slots", "n_tasks",
                                         "attn_splits", "validator", "xcd_local")] + [
        ("workspace_bytes", C.c_int64)]


# Every function the header declares (checked by the CPU test suite).
EXPORTS = ["pre_workspace_size", "pre_engine_create", "pre_engine_set_positions",
           "pre_engine_get_positions", "pre_engine_decode", "pre_baseline_decode",
           "pre_engine_status", "pre_engine_reset", "pre_engine_set_watchdog",
           "pre_engine_set_trace", "pre_engine_destroy", "pre_strerror", "pre_plan_describe",
           "pre_plan_validate", "pre_step_bytes"]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run persistent_resident_execution_amd.build")
        L = C.CDLL(LIB_PATH)
        vp, i32 = C.c_void_p, C.c_int32
        L.pre_workspace_size.argtypes = [C.POINTER(Config), C.POINTER(C.c_size_t)]
        L.pre_engine_create.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.POINTER(KV), vp,
                                        C.c_size_t, vp, C.POINTER(vp)]
        L.pre_engine_set_positions.argtypes = [vp, C.POINTER(i32)]
        L.pre_engine_get_positions.argtypes = [vp, C.POINTER(i32)]
        for f in (L.pre_engine_decode, L.pre_baseline_decode):
            f.argtypes = [vp, i32, vp, vp, vp, C.POINTER(Check), vp]
        L.pre_engine_status.argtypes = [vp, C.POINTER(Status)]
        L.pre_engine_reset.argtypes = [vp, vp]
        L.pre_engine_set_watchdog.argtypes = [vp, C.c_uint32]
        L.pre_engine_set_trace.argtypes = [vp, vp, C.c_size_t]
        L.pre_engine_destroy.argtypes = [vp]
        L.pre_strerror.restype = C.c_char_p
        L.pre_strerror.argtypes = [C.c_int]
        L.pre_plan_describe.argtypes = [C.POINTER(Config), C.POINTER(PlanInfo), vp, i32]
        L.pre_plan_validate.argtypes = [C.POINTER(Config), vp, i32]
        L.pre_step_bytes.restype = C.c_int64
        L.pre_step_bytes.argtypes = [C.POINTER(Config), C.POINTER(i32)]
        # debug entries (not part of the C ABI header)
        debug = {"pre_debug_fp8_decode": [vp, vp, C.c_int, vp], "pre_debug_layout": [vp, vp],
                 "pre_debug_lane_ops": [vp, vp, vp],
                 "pre_debug_gemv": [C.c_int, vp, C.c_int, C.c_int, vp, vp, C.c_int, C.c_int, C.c_int, vp],
                 "pre_debug_copy": [vp, vp, C.c_size_t, vp], "pre_debug_mfma": [vp, vp, vp, vp]}
        for name, at in debug.items():
            if hasattr(L, name):
                getattr(L, name).argtypes = at
        _lib = L
    return _lib


def make_config(m: synth.ModelConfig, grid_wgs=0, wg_threads=0, attn_splits=0, xcd_local=0) -> Config:
    c = Config()
    for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
              "batch", "max_ctx", "n_experts", "top_k", "n_shared", "expert_ffn"):
        setattr(c, n, int(getattr(m, n)))
    c.rope_theta = float(m.rope_theta)
    c.rms_eps = float(m.rms_eps)
    c.expert_dtype = 1 if m.is_moe else 0
    c.grid_wgs, c.wg_threads, c.attn_splits = int(grid_wgs), int(wg_threads), int(attn_splits)
    c.xcd_local = int(xcd_local)
    return c


def _check(rc, what):
    if rc != PRE_OK:
        raise PreError(rc, what)


def plan_describe(m: synth.ModelConfig, with_tasks=False, **kw):
    import numpy as np
    cfg = make_config(m, **kw)
    info = PlanInfo()
    _check(lib().pre_plan_describe(C.byref(cfg), C.byref(info), None, 0), "plan_describe")
    tasks = None
    if with_tasks:
        tasks = np.zeros((info.n_tasks, 8), np.int32)
        _check(lib().pre_plan_describe(C.byref(cfg), C.byref(info),
                                       C.c_void_p(tasks.ctypes.data), info.n_tasks), "plan_describe")
    return info, tasks


def plan_validate(m: synth.ModelConfig, tasks, **kw) -> int:
    import numpy as np
    cfg = make_config(m, **kw)
    t = np.ascontiguousarray(tasks, dtype=np.int32)
    return int(lib().pre_plan_validate(C.byref(cfg), C.c_void_p(t.ctypes.data), t.shape[0]))


def step_bytes(m: synth.ModelConfig, positions) -> int:
    cfg = make_config(m)
    pos = (C.c_int32 * m.batch)(*[int(p) for p in positions])
    return int(lib().pre_step_bytes(C.byref(cfg), pos))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


class Engine:
    """A decode engine bound to device weights and a KV cache (torch tensors).

    weights: the nested dict of ``synth.gen_weights`` (device tensors);
    k_cache, v_cache: bf16 [n_layers][batch][n_kv_heads][max_ctx][head_dim].
    """

    def __init__(self, m: synth.ModelConfig, weights: dict, k_cache, v_cache, grid_wgs=0,
                 wg_threads=0, attn_splits=0, stream=None, xcd_local=0):
        self.m = m
        self.cfg = make_config(m, grid_wgs, wg_threads, attn_splits, xcd_local)
        L = lib()
        nbytes = C.c_size_t()
        _check(L.pre_workspace_size(C.byref(self.cfg), C.byref(nbytes)), "workspace_size")
        dev = k_cache.device
        self.workspace = torch.empty(int(nbytes.value), dtype=torch.uint8, device=dev)
        self._keep = [weights, k_cache, v_cache]
        self.layers = (LayerW * m.n_layers)()
        for l, lw in enumerate(weights["layers"]):
            for n in LAYER_FIELDS:
                t = lw.get(n)
                if t is not None:
                    setattr(self.layers[l], n, t.data_ptr())
        self.w = Weights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                         weights["lm_head"].data_ptr(), self.layers)
        self.kv = KV(k_cache.data_ptr(), v_cache.data_ptr())
        h = C.c_void_p()
        _check(L.pre_engine_create(C.byref(self.cfg), C.byref(self.w), C.byref(self.kv),
                                   C.c_void_p(self.workspace.data_ptr()), nbytes.value,
                                   _stream(stream), C.byref(h)), "engine_create")
        self.h = h

    # -- positions -----------------------------------------------------------
    def set_positions(self, pos):
        arr = (C.c_int32 * self.m.batch)(*[int(p) for p in pos])
        _check(lib().pre_engine_set_positions(self.h, arr), "set_positions")

    def positions(self):
        arr = (C.c_int32 * self.m.batch)()
        _check(lib().pre_engine_get_positions(self.h, arr), "get_positions")
        return list(arr)

    # -- decode ----------------------------------------------------------------
    def _run(self, fn, n_steps, in_tokens, forced, out_tokens, logits, hidden, stream):
        chk = Check(logits.data_ptr() if logits is not None else None,
                    hidden.data_ptr() if hidden is not None else None)
        _check(fn(self.h, int(n_steps), _ptr(in_tokens), _ptr(forced), _ptr(out_tokens),
                  C.byref(chk), _stream(stream)), fn.__name__)

    def decode(self, n_steps, in_tokens=None, forced=None, out_tokens=None, logits=None,
               hidden=None, stream=None):
        """One persistent launch of n_steps; returns out_tokens [n_steps, batch] (int32)."""
        if out_tokens is None:
            out_tokens = torch.empty((n_steps, self.m.batch), dtype=torch.int32,
                                     device=self.workspace.device)
        self._run(lib().pre_engine_decode, n_steps, in_tokens, forced, out_tokens, logits, hidden,
                  stream)
        return out_tokens

    def baseline_decode(self, n_steps, in_tokens=None, forced=None, out_tokens=None, logits=None,
                        hidden=None, stream=None):
        if out_tokens is None:
            out_tokens = torch.empty((n_steps, self.m.batch), dtype=torch.int32,
                                     device=self.workspace.device)
        self._run(lib().pre_baseline_decode, n_steps, in_tokens, forced, out_tokens, logits,
                  hidden, stream)
        return out_tokens

    def status(self, raise_on_error=True):
        st = Status()
        rc = lib().pre_engine_status(self.h, C.byref(st))
        d = {f: getattr(st, f) for f, _ in Status._fields_}
        if rc != PRE_OK and raise_on_error:
            raise PreError(rc, f"device status {DEV_ERRORS.get(st.error, st.error)} {d}")
        return d

    def reset(self, stream=None):
        _check(lib().pre_engine_reset(self.h, _stream(stream)), "reset")

    def set_watchdog(self, ms):
        _check(lib().pre_engine_set_watchdog(self.h, int(ms)), "set_watchdog")

    def set_trace(self, buf):
        _check(lib().pre_engine_set_trace(self.h, _ptr(buf), 0 if buf is None else buf.numel() *
                                          buf.element_size()), "set_trace")

    LAYOUT = ["status", "flags", "layers", "tasks", "rope", "xcc", "x_out", "pbuf", "q", "u", "rl",
              "part", "lmp", "x_emb", "a_norm", "tok", "xmid", "pk", "ssq", "total"]

    def debug_slot(self, name, count, dtype=torch.float32, offset=0):
        """A view of a workspace region (debugging)."""
        import numpy as np
        off = np.zeros(len(self.LAYOUT), np.int64)
        _check(lib().pre_debug_layout(self.h, C.c_void_p(off.ctypes.data)), "debug_layout")
        start = int(off[self.LAYOUT.index(name)]) + offset
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.workspace[start:start + count * esz].view(dtype)

    def close(self):
        if getattr(self, "h", None):
            lib().pre_engine_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fp8_decode_table(device="cuda"):
    """The kernels' fp8 unpacking applied to all 256 codes (debug entry)."""
    codes = torch.arange(256, dtype=torch.uint8, device=device)
    out = torch.empty(256, dtype=torch.float32, device=device)
    _check(lib().pre_debug_fp8_decode(_ptr(codes), _ptr(out), 256, _stream()), "fp8_decode")
    torch.cuda.synchronize()
    return out.cpu()


def debug_gemv(variant, W, x, y, grid=256, threads=512, lds_min=96 * 1024):
    """Tuning entry: y = W x with the streamed GEMV variant (see pre_debug_gemv)."""
    rows, K = W.shape
    _check(lib().pre_debug_gemv(int(variant), _ptr(W), rows, K, _ptr(x), _ptr(y), int(grid),
                                int(threads), int(lds_min), _stream()), "debug_gemv")


def debug_lane_ops(x):
    """Wavefront primitives applied to 64 floats (debug entry pre_debug_lane_ops)."""
    inp = x.to(device="cuda", dtype=torch.float32).contiguous()
    out = torch.zeros(320, dtype=torch.float32, device="cuda")
    _check(lib().pre_debug_lane_ops(_ptr(inp), _ptr(out), _stream()), "debug_lane_ops")
    torch.cuda.synchronize()
    return out.cpu()


def debug_copy(src, dst):
    """dst[:] = src[:] with the library's plain copy kernel (byte counts must
    match and be a multiple of 16); the reference for traffic counters."""
    n = src.numel() * src.element_size()
    assert n == dst.numel() * dst.element_size() and n % 16 == 0
    _check(lib().pre_debug_copy(_ptr(src), _ptr(dst), n, _stream()), "debug_copy")


def debug_mfma(a, b):
    """A (16 x 32) @ B (32 x 16), bf16 in, fp32 out, through the matrix-core
    instruction with the operand lane layout the micro-batch GEMMs use."""
    A = a.to(device="cuda", dtype=torch.bfloat16).contiguous()
    Bm = b.to(device="cuda", dtype=torch.bfloat16).contiguous()
    assert A.shape == (16, 32) and Bm.shape == (32, 16)
    out = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    _check(lib().pre_debug_mfma(_ptr(A), _ptr(Bm), _ptr(out), _stream()), "debug_mfma")
    torch.cuda.synchronize()
    return out.cpu()
