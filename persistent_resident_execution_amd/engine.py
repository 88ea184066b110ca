"""ctypes binding of the C ABI in include/pre.h (argument marshalling only).

Every step of the decode runs in the HIP kernels of libpre.so; this module
only turns torch tensors into device pointers and streams.  It raises if the
library has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os

import torch

from . import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpre.so")
_lib = None

PRE_OK = 0
ERRORS = {-1: "PRE_ERR_ARG", -2: "PRE_ERR_SHAPE", -3: "PRE_ERR_ALIGN", -4: "PRE_ERR_WORKSPACE",
          -5: "PRE_ERR_HIP", -6: "PRE_ERR_UNSUPPORTED", -7: "PRE_ERR_DEVICE", -8: "PRE_ERR_BROKEN",
          -9: "PRE_ERR_CONTEXT", -10: "PRE_ERR_BUSY"}
DEV_ERRORS = {0: "ok", 1: "timeout", 2: "bad token", 3: "nan", 4: "placement", 5: "context"}


class PreError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({lib().pre_strerror(code).decode()})")
        self.code = code


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
        "batch", "max_ctx")] + [("rope_theta", C.c_float), ("rms_eps", C.c_float)] + [
        (n, C.c_int32) for n in ("n_experts", "top_k", "n_shared", "expert_ffn", "expert_dtype",
                                 "grid_wgs", "wg_threads", "attn_splits", "xcd_local", "chunk", "kv_dtype",
                                 "fold_ffn", "fold_attn")]


LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd", "router",
                "e_wg", "e_wu", "e_wd", "e_sg", "e_su", "e_sd", "s_wg", "s_wu", "s_wd", "s_sg",
                "s_su", "s_sd"]


class LayerW(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in LAYER_FIELDS]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(LayerW))]


class KV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("d_ctx_len", C.c_void_p), ("k_scale", C.c_void_p),
                ("v_scale", C.c_void_p)]


class Check(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("hidden", C.c_void_p)]


class Status(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("error", "step", "stage", "slot", "wg")] + [
        ("observed", C.c_uint32), ("expected", C.c_uint32), ("xcc_mismatch", C.c_int32)]


class ServeStats(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("steps", "served", "error")]


class PlanInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_stage_inst", "n_wgs", "n_slots", "n_tasks",
                                         "attn_splits", "validator", "xcd_local", "fold_ffn",
                                         "fold_attn")] + [
        ("workspace_bytes", C.c_int64)]


# Every function the header declares (checked by the CPU test suite).
EXPORTS = ["pre_workspace_size", "pre_engine_create", "pre_engine_create_static", "pre_engine_set_positions",
           "pre_engine_get_positions", "pre_engine_decode", "pre_baseline_decode",
           "pre_engine_status", "pre_engine_reset", "pre_engine_set_watchdog",
           "pre_engine_set_trace", "pre_engine_destroy", "pre_strerror", "pre_plan_describe",
           "pre_plan_validate", "pre_step_bytes", "pre_serve_start", "pre_serve_submit", "pre_serve_poll",
           "pre_serve_stop", "pre_engine_prefill", "pre_engine_verify"]


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
        L.pre_engine_create_static.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.POINTER(KV), vp,
                                               C.POINTER(vp)]
        L.pre_engine_set_positions.argtypes = [vp, C.POINTER(i32)]
        L.pre_engine_get_positions.argtypes = [vp, C.POINTER(i32)]
        for f in (L.pre_engine_decode, L.pre_baseline_decode):
            f.argtypes = [vp, i32, vp, vp, vp, C.POINTER(Check), vp]
        L.pre_engine_prefill.argtypes = [vp, i32, vp, vp, C.POINTER(Check), vp]
        L.pre_engine_verify.argtypes = [vp, i32, vp, vp, vp, C.POINTER(Check), vp]
        L.pre_engine_status.argtypes = [vp, C.POINTER(Status)]
        L.pre_engine_reset.argtypes = [vp, vp]
        L.pre_engine_set_watchdog.argtypes = [vp, C.c_uint32]
        L.pre_engine_set_trace.argtypes = [vp, vp, C.c_size_t]
        L.pre_engine_destroy.argtypes = [vp]
        L.pre_strerror.restype = C.c_char_p
        L.pre_strerror.argtypes = [C.c_int]
        L.pre_plan_describe.argtypes = [C.POINTER(Config), C.POINTER(PlanInfo), vp, i32]
        L.pre_plan_validate.argtypes = [C.POINTER(Config), vp, i32]
        L.pre_serve_start.argtypes = [vp, i32, i32, i32, C.c_uint32, vp, C.POINTER(vp)]
        L.pre_serve_submit.argtypes = [vp, C.POINTER(i32), i32, i32, i32, i32, C.POINTER(i32)]
        L.pre_serve_poll.argtypes = [vp, i32, C.POINTER(i32), i32, C.POINTER(i32), C.POINTER(i32),
                                     C.POINTER(i32)]
        L.pre_serve_stop.argtypes = [vp, C.POINTER(ServeStats)]
        L.pre_step_bytes.restype = C.c_int64
        L.pre_step_bytes.argtypes = [C.POINTER(Config), C.POINTER(i32)]
        # debug entries (not part of the C ABI header)
        debug = {"pre_debug_fp8_decode": [vp, vp, C.c_int, vp], "pre_debug_layout": [vp, vp],
                 "pre_debug_lane_ops": [vp, vp, vp],
                 "pre_debug_gemv": [C.c_int, vp, C.c_int, C.c_int, vp, vp, C.c_int, C.c_int, C.c_int, vp],
                 "pre_debug_copy": [vp, vp, C.c_size_t, vp], "pre_debug_mfma": [vp, vp, vp, vp],
                 "pre_debug_drop_signal": [vp, i32], "pre_debug_fp8_encode": [vp, vp, C.c_int, vp]}
        for name, at in debug.items():
            if hasattr(L, name):
                getattr(L, name).argtypes = at
        _lib = L
    return _lib


def make_config(m: synth.ModelConfig, grid_wgs=0, wg_threads=0, attn_splits=0, xcd_local=0, chunk=0,
                fold_ffn=0, fold_attn=0) -> Config:
    c = Config()
    for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
              "batch", "max_ctx", "n_experts", "top_k", "n_shared", "expert_ffn"):
        setattr(c, n, int(getattr(m, n)))
    c.rope_theta = float(m.rope_theta)
    c.rms_eps = float(m.rms_eps)
    c.expert_dtype = 1 if m.is_moe else 0
    c.grid_wgs, c.wg_threads, c.attn_splits = int(grid_wgs), int(wg_threads), int(attn_splits)
    c.xcd_local = int(xcd_local)
    c.chunk = int(chunk)
    c.kv_dtype = 1 if getattr(m, "kv_fp8", False) else 0
    c.fold_ffn = int(fold_ffn)
    c.fold_attn = int(fold_attn)
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


# ---- argument checks ----------------------------------------------------------
# The C ABI receives raw device pointers and cannot tell a host tensor, a wrong
# dtype or a short buffer from a good one; any of these would make a kernel
# read or write out of bounds.  Every tensor is checked here before a call.

def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def check_tensor(t, name, dtype, shape=None, numel=None, device_type="cuda"):
    """t must be a contiguous tensor of `dtype` on a `device_type` device,
    of exactly `shape` (if given) and at least `numel` elements (if given)."""
    _need(torch.is_tensor(t), f"{name}: expected a tensor, got {type(t).__name__}")
    _need(t.device.type == device_type, f"{name}: on {t.device}, expected a {device_type} tensor")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    _need(t.dtype in dts, f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dts))}")
    _need(t.is_contiguous(), f"{name}: not contiguous")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None:
        _need(t.numel() >= numel, f"{name}: {t.numel()} elements, needs at least {numel}")


FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


def weight_shapes(m: synth.ModelConfig) -> dict:
    """Expected (dtype, shape) of every weight tensor (top level and per layer)."""
    h, d, bf = m.hidden, m.head_dim, torch.bfloat16
    top = {"embed": (bf, (m.vocab, h)), "final_norm": (bf, (h,)), "lm_head": (bf, (m.vocab, h))}
    lay = {"attn_norm": (bf, (h,)), "wq": (bf, (m.n_q_heads * d, h)), "wk": (bf, (m.n_kv_heads * d, h)),
           "wv": (bf, (m.n_kv_heads * d, h)), "wo": (bf, (h, m.n_q_heads * d)), "ffn_norm": (bf, (h,))}
    if m.is_moe:
        f, E, S = m.expert_ffn, m.n_experts, m.n_shared
        fb, hb = (f + 127) // 128, (h + 127) // 128
        lay["router"] = (bf, (E, h))
        for pre, n in (("e_", E), ("s_", S)):
            if n == 0:
                continue
            lay[pre + "wg"] = (FP8_DTYPES, (n, f, h))
            lay[pre + "wu"] = (FP8_DTYPES, (n, f, h))
            lay[pre + "wd"] = (FP8_DTYPES, (n, h, f))
            lay[pre + "sg"] = (bf, (n, fb, hb))
            lay[pre + "su"] = (bf, (n, fb, hb))
            lay[pre + "sd"] = (bf, (n, hb, fb))
    else:
        f = m.ffn_dim
        lay.update({"wg": (bf, (f, h)), "wu": (bf, (f, h)), "wd": (bf, (h, f))})
    return {"top": top, "layer": lay}


def check_model_args(m: synth.ModelConfig, weights: dict, k_cache, v_cache, ctx_len=None,
                     device_type="cuda", k_scale=None, v_scale=None):
    """Weights, cache (and its row scales, for an fp8 cache) and position
    array of an engine, before create."""
    ws = weight_shapes(m)
    for n, (dt, sh) in ws["top"].items():
        check_tensor(weights.get(n), n, dt, shape=sh, device_type=device_type)
    _need(len(weights.get("layers", [])) == m.n_layers, f"weights: {m.n_layers} layers expected")
    for l, lw in enumerate(weights["layers"]):
        for n, (dt, sh) in ws["layer"].items():
            check_tensor(lw.get(n), f"layers[{l}].{n}", dt, shape=sh, device_type=device_type)
    kv_shape = (m.n_layers, m.batch, m.n_kv_heads, m.max_ctx, m.head_dim)
    kv_dt = torch.uint8 if m.kv_fp8 else torch.bfloat16
    check_tensor(k_cache, "k_cache", kv_dt, shape=kv_shape, device_type=device_type)
    check_tensor(v_cache, "v_cache", kv_dt, shape=kv_shape, device_type=device_type)
    if m.kv_fp8:
        check_tensor(k_scale, "k_scale", torch.float32, shape=kv_shape[:4], device_type=device_type)
        check_tensor(v_scale, "v_scale", torch.float32, shape=kv_shape[:4], device_type=device_type)
    else:
        _need(k_scale is None and v_scale is None, "k_scale / v_scale are for an fp8 cache only")
    if ctx_len is not None:
        check_tensor(ctx_len, "ctx_len", torch.int32, shape=(m.batch,), device_type=device_type)


def check_decode_args(m: synth.ModelConfig, n_steps, in_tokens, forced, out_tokens, logits, hidden,
                      device_type="cuda"):
    """The buffers of one decode call, sized for n_steps steps of m.batch sequences."""
    _need(isinstance(n_steps, int) and n_steps >= 0, f"n_steps: {n_steps!r} is not a count")
    if n_steps == 0:
        return
    B = m.batch
    _need(in_tokens is not None or forced is not None, "in_tokens or forced is required")
    if in_tokens is not None:
        check_tensor(in_tokens, "in_tokens", torch.int32, numel=B, device_type=device_type)
    if forced is not None:
        check_tensor(forced, "forced", torch.int32, numel=n_steps * B, device_type=device_type)
    check_tensor(out_tokens, "out_tokens", torch.int32, numel=n_steps * B, device_type=device_type)
    if logits is not None:
        check_tensor(logits, "logits", torch.float32, numel=n_steps * B * m.vocab, device_type=device_type)
    if hidden is not None:
        check_tensor(hidden, "hidden", torch.float32, numel=n_steps * B * m.hidden, device_type=device_type)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


class Engine:
    """A decode engine bound to device weights and a KV cache (torch tensors).

    weights: the nested dict of ``synth.gen_weights`` (device tensors);
    k_cache, v_cache: bf16 [n_layers][batch][n_kv_heads][max_ctx][head_dim].
    """

    def __init__(self, m: synth.ModelConfig, weights: dict, k_cache, v_cache, grid_wgs=0,
                 wg_threads=0, attn_splits=0, stream=None, xcd_local=0, ctx_len=None,
                 static_workspace=False, chunk=0, k_scale=None, v_scale=None, fold_ffn=0,
                 fold_attn=0):
        """static_workspace: create with pre_engine_create_static (the
        library's static device workspace; no allocation) instead of a
        workspace tensor.  fold_ffn: 0 = fold the down projection into the
        gate/up stage where the engine supports it (small one-XCD dense
        models), -1 = never.  fold_attn: 0 = each output-projection task
        computes its KV head's attention itself where supported (small
        one-XCD batch-1 engines, bf16 cache), -1 = never."""
        self.m = m
        self.h = None
        check_model_args(m, weights, k_cache, v_cache, ctx_len, k_scale=k_scale, v_scale=v_scale)
        dev = k_cache.device
        for t in [weights["embed"], v_cache] + ([ctx_len] if ctx_len is not None else []):
            _need(t.device == dev, f"every tensor must be on {dev}, found one on {t.device}")
        self.device = dev
        self.cfg = make_config(m, grid_wgs, wg_threads, attn_splits, xcd_local, chunk, fold_ffn, fold_attn)
        self.chunk = int(chunk)
        L = lib()
        nbytes = C.c_size_t()
        _check(L.pre_workspace_size(C.byref(self.cfg), C.byref(nbytes)), "workspace_size")
        self.workspace = None if static_workspace else torch.empty(int(nbytes.value), dtype=torch.uint8,
                                                                   device=dev)
        self.ctx_len = ctx_len
        self._keep = [weights, k_cache, v_cache, ctx_len, k_scale, v_scale]
        self.layers = (LayerW * m.n_layers)()
        for l, lw in enumerate(weights["layers"]):
            for n in LAYER_FIELDS:
                t = lw.get(n)
                if t is not None:
                    setattr(self.layers[l], n, t.data_ptr())
        self.w = Weights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                         weights["lm_head"].data_ptr(), self.layers)
        self.kv = KV(k_cache.data_ptr(), v_cache.data_ptr(),
                     ctx_len.data_ptr() if ctx_len is not None else None,
                     k_scale.data_ptr() if k_scale is not None else None,
                     v_scale.data_ptr() if v_scale is not None else None)
        h = C.c_void_p()
        if static_workspace:
            _check(L.pre_engine_create_static(C.byref(self.cfg), C.byref(self.w), C.byref(self.kv),
                                              _stream(stream), C.byref(h)), "engine_create_static")
        else:
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
        _need(self.h is not None, "engine is closed")
        check_decode_args(self.m, n_steps, in_tokens, forced, out_tokens, logits, hidden)
        dev = self.device
        for t in (in_tokens, forced, out_tokens, logits, hidden):
            _need(t is None or t.device == dev, f"every buffer must be on {dev}, found one on "
                                                f"{None if t is None else t.device}")
        chk = Check(logits.data_ptr() if logits is not None else None,
                    hidden.data_ptr() if hidden is not None else None)
        _check(fn(self.h, int(n_steps), _ptr(in_tokens), _ptr(forced), _ptr(out_tokens),
                  C.byref(chk), _stream(stream)), fn.__name__)

    def decode(self, n_steps, in_tokens=None, forced=None, out_tokens=None, logits=None,
               hidden=None, stream=None):
        """One persistent launch of n_steps; returns out_tokens [n_steps, batch] (int32)."""
        if out_tokens is None:
            out_tokens = torch.empty((n_steps, self.m.batch), dtype=torch.int32,
                                     device=self.device)
        self._run(lib().pre_engine_decode, n_steps, in_tokens, forced, out_tokens, logits, hidden,
                  stream)
        return out_tokens

    def baseline_decode(self, n_steps, in_tokens=None, forced=None, out_tokens=None, logits=None,
                        hidden=None, stream=None):
        if out_tokens is None:
            out_tokens = torch.empty((n_steps, self.m.batch), dtype=torch.int32,
                                     device=self.device)
        self._run(lib().pre_baseline_decode, n_steps, in_tokens, forced, out_tokens, logits,
                  hidden, stream)
        return out_tokens

    def prefill(self, tokens, out_tokens=None, logits=None, hidden=None, stream=None):
        """Prefill through the chunk task set (pre_engine_prefill): tokens
        int32 [n] on the device; returns the greedy successor of each token
        (int32 [n]; the last one is the first generated token)."""
        _need(self.h is not None, "engine is closed")
        n = int(tokens.numel())
        if out_tokens is None:
            out_tokens = torch.empty(n, dtype=torch.int32, device=self.device)
        mm = dataclasses.replace(self.m, batch=1)
        check_tensor(tokens, "tokens", torch.int32, numel=n)
        check_decode_args(mm, n, None, tokens, out_tokens, logits, hidden)
        for t in (tokens, out_tokens, logits, hidden):
            _need(t is None or t.device == self.device, f"every buffer must be on {self.device}")
        chk = Check(_ptr(logits), _ptr(hidden))
        _check(lib().pre_engine_prefill(self.h, n, _ptr(tokens), _ptr(out_tokens), C.byref(chk), _stream(stream)),
               "engine_prefill")
        return out_tokens

    def verify(self, tokens, out_tokens=None, accepted=None, logits=None, stream=None):
        """Speculative verify (pre_engine_verify): tokens int32 [1 + k] on the
        device (the current token, then k drafts); returns (greedy successors
        [1 + k], accepted count [1]) as device tensors."""
        _need(self.h is not None, "engine is closed")
        n = int(tokens.numel())
        if out_tokens is None:
            out_tokens = torch.empty(n, dtype=torch.int32, device=self.device)
        if accepted is None:
            accepted = torch.empty(1, dtype=torch.int32, device=self.device)
        mm = dataclasses.replace(self.m, batch=1)
        check_tensor(tokens, "tokens", torch.int32, numel=n)
        check_decode_args(mm, n, None, tokens, out_tokens, logits, None)
        check_tensor(accepted, "accepted", torch.int32, numel=1)
        chk = Check(_ptr(logits), None)
        _check(lib().pre_engine_verify(self.h, n - 1, _ptr(tokens), _ptr(out_tokens), _ptr(accepted),
                                       C.byref(chk), _stream(stream)), "engine_verify")
        return out_tokens, accepted

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

    def debug_drop_signal(self, slot):
        """Debug: the task setting ready flag `slot` skips the store from the
        next call on (-1: off) -- drives the watchdog path."""
        _check(lib().pre_debug_drop_signal(self.h, int(slot)), "debug_drop_signal")

    LAYOUT = ["status", "flags", "layers", "tasks", "rope", "xcc", "x_out", "pbuf", "q", "u", "rl",
              "part", "lmp", "x_emb", "a_norm", "tok", "xmid", "pk", "ssq", "ctx", "kvnew", "total"]

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


class Server:
    """The serving loop of an engine (pre_serve_*): one resident launch that
    takes requests from a ring in host memory until stop().  submit / poll /
    wait touch host memory only; no GPU work of the device may be waited on
    while the loop runs (it holds every CU)."""

    def __init__(self, eng: Engine, n_slots=8, max_prompt=256, max_out=256, idle_ms=10000, stream=None):
        self.eng, self.max_out = eng, int(max_out)
        self.h = None
        h = C.c_void_p()
        _check(lib().pre_serve_start(eng.h, int(n_slots), int(max_prompt), int(max_out), int(idle_ms),
                                     _stream(stream), C.byref(h)), "serve_start")
        self.h = h

    def submit(self, prompt, pos=0, budget=16, eos=-1):
        """Queue a request; returns its slot."""
        toks = [int(t) for t in prompt]
        arr = (C.c_int32 * len(toks))(*toks)
        slot = C.c_int32()
        _check(lib().pre_serve_submit(self.h, arr, len(toks), int(pos), int(budget), int(eos),
                                      C.byref(slot)), "serve_submit")
        return slot.value

    def poll(self, slot):
        """(tokens so far, done, request error)."""
        buf = (C.c_int32 * self.max_out)()
        n, done, err = C.c_int32(), C.c_int32(), C.c_int32()
        _check(lib().pre_serve_poll(self.h, int(slot), buf, self.max_out, C.byref(n), C.byref(done),
                                    C.byref(err)), "serve_poll")
        return list(buf[:min(n.value, self.max_out)]), bool(done.value), err.value

    def wait(self, slot, timeout_s=60.0):
        """Poll until the request is done; returns (tokens, request error)."""
        import time
        t0 = time.time()
        while True:
            toks, done, err = self.poll(slot)
            if done:
                return toks, err
            if time.time() - t0 > timeout_s:
                raise TimeoutError(f"request in slot {slot} not done after {timeout_s}s ({len(toks)} tokens)")
            time.sleep(0.0005)

    def stop(self):
        """End the loop; returns its counts (steps, served, error)."""
        if self.h is None:
            return None
        st = ServeStats()
        h, self.h = self.h, None
        _check(lib().pre_serve_stop(h, C.byref(st)), "serve_stop")
        return {"steps": st.steps, "served": st.served, "error": st.error}

    def __del__(self):
        try:
            self.stop()
        except Exception:
            pass


def fp8_decode_table(device="cuda"):
    """The kernels' fp8 unpacking applied to all 256 codes (debug entry)."""
    codes = torch.arange(256, dtype=torch.uint8, device=device)
    out = torch.empty(256, dtype=torch.float32, device=device)
    _check(lib().pre_debug_fp8_decode(_ptr(codes), _ptr(out), 256, _stream()), "fp8_decode")
    torch.cuda.synchronize()
    return out.cpu()


def fp8_encode(values):
    """The fp8 cache's e4m3 encoder applied on the device to fp32 values
    (debug entry); returns the codes on the host."""
    x = torch.as_tensor(values, dtype=torch.float32).to("cuda").contiguous()
    out = torch.zeros(x.numel(), dtype=torch.uint8, device="cuda")
    _check(lib().pre_debug_fp8_encode(_ptr(x), _ptr(out), x.numel(), _stream()), "fp8_encode")
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
