"""CPU oracle of the decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU engine never imports, links or
calls it, and the two share no code: the only thing both sides consume is the
seeded synthetic input (weights, tokens) built by
``persistent_resident_execution_amd.synth``.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one sequential sum per
dot product); this module only compiles it with gcc and marshals numpy
arrays through ctypes.  Readings of the pages are listed in ``oracle.h``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrcConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim",
        "vocab", "max_ctx")] + [("rope_theta", C.c_double), ("rms_eps", C.c_double)] + [
        (n, C.c_int32) for n in ("n_experts", "top_k", "n_shared", "expert_ffn")]


_LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd",
                 "router", "e_wg", "e_wu", "e_wd", "e_sg", "e_su", "e_sd",
                 "s_wg", "s_wu", "s_wd", "s_sg", "s_su", "s_sd"]


class OrcLayer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _LAYER_FIELDS]


class OrcKV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("k_scale", C.c_void_p), ("v_scale", C.c_void_p),
                ("layer_stride", C.c_int64), ("scale_layer_stride", C.c_int64), ("fp8", C.c_int32)]


class OrcWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(OrcLayer))]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = C.CDLL(_LIB)
        dp, vp, i32, i64 = C.POINTER(C.c_double), C.c_void_p, C.c_int, C.c_int64
        L.orc_bf16_to_double.restype = C.c_double
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_float_to_bf16.restype = C.c_uint16
        L.orc_float_to_bf16.argtypes = [C.c_float]
        L.orc_fp8e4m3_to_double.restype = C.c_double
        L.orc_fp8e4m3_to_double.argtypes = [C.c_uint8]
        L.orc_silu.restype = C.c_double
        L.orc_silu.argtypes = [C.c_double]
        L.orc_rmsnorm.argtypes = [dp, vp, i32, C.c_double, dp]
        L.orc_gemv_bf16.argtypes = [vp, i32, i32, dp, dp]
        L.orc_gemv_fp8.argtypes = [vp, vp, i32, i32, dp, dp]
        L.orc_rope.argtypes = [dp, i32, i32, C.c_double]
        L.orc_softmax.argtypes = [dp, i32, dp]
        L.orc_attend.argtypes = [dp, vp, vp, i32, i32, dp]
        L.orc_argmax.restype = C.c_int
        L.orc_argmax.argtypes = [dp, i32]
        L.orc_topk.argtypes = [dp, i32, i32, vp]
        L.orc_moe_ffn.argtypes = [C.POINTER(OrcConfig), C.POINTER(OrcLayer), dp, dp, vp, dp]
        L.orc_decode_step.restype = C.c_int
        L.orc_decode_step.argtypes = [C.POINTER(OrcConfig), C.POINTER(OrcWeights), vp, vp, i64,
                                      i32, i32, dp, dp]
        L.orc_forward_full.restype = C.c_int
        L.orc_forward_full.argtypes = [C.POINTER(OrcConfig), C.POINTER(OrcWeights), vp, i32, dp, dp]
        L.orc_prefill.restype = C.c_int
        L.orc_prefill.argtypes = [C.POINTER(OrcConfig), C.POINTER(OrcWeights), vp, vp, i64, vp, i32]
        L.orc_float_to_fp8e4m3.restype = C.c_uint8
        L.orc_float_to_fp8e4m3.argtypes = [C.c_float]
        L.orc_quantize_row_fp8.argtypes = [vp, i32, vp, vp]
        L.orc_attend_fp8.argtypes = [dp, vp, vp, vp, vp, i32, i32, dp]
        L.orc_decode_step_kv.restype = C.c_int
        L.orc_decode_step_kv.argtypes = [C.POINTER(OrcConfig), C.POINTER(OrcWeights), C.POINTER(OrcKV), i32,
                                         i32, dp, dp]
        L.orc_num_threads.restype = C.c_int
        L.orc_set_num_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _dp(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _vp(a):
    if a is None:
        return None
    assert a.flags.c_contiguous, "oracle inputs must be C-contiguous"
    return C.c_void_p(a.ctypes.data)


# ---- primitives (used by the pins) ------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_bf16_to_double(int(v)) for v in b], dtype=np.float64)


def f32_to_bf16(vals) -> np.ndarray:
    L = lib()
    v = np.asarray(vals, dtype=np.float32).ravel()
    return np.array([L.orc_float_to_bf16(float(x)) for x in v], dtype=np.uint16)


def fp8_to_f64(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_fp8e4m3_to_double(int(x)) for x in c], dtype=np.float64)


def f32_to_fp8(vals) -> np.ndarray:
    L = lib()
    v = np.asarray(vals, dtype=np.float32).ravel()
    return np.array([L.orc_float_to_fp8e4m3(float(x)) for x in v], dtype=np.uint8)


def quantize_row_fp8(x):
    """(codes uint8 [n], fp32 scale) of one cached row."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.size, np.uint8)
    sc = np.empty(1, np.float32)
    lib().orc_quantize_row_fp8(_vp(x), x.size, _vp(codes), _vp(sc))
    return codes, float(sc[0])


def attend_fp8(q, Kc, Ks, Vc, Vs):
    q = np.ascontiguousarray(q, dtype=np.float64)
    Kc, Vc = np.ascontiguousarray(Kc, dtype=np.uint8), np.ascontiguousarray(Vc, dtype=np.uint8)
    Ks, Vs = np.ascontiguousarray(Ks, dtype=np.float32), np.ascontiguousarray(Vs, dtype=np.float32)
    n, d = Kc.shape
    o = np.empty(d, dtype=np.float64)
    lib().orc_attend_fp8(_dp(q), _vp(Kc), _vp(Ks), _vp(Vc), _vp(Vs), n, d, _dp(o))
    return o


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def rmsnorm(x, g_bits, eps):
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_dp(x), _vp(g), x.size, float(eps), _dp(out))
    return out


def gemv_bf16(W_bits, x):
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float64)
    m, k = W.shape
    y = np.empty(m, dtype=np.float64)
    lib().orc_gemv_bf16(_vp(W), m, k, _dp(x), _dp(y))
    return y


def gemv_fp8(Q, scales_bits, x):
    Q = np.ascontiguousarray(Q, dtype=np.uint8)
    S = np.ascontiguousarray(scales_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float64)
    m, k = Q.shape
    y = np.empty(m, dtype=np.float64)
    lib().orc_gemv_fp8(_vp(Q), _vp(S), m, k, _dp(x), _dp(y))
    return y


def rope(v, pos, theta):
    v = np.array(v, dtype=np.float64, copy=True)
    lib().orc_rope(_dp(v), v.size, int(pos), float(theta))
    return v


def softmax(s):
    s = np.ascontiguousarray(s, dtype=np.float64)
    p = np.empty_like(s)
    lib().orc_softmax(_dp(s), s.size, _dp(p))
    return p


def attend(q, K_bits, V_bits):
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K_bits, dtype=np.uint16)
    V = np.ascontiguousarray(V_bits, dtype=np.uint16)
    n, d = K.shape
    o = np.empty(d, dtype=np.float64)
    lib().orc_attend(_dp(q), _vp(K), _vp(V), n, d, _dp(o))
    return o


def argmax(v) -> int:
    v = np.ascontiguousarray(v, dtype=np.float64)
    return int(lib().orc_argmax(_dp(v), v.size))


def topk(p, k):
    p = np.ascontiguousarray(p, dtype=np.float64)
    idx = np.empty(k, dtype=np.int32)
    lib().orc_topk(_dp(p), p.size, k, _vp(idx))
    return idx


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


# ---- whole model --------------------------------------------------------------

@dataclass
class _Keep:
    arrays: list


class OracleModel:
    """Binds host weight arrays (numpy, raw bf16/fp8 bits) to the C oracle.

    ``cfg`` is any object with the fields of the model config; ``weights`` is the
    nested dict produced by ``synth.weights_to_numpy``.
    """

    def __init__(self, cfg, weights: dict):
        self.cfg = cfg
        self._keep = _Keep([])
        c = OrcConfig()
        for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim",
                  "vocab", "max_ctx", "n_experts", "top_k", "n_shared", "expert_ffn"):
            setattr(c, n, int(getattr(cfg, n)))
        c.rope_theta = float(cfg.rope_theta)
        c.rms_eps = float(cfg.rms_eps)
        self.c = c
        layers = (OrcLayer * cfg.n_layers)()
        for l, lw in enumerate(weights["layers"]):
            for n in _LAYER_FIELDS:
                a = lw.get(n)
                if a is not None:
                    a = np.ascontiguousarray(a)
                    self._keep.arrays.append(a)
                    setattr(layers[l], n, a.ctypes.data)
        self._layers = layers
        w = OrcWeights()
        for n in ("embed", "final_norm", "lm_head"):
            a = np.ascontiguousarray(weights[n])
            self._keep.arrays.append(a)
            setattr(w, n, a.ctypes.data)
        w.layers = layers
        self.w = w

    def new_cache(self):
        """Zeroed bf16 caches [n_layers][n_kv_heads][max_ctx][head_dim] (K, V)."""
        c = self.cfg
        shape = (c.n_layers, c.n_kv_heads, c.max_ctx, c.head_dim)
        return np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)

    def decode_step(self, kc, vc, token, pos, want_logits=True, want_hidden=True):
        """One decode step; kc/vc are [L][Hkv][max_ctx][d] uint16 views (layer
        stride taken from the array).  Returns (token, logits, hidden)."""
        c = self.cfg
        assert kc.dtype == np.uint16 and kc.shape[1:] == (c.n_kv_heads, c.max_ctx, c.head_dim)
        assert kc.strides == vc.strides and kc.strides[1:] == (
            c.max_ctx * c.head_dim * 2, c.head_dim * 2, 2), "inner K/V dims must be contiguous"
        stride = kc.strides[0] // 2
        lg = np.empty(c.vocab, np.float64) if want_logits else None
        hd = np.empty(c.hidden, np.float64) if want_hidden else None
        tok = lib().orc_decode_step(C.byref(self.c), C.byref(self.w), C.c_void_p(kc.ctypes.data),
                                    C.c_void_p(vc.ctypes.data), stride, int(token), int(pos),
                                    _dp(lg) if lg is not None else None,
                                    _dp(hd) if hd is not None else None)
        return tok, lg, hd

    def new_cache_fp8(self):
        """Zeroed fp8 caches: codes uint8 [n_layers][n_kv_heads][max_ctx][head_dim]
        (K, V) and fp32 row scales [n_layers][n_kv_heads][max_ctx] (K, V)."""
        c = self.cfg
        shape = (c.n_layers, c.n_kv_heads, c.max_ctx, c.head_dim)
        return (np.zeros(shape, np.uint8), np.zeros(shape, np.uint8), np.zeros(shape[:3], np.float32),
                np.zeros(shape[:3], np.float32))

    def decode_step_fp8(self, kc8, vc8, ks, vs, token, pos, want_logits=True, want_hidden=True):
        """decode_step over an fp8 cache (codes [L][Hkv][max_ctx][d] uint8 and
        fp32 row scales [L][Hkv][max_ctx]; inner dimensions contiguous)."""
        c = self.cfg
        assert kc8.dtype == np.uint8 and vc8.dtype == np.uint8 and ks.dtype == np.float32
        assert kc8.shape[1:] == (c.n_kv_heads, c.max_ctx, c.head_dim) and ks.shape[1:] == (c.n_kv_heads, c.max_ctx)
        assert kc8.strides == vc8.strides and kc8.strides[1:] == (c.max_ctx * c.head_dim, c.head_dim, 1)
        assert ks.strides == vs.strides and ks.strides[1:] == (c.max_ctx * 4, 4)
        kv = OrcKV(kc8.ctypes.data, vc8.ctypes.data, ks.ctypes.data, vs.ctypes.data, kc8.strides[0],
                   ks.strides[0] // 4, 1)
        lg = np.empty(c.vocab, np.float64) if want_logits else None
        hd = np.empty(c.hidden, np.float64) if want_hidden else None
        tok = lib().orc_decode_step_kv(C.byref(self.c), C.byref(self.w), C.byref(kv), int(token), int(pos),
                                       _dp(lg) if lg is not None else None, _dp(hd) if hd is not None else None)
        return tok, lg, hd

    def prefill(self, kc, vc, tokens):
        c = self.cfg
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        stride = kc.strides[0] // 2
        return int(lib().orc_prefill(C.byref(self.c), C.byref(self.w), C.c_void_p(kc.ctypes.data),
                                     C.c_void_p(vc.ctypes.data), stride, _vp(t), t.size))

    def forward_full(self, tokens):
        c = self.cfg
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        lg = np.empty((t.size, c.vocab), np.float64)
        hd = np.empty((t.size, c.hidden), np.float64)
        tok = lib().orc_forward_full(C.byref(self.c), C.byref(self.w), _vp(t), t.size, _dp(lg),
                                     _dp(hd))
        return tok, lg, hd

    def moe_ffn(self, layer, b):
        c = self.cfg
        b = np.ascontiguousarray(b, dtype=np.float64)
        out = np.empty(c.hidden, np.float64)
        sel = np.empty(c.top_k, np.int32)
        selw = np.empty(c.top_k, np.float64)
        lib().orc_moe_ffn(C.byref(self.c), C.byref(self._layers[layer]), _dp(b), _dp(out),
                          _vp(sel), _dp(selw))
        return out, sel, selw
