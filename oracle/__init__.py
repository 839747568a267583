"""Oracle for the decode step — TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import
this package.  It wraps ``liboracle.so`` (built from oracle.c, plain fp64 C with
OpenMP over independent rows and heads) with ctypes; the arithmetic is all in
oracle.c.  It shares no code with the HIP path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATHS = {"f64": os.path.join(_HERE, "liboracle.so"), "f32": os.path.join(_HERE, "liboracle_f32.so")}
_LIB_PATH = _LIB_PATHS["f64"]
_libs = {}
_default_precision = "f64"


def set_default_precision(precision: str) -> str:
    """Select the build the piece functions below call ("f64", the parity reference, or "f32"); returns
    the previous choice. Used by the pins that check the fp32 build on its own."""
    global _default_precision
    if precision not in _LIB_PATHS:
        raise ValueError(precision)
    old, _default_precision = _default_precision, precision
    return old

_dp = ctypes.POINTER(ctypes.c_double)
_u16p = ctypes.c_void_p


class OrcConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("d", ctypes.c_int), ("hq", ctypes.c_int), ("hk", ctypes.c_int),
                ("dh", ctypes.c_int), ("f", ctypes.c_int), ("v", ctypes.c_int), ("eps", ctypes.c_double),
                ("theta", ctypes.c_double), ("tied", ctypes.c_int), ("qkv_bias", ctypes.c_int)]


def build_lib(force: bool = False) -> str:
    """Build liboracle.so (fp64) and liboracle_f32.so (fp32 arithmetic, same definition)."""
    src = os.path.join(_HERE, "oracle.c")
    hdr = os.path.join(_HERE, "oracle.h")
    newest = max(os.path.getmtime(src), os.path.getmtime(hdr))
    for prec, path in _LIB_PATHS.items():
        if force or not os.path.exists(path) or os.path.getmtime(path) < newest:
            tmp = path + ".tmp%d" % os.getpid()
            extra = ["-DORC_FP32"] if prec == "f32" else []
            subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall"] + extra
                                  + [src, "-o", tmp, "-lm"])
            os.replace(tmp, path)
    return _LIB_PATH


def lib(precision: str | None = None):
    precision = precision or _default_precision
    if precision not in _libs:
        path = _LIB_PATHS[precision]
        if not os.path.exists(path):
            build_lib()
        L = ctypes.CDLL(path)
        L.orc_create.restype = ctypes.c_void_p
        L.orc_create.argtypes = [ctypes.POINTER(OrcConfig), ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        L.orc_destroy.restype = None
        L.orc_destroy.argtypes = [ctypes.c_void_p]
        L.orc_set_kv.restype = ctypes.c_int
        L.orc_set_kv.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 4 + [_u16p, _u16p]
        L.orc_get_kv.restype = ctypes.c_int
        L.orc_get_kv.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 4 + [_u16p, _u16p]
        L.orc_step.restype = ctypes.c_int
        L.orc_step.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, _dp]
        L.orc_forward_nocache.restype = ctypes.c_int
        L.orc_forward_nocache.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double, _dp]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm.argtypes = [_dp, _u16p, ctypes.c_int, ctypes.c_double, _dp]
        L.orc_gemv.restype = None
        L.orc_gemv.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _dp, _u16p, _dp]
        L.orc_rope.restype = None
        L.orc_rope.argtypes = [_dp, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.orc_softmax.restype = None
        L.orc_softmax.argtypes = [_dp, ctypes.c_int]
        L.orc_attention.restype = None
        L.orc_attention.argtypes = [_dp, _u16p, _u16p] + [ctypes.c_int] * 4 + [_dp]
        L.orc_silu.restype = ctypes.c_double
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_swiglu.restype = None
        L.orc_swiglu.argtypes = [_dp, _dp, ctypes.c_int, _dp]
        L.orc_argmax.restype = ctypes.c_int
        L.orc_argmax.argtypes = [_dp, ctypes.c_int]
        L.orc_bf16.restype = ctypes.c_uint16
        L.orc_bf16.argtypes = [ctypes.c_double]
        L.orc_from_bf16.restype = ctypes.c_double
        L.orc_from_bf16.argtypes = [ctypes.c_uint16]
        L.orc_threads.restype = ctypes.c_int
        L.orc_threads.argtypes = []
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [ctypes.c_int]
        _u8p = ctypes.POINTER(ctypes.c_uint8)
        _i32p = ctypes.POINTER(ctypes.c_int32)
        L.orc_fp8_decode.restype = ctypes.c_double
        L.orc_fp8_decode.argtypes = [ctypes.c_uint8]
        L.orc_fp8_encode.restype = ctypes.c_uint8
        L.orc_fp8_encode.argtypes = [ctypes.c_double]
        L.orc_fp8_row_exp.restype = ctypes.c_int
        L.orc_fp8_row_exp.argtypes = [_u16p, ctypes.c_int]
        L.orc_fp8_quantize.restype = None
        L.orc_fp8_quantize.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u8p, _i32p]
        L.orc_fp8_dequantize.restype = None
        L.orc_fp8_dequantize.argtypes = [_u8p, _i32p, ctypes.c_int, ctypes.c_int, _u16p]
        _libs[precision] = L
    return _libs[precision]


def _d(a):
    return a.ctypes.data_as(_dp)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


# ----------------------------------------------------------------- pieces
def rmsnorm(x, g, eps):
    x = _f64(x); g = _u16(g); out = np.empty_like(x)
    lib().orc_rmsnorm(_d(x), g.ctypes.data, x.size, eps, _d(out))
    return out


def gemv(w, x, bias=None):
    w = _u16(w); x = _f64(x); n, k = w.shape
    assert x.size == k
    y = np.empty(n, dtype=np.float64)
    b = _u16(bias) if bias is not None else None
    lib().orc_gemv(w.ctypes.data, n, k, _d(x), b.ctypes.data if b is not None else None, _d(y))
    return y


def rope(u, pos, theta):
    u = _f64(u).copy()
    lib().orc_rope(_d(u), u.size, float(pos), float(theta))
    return u


def softmax(s):
    s = _f64(s).copy()
    lib().orc_softmax(_d(s), s.size)
    return s


def attention(q, kc, vc, hq, hk, dh):
    """q [hq*dh] float; kc, vc [npos, hk, dh] bf16 bits -> out [hq*dh]."""
    q = _f64(q); kc = _u16(kc); vc = _u16(vc)
    npos = kc.shape[0]
    out = np.empty(hq * dh, dtype=np.float64)
    lib().orc_attention(_d(q), kc.ctypes.data, vc.ctypes.data, npos, hq, hk, dh, _d(out))
    return out


def silu(z):
    return lib().orc_silu(float(z))


def swiglu(a, b):
    a = _f64(a); b = _f64(b); h = np.empty_like(a)
    lib().orc_swiglu(_d(a), _d(b), a.size, _d(h))
    return h


def argmax(v):
    v = _f64(v)
    return lib().orc_argmax(_d(v), v.size)


def bf16(x):
    return lib().orc_bf16(float(x))


def from_bf16(b):
    return lib().orc_from_bf16(int(b))


def bf16_to_f64(a):
    """bf16 bit patterns -> float64 (exact)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def threads():
    return lib().orc_threads()


def set_threads(n):
    lib().orc_set_threads(int(n))


# ----------------------------------------------------------------- FP8 weights
def fp8_decode(code: int) -> float:
    """The value of one OCP E4M3 code."""
    return lib().orc_fp8_decode(int(code))


def fp8_encode(x: float) -> int:
    """The nearest finite E4M3 code to x (|x| <= 448), ties to an even mantissa."""
    return int(lib().orc_fp8_encode(float(x)))


def fp8_row_exp(row) -> int:
    r = _u16(row)
    return int(lib().orc_fp8_row_exp(r.ctypes.data, r.size))


def fp8_quantize(w):
    """[n, k] bf16 bits -> (codes [n, k] uint8, exps [n] int32): each row scaled by its own 2^-e."""
    w = _u16(w)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    exps = np.empty(n, dtype=np.int32)
    lib().orc_fp8_quantize(w.ctypes.data, n, k,
                           codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                           exps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return codes, exps


def fp8_dequantize(codes, exps):
    """bf16 bits of decode(codes) * 2^exps per row (exact)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    exps = np.ascontiguousarray(exps, dtype=np.int32)
    n, k = codes.shape
    out = np.empty((n, k), dtype=np.uint16)
    lib().orc_fp8_dequantize(codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                             exps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, k, out.ctypes.data)
    return out


FP8_MATRICES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def fp8_model(shape, weights: dict):
    """The model whose GEMV matrices are FP8-quantised: every projection and the LM head replaced by
    its exact dequantised values; embeddings, norm gains and biases unchanged. A tied LM head becomes
    an untied one (the embedding lookup keeps the bf16 table). Returns (shape, weights)."""
    import dataclasses
    d = shape.d_model
    out = dict(weights)
    for l in range(shape.n_layers):
        for t in FP8_MATRICES:
            name = "layers.%d.%s" % (l, t)
            w = _u16(weights[name])
            rows = w.size // (shape.d_ffn if t == "wd" else shape.n_q_heads * shape.head_dim if t == "wo" else d)
            out[name] = fp8_dequantize(*fp8_quantize(w.reshape(rows, -1))).reshape(w.shape)
    head = weights["embed"] if shape.tied_embeddings else weights["lm_head"]
    out["lm_head"] = fp8_dequantize(*fp8_quantize(_u16(head).reshape(shape.vocab, d))).reshape(np.shape(head))
    return dataclasses.replace(shape, name=shape.name + "-fp8", tied_embeddings=False), out


# ----------------------------------------------------------------- model
class OracleModel:
    """The decode step of one model over n_seqs sequences with max_pos cache positions each."""

    def __init__(self, shape, weights: dict, n_seqs: int = 1, max_pos: int = 64, precision: str = "f64"):
        self.shape = shape
        self.L = lib(precision)
        m = shape
        self.cfg = OrcConfig(m.n_layers, m.d_model, m.n_q_heads, m.n_kv_heads, m.head_dim, m.d_ffn, m.vocab,
                             float(m.rms_eps), float(m.rope_theta), int(bool(m.tied_embeddings)),
                             int(bool(m.qkv_bias)))
        names = ["embed", "final_norm", None if m.tied_embeddings else "lm_head"]
        for l in range(m.n_layers):
            p = "layers.%d." % l
            for t in ["attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo", "ffn_norm", "wg", "wu", "wd"]:
                names.append(p + t if (m.qkv_bias or t not in ("bq", "bk", "bv")) else None)
        self._keep = []
        ptrs = (ctypes.c_void_p * len(names))()
        for i, nme in enumerate(names):
            if nme is None:
                ptrs[i] = None
            else:
                a = _u16(weights[nme])
                self._keep.append(a)
                ptrs[i] = a.ctypes.data
        self._ptrs = ptrs
        self.n_seqs, self.max_pos = n_seqs, max_pos
        self._h = self.L.orc_create(ctypes.byref(self.cfg), ctypes.cast(ptrs, ctypes.c_void_p), n_seqs, max_pos)
        if not self._h:
            raise ValueError("orc_create rejected the model or could not allocate its cache")

    def close(self):
        if self._h:
            self.L.orc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, seq, token, pos, rope_pos=None):
        logits = np.empty(self.shape.vocab, dtype=np.float64)
        tok = self.L.orc_step(self._h, seq, int(token), pos, float(pos if rope_pos is None else rope_pos), _d(logits))
        if tok < 0:
            raise ValueError("orc_step rejected its arguments")
        return tok, logits

    def set_kv(self, layer, seq, pos0, k, v):
        k = _u16(k); v = _u16(v)
        npos = k.shape[0]
        if self.L.orc_set_kv(self._h, layer, seq, pos0, npos, k.ctypes.data, v.ctypes.data):
            raise ValueError("orc_set_kv rejected its arguments")

    def get_kv(self, layer, seq, pos0, npos):
        m = self.shape
        k = np.empty((npos, m.n_kv_heads, m.head_dim), dtype=np.uint16)
        v = np.empty_like(k)
        if self.L.orc_get_kv(self._h, layer, seq, pos0, npos, k.ctypes.data, v.ctypes.data):
            raise ValueError("orc_get_kv rejected its arguments")
        return k, v

    def forward_nocache(self, tokens, rope_off=0.0):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        logits = np.empty(self.shape.vocab, dtype=np.float64)
        tok = self.L.orc_forward_nocache(self._h, t.ctypes.data, t.size, float(rope_off), _d(logits))
        if tok < 0:
            raise ValueError("orc_forward_nocache rejected its arguments")
        return tok, logits
