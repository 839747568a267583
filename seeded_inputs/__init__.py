"""Seeded synthetic inputs for the decode step: model shapes, weights, prompts,
pre-filled KV contents, page tables and context lengths.

Both the oracle and the HIP path read these as inputs; this module holds none of
the decode step's arithmetic.  Every tensor is drawn from its own counter-based
stream (SplitMix64 + Box-Muller, see gen.c) whose seed is the CRC32 of
"<workload>/<tensor name>", so values are identical on any machine and thread count.

The workload shapes are a Llama-style decoder at three sizes (tiny, a Qwen2.5-0.5B
shape and a Llama-3-8B shape), plus two 8B-shaped decode workloads: one long-context
sequence over a paged KV cache pre-filled to 32768 tokens, and sixteen sequences
decoded together.  The latency workload (39-token prompt, 512 generated tokens, no
speculative decoding) is the one the MegaKernel article ("Compiling LLMs into a
MegaKernel", section on MPK's value) measures with; trained weights of the models the
pages name are not used — weights are N(0, 0.02) rounded to bf16.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import struct
import subprocess
import zlib

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libseeded_inputs.so")
_lib = None


# --------------------------------------------------------------------------- shapes
@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rms_eps: float
    rope_theta: float
    tied_embeddings: bool
    qkv_bias: bool


@dataclasses.dataclass(frozen=True)
class Workload:
    """A decode workload: a model shape plus how its sequences start.

    prompt_len > 0: each sequence starts from a prompt of uniform token ids that is
    run through the step position by position (prefill), then `steps` greedy steps.
    prefill_ctx > 0 (or ctx_range): the KV cache is pre-filled with N(0, 1) bf16
    values for positions < ctx and decode starts from a uniform first token.
    """
    name: str
    model: ModelShape
    n_seqs: int = 1
    prompt_len: int = 0
    steps: int = 0
    prefill_ctx: int = 0
    ctx_range: tuple = ()
    paging: str = "identity"     # "identity" or "permuted" block tables
    block_size: int = 16


TINY = ModelShape("tiny", 2, 256, 4, 2, 64, 688, 4096, 1e-5, 1e4, False, False)
QWEN05B = ModelShape("qwen0.5b", 24, 896, 14, 2, 64, 4864, 151936, 1e-6, 1e6, True, True)
LLAMA8B = ModelShape("llama8b", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 5e5, False, False)
# A two-layer shape between tiny and 8B (8B head geometry, GQA 4:1), for batched-decode tests at a size
# the oracle runs in seconds.
MID = ModelShape("mid", 2, 2048, 16, 4, 128, 5632, 16384, 1e-5, 5e5, False, False)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, 1, prompt_len=16, steps=32),
    "qwen0.5b": Workload("qwen0.5b", QWEN05B, 1, prompt_len=39, steps=512),
    "llama8b": Workload("llama8b", LLAMA8B, 1, prompt_len=39, steps=512),
    "llama8b_long": Workload("llama8b_long", LLAMA8B, 1, steps=64, prefill_ctx=32768, paging="permuted"),
    # the 8B decode's last steps: a cache already holding 530 positions (near the end of the 39 + 512
    # workload), for parity on the same 35-block cache and graph
    "llama8b_pf530": Workload("llama8b_pf530", LLAMA8B, 1, steps=16, prefill_ctx=530),
    "llama8b_b16": Workload("llama8b_b16", LLAMA8B, 16, steps=128, ctx_range=(512, 8192), paging="permuted"),
    # small batched workloads with the same structure (per-sequence contexts, permuted pages)
    "tiny_b4": Workload("tiny_b4", TINY, 4, steps=8, ctx_range=(5, 60), paging="permuted"),
    "mid_b16": Workload("mid_b16", MID, 16, steps=4, ctx_range=(16, 300), paging="permuted"),
    # longer mixed contexts: with one split per KV head an attention task holds up to three pieces
    "mid_b16_long": Workload("mid_b16_long", MID, 16, steps=2, ctx_range=(256, 2048), paging="permuted"),
}


def shrink(model: ModelShape, name: str, **kw) -> ModelShape:
    return dataclasses.replace(model, name=name, **kw)


# --------------------------------------------------------------------------- library
def build_lib(force: bool = False) -> str:
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", src,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        L.si_splitmix_out.restype = ctypes.c_uint64
        L.si_splitmix_out.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.si_normal_at.restype = ctypes.c_double
        L.si_normal_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.si_normal_bf16.restype = None
        L.si_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_void_p]
        L.si_uniform_int.restype = None
        L.si_uniform_int.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]
        L.si_permutation.restype = None
        L.si_permutation.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        _lib = L
    return _lib


def tensor_seed(workload: str, tensor: str) -> int:
    return zlib.crc32(("%s/%s" % (workload, tensor)).encode())


def normal_bf16(seed: int, n: int, mean: float = 0.0, std: float = 1.0, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    if n:
        lib().si_normal_bf16(seed, offset, n, mean, std, out.ctypes.data)
    return out


def uniform_int(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        lib().si_uniform_int(seed, n, lo, hi, out.ctypes.data)
    return out


def permutation(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        lib().si_permutation(seed, n, out.ctypes.data)
    return out


# ------------------------------------------------- pure-Python copy of the generator
# Used only to pin the C generator on small slices (same libm calls, same rounding).
_M64 = (1 << 64) - 1


def py_splitmix_out(seed: int, k: int) -> int:
    z = (seed + (k + 1) * 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def py_normal_at(seed: int, i: int) -> float:
    j = i >> 1
    a, b = py_splitmix_out(seed, 2 * j), py_splitmix_out(seed, 2 * j + 1)
    u1 = float((a >> 11) + 1) * 2.0 ** -53
    u2 = float(b >> 11) * 2.0 ** -53
    r = math.sqrt(-2.0 * math.log(u1))
    t = math.tau * u2
    return r * math.sin(t) if (i & 1) else r * math.cos(t)


def py_bf16_from_double(v: float) -> int:
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFFFFFF
    return u >> 16


# --------------------------------------------------------------------------- weights
def tensor_specs(m: ModelShape):
    """(name, shape, kind) for every model tensor; kind is 'w' (N(0, 0.02)) or 'g' (gain)."""
    d, hq, hk, dh, f, v = m.d_model, m.n_q_heads, m.n_kv_heads, m.head_dim, m.d_ffn, m.vocab
    specs = [("embed", (v, d), "w")]
    for l in range(m.n_layers):
        p = "layers.%d." % l
        specs += [(p + "attn_norm", (d,), "g"), (p + "wq", (hq * dh, d), "w"), (p + "wk", (hk * dh, d), "w"),
                  (p + "wv", (hk * dh, d), "w")]
        if m.qkv_bias:
            specs += [(p + "bq", (hq * dh,), "w"), (p + "bk", (hk * dh,), "w"), (p + "bv", (hk * dh,), "w")]
        specs += [(p + "wo", (d, hq * dh), "w"), (p + "ffn_norm", (d,), "g"), (p + "wg", (f, d), "w"),
                  (p + "wu", (f, d), "w"), (p + "wd", (d, f), "w")]
    specs.append(("final_norm", (d,), "g"))
    if not m.tied_embeddings:
        specs.append(("lm_head", (v, d), "w"))
    return specs


def gen_weights(m: ModelShape, seed_ns: str | None = None, gain_std: float = 0.0, w_std: float = 0.02):
    """All weights as bf16 bit patterns (np.uint16).  Matrices ~ N(0, w_std); RMSNorm gains
    are 1.0 unless gain_std > 0, then N(1, gain_std).  `seed_ns` names the seed namespace
    (defaults to the model name)."""
    ns = seed_ns or m.name
    out = {}
    for name, shape, kind in tensor_specs(m):
        n = int(np.prod(shape))
        if kind == "g":
            if gain_std > 0:
                a = normal_bf16(tensor_seed(ns, name), n, 1.0, gain_std)
            else:
                a = np.full(n, 0x3F80, dtype=np.uint16)   # bf16 1.0
        else:
            a = normal_bf16(tensor_seed(ns, name), n, 0.0, w_std)
        out[name] = a.reshape(shape)
    return out


def weight_bytes(m: ModelShape) -> int:
    return sum(int(np.prod(s)) * 2 for _, s, _ in tensor_specs(m))


# --------------------------------------------------------------------------- workload state
def prompt_tokens(w: Workload, seq: int = 0) -> np.ndarray:
    return uniform_int(tensor_seed(w.name, "prompt.%d" % seq), w.prompt_len, 0, w.model.vocab - 1)


def first_tokens(w: Workload) -> np.ndarray:
    return uniform_int(tensor_seed(w.name, "first_tokens"), w.n_seqs, 0, w.model.vocab - 1)


def context_lengths(w: Workload) -> np.ndarray:
    """KV positions already filled per sequence when decode starts."""
    if w.ctx_range:
        lo, hi = w.ctx_range
        return uniform_int(tensor_seed(w.name, "ctx"), w.n_seqs, lo, hi)
    return np.full(w.n_seqs, w.prefill_ctx, dtype=np.int32)


def kv_fill(w: Workload, layer: int, seq: int, n_pos: int, which: str) -> np.ndarray:
    """Pre-filled K or V for logical positions [0, n_pos) of one sequence and layer,
    N(0, 1) in bf16, laid out [pos, kv_head, head_dim].  K is taken as already rotated."""
    m = w.model
    a = normal_bf16(tensor_seed(w.name, "kv.%d.%s.%d" % (layer, which, seq)), n_pos * m.n_kv_heads * m.head_dim)
    return a.reshape(n_pos, m.n_kv_heads, m.head_dim)


def block_tables(w: Workload, capacity: np.ndarray):
    """Per-sequence block tables for `capacity[s]` positions.  Returns (table [n_seqs,
    max_blocks] int32, num_blocks).  Identity paging hands out blocks in order; permuted
    paging takes them from a seeded random permutation of the pool."""
    bs = w.block_size
    nb = [(int(c) + bs - 1) // bs for c in capacity]
    total = int(sum(nb))
    order = permutation(tensor_seed(w.name, "pages"), total) if w.paging == "permuted" else np.arange(total, dtype=np.int32)
    mb = max(nb) if nb else 0
    table = np.zeros((len(nb), max(mb, 1)), dtype=np.int32)
    off = 0
    for s, n in enumerate(nb):
        table[s, :n] = order[off:off + n]
        off += n
    return table, total
