"""Python binding of libmk.so, the persistent decode megakernel for MI355X (gfx950).

This layer only marshals arguments. Every step of the decode path runs in the HIP
kernels behind the C ABI declared in include/mk.h, and the functions here carry the
same names. PyTorch supplies device memory and streams. If the library is missing,
``lib()`` raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libmk.so")
_SOURCES = ["csrc/mk_kernel.hip", "csrc/mk_api.cpp", "csrc/mk_graph.cpp"]
_HEADERS = ["csrc/mk_graph.h", "csrc/mk_host.h", "../include/mk.h"]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

MK_OK = 0
STATUS = {0: "MK_OK", -1: "MK_ERR_INVALID_ARG", -2: "MK_ERR_SHAPE", -3: "MK_ERR_STATE", -4: "MK_ERR_HIP",
          -5: "MK_ERR_DEVICE_TIMEOUT", -6: "MK_ERR_DEVICE_FAULT", -7: "MK_ERR_UNSUPPORTED"}


class MKError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status


class mk_model_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("tied_embeddings", ctypes.c_int32), ("qkv_bias", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("attn_splits", ctypes.c_int32), ("attn_min_blocks", ctypes.c_int32),
                ("prefill_rows", ctypes.c_int32), ("weight_format", ctypes.c_int32)]


class mk_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ptr", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class mk_graph_info(ctypes.Structure):
    _fields_ = [("n_tasks", ctypes.c_int64), ("n_events", ctypes.c_int64), ("n_flag_slots", ctypes.c_int64),
                ("n_attn_groups", ctypes.c_int64), ("max_queue_len", ctypes.c_int64), ("weight_bytes", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int64), ("hash", ctypes.c_uint64), ("n_stages", ctypes.c_int64),
                ("attn_tasks", ctypes.c_int64), ("n_cus", ctypes.c_int64)]


EXPORTS = ["mk_create", "mk_create_host", "mk_workspace_size", "mk_bind_memory", "mk_load_weights", "mk_decode_step",
           "mk_decode_n", "mk_decode_step_static", "mk_decode_step_dynamic", "mk_decode_step_staged", "mk_prefill", "mk_read_fp8_weights", "mk_read_logits",
           "mk_sync_check", "mk_graph_stats", "mk_graph_validate",
           "mk_graph_simulate", "mk_graph_corrupt", "mk_set_trace", "mk_destroy", "mk_status_str", "mk_last_error"]


def build(force: bool = True) -> str:
    """Compile libmk.so for gfx950 with hipcc (in-tree)."""
    srcs = [os.path.join(_HERE, s) for s in _SOURCES]
    deps = srcs + [os.path.normpath(os.path.join(_HERE, h)) for h in _HEADERS]
    if not force and os.path.exists(LIB_PATH) and os.path.getmtime(LIB_PATH) >= max(map(os.path.getmtime, deps)):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["hipcc"] + HIPCC_FLAGS + srcs + ["-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmk.so is not built (run __graft_entry__.build()); the decode path has no fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "mk_create": [ctypes.POINTER(mk_model_config), ctypes.c_int, ctypes.POINTER(vp)],
            "mk_create_host": [ctypes.POINTER(mk_model_config), ctypes.c_int, ctypes.POINTER(vp)],
            "mk_workspace_size": [vp, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)],
            "mk_bind_memory": [vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp],
            "mk_load_weights": [vp, ctypes.POINTER(mk_tensor), ctypes.c_int, vp],
            "mk_decode_step": [vp, vp, ctypes.c_int, vp, vp],
            "mk_decode_n": [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp],
            "mk_decode_step_static": [vp, vp, ctypes.c_int, vp, vp],
            "mk_decode_step_staged": [vp, vp, ctypes.c_int, vp, vp],
            "mk_decode_step_dynamic": [vp, vp, ctypes.c_int, vp, vp],
            "mk_prefill": [vp, ctypes.c_int, ctypes.POINTER(i32), ctypes.c_int, vp, vp],
            "mk_read_fp8_weights": [vp, ctypes.c_char_p, vp, vp, vp],
            "mk_read_logits": [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_float), sz, vp],
            "mk_sync_check": [vp, vp],
            "mk_graph_stats": [vp, ctypes.POINTER(mk_graph_info)],
            "mk_graph_validate": [vp],
            "mk_graph_simulate": [vp, ctypes.c_uint64, ctypes.c_int],
            "mk_graph_corrupt": [vp, ctypes.c_int],
            "mk_set_trace": [vp, vp, sz],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = i32
        L.mk_destroy.argtypes = [vp]
        L.mk_destroy.restype = None
        L.mk_status_str.argtypes = [i32]
        L.mk_status_str.restype = ctypes.c_char_p
        L.mk_last_error.argtypes = []
        L.mk_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


TRACE_REC_BYTES = 48


def trace_dtype():
    """numpy dtype of one task record written by mk_set_trace's buffer (48 bytes)."""
    import numpy as np
    return np.dtype([("t_queue", "<u8"), ("t_ready", "<u8"), ("t_streamed", "<u8"), ("t_done", "<u8"), ("cu", "<u2"),
                     ("type", "u1"), ("layer", "u1"), ("epoch", "<u4"), ("xcc", "<u4"), ("step", "<u4")])


def _check(status):
    if status != MK_OK:
        raise MKError(status, lib().mk_last_error().decode())
    return status


def _vp(x):
    """Device pointer of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    return ctypes.c_void_p(x.data_ptr())


# ------------------------------------------------------------------- ABI functions
def mk_create(cfg: mk_model_config, device: int = 0):
    h = ctypes.c_void_p()
    _check(lib().mk_create(ctypes.byref(cfg), device, ctypes.byref(h)))
    return h


def mk_create_host(cfg: mk_model_config, n_cus: int):
    h = ctypes.c_void_p()
    _check(lib().mk_create_host(ctypes.byref(cfg), n_cus, ctypes.byref(h)))
    return h


def mk_workspace_size(ctx):
    w, kv, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().mk_workspace_size(ctx, ctypes.byref(w), ctypes.byref(kv), ctypes.byref(s)))
    return w.value, kv.value, s.value


def mk_bind_memory(ctx, weights, k_pools, v_pools, scratch, page_table, ctx_lens, logits):
    n = len(k_pools)
    kp = (ctypes.c_void_p * n)(*[_vp(t).value for t in k_pools])
    vp = (ctypes.c_void_p * n)(*[_vp(t).value for t in v_pools])
    _check(lib().mk_bind_memory(ctx, _vp(weights), kp, vp, _vp(scratch), _vp(page_table), _vp(ctx_lens), _vp(logits)))


def mk_load_weights(ctx, named: dict, stream=None):
    """named: name -> bf16 device tensor (contiguous)."""
    arr = (mk_tensor * len(named))()
    keep = []
    for i, (k, t) in enumerate(named.items()):
        b = k.encode()
        keep.append(b)
        arr[i] = mk_tensor(b, t.data_ptr(), t.numel())
    _check(lib().mk_load_weights(ctx, arr, len(named), _vp(stream)))


def mk_decode_step(ctx, tokens_in, n_seqs, tokens_out, stream=None):
    _check(lib().mk_decode_step(ctx, _vp(tokens_in), n_seqs, _vp(tokens_out), _vp(stream)))


def mk_decode_n(ctx, tokens_in, n_seqs, n_steps, tokens_out, stream=None):
    _check(lib().mk_decode_n(ctx, _vp(tokens_in), n_seqs, n_steps, _vp(tokens_out), _vp(stream)))


def mk_decode_step_static(ctx, tokens_in, n_seqs, tokens_out, stream=None):
    _check(lib().mk_decode_step_static(ctx, _vp(tokens_in), n_seqs, _vp(tokens_out), _vp(stream)))


def mk_decode_step_dynamic(ctx, tokens_in, n_seqs, tokens_out, stream=None):
    _check(lib().mk_decode_step_dynamic(ctx, _vp(tokens_in), n_seqs, _vp(tokens_out), _vp(stream)))


def mk_decode_step_staged(ctx, tokens_in, n_seqs, tokens_out, stream=None):
    _check(lib().mk_decode_step_staged(ctx, _vp(tokens_in), n_seqs, _vp(tokens_out), _vp(stream)))


def mk_read_fp8_weights(ctx, name, rows, cols, stream=None):
    """(codes [rows, cols] uint8, exps [rows] int32) of one FP8 matrix, read back in natural layout."""
    import numpy as np
    codes = np.zeros((rows, cols), dtype=np.uint8)
    exps = np.zeros(rows, dtype=np.int32)
    _check(lib().mk_read_fp8_weights(ctx, name.encode(), codes.ctypes.data, exps.ctypes.data, _vp(stream)))
    return codes, exps


def mk_prefill(ctx, seq, tokens, token_out=None, stream=None):
    n = len(tokens)
    arr = (ctypes.c_int32 * max(n, 1))(*[int(t) for t in tokens])
    _check(lib().mk_prefill(ctx, seq, arr, n, _vp(token_out), _vp(stream)))


def mk_read_logits(ctx, seq, n, stream=None):
    import numpy as np
    out = np.empty(n, dtype=np.float32)
    _check(lib().mk_read_logits(ctx, seq, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n, _vp(stream)))
    return out


def mk_sync_check(ctx, stream=None):
    _check(lib().mk_sync_check(ctx, _vp(stream)))


def mk_graph_stats(ctx) -> mk_graph_info:
    info = mk_graph_info()
    _check(lib().mk_graph_stats(ctx, ctypes.byref(info)))
    return info


def mk_graph_validate(ctx):
    _check(lib().mk_graph_validate(ctx))


def mk_graph_simulate(ctx, seed: int, n_steps: int):
    _check(lib().mk_graph_simulate(ctx, seed, n_steps))


def mk_graph_corrupt(ctx, kind: int):
    _check(lib().mk_graph_corrupt(ctx, kind))


def mk_set_trace(ctx, buf, nbytes):
    _check(lib().mk_set_trace(ctx, _vp(buf), nbytes))


def mk_destroy(ctx):
    lib().mk_destroy(ctx)


def mk_status_str(s: int) -> str:
    return lib().mk_status_str(s).decode()


def mk_last_error() -> str:
    return lib().mk_last_error().decode()


# ------------------------------------------------------------------- convenience
def make_config(shape, max_seqs=1, max_blocks_per_seq=64, num_blocks=64, attn_splits=0, block_size=16,
                attn_min_blocks=0, prefill_rows=0, weight_format=0):
    """mk_model_config from any object with the model-shape attributes."""
    return mk_model_config(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                           shape.d_ffn, shape.vocab, float(shape.rms_eps), float(shape.rope_theta),
                           int(bool(shape.tied_embeddings)), int(bool(shape.qkv_bias)), max_seqs, block_size,
                           max_blocks_per_seq, num_blocks, attn_splits, attn_min_blocks, prefill_rows,
                           weight_format)


class Decoder:
    """Allocates the caller-owned device buffers with torch, binds them, and forwards calls.

    Argument marshalling and memory plumbing only. The decode step itself is the
    C ABI's mk_decode_step.
    """

    def __init__(self, cfg: mk_model_config, device: int = 0):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.dev = torch.device("cuda", device)
        self.ctx = mk_create(cfg, device)
        wb, kvb, sb = mk_workspace_size(self.ctx)
        self.sizes = (wb, kvb, sb)
        u8 = torch.uint8
        self.weights = torch.empty(wb, dtype=u8, device=self.dev)
        self.k_pools = [torch.zeros(kvb // 2, dtype=torch.int16, device=self.dev) for _ in range(cfg.n_layers)]
        self.v_pools = [torch.zeros(kvb // 2, dtype=torch.int16, device=self.dev) for _ in range(cfg.n_layers)]
        self.scratch = torch.zeros(sb, dtype=u8, device=self.dev)
        self.page_table = torch.zeros((cfg.max_seqs, cfg.max_blocks_per_seq), dtype=torch.int32, device=self.dev)
        self.ctx_lens = torch.zeros(cfg.max_seqs, dtype=torch.int32, device=self.dev)
        self.logits = torch.zeros((cfg.max_seqs, cfg.vocab), dtype=torch.float32, device=self.dev)
        self.tokens = torch.zeros(max(cfg.max_seqs, 1), dtype=torch.int32, device=self.dev)
        mk_bind_memory(self.ctx, self.weights, self.k_pools, self.v_pools, self.scratch, self.page_table,
                       self.ctx_lens, self.logits)

    def load_weights(self, host_weights: dict, stream=None):
        """host_weights: name -> numpy uint16 (bf16 bits). Uploaded, re-laid out, then freed."""
        torch = self.torch
        named = {k: torch.from_numpy(v.reshape(-1).view("int16")).to(self.dev) for k, v in host_weights.items()}
        mk_load_weights(self.ctx, named, stream)
        torch.cuda.synchronize(self.dev)
        del named

    def set_page_table(self, table):
        self.page_table.copy_(self.torch.as_tensor(table, dtype=self.torch.int32))

    def set_ctx_lens(self, lens):
        self.ctx_lens.copy_(self.torch.as_tensor(lens, dtype=self.torch.int32))

    def stream_ptr(self):
        return self.torch.cuda.current_stream(self.dev).cuda_stream

    def prefill(self, tokens, token_out=None, seq=0):
        mk_prefill(self.ctx, seq, tokens, token_out, self.stream_ptr())

    def step(self, tokens_in, n_seqs=1, tokens_out=None):
        mk_decode_step(self.ctx, tokens_in, n_seqs, tokens_out if tokens_out is not None else tokens_in,
                       self.stream_ptr())

    def decode_n(self, tokens_in, n_steps, n_seqs=1, tokens_out=None):
        """n_steps greedy steps in one launch; returns the [n_steps, n_seqs] int32 device tensor of tokens."""
        if tokens_out is None:
            tokens_out = self.torch.empty((n_steps, n_seqs), dtype=self.torch.int32, device=self.dev)
        mk_decode_n(self.ctx, tokens_in, n_seqs, n_steps, tokens_out, self.stream_ptr())
        return tokens_out

    def step_dynamic(self, tokens_in, n_seqs=1, tokens_out=None):
        """The same step with its tasks taken from a device-side ready queue at run time."""
        mk_decode_step_dynamic(self.ctx, tokens_in, n_seqs, tokens_out if tokens_out is not None else tokens_in,
                               self.stream_ptr())

    def step_staged(self, tokens_in, n_seqs=1, tokens_out=None):
        """The same step as one kernel dispatch per dependency stage (to measure pass-to-pass gaps)."""
        mk_decode_step_staged(self.ctx, tokens_in, n_seqs, tokens_out if tokens_out is not None else tokens_in,
                              self.stream_ptr())

    def read_logits(self, seq=0):
        return mk_read_logits(self.ctx, seq, self.cfg.vocab, self.stream_ptr())

    def sync_check(self):
        mk_sync_check(self.ctx, self.stream_ptr())

    def enable_trace(self):
        n = mk_graph_stats(self.ctx).n_tasks
        self.trace_buf = self.torch.zeros(n * TRACE_REC_BYTES, dtype=self.torch.uint8, device=self.dev)
        mk_set_trace(self.ctx, self.trace_buf, n * TRACE_REC_BYTES)

    def disable_trace(self):
        mk_set_trace(self.ctx, None, 0)
        self.trace_buf = None

    def read_trace(self):
        """Per-task records of the last step: structured numpy array (t_queue, t_ready, t_streamed, t_done,
        cu, type, layer, epoch, xcc, step), indexed by the task's position in the global order."""
        self.torch.cuda.synchronize(self.dev)
        return self.trace_buf.cpu().numpy().view(trace_dtype())

    def close(self):
        if self.ctx:
            mk_destroy(self.ctx)
            self.ctx = None
