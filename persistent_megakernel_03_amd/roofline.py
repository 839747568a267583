"""Bytes-moved accounting for the decode step (host logic, no GPU).

The bound follows the MegaKernel article's lower limit ("LLMs in einen MegaKernel
kompilieren", section on MPK's value): decode must read every weight once per token,
so time >= bytes / peak bandwidth (16 GB at 1.6 TB/s gives 10 ms there). Here the bytes
are the weights a step reads plus the KV-cache rows its attention reads. The KV size
formula 2 * batch * layers * seq * head_dim * heads * bytes is the one the slide deck
works through (slide 9).
"""
from __future__ import annotations

MI355X_HBM_PEAK_GBS = 8000.0   # GB/s, published peak of one MI355X


def gemv_weight_bytes(m) -> int:
    """All matrices a step streams: QKV, O, gate/up, down per layer, plus the LM head."""
    per_layer = ((m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim * m.d_model + m.d_model * m.n_q_heads * m.head_dim
                 + 3 * m.d_ffn * m.d_model)
    return 2 * (m.n_layers * per_layer + m.vocab * m.d_model)


def weight_bytes_per_token(m) -> int:
    """Weights read per token: every GEMV matrix, one embedding row, the RMSNorm gains and
    the QKV bias (the tied LM head counts once, as the LM head)."""
    b = gemv_weight_bytes(m) + 2 * m.d_model + 2 * (2 * m.n_layers + 1) * m.d_model
    if m.qkv_bias:
        b += 2 * m.n_layers * (m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim
    return b


def gemv_rows(m) -> int:
    """Output rows of every GEMV matrix a step streams (each FP8 row carries one fp32 scale)."""
    return m.n_layers * ((m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim + m.d_model + 2 * m.d_ffn + m.d_model) + m.vocab


def weight_bytes_per_token_fp8(m) -> int:
    """Weights read per token with FP8 GEMV matrices: one byte per matrix weight plus a 4-byte scale per
    row; the embedding row, the gains and the bias stay bf16."""
    b = gemv_weight_bytes(m) // 2 + 4 * gemv_rows(m) + 2 * m.d_model + 2 * (2 * m.n_layers + 1) * m.d_model
    if m.qkv_bias:
        b += 2 * m.n_layers * (m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim
    return b


def kv_bytes(batch: int, layers: int, seq: int, head_dim: int, heads: int, elem_bytes: int = 2) -> int:
    """Size of a K+V cache: 2 (K and V) * batch * layers * seq * head_dim * heads * bytes."""
    return 2 * batch * layers * seq * head_dim * heads * elem_bytes


def kv_read_bytes_per_token(m, ctx: int) -> int:
    """KV rows one sequence's step reads when attending to ctx positions (bf16)."""
    return kv_bytes(1, m.n_layers, ctx, m.head_dim, m.n_kv_heads, 2)


def step_bytes(m, ctxs, fp8: bool = False) -> int:
    """Algorithmic bytes of one decode step over sequences with the given attended lengths:
    the weights once plus each sequence's KV rows."""
    w = weight_bytes_per_token_fp8(m) if fp8 else weight_bytes_per_token(m)
    return w + sum(kv_read_bytes_per_token(m, c) for c in ctxs)


def roofline_ms(bytes_: float, peak_gbs: float = MI355X_HBM_PEAK_GBS) -> float:
    return bytes_ / (peak_gbs * 1e9) * 1e3


# Sources whose change alters what the decode kernel reads or writes per launch: the kernel
# itself and the graph builder that lays out its tasks.
_KERNEL_SOURCES = ("csrc/mk_kernel.hip", "csrc/mk_graph.h", "csrc/mk_graph.cpp")


def kernel_source_hash() -> str:
    """First 16 hex digits of SHA-256 over the decode kernel's sources."""
    import hashlib
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES:
        with open(os.path.join(here, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(summary_path: str):
    """HBM bytes per decode step measured with FETCH_SIZE/WRITE_SIZE (scaled by a copy-kernel
    calibration) over a resident launch, as recorded in a profile summary, or None when the summary is
    missing or the kernel sources have changed since it was taken."""
    import os
    import re
    if not os.path.exists(summary_path):
        return None
    txt = open(summary_path).read()
    mb = re.search(r"traffic_bytes_per_step = (\d+)", txt)
    mh = re.search(r"source_sha256_16 = ([0-9a-f]{16})", txt)
    if not mb or not mh or mh.group(1) != kernel_source_hash():
        return None
    return int(mb.group(1))
