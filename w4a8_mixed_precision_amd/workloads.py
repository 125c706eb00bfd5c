"""Layer shapes and seeded synthetic inputs.

This module draws random numbers and nothing else: it holds none of the
quantization or GEMM arithmetic, so both the HIP path and the CPU oracle can be
fed from it.

Shapes follow the model tables of the pages: Llama-3-8B (d_model 4096, 32 query
heads and 8 KV heads of 128 -> fused QKV N = 6144, FFN width 14336) and a
Qwen-72B-class model (d_model 8192, 64/8 heads -> QKV N = 10240, FFN width 29568),
"01 inference papers and experiments", §1.1 dense-model table.  The value
distributions follow the outlier observations on the same pages: a few percent of
input channels carry values 10-20x larger than the rest ("01 inference papers and
experiments", §4.3 SmoothQuant; "QServe：把 W4A8KV4 ..." §3.1 SmoothAttention
notes ~10x Key outliers).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202
GROUP = 128


@dataclass(frozen=True)
class Layer:
    cfg: int          # workload family index (0..4)
    layer: int        # index of the layer inside the family
    name: str
    K: int
    N: int
    Ms: tuple


# family 0: tiny case the oracle finishes in well under a second
# family 1: Llama-3-8B fused QKV projection at decode batch sizes
# family 2: Llama-3-8B MLP at decode batch sizes
# family 3: Qwen-72B-class layers
# family 4: Llama-3-8B MLP at prefill token counts
LAYERS = (
    Layer(0, 0, "tiny", 512, 512, (8,)),
    Layer(1, 0, "llama3_8b_qkv", 4096, 6144, (1, 16, 64)),
    Layer(2, 0, "llama3_8b_gate_up", 4096, 28672, (64, 256, 1024)),
    Layer(2, 1, "llama3_8b_down", 14336, 4096, (64, 256, 1024)),
    Layer(3, 0, "qwen72b_qkv", 8192, 10240, (1, 128, 512)),
    Layer(3, 1, "qwen72b_gate_up", 8192, 59136, (1, 128, 512)),
    Layer(3, 2, "qwen72b_down", 29568, 8192, (1, 128, 512)),
    Layer(4, 0, "llama3_8b_gate_up_prefill", 4096, 28672, (2048, 4096, 8192)),
    Layer(4, 1, "llama3_8b_down_prefill", 14336, 4096, (2048, 4096, 8192)),
)


def layers(cfg: int | None = None):
    return [L for L in LAYERS if cfg is None or L.cfg == cfg]


def find(name: str) -> Layer:
    for L in LAYERS:
        if L.name == name:
            return L
    raise KeyError(name)


def _rng(cfg: int, layer: int, role: int, m: int) -> np.random.Generator:
    ss = np.random.SeedSequence([SEED_BASE, cfg, layer, role, m])
    return np.random.Generator(np.random.PCG64(ss))


def weights_fp16(L: Layer, N: int | None = None, K: int | None = None) -> np.ndarray:
    """W fp16 [N, K]: N(0, 0.02) with 2% of input channels scaled x10."""
    N = L.N if N is None else N
    K = L.K if K is None else K
    w = _rng(L.cfg, L.layer, 0, 0).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(0.02)
    cols = _rng(L.cfg, L.layer, 1, 0).choice(K, round(0.02 * K), replace=False)
    w[:, cols] *= np.float32(10.0)
    return w.astype(np.float16)


def activations_fp16(L: Layer, M: int, K: int | None = None) -> np.ndarray:
    """X fp16 [M, K]: N(0, 1) with 1% of channels scaled x20 (same channels for every M)."""
    K = L.K if K is None else K
    x = _rng(L.cfg, L.layer, 2, M).standard_normal((M, K), dtype=np.float32)
    cols = _rng(L.cfg, L.layer, 3, 0).choice(K, round(0.01 * K), replace=False)
    x[:, cols] *= np.float32(20.0)
    return x.astype(np.float16)


def algorithmic_bytes(M: int, N: int, K: int, per_channel: bool = False) -> dict:
    """Bytes the GEMM must move at least once: packed weights (4 bit), group metadata
    counted at its UINT4 zero + UINT8 scale size (1.5 B per group), fp16 channel
    scales, INT8 activations, fp16 token scales and the fp16 output.  Per-channel
    format: no group metadata, a UINT4 zero per channel (0.5 B) and an INT32 code sum
    per token."""
    if per_channel:
        weight = N * K // 2 + N // 2 + 2 * N
        act = M * K + 2 * M + 4 * M
    else:
        weight = N * K // 2 + (3 * N * (K // GROUP)) // 2 + 2 * N
        act = M * K + 2 * M
    out = 2 * M * N
    return {"weight": weight, "act": act, "out": out, "total": weight + act + out}


def algorithmic_ops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


# KV4 decode attention shapes: one new token per sequence attending to its cache.
# Llama-3-8B (32 query heads, 8 KV heads of 128), the Qwen-72B-class model (64 / 8)
# and Llama-2-7B (32 / 32) at decode batch sizes and contexts of a serving mix (the
# pages' throughput runs use 1024 input tokens; the long single sequence exercises
# the split over the sequence).
@dataclass(frozen=True)
class KvShape:
    name: str
    B: int
    seq_len: int
    h: int
    h_kv: int


KV_SHAPES = (
    KvShape("llama3_8b_b64_l1024", 64, 1024, 32, 8),
    KvShape("llama3_8b_b256_l512", 256, 512, 32, 8),
    KvShape("llama3_8b_b16_l4096", 16, 4096, 32, 8),
    KvShape("llama3_8b_b1_l32768", 1, 32768, 32, 8),
    KvShape("qwen72b_b64_l1024", 64, 1024, 64, 8),
    # Llama-2-7B (32 heads, no grouping): the pages' KV4 attention breakdown runs 64
    # requests of 1024 input tokens on this model
    KvShape("llama2_7b_b64_l1024", 64, 1024, 32, 32),
)

KV_PAGE_TOKENS = 64
KV_HEAD_DIM = 128
# bytes per cached token per KV head: 128 K codes + 128 V codes at 4 bits, fp16
# scale and zero for each of K and V
KV_TOKEN_HEAD_BYTES = KV_HEAD_DIM + 8


def find_kv(name: str) -> KvShape:
    for s in KV_SHAPES:
        if s.name == name:
            return s
    raise KeyError(name)


def kv_fp16(S: KvShape, b: int, n: int, role: int, scale: float = 1.0) -> np.ndarray:
    """Keys (role 0) or values (role 1) fp16 [n, h_kv, 128] for sequence b: N(0, scale)
    with 3 outlier channels per head scaled x8 (the Key outliers the pages report)."""
    r = _rng(5, b, 4 + role, n)
    x = r.standard_normal((n, S.h_kv, KV_HEAD_DIM), dtype=np.float32) * np.float32(scale)
    cols = _rng(5, 0, 6 + role, 0).choice(KV_HEAD_DIM, 3, replace=False)
    x[:, :, cols] *= np.float32(8.0)
    return x.astype(np.float16)


def kv_queries_fp16(S: KvShape) -> np.ndarray:
    return _rng(5, 0, 8, S.B).standard_normal((S.B, S.h, KV_HEAD_DIM), dtype=np.float32).astype(np.float16)


def kv_attention_bytes(B: int, seq_len: int, h: int, h_kv: int) -> int:
    """Bytes decode attention must move at least once: every cached token's codes and
    statistics of every KV head, the fp16 queries and outputs, the page table entries
    and lengths."""
    pages = -(-seq_len // KV_PAGE_TOKENS)
    return B * seq_len * h_kv * KV_TOKEN_HEAD_BYTES + 2 * 2 * B * h * KV_HEAD_DIM + 4 * B * pages + 4 * B


def kv_attention_flops(B: int, seq_len: int, h: int) -> int:
    return 2 * 2 * B * h * seq_len * KV_HEAD_DIM
