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
