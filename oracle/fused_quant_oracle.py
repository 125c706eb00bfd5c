"""CPU oracle for the kernels that produce the GEMM's INT8 activations: RMSNorm +
per-token quantization (before the QKV projection and the first FFN layer) and
SiLU(gate) * up + per-token quantization (before the second FFN layer).
TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP library.

Sources (cited by title and section):

* [QServe review] "QServe：把 W4A8KV4 的理论收益做成实测吞吐的量化—系统协同设计",
  section 3.2 "运行时精度映射" and section 4 step 2: every GEMM takes W4A8 inputs;
  the activation quantization is fused into the preceding normalization kernel (QKV
  projection, first FFN layer) or the preceding activation kernel (second FFN
  layer); blocks are FP16 in and FP16 out.
* [QServe summary] "QServe: W4A8KV4 Quantization and System Co-design for Efficient
  LLM Serving", per-channel fast dequantization: t_X = X 1_k is precomputed by the
  memory-bound kernel that precedes each W4A8 GEMM.

The pages name the kernels but not their formulas.  Readings (also listed with the
design notes):

R14 The normalization of the workloads' models (Llama-3, Qwen) is RMSNorm:
    y = x / sqrt(mean_k x^2 + eps) * gamma, FP16 in and out.  Precision: the sum of
    squares in fp64 (each fp16 square is exact there), mean = fp32(sum / K),
    inv = fp32(1 / fp32(sqrt(fp32(mean + eps)))) with IEEE operations, then
    y = fp16(fp32(fp32(x * inv) * gamma)).  eps > 0.
R15 The FFN activation of those models is SwiGLU: h = SiLU(gate) * up =
    gate * up / (1 + exp(-gate)), computed in fp64 and rounded once to fp16 (fp64
    stands in for the exact value; the pages fix only FP16 in and out).
R16 The fused kernel's INT8 output is the per-token quantization of that fp16
    value, exactly as the standalone quantizer (readings R1, R6, R8), so fusing
    changes where the fp16 value lives (registers, not memory), not the codes.

Pins: tests/test_oracle_pins.py (closed forms, power-of-two scale invariance,
exact rational arithmetic, the SiLU symmetry identity, special cases).
"""

from __future__ import annotations

import math

import numpy as np

from oracle import qoq_oracle as o


def rms_inverse(x16: np.ndarray, eps: float) -> np.ndarray:
    """Per row: inv = fp32(1 / sqrt(fp32(fp32(sum x^2 / K) + eps))) (R14)."""
    x = np.asarray(x16, dtype=np.float16)
    M, K = x.shape
    inv = np.empty(M, dtype=np.float32)
    for m in range(M):
        sq = [float(v) * float(v) for v in x[m].astype(np.float64)]   # exact in fp64
        mean = np.float32(math.fsum(sq) / K)
        inv[m] = np.float32(1.0) / np.sqrt(np.float32(mean + np.float32(eps)))
    return inv


def rmsnorm_fp16(x16: np.ndarray, gamma16: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with FP16 output (R14)."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    g = np.asarray(gamma16, dtype=np.float16).astype(np.float32)
    inv = rms_inverse(x16, eps)
    t = (x * inv[:, None]).astype(np.float32)
    return (t * g[None, :]).astype(np.float32).astype(np.float16)


def rmsnorm_quantize(x16: np.ndarray, gamma16: np.ndarray, eps: float):
    """Fused RMSNorm + per-token INT8 quantization (R14, R16): (qx, s_X, t_X)."""
    y = rmsnorm_fp16(x16, gamma16, eps)
    q, s = o.quantize_activations(y)
    return q, s, o.activation_row_sums(q)


def silu_mul_f64(gate16: np.ndarray, up16: np.ndarray) -> np.ndarray:
    """gate * up / (1 + exp(-gate)) in fp64 (R15), before the fp16 rounding."""
    g = np.asarray(gate16, dtype=np.float16).astype(np.float64)
    u = np.asarray(up16, dtype=np.float16).astype(np.float64)
    with np.errstate(over="ignore"):
        return g * u / (1.0 + np.exp(-g))


def silu_mul_fp16(gate16: np.ndarray, up16: np.ndarray) -> np.ndarray:
    """SwiGLU activation with FP16 output (R15)."""
    return silu_mul_f64(gate16, up16).astype(np.float16)


def silu_mul_quantize(gate16: np.ndarray, up16: np.ndarray):
    """Fused SiLU(gate) * up + per-token INT8 quantization (R15, R16): (qx, s_X, t_X)."""
    h = silu_mul_fp16(gate16, up16)
    q, s = o.quantize_activations(h)
    return q, s, o.activation_row_sums(q)
