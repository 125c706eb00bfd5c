"""CPU oracle for the KV4 path: per-head dynamic INT4 quantization of new key /
value vectors (the KV write) and decode attention over the quantized cache.
TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP library.

Sources (cited by title and section):

* [QServe summary] "QServe: W4A8KV4 Quantization and System Co-design for Efficient
  LLM Serving": the attention of one layer, o_h = softmax(q_h K_{h_KV}^T / sqrt(D))
  V_{h_KV} with h_KV = floor(h / r) (grouped heads, r = H / H_KV); integer
  quantization Q = round(X / s + z), s = (X_max - X_min) / (q_max - q_min),
  z = round(q_min - X_min / s), dequantized (Q - z) s; the KV cache is paged, with
  each head's FP16 scale and zero stored in the page right after its quantized
  features; KV4 attention computes in FP16.
* [QServe review] "QServe：把 W4A8KV4 ..." §3.2 (KV cache management: per-head
  dynamic KV quantization, FP16 scale and zero per head inside each page, updated
  online) and §4 steps 4-5 (decode attention reads INT4 K / V from pages, FP16 math;
  the write path quantizes each new token's k / v per head, asymmetric INT4).

Readings (also listed with the design notes):

R17 "Per-head dynamic" quantization is per token and per KV head: the D values of
    one head's key (or value) vector of one token share one (s, z).  UINT4 codes
    (q_min = 0, q_max = 15) by the summary's asymmetric quantizer over the vector's
    own range [lo, hi] = [min x, max x]: s = fp16(fp32(hi - lo) / 15) (fp32 IEEE,
    then fp16; the stored value is the one used), z = rne(-lo / s) (fp32 quotient),
    stored as FP16 (the review's per-head FP16 zero); codes q = clamp(z + rne(x /
    s), 0, 15) (fp32 quotient, zero added after rounding as reading R2 of the
    weights).  The zero is an integer, so q - z is exact in FP16 arithmetic while
    |z| <= 1024 (|q - z| <= 1039 < 2048).  Where that quantizer has no usable
    result -- s = 0 (a constant vector) or |z| > 1024 (a narrow range far from 0,
    where one step is below 1/68 of the offset) -- the range widened to contain 0
    is used instead (lo = min(lo, 0), hi = max(hi, 0): z then lies in [0, 15]).
    An all-zero vector: s = 0, every code and z are 0.
R18 The dequantized cache value is K_hat = fp16((q - z) * s): q - z is an exact
    small integer and the product is rounded once to fp16 (the pages' FP16 math).
R19 Decode attention over the dequantized values is the plain definition, computed
    here in fp64: scores q . K_hat / sqrt(D), softmax, P V_hat, output rounded to fp16.
    The GPU's contractions use FP16 inputs with FP32 accumulation (the pages' FP16
    CUDA-core math mapped to MI355X matrix cores); the comparison tolerance follows
    from that arithmetic (design notes).

R20 SmoothAttention (the summary's SmoothAttention section, its scaling equation and
    the RoPE constraint; review §4.2): per KV head g and channel i over key samples,
    a_i = max_n |K[n, g, i]| (exact), the RoPE pair (i, i + D/2) shares
    lambda_i = lambda_{i+D/2} = max(a_i, a_{i+D/2})^alpha; alpha = 0.5 (the pages'
    choice) is the IEEE fp32 square root, other alpha the fp64 power rounded to fp32;
    a pair that never leaves 0 keeps lambda = 1 (the pages leave it open; 1 is the
    identity).  Folding: W_Q rows of query head h, channel i become fp16(fp32(w) *
    lambda[h // r, i]), W_K rows of KV head g, channel i become fp16(w / lambda[g, i])
    (fp32 IEEE quotient), so q' . k' = q . k before rounding (Z = (Q Lambda)(K
    Lambda^-1)^T).

Pins: tests/test_oracle_kv4_pins.py.
"""

from __future__ import annotations

import numpy as np

Q_MAX = 15
Z_LIMIT = 1024          # |z| beyond this: the widened range is used (R17)


def _scale_zero(lo: np.ndarray, hi: np.ndarray):
    """s = fp16(fp32(hi - lo) / 15) and z = rne(fp32(-lo / s)) (0 where s = 0)."""
    rng = (hi - lo).astype(np.float32)
    s = (rng / np.float32(Q_MAX)).astype(np.float16)
    s32 = s.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    z = np.where(s32 == 0, np.float32(0), np.rint(-lo / safe)).astype(np.float32)
    return s, s32, safe, z


def kv_quantize(x16: np.ndarray):
    """Per-vector asymmetric UINT4 (R17).  x16: fp16 [..., D] -> (codes uint8
    [..., D], s fp16 [...], z fp16 [...])."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    s, s32, safe, z = _scale_zero(lo, hi)
    widen = (s32 == 0) | (np.abs(z) > Z_LIMIT)
    lo = np.where(widen, np.minimum(lo, np.float32(0)), lo)
    hi = np.where(widen, np.maximum(hi, np.float32(0)), hi)
    s, s32, safe, z = _scale_zero(lo, hi)
    q = np.where(s32[..., None] == 0, 0, z[..., None] + np.rint(x / safe[..., None]))
    q = np.clip(q, 0, Q_MAX).astype(np.uint8)
    return q, s, z.astype(np.float16)


def kv_dequantize(q: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """fp16((q - z) * s) (R18)."""
    d = q.astype(np.float32) - np.asarray(z16, np.float16).astype(np.float32)[..., None]   # exact
    return (d * np.asarray(s16, np.float16).astype(np.float32)[..., None]).astype(np.float16)


def decode_attention(q16: np.ndarray, k_hat16: np.ndarray, v_hat16: np.ndarray, h_kv: int) -> np.ndarray:
    """One decode step for one sequence (R19).  q16: [H, D]; k_hat16, v_hat16:
    [S, H_KV, D] (the dequantized cache, S tokens); GQA h -> h // (H / H_KV).
    Returns o fp16 [H, D]."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    K = np.asarray(k_hat16, dtype=np.float16).astype(np.float64)
    V = np.asarray(v_hat16, dtype=np.float16).astype(np.float64)
    H, D = q.shape
    r = H // h_kv
    out = np.empty((H, D), np.float64)
    for h in range(H):
        g = h // r
        sc = K[:, g, :] @ q[h] / np.sqrt(D)
        w = np.exp(sc - sc.max())
        w /= w.sum()
        out[h] = w @ V[:, g, :]
    return out.astype(np.float16)


def attention_reference(q16, k16, v16, h_kv: int):
    """Quantize the cache (R17), dequantize (R18), attend (R19): o fp16 [H, D] for
    k16, v16 fp16 [S, H_KV, D] as written token by token."""
    kq, ks, kz = kv_quantize(k16)
    vq, vs, vz = kv_quantize(v16)
    return decode_attention(q16, kv_dequantize(kq, ks, kz), kv_dequantize(vq, vs, vz), h_kv)


def smooth_attention_lambda(k16: np.ndarray, alpha: float = 0.5) -> np.ndarray:
    """R20: lambda fp32 [H_KV, D] from key samples fp16 [n, H_KV, D]."""
    a = np.abs(np.asarray(k16, np.float16).astype(np.float32)).max(axis=0)      # [H_KV, D], exact
    D = a.shape[-1]
    pair = np.maximum(a[:, : D // 2], a[:, D // 2:])
    if alpha == 0.5:
        lam = np.sqrt(pair)                                                      # IEEE fp32 square root
    else:
        lam = np.power(pair.astype(np.float64), float(alpha)).astype(np.float32)
    lam = np.where(pair == 0, np.float32(1), lam).astype(np.float32)
    return np.concatenate([lam, lam], axis=1)


def smooth_attention_fold(wq16: np.ndarray, wk16: np.ndarray, lam: np.ndarray, h: int, h_kv: int):
    """R20: fold Lambda into the query and key projections.  wq16 fp16 [h*D, d_model],
    wk16 fp16 [h_kv*D, d_model], lam fp32 [h_kv, D] -> (wq', wk') fp16."""
    lam = np.asarray(lam, np.float32)
    D = lam.shape[1]
    r = h // h_kv
    row_q = np.repeat(lam, r, axis=0).reshape(h * D, 1)      # query head hq uses KV head hq // r
    row_k = lam.reshape(h_kv * D, 1)
    wq = (np.asarray(wq16, np.float16).astype(np.float32) * row_q).astype(np.float16)
    wk = (np.asarray(wk16, np.float16).astype(np.float32) / row_k).astype(np.float16)
    return wq, wk
