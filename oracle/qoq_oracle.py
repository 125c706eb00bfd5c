"""CPU oracle for the QoQ W4A8 GEMM (per-group, and the per-channel variant).
TEST INFRASTRUCTURE ONLY.

This module is the plain, slow, obviously-correct statement of what the GPU path
computes.  Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  It shares no code with the HIP library (no
kernels, headers, helpers, tables or constants): every number below is derived
here from the pages' definitions.

Sources (web pages; cited by title and section):

* [QServe review]  "QServe：把 W4A8KV4 的理论收益做成实测吞吐的量化—系统协同设计"
  (zenmind.me gpu-llm papers #10), section 3.1 "渐进分组量化与保护区间" and
  section 4 "GPU/系统数据路径" step 3.
* [QServe summary] "QServe: W4A8KV4 Quantization and System Co-design for Efficient
  LLM Serving" (papercache.org summary of arXiv:2405.04532), sections
  "整数量化" (integer quantization), "渐进式组量化" (progressive group
  quantization), "保护性量化范围" (protective quantization range) and the
  epilogue formula O = (Q_X Q_W) ⊙ (s_W × s_X) − ... in "怎么做的".
* [Inference chapter] "01 inference papers and experiments" (cklxx.github.io),
  section 4.1 "均匀量化的数学基础" (symmetric / asymmetric uniform quantization).

Readings taken where the pages are silent or garbled (each is also listed in the
design notes of the repository):

R1  Every rounding is round-half-to-even (IEEE default).
R2  Level-1 code: q = z + rne(x / s) (zero added after rounding).  This is the only
    reading that reproduces the worked example value 120 -> code 15 under R1, and it
    makes the dequantized value equal rne(x/s)*s whenever no clamp fires, which is
    the identity the protective-range derivation uses.
R3  The integer group scale is s_u8 = max(1, ceil((max - min) / 15)).
R4  Each group's range is widened to contain 0 (min <= 0 <= max) so that z fits
    the UINT4 range [0, 15].
R5  Level-0 scale s_W = fp16(absmax / 119) (protective range), computed as an IEEE
    fp32 divide then rounded to fp16; the fp16 value is the one used to quantize.
R6  Activations: per-token symmetric INT8 in [-127, 127], s_X = fp16(absmax / 127).
R7  Epilogue: out = fp16( float32(acc) * (float32(s_X[m]) * float32(s_W[n])) ).
R8  An all-zero row (or a scale that rounds to fp16 zero) quantizes to code 0.
R12 Per-channel variant (the format without groups): per output channel asymmetric
    UINT4 with an integer UINT4 zero and an fp16 scale s_W = fp16((max - min) / 15)
    over the channel's range widened to contain 0 (R4), fp32 subtract and divide,
    code q = clamp(z + rne(w / s_W), 0, 15) (R2), z = clamp(rne(-min / s_W), 0, 15).
R13 Its epilogue term t_X x (z_W ⊙ s_W) takes t_X over the quantized activations,
    t[m] = sum_k qx[m, k] (so s_X t is the row sum of X_hat = Q_X s_X): the epilogue
    is then an exact rearrangement of sum_k X_hat W_hat, and the GEMM result is the
    plain integer contraction sum_k qx (q - z) with the fp16 epilogue of R7.
(R9-R11 concern the protective-range bound, the level-1 equation and the unpack
count; they are listed with the design notes.)

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
the worked example printed on the pages, exhaustive bound sweeps of the protective
range derivation, closed-form special cases and brute force on tiny inputs.  The
packed byte layout (``pack_weights``) is this library's own storage format; the
pages do not fix it, so that function is pinned only by round-trip and hand-computed
bytes ("parity unpinned by the pages" for the byte order itself).
"""

from __future__ import annotations

import numpy as np

GROUP = 128          # group size g along the reduction dimension
W_QMAX = 119         # protective range of the level-0 INT8 weight codes
X_QMAX = 127         # symmetric INT8 activation range
U4_MAX = 15          # UINT4 code range [0, 15]


# ---------------------------------------------------------------------------
# integer helper
# ---------------------------------------------------------------------------
def rne_div(a, b):
    """Exact integer a / b (b > 0) rounded to nearest, ties to even (reading R1).

    Works on int64 numpy arrays.  floor-divide first, then round up when the
    remainder is more than half of b, or exactly half and the floor is odd.
    """
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    q, r = np.divmod(a, b)              # q = floor(a/b), 0 <= r < b
    twice = 2 * r
    up = (twice > b) | ((twice == b) & (q % 2 == 1))
    return q + up.astype(np.int64)


# ---------------------------------------------------------------------------
# O1  level 0: per-output-channel symmetric INT8 in the protective range
#     [QServe summary] "渐进式组量化" first equation (W_hat = Q_s8 * s_fp16, one
#     fp16 scale per output channel); [QServe review] §3.1 protective range
#     [-119, 119]; [Inference chapter] §4.1 symmetric quantizer
#     x_q = clip(round(x / s), Qmin, Qmax).
# ---------------------------------------------------------------------------
def quantize_weights_level0(w16: np.ndarray):
    """W fp16 [N, K] -> (q_s8 int8 [N, K], s_W fp16 [N])."""
    w = np.asarray(w16, dtype=np.float16).astype(np.float32)
    absmax = np.max(np.abs(w), axis=1)                       # exact in fp32
    s_w = (absmax / np.float32(W_QMAX)).astype(np.float16)   # fp32 divide, RNE to fp16
    sw = s_w.astype(np.float32)
    q = np.zeros(w.shape, dtype=np.int8)
    rows = np.nonzero(sw != 0)[0]                            # R8: zero scale -> code 0
    if rows.size:
        ratio = w[rows] / sw[rows, None]                     # fp32 divide
        q[rows] = np.clip(np.rint(ratio), -W_QMAX, W_QMAX).astype(np.int8)
    return q, s_w


# ---------------------------------------------------------------------------
# O2  level 1: per-group asymmetric UINT4 with UINT4 zero and UINT8 scale
#     [QServe summary] "整数量化": Q = round(X/s + z), s = (Xmax - Xmin)/(qmax - qmin),
#     z = round(qmin - Xmin/s); "渐进式组量化": Q_u4 in N^{n x k}, z_u4 and s_u8 in
#     N^{n x k/g}; readings R2-R4.
# ---------------------------------------------------------------------------
def quantize_weights_level1(q_s8: np.ndarray, group: int = GROUP):
    """q_s8 int [N, K] -> (q_u4 uint8 [N, K], z uint8 [N, K/g], s_u8 uint8 [N, K/g]).

    ``group`` is 128 for the GEMM; the bound sweeps in the tests call it with other
    group lengths to enumerate groups exhaustively.
    """
    x = np.asarray(q_s8, dtype=np.int64)
    n, k = x.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    xg = x.reshape(n, k // group, group)
    lo = np.minimum(xg.min(axis=2), 0)                       # R4
    hi = np.maximum(xg.max(axis=2), 0)
    s = np.maximum((hi - lo + (U4_MAX - 1)) // U4_MAX, 1)    # R3: ceil((hi-lo)/15), >= 1
    z = np.clip(rne_div(-lo, s), 0, U4_MAX)                  # z = round(qmin - Xmin/s), qmin = 0
    q = np.clip(z[..., None] + rne_div(xg, s[..., None]), 0, U4_MAX)   # R2
    return (q.reshape(n, k).astype(np.uint8), z.astype(np.uint8), s.astype(np.uint8))


# ---------------------------------------------------------------------------
# O3  dequantize level 1 back to the INT8 intermediate: (q_u4 - z) * s_u8
#     [QServe review] §3.1 worked example "(15-7) x 16 = 128"; [Inference chapter]
#     §4.1 asymmetric dequantization x_hat = (x_q - z) * s.
# ---------------------------------------------------------------------------
def dequantize_level1(q_u4: np.ndarray, z: np.ndarray, s_u8: np.ndarray, group: int = GROUP):
    """-> w_hat int16 [N, K] (values fit INT8 when level 0 used the protective range)."""
    q = np.asarray(q_u4, dtype=np.int16)
    n, k = q.shape
    zz = np.repeat(np.asarray(z, dtype=np.int16), group, axis=1)
    ss = np.repeat(np.asarray(s_u8, dtype=np.int16), group, axis=1)
    return (q - zz) * ss


# ---------------------------------------------------------------------------
# O4  per-token symmetric INT8 activation quantization (reading R6)
#     [QServe summary] epilogue term (s_W x s_X): one activation scale per token;
#     [Inference chapter] §4.1 symmetric quantizer with Qmax = 127.
# ---------------------------------------------------------------------------
def quantize_activations(x16: np.ndarray):
    """X fp16 [M, K] -> (qx int8 [M, K], s_X fp16 [M])."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    absmax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s_x = (absmax / np.float32(X_QMAX)).astype(np.float16)
    sx = s_x.astype(np.float32)
    q = np.zeros(x.shape, dtype=np.int8)
    rows = np.nonzero(sx != 0)[0]
    if rows.size:
        q[rows] = np.clip(np.rint(x[rows] / sx[rows, None]), -X_QMAX, X_QMAX).astype(np.int8)
    return q, s_x


# ---------------------------------------------------------------------------
# O5  exact integer contraction acc[m, n] = sum_k qx[m, k] * w_hat[n, k]
#     [QServe summary] "渐进式组量化": after dequantizing to the INT8 intermediate the
#     GEMM runs as a W8A8 INT8 matmul; [QServe review] §4 step 3 (INT8 x INT8 with
#     INT32 accumulation).  An fp64 matmul of integer-valued arrays is exact here:
#     every partial sum is below 2^53.
# ---------------------------------------------------------------------------
def contract(qx: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    a = np.asarray(qx, dtype=np.float64)
    b = np.asarray(w_hat, dtype=np.float64)
    k = a.shape[1]
    assert k * 127 * 128 < 2 ** 53
    acc = a @ b.T
    if acc.size:
        assert np.all(np.abs(acc) < 2 ** 31), "INT32 accumulator range exceeded"
    return acc.astype(np.int32)


# ---------------------------------------------------------------------------
# O6  epilogue out = acc * (s_X[m] * s_W[n]) in fp32, rounded to fp16 (reading R7)
#     [QServe summary] O = (Q_X Q_W) ⊙ (s_W × s_X) - ...  (the subtracted zero-point
#     term is absent in the per-group kernel: zeros are applied in the main loop).
# ---------------------------------------------------------------------------
def epilogue_fp32(acc: np.ndarray, s_x16: np.ndarray, s_w16: np.ndarray) -> np.ndarray:
    sx = np.asarray(s_x16, dtype=np.float16).astype(np.float32)
    sw = np.asarray(s_w16, dtype=np.float16).astype(np.float32)
    scale = sx[:, None] * sw[None, :]                        # exact (fp16 x fp16 fits fp32)
    return np.asarray(acc).astype(np.float32) * scale


def epilogue(acc: np.ndarray, s_x16: np.ndarray, s_w16: np.ndarray) -> np.ndarray:
    return epilogue_fp32(acc, s_x16, s_w16).astype(np.float16)


# ---------------------------------------------------------------------------
# O7  storage layout of the packed weights and their group metadata.
#     [QServe review] §3.2 compute-aware weight reordering: weights are stored offline
#     in the order the kernel consumes them, so each lane issues one 128-bit load per
#     step; zeros and scales are reordered the same way.  The byte order below is this
#     library's own (the pages fix only the principle):
#
#       strip b = n // 16, column-in-strip c = n % 16, group j = k // 128,
#       within the group k = 128 j + 64 half + 16 h + i  (half in {0,1}, h in 0..3,
#       i in 0..15).
#       packed[((b * G + j) * 64 + 16 h + c) * 16 + i]
#           = q_u4[n, 128 j + 16 h + i] | q_u4[n, 128 j + 64 + 16 h + i] << 4
#       meta[(b * G + j) * 16 + c] = s_u8[n, j] | z[n, j] << 8       (uint16)
#       s_W stays fp16 [N] in natural order.
# ---------------------------------------------------------------------------
def pack_codes(q_u4: np.ndarray) -> np.ndarray:
    """UINT4 codes [N, K] -> packed uint8 [N*K/2] in the order above."""
    q = np.asarray(q_u4, dtype=np.uint16)
    n_total, k_total = q.shape
    if n_total % 16 or k_total % GROUP:
        raise ValueError("N must be a multiple of 16 and K a multiple of 128")
    g_total = k_total // GROUP
    off = np.arange(n_total * k_total // 2, dtype=np.int64)
    i = off % 16
    c = (off // 16) % 16
    h = (off // 256) % 4
    j = (off // 1024) % g_total
    b = off // (1024 * g_total)
    n = 16 * b + c
    k_lo = GROUP * j + 16 * h + i
    return (q[n, k_lo] | (q[n, k_lo + 64] << 4)).astype(np.uint8)


def pack_weights(q_u4: np.ndarray, z: np.ndarray, s_u8: np.ndarray):
    """-> (packed uint8 [N*K/2], meta uint16 [N*K/128])."""
    packed = pack_codes(q_u4)
    n_total, k_total = np.asarray(q_u4).shape
    g_total = k_total // GROUP

    moff = np.arange(n_total * g_total, dtype=np.int64)
    mc = moff % 16
    mj = (moff // 16) % g_total
    mb = moff // (16 * g_total)
    mn = 16 * mb + mc
    meta = (np.asarray(s_u8, dtype=np.uint16)[mn, mj]
            | (np.asarray(z, dtype=np.uint16)[mn, mj] << 8)).astype(np.uint16)
    return packed, meta


def quantize_pack_weights(w16: np.ndarray):
    """The whole offline step: W fp16 [N, K] -> (packed, meta, s_W fp16 [N])."""
    q_s8, s_w = quantize_weights_level0(w16)
    q_u4, z, s_u8 = quantize_weights_level1(q_s8)
    packed, meta = pack_weights(q_u4, z, s_u8)
    return packed, meta, s_w


# ---------------------------------------------------------------------------
# the whole runtime path, from fp16 inputs to the GEMM result
# ---------------------------------------------------------------------------
def w4a8_reference(x16: np.ndarray, w16: np.ndarray):
    """Returns a dict with every intermediate of the path for X fp16 [M,K], W fp16 [N,K]."""
    q_s8, s_w = quantize_weights_level0(w16)
    q_u4, z, s_u8 = quantize_weights_level1(q_s8)
    w_hat = dequantize_level1(q_u4, z, s_u8)
    qx, s_x = quantize_activations(x16)
    acc = contract(qx, w_hat)
    ref32 = epilogue_fp32(acc, s_x, s_w)
    return {
        "q_s8": q_s8, "s_w": s_w, "q_u4": q_u4, "z": z, "s_u8": s_u8, "w_hat": w_hat,
        "qx": qx, "s_x": s_x, "acc": acc, "ref32": ref32, "out": ref32.astype(np.float16),
    }


# ---------------------------------------------------------------------------
# O8  per-channel W4A8 (the format without groups): per output channel asymmetric
#     UINT4 with an integer zero and an fp16 scale
#     [QServe summary] "整数量化": Q = round(X/s + z), s = (Xmax - Xmin)/(qmax - qmin),
#     z = round(qmin - Xmin/s), here with one (s, z) per output channel ("逐通道W4A8
#     GEMM中的快速反量化": the zero point is per channel, so it can leave the main
#     loop); [Inference chapter] §4.1 asymmetric quantizer; readings R1, R2, R4, R8, R12.
# ---------------------------------------------------------------------------
def quantize_weights_per_channel(w16: np.ndarray):
    """W fp16 [N, K] -> (q_u4 uint8 [N, K], z uint8 [N], s_W fp16 [N])."""
    w = np.asarray(w16, dtype=np.float16).astype(np.float32)
    lo = np.minimum(w.min(axis=1), np.float32(0))                   # R4
    hi = np.maximum(w.max(axis=1), np.float32(0))
    s_w = ((hi - lo) / np.float32(U4_MAX)).astype(np.float16)     # fp32 subtract, divide; RNE
    sw = s_w.astype(np.float32)
    q = np.zeros(w.shape, dtype=np.uint8)
    z = np.zeros(w.shape[0], dtype=np.uint8)
    rows = np.nonzero(sw != 0)[0]                                  # R8
    if rows.size:
        zr = np.clip(np.rint(-lo[rows] / sw[rows]), 0, U4_MAX)     # z = round(qmin - Xmin/s)
        qr = np.clip(zr[:, None] + np.rint(w[rows] / sw[rows, None]), 0, U4_MAX)   # R2
        z[rows] = zr.astype(np.uint8)
        q[rows] = qr.astype(np.uint8)
    return q, z, s_w


def dequantize_per_channel(q_u4: np.ndarray, z: np.ndarray) -> np.ndarray:
    """-> (q - z) int16 [N, K], the weight in units of its channel scale s_W."""
    return np.asarray(q_u4, dtype=np.int16) - np.asarray(z, dtype=np.int16)[:, None]


# ---------------------------------------------------------------------------
# O9  t[m] = sum_k qx[m, k], the activation row sum of the per-channel epilogue
#     [QServe summary] "逐通道W4A8 GEMM中的快速反量化": the second term becomes
#     t_X x (z_W ⊙ s_W) with t_X = X 1_k, precomputed by the preceding memory-bound
#     kernel; reading R13 (over the quantized activations).
# ---------------------------------------------------------------------------
def activation_row_sums(qx: np.ndarray) -> np.ndarray:
    return np.asarray(qx, dtype=np.int64).sum(axis=1).astype(np.int32)


def w4a8_pc_reference(x16: np.ndarray, w16: np.ndarray):
    """Every intermediate of the per-channel path for X fp16 [M,K], W fp16 [N,K].
    acc = sum_k qx (q - z) (exact), out = fp16(acc * (s_X * s_W)) (R7, R13)."""
    q_u4, z, s_w = quantize_weights_per_channel(w16)
    w_hat = dequantize_per_channel(q_u4, z)
    qx, s_x = quantize_activations(x16)
    acc = contract(qx, w_hat)
    ref32 = epilogue_fp32(acc, s_x, s_w)
    return {
        "q_u4": q_u4, "z": z, "s_w": s_w, "w_hat": w_hat, "qx": qx, "s_x": s_x,
        "t": activation_row_sums(qx), "acc": acc, "ref32": ref32, "out": ref32.astype(np.float16),
    }
