"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Each test checks the oracle against something other than itself: the worked example
printed on the pages, exhaustive sweeps of the protective-range derivation,
hand-computed textbook cases, exact rational arithmetic, closed-form error bounds,
invariances, and brute force on tiny inputs.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import qoq_oracle as o
from tests.exact_float import FP16, FP32, round_float, rne_int
from w4a8_mixed_precision_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# P1: the pages' worked overflow example
# ---------------------------------------------------------------------------
def test_worked_example_overflow():
    g = _golden("worked_example_overflow.json")
    grp = np.zeros((1, 128), np.int64)
    grp[0, 0] = g["group_min"]
    grp[0, 1] = g["group_max"]
    grp[0, 2:] = np.linspace(g["group_min"], g["group_max"], 126).round()
    q, z, s = o.quantize_weights_level1(grp)
    assert int(s[0, 0]) == g["expected_scale"]
    assert int(z[0, 0]) == g["expected_zero"]
    idx = int(np.nonzero(grp[0] == g["value"])[0][0])
    assert int(q[0, idx]) == g["expected_code_of_value"]
    w_hat = o.dequantize_level1(q, z, s)
    assert int(w_hat[0, idx]) == g["expected_dequantized_value"]
    assert int(w_hat.max()) > g["int8_max"]          # the overflow the pages warn about


def test_worked_example_rejects_joint_rounding():
    """Rounding x/s + z jointly (half to even) would give code 14 for the value 120,
    contradicting the pages' 15; the oracle adds z after rounding (reading R2)."""
    g = _golden("worked_example_overflow.json")
    s, z, v = g["expected_scale"], g["expected_zero"], g["value"]
    assert rne_int(Fraction(v, s) + z) == 14
    assert z + rne_int(Fraction(v, s)) == g["expected_code_of_value"]


# ---------------------------------------------------------------------------
# P2: the protective-range derivation, swept exhaustively
# ---------------------------------------------------------------------------
def _all_groups(limit):
    """Every (lo, hi, x) with -limit <= lo <= 0 <= hi <= limit and lo <= x <= hi,
    as 3-element groups [lo, hi, x]."""
    rows = []
    for lo in range(-limit, 1):
        for hi in range(0, limit + 1):
            xs = np.arange(lo, hi + 1, dtype=np.int64)
            blk = np.empty((xs.size, 3), np.int64)
            blk[:, 0] = lo
            blk[:, 1] = hi
            blk[:, 2] = xs
            rows.append(blk)
    return np.concatenate(rows)


def test_protective_range_exhaustive_bounds():
    g = _golden("worked_example_overflow.json")
    lo_r, hi_r = g["protective_range"]
    groups = _all_groups(hi_r)
    assert -lo_r == hi_r
    q, z, s = o.quantize_weights_level1(groups, group=3)
    w_hat = o.dequantize_level1(q, z, s, group=3).astype(np.int64)
    s64 = s.astype(np.int64)[:, 0]
    z64 = z.astype(np.int64)[:, 0]
    q64 = q.astype(np.int64)
    assert s64.max() <= g["scale_upper_bound"]
    assert z64.max() <= 15 and q64.max() <= 15 and q64.min() >= 0
    # the dequantized intermediate stays inside INT8 (the point of the range)
    assert w_hat.max() <= 127 and w_hat.min() >= -128
    # dequantized value within half a group step of the level-0 code
    assert np.all(2 * np.abs(w_hat - groups) <= s64[:, None])
    # byte-lane products of the multiply-then-subtract order never exceed a byte
    assert (q64 * s64[:, None]).max() <= 255
    assert (z64 * s64).max() <= 255


def test_unprotected_range_overflows():
    """Without the protective range ([-127, 127]) the same cascade leaves INT8."""
    groups = _all_groups(127)
    q, z, s = o.quantize_weights_level1(groups, group=3)
    w_hat = o.dequantize_level1(q, z, s, group=3)
    assert w_hat.max() > 127


def test_scale_bound_formula():
    g = _golden("worked_example_overflow.json")
    assert Fraction(127 - (-128), 15 - 0) == g["scale_upper_bound"]


# ---------------------------------------------------------------------------
# textbook symmetric quantization cases, hand computed
# ---------------------------------------------------------------------------
def test_level0_textbook_ties_to_even():
    # absmax 119 -> scale exactly 1, codes are the values rounded half to even
    row = np.array([119.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -118.5] + [0.0] * 120, np.float16)
    q, s = o.quantize_weights_level0(row[None, :])
    assert float(s[0]) == 1.0
    assert q[0, :8].tolist() == [119, 2, 4, -2, 0, 0, 2, -118]
    # absmax 238 -> scale exactly 2
    row2 = np.array([-238.0, 5.0, 7.0, -5.0, 1.0, 3.0] + [0.0] * 122, np.float16)
    q2, s2 = o.quantize_weights_level0(row2[None, :])
    assert float(s2[0]) == 2.0
    assert q2[0, :6].tolist() == [-119, 2, 4, -2, 0, 2]


def test_activation_textbook_ties_to_even():
    row = np.array([[-127.0, 2.5, 3.5, -2.5, 126.5, 0.5]], np.float16)
    q, s = o.quantize_activations(row)
    assert float(s[0]) == 1.0
    assert q[0].tolist() == [-127, 2, 4, -2, 126, 0]


def test_zero_rows():
    q, s = o.quantize_weights_level0(np.zeros((2, 256), np.float16))
    assert np.all(q == 0) and np.all(s == 0)
    q_u4, z, su = o.quantize_weights_level1(q)
    assert np.all(su == 1) and np.all(z == 0) and np.all(q_u4 == 0)
    qx, sx = o.quantize_activations(np.zeros((3, 256), np.float16))
    assert np.all(qx == 0) and np.all(sx == 0)
    acc = o.contract(qx, o.dequantize_level1(q_u4, z, su))
    assert acc.shape == (3, 2) and np.all(acc == 0)


# ---------------------------------------------------------------------------
# fp32 / fp16 steps checked with exact rational arithmetic
# ---------------------------------------------------------------------------
def _exact_sym_quant(row16, qmax):
    vals = [Fraction(float(v)) for v in row16]
    a = max(abs(v) for v in vals)
    s = round_float(round_float(a / qmax, FP32), FP16)
    if s == 0:
        return [0] * len(vals), s
    codes = []
    for v in vals:
        r = round_float(v / s, FP32)
        codes.append(max(-qmax, min(qmax, rne_int(r))))
    return codes, s


@pytest.mark.parametrize("qmax,fn", [(119, o.quantize_weights_level0), (127, o.quantize_activations)])
def test_symmetric_quant_exact_rational(qmax, fn):
    rng = np.random.default_rng(7)
    rows = [rng.standard_normal(64).astype(np.float16) * np.float16(sc)
            for sc in (1e-3, 0.02, 1.0, 30.0)]
    # fp16 subnormal territory: scale itself rounds coarsely, the clamp must fire
    rows.append((rng.standard_normal(64) * 2e-6).astype(np.float16))
    rows.append(np.array([6e-8] + [0.0] * 63, np.float16))
    x = np.stack(rows)
    q, s = fn(x)
    for r in range(x.shape[0]):
        codes, sc = _exact_sym_quant(x[r], qmax)
        assert Fraction(float(s[r])) == sc
        assert q[r].tolist() == codes


def test_level0_absmax_maps_to_119():
    L = wl.find("tiny")
    w = wl.weights_fp16(L)
    q, s = o.quantize_weights_level0(w)
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 119)
    assert q.min() >= -119 and q.max() <= 119


# ---------------------------------------------------------------------------
# P3: lossless special case -> the GEMM is a per-channel W8A8 integer GEMM
# ---------------------------------------------------------------------------
def test_lossless_groups_reduce_to_w8a8():
    rng = np.random.default_rng(11)
    N, K, M = 32, 256, 5
    q_s8 = np.zeros((N, K), np.int64)
    for n in range(N):
        for j in range(K // 128):
            lo = -int(rng.integers(0, 16))
            hi = lo + 15 if lo + 15 >= 0 else 0
            hi = max(0, min(hi, 15 + lo))
            q_s8[n, 128 * j:128 * (j + 1)] = rng.integers(lo, hi + 1, 128)
    q, z, s = o.quantize_weights_level1(q_s8)
    assert np.all(s == 1)
    w_hat = o.dequantize_level1(q, z, s)
    assert np.array_equal(w_hat.astype(np.int64), q_s8)
    qx = rng.integers(-127, 128, (M, K)).astype(np.int8)
    acc = o.contract(qx, w_hat)
    assert np.array_equal(acc.astype(np.int64), qx.astype(np.int64) @ q_s8.T)


# ---------------------------------------------------------------------------
# P4: brute force on tiny shapes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 32, 256), (8, 16, 256)])
def test_contraction_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N + K)
    x16 = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    w16 = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    r = o.w4a8_reference(x16, w16)
    qx = r["qx"].astype(int).tolist()
    wh = r["w_hat"].astype(int).tolist()
    for m in range(M):
        for n in range(N):
            acc = 0
            for k in range(K):
                acc += qx[m][k] * wh[n][k]
            assert acc == int(r["acc"][m, n])
    # fp64 product of the dequantized operands vs the fp16 output: one fp16 rounding
    # (2^-11 relative) plus two fp32 roundings separate them
    sx = r["s_x"].astype(np.float64)
    sw = r["s_w"].astype(np.float64)
    ref64 = (r["qx"].astype(np.float64) * sx[:, None]) @ (r["w_hat"].astype(np.float64) * sw[:, None]).T
    out = r["out"].astype(np.float64)
    bound = np.abs(ref64) * (2.0 ** -11 + 2.0 ** -22) + 2.0 ** -25
    assert np.all(np.abs(out - ref64) <= bound)


def test_pipeline_approximates_fp_matmul():
    """End-to-end: the quantized GEMM approximates the fp matmul within the error the
    two quantizers allow (closed form: per element, |x - qx sx| <= sx/2 and
    |w - w_hat sw| <= sw (1 + s_u8) / 2)."""
    L = wl.find("tiny")
    w16 = wl.weights_fp16(L)
    x16 = wl.activations_fp16(L, 8)
    r = o.w4a8_reference(x16, w16)
    x = x16.astype(np.float64)
    w = w16.astype(np.float64)
    sx = r["s_x"].astype(np.float64)[:, None]
    sw = r["s_w"].astype(np.float64)[:, None]
    ex = np.abs(x - r["qx"] * sx)
    assert np.all(ex <= sx / 2 * (1 + 1e-6))
    e0 = np.abs(w - r["q_s8"] * sw)
    assert np.all(e0 <= sw / 2 * (1 + 1e-6))
    su = np.repeat(r["s_u8"].astype(np.float64), 128, axis=1)
    ew = np.abs(w - r["w_hat"] * sw)
    assert np.all(ew <= sw * (1 + su) / 2 * (1 + 1e-6))
    exact = x @ w.T
    xq = r["qx"] * sx
    wq = r["w_hat"] * sw
    bound = ex @ np.abs(w).T + np.abs(xq) @ ew.T
    assert np.all(np.abs(r["ref32"] - exact) <= bound * (1 + 1e-3) + np.abs(exact) * 1e-6 + 1e-6)


# ---------------------------------------------------------------------------
# P6: invariances
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("j", [-3, 2])
def test_power_of_two_scaling_invariance(j):
    L = wl.find("tiny")
    w16 = wl.weights_fp16(L)[:64]
    x16 = wl.activations_fp16(L, 8)
    r = o.w4a8_reference(x16, w16)
    f = np.float16(2.0 ** j)
    r2 = o.w4a8_reference(x16 * f, w16 * f)
    for key in ("qx", "q_u4", "z", "s_u8", "acc"):
        assert np.array_equal(r[key], r2[key]), key
    assert np.array_equal(r2["s_x"].astype(np.float32), r["s_x"].astype(np.float32) * 2.0 ** j)
    assert np.array_equal(r2["s_w"].astype(np.float32), r["s_w"].astype(np.float32) * 2.0 ** j)


def test_row_permutation_equivariance():
    L = wl.find("tiny")
    w16 = wl.weights_fp16(L)[:32]
    x16 = wl.activations_fp16(L, 8)
    perm = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    r = o.w4a8_reference(x16, w16)
    r2 = o.w4a8_reference(x16[perm], w16)
    assert np.array_equal(r2["acc"], r["acc"][perm])
    assert np.array_equal(r2["out"], r["out"][perm])


# ---------------------------------------------------------------------------
# rne_div against exact rationals
# ---------------------------------------------------------------------------
def test_rne_div_exhaustive_small():
    a = np.arange(-300, 301)
    for b in range(1, 20):
        got = o.rne_div(a, b)
        want = np.array([round(Fraction(int(v), b)) for v in a])
        assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# packed layout: round trip by the inverse mapping and hand-computed bytes
# ---------------------------------------------------------------------------
def _unpack_by_position(packed, meta, N, K):
    """Inverse of the storage layout, written per (n, k) rather than per byte."""
    G = K // 128
    q = np.zeros((N, K), np.uint8)
    for n in range(N):
        b, c = divmod(n, 16)
        for k in range(K):
            j, kk = divmod(k, 128)
            half, rest = divmod(kk, 64)
            h, i = divmod(rest, 16)
            byte = int(packed[((b * G + j) * 64 + 16 * h + c) * 16 + i])
            q[n, k] = (byte >> 4) if half else (byte & 15)
    s = np.zeros((N, G), np.uint8)
    z = np.zeros((N, G), np.uint8)
    for n in range(N):
        b, c = divmod(n, 16)
        for j in range(G):
            v = int(meta[(b * G + j) * 16 + c])
            s[n, j] = v & 255
            z[n, j] = v >> 8
    return q, z, s


def test_pack_round_trip():
    rng = np.random.default_rng(3)
    N, K = 48, 384
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    z = rng.integers(0, 16, (N, K // 128)).astype(np.uint8)
    s = rng.integers(1, 18, (N, K // 128)).astype(np.uint8)
    packed, meta = o.pack_weights(q, z, s)
    assert packed.size == N * K // 2 and meta.size == N * K // 128
    q2, z2, s2 = _unpack_by_position(packed, meta, N, K)
    assert np.array_equal(q, q2) and np.array_equal(z, z2) and np.array_equal(s, s2)


def test_pack_hand_computed_bytes():
    N, K = 32, 256
    n_idx, k_idx = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    q = ((n_idx + 3 * k_idx) % 16).astype(np.uint8)
    z = np.zeros((N, 2), np.uint8)
    s = np.ones((N, 2), np.uint8)
    packed, _ = o.pack_weights(q, z, s)
    # byte 0: n=0, k=0 (lo) and k=64 (hi): q=0 and (3*64)%16=0 -> 0x00
    assert packed[0] == 0x00
    # byte 1: n=0, k=1 -> 3 ; k=65 -> 195%16=3 -> 0x33
    assert packed[1] == 0x33
    # byte 16: column c=1 (n=1), k=0 -> 1 ; k=64 -> (1+192)%16=1 -> 0x11
    assert packed[16] == 0x11
    # byte 256: h=1 -> k=16 for n=0: 48%16=0 ; k=80: 240%16=0 -> 0x00
    assert packed[256] == 0x00
    # byte 257: n=0, k=17: 51%16=3 ; k=81: 243%16=3 -> 0x33
    assert packed[257] == 0x33
    # byte 1024: next group j=1 of strip 0, n=0, k=128 -> 384%16=0
    assert packed[1024] == 0x00
    # byte 2048: strip b=1 (n=16), group 0, k=0 -> 16%16=0 ; k=64 -> 208%16=0
    assert packed[2048] == 0x00
    # byte 2049: n=16, k=1 -> 19%16=3 ; k=65 -> (16+195)%16=3
    assert packed[2049] == 0x33
    # byte 2048+16*5+2: n=21, k=2 -> 27%16=11 ; k=66 -> (21+198)%16=11
    assert packed[2048 + 80 + 2] == 0xBB


def test_generator_is_seeded():
    L = wl.find("tiny")
    a = wl.weights_fp16(L)
    b = wl.weights_fp16(L)
    assert np.array_equal(a, b)
    x1 = wl.activations_fp16(L, 8)
    assert np.array_equal(x1, wl.activations_fp16(L, 8))
    # outlier channels: about 2% of weight columns and 1% of activation columns are large
    big = (np.abs(a.astype(np.float32)).max(axis=0) > 0.15).sum()
    assert 5 <= big <= 20


# ---------------------------------------------------------------------------
# per-channel variant (readings R12, R13)
# ---------------------------------------------------------------------------
def _exact_pc_quant(row):
    """Per-channel asymmetric UINT4 of one fp16 row by exact rational arithmetic
    (IEEE fp32 subtract / divide and the fp16 scale rounding done on Fractions)."""
    vals = [Fraction(float(v)) for v in row]
    lo = min(min(vals), Fraction(0))
    hi = max(max(vals), Fraction(0))
    diff = round_float(hi - lo, FP32)
    s = round_float(round_float(diff / 15, FP32), FP16)
    if s == 0:
        return [0] * len(vals), 0, s
    z = max(0, min(15, rne_int(round_float(-lo / s, FP32))))
    q = [max(0, min(15, z + rne_int(round_float(v / s, FP32)))) for v in vals]
    return q, z, s


def test_per_channel_exact_rational():
    rng = np.random.default_rng(11)
    rows = [(rng.standard_normal(128) * sc).astype(np.float16) for sc in (1e-3, 0.02, 1.0, 40.0)]
    rows.append(np.abs(rng.standard_normal(128) * 0.1).astype(np.float16))        # all >= 0: z = 0
    rows.append(-np.abs(rng.standard_normal(128) * 0.1).astype(np.float16))       # all <= 0: z = 15
    rows.append((rng.standard_normal(128) * 3e-6).astype(np.float16))             # subnormal scale
    rows.append(np.zeros(128, np.float16))                                          # R8
    w = np.stack(rows)
    q, z, s = o.quantize_weights_per_channel(w)
    for r in range(w.shape[0]):
        qe, ze, se = _exact_pc_quant(w[r])
        assert Fraction(float(s[r])) == se
        assert int(z[r]) == ze
        assert q[r].tolist() == qe
    assert int(z[4]) == 0 and int(z[5]) == 15
    assert float(s[7]) == 0 and not q[7].any() and int(z[7]) == 0


@pytest.mark.parametrize("z0,e", [(0, 6), (7, 3), (15, 10), (4, 14)])
def test_per_channel_lossless_rows(z0, e):
    """Rows on the grid (k - z0) * 2^-e using all 16 codes: the scale, zero and codes
    are recovered exactly and the reconstruction is lossless."""
    rng = np.random.default_rng(z0 + e)
    k = rng.integers(0, 16, (3, 256))
    k[:, 0], k[:, 1] = 0, 15
    w = ((k - z0) * 2.0 ** -e).astype(np.float16)
    q, z, s = o.quantize_weights_per_channel(w)
    assert np.all(s.astype(np.float64) == 2.0 ** -e)
    assert np.all(z == z0)
    assert np.array_equal(q, k.astype(np.uint8))
    w_hat = o.dequantize_per_channel(q, z).astype(np.float64) * s.astype(np.float64)[:, None]
    assert np.array_equal(w_hat, w.astype(np.float64))


def test_per_channel_error_bound():
    """|(q - z) s - w| <= s/2 (plus the fp32 division's half-ulp) for every element
    that does not clamp; a clamp can only fire at the top of the range and then
    costs at most one step: the zero makes the bottom of the range code 0 exactly."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 512)) * rng.uniform(1e-3, 10, (64, 1))).astype(np.float16)
    q, z, s = o.quantize_weights_per_channel(w)
    wf = w.astype(np.float64)
    sf = s.astype(np.float64)[:, None]
    err = np.abs((q.astype(np.float64) - z.astype(np.float64)[:, None]) * sf - wf)
    unclamped = z.astype(np.int64)[:, None] + np.rint(w.astype(np.float32) / s.astype(np.float32)[:, None]) <= 15
    assert np.all(err[unclamped] <= sf.repeat(512, 1)[unclamped] * (0.5 + 2.0 ** -20))
    assert np.all(err <= sf * 1.01)
    assert np.all(q[np.arange(64), np.argmin(np.minimum(w, 0), axis=1)] == 0) or np.all(w.min(axis=1) >= 0)


def test_per_channel_matches_pages_affine_formula():
    """Away from exact ties, q = clip(round(w/s + z), 0, 15) with the pages' formula
    in fp64 gives the same codes as R2's z + rne(w/s)."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((32, 384)) * 0.05).astype(np.float16)
    q, z, s = o.quantize_weights_per_channel(w)
    ref = np.clip(np.rint(w.astype(np.float64) / s.astype(np.float64)[:, None] + z[:, None]), 0, 15)
    assert np.array_equal(q, ref.astype(np.uint8))


@pytest.mark.parametrize("j", [-3, 2])
def test_per_channel_power_of_two_invariance(j):
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float16)
    q1, z1, s1 = o.quantize_weights_per_channel(w)
    q2, z2, s2 = o.quantize_weights_per_channel((w.astype(np.float32) * 2.0 ** j).astype(np.float16))
    assert np.array_equal(q1, q2) and np.array_equal(z1, z2)
    assert np.array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0 ** j)


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 16, 256), (5, 32, 128)])
def test_per_channel_contraction_brute_force(M, N, K):
    """Pure-Python sums: acc = sum_k qx (q - z), and the pages' rearrangement
    sum_k qx q - z t with t = sum_k qx gives the same integers; the fp16 output is
    the fp32 product of acc and the two scales, rounded once."""
    rng = np.random.default_rng(M * 100 + N + K)
    x16 = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    w16 = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    r = o.w4a8_pc_reference(x16, w16)
    qx, q, z = r["qx"].tolist(), r["q_u4"].tolist(), r["z"].tolist()
    for m in range(M):
        t = sum(qx[m])
        assert t == int(r["t"][m])
        for n in range(N):
            direct = sum(qx[m][k] * (q[n][k] - z[n]) for k in range(K))
            split = sum(qx[m][k] * q[n][k] for k in range(K)) - z[n] * t
            assert direct == split == int(r["acc"][m, n])
            exact = Fraction(direct) * Fraction(float(r["s_x"][m])) * Fraction(float(r["s_w"][n]))
            assert float(r["out"][m, n]) == float(round_float(round_float(exact, FP32), FP16))
