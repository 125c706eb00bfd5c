"""Pins of the KV4 oracle (oracle/kv4_oracle.py): the per-head INT4 quantizer against
exact rational arithmetic and its error bound, degenerate vectors, scale
invariance; decode attention against closed forms and a pure-Python evaluation."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import kv4_oracle as kv
from tests.exact_float import FP16, FP32, round_float, rne_int


def _scale_zero_exact(lo, hi):
    s = round_float(round_float(round_float(hi - lo, FP32) / 15, FP32), FP16)
    return s, (rne_int(round_float(-lo / s, FP32)) if s != 0 else 0)


def _quant_exact(x16):
    """R17 by rationals: over [lo, hi] = [min x, max x], s = RN16(RN32(RN32(hi - lo) /
    15)), z = rne(RN32(-lo / s)); if s = 0 or |z| > 1024, the same over [min(lo, 0),
    max(hi, 0)]; q = clamp(z + rne(RN32(x / s)), 0, 15)."""
    xs = [Fraction(float(v)) for v in x16]
    lo, hi = min(xs), max(xs)
    s, z = _scale_zero_exact(lo, hi)
    if s == 0 or abs(z) > 1024:
        s, z = _scale_zero_exact(min(lo, 0), max(hi, 0))
    if s == 0:
        return [0] * len(xs), s, 0
    q = [min(max(z + rne_int(round_float(x / s, FP32)), 0), 15) for x in xs]
    return q, s, z


@pytest.mark.parametrize("scale", [1e-3, 0.7, 40.0])
def test_kv_quantize_matches_exact_rationals(scale):
    rng = np.random.default_rng(int(scale * 1000))
    x = (rng.standard_normal((10, 128)) * scale).astype(np.float16)
    x[1] = np.abs(x[1])                              # one-signed vectors: z < 0 / z > 15
    x[2] = -np.abs(x[2])
    x[3] = np.abs(x[3]) + np.float16(3 * scale)      # one-signed, offset from 0
    x[4] = -x[3]
    x[5] = (np.float16(40 * scale) + x[5] * np.float16(0.02)).astype(np.float16)   # narrow, far from 0
    x[6] = np.float16(2.5 * scale)                   # constant: s = 0 over its own range
    x[7] = (np.float16(1000 * scale) + np.abs(x[7]) * np.float16(0.01)).astype(np.float16)  # |z| > 1024
    x[8, :64] = np.float16(scale)                    # two values only
    x[8, 64:] = np.float16(3 * scale)
    q, s, z = kv.kv_quantize(x)
    for i in range(10):
        wq, ws, wz = _quant_exact(x[i])
        assert [int(v) for v in q[i]] == wq
        assert Fraction(float(s[i])) == ws and float(z[i]) == wz


def test_kv_quantize_error_bound():
    """|x - (q - z) s| <= s / 2 (+ the fp16 rounding of s: relative 2^-11 of the
    range, 15 s) for every element; zeros are integers in [-1024, 1024]; codes span
    [0, 15]; one-signed vectors take the step of their own range (the widened range
    would double it or more)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 128)) * rng.uniform(0.01, 10, (200, 1))).astype(np.float16)
    x[::7] = np.abs(x[::7]) + np.float16(3)              # one-signed, offset away from 0
    q, s, z = kv.kv_quantize(x)
    s64 = s.astype(np.float64)[:, None]
    xd = (q.astype(np.float64) - z.astype(np.float64)[:, None]) * s64
    err = np.abs(xd - x.astype(np.float64))
    assert np.all(err <= s64 / 2 + 15 * s64 * 2.0 ** -10)
    assert q.max() == 15 and q.min() == 0
    assert np.all(np.abs(z) <= 1024) and np.array_equal(z, np.rint(z))
    own = (x[::7].max(1).astype(np.float32) - x[::7].min(1).astype(np.float32)) / 15
    assert np.allclose(s[::7].astype(np.float32), own, rtol=2.0 ** -10)
    assert np.all(z[::7] < 0)


def test_kv_quantize_degenerate_vectors():
    """All zero; constant (own range 0: the widened range [0, 2.5]); a single
    non-zero; a narrow range far from 0 (z beyond 1024: widened); a two-valued
    one-signed vector (own range: exact)."""
    x = np.zeros((6, 128), np.float16)
    x[1] = 2.5                                            # constant: lo = 0, s = 1/6, z = 0, q = 15
    x[2, 7] = -0.375                                      # a single non-zero
    x[3] = 100.0
    x[3, ::2] = 100.0625                                  # own range 1/16: z = -24000 -> widened
    x[4, :64] = 1.0                                       # own range [1, 2.5]: s = 0.1, z = -10
    x[4, 64:] = 2.5
    x[5] = -x[4]                                          # [-2.5, -1]: s = 0.1, z = 25
    q, s, z = kv.kv_quantize(x)
    assert float(s[3]) == float(np.float16(np.float32(100.0625) / 15)) and float(z[3]) == 0
    assert np.all(q[3] == 15)
    assert float(s[4]) == float(np.float16(0.1)) and float(z[4]) == -10
    assert np.all(q[4, :64] == 0) and np.all(q[4, 64:] == 15)
    assert float(z[5]) == 25 and np.all(q[5, :64] == 15) and np.all(q[5, 64:] == 0)
    back = kv.kv_dequantize(q, s, z).astype(np.float64)
    assert float(s[0]) == 0 and float(z[0]) == 0 and not q[0].any() and not back[0].any()
    assert float(z[1]) == 0 and np.all(q[1] == 15) and np.allclose(back[1], 2.5, rtol=2.0 ** -10)
    assert float(z[2]) == 15 and q[2, 7] == 0 and np.all(np.delete(q[2], 7) == 15)
    assert abs(back[2, 7] + 0.375) <= 2.0 ** -10 and not np.delete(back[2], 7).any()


@pytest.mark.parametrize("j", [-5, 4])
def test_kv_quantize_power_of_two_invariance(j):
    rng = np.random.default_rng(j + 20)
    x = rng.standard_normal((8, 128)).astype(np.float16)
    q1, s1, z1 = kv.kv_quantize(x)
    q2, s2, z2 = kv.kv_quantize((x.astype(np.float32) * 2.0 ** j).astype(np.float16))
    assert np.array_equal(q1, q2) and np.array_equal(z1, z2)
    assert np.array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0 ** j)


def test_kv_dequantize_single_rounding():
    q = np.array([[0, 15, 7, 3]], np.uint8)
    s = np.array([0.1], np.float16)
    z = np.array([6.0], np.float16)
    got = kv.kv_dequantize(q, s, z)[0].astype(np.float64)
    for k in range(4):
        exact = (Fraction(int(q[0, k])) - 6) * Fraction(float(s[0]))
        assert got[k] == float(round_float(exact, FP16))


def test_attention_uniform_keys_average_values():
    """Equal keys: every score is the same, the output is the mean of the values."""
    rng = np.random.default_rng(4)
    S, HKV, D, H = 37, 2, 128, 8
    K = np.repeat(rng.standard_normal((1, HKV, D)).astype(np.float16), S, 0)
    V = rng.standard_normal((S, HKV, D)).astype(np.float16)
    q = rng.standard_normal((H, D)).astype(np.float16)
    o = kv.decode_attention(q, K, V, HKV).astype(np.float64)
    for h in range(H):
        assert np.allclose(o[h], V[:, h // 4, :].astype(np.float64).mean(0), atol=2e-3, rtol=2e-3)


def test_attention_one_dominant_key():
    """One key aligned with q and far larger than the rest: its value comes out."""
    D = 128
    q = np.zeros((1, D), np.float16)
    q[0, 0] = 8.0
    K = np.zeros((5, 1, D), np.float16)
    K[3, 0, 0] = 200.0                                  # score 1600 / sqrt(128) ~ 141
    V = np.arange(5 * D, dtype=np.float32).reshape(5, 1, D).astype(np.float16) / 64
    o = kv.decode_attention(q, K, V, 1)
    assert np.array_equal(o[0].view(np.uint16), V[3, 0].view(np.uint16))


def test_attention_gqa_head_mapping():
    """Head h reads KV head h // r: give each KV head distinct constant values."""
    S, HKV, D, H = 9, 4, 128, 16
    K = np.zeros((S, HKV, D), np.float16)
    V = np.zeros((S, HKV, D), np.float16)
    for g in range(HKV):
        V[:, g, :] = g + 1
    q = np.ones((H, D), np.float16)
    o = kv.decode_attention(q, K, V, HKV)
    for h in range(H):
        assert np.all(o[h] == h // 4 + 1)


def test_attention_brute_force_python():
    """Pure-Python loops with math.exp on a small case."""
    rng = np.random.default_rng(5)
    S, HKV, D, H = 6, 2, 128, 4
    q = rng.standard_normal((H, D)).astype(np.float16)
    K = rng.standard_normal((S, HKV, D)).astype(np.float16)
    V = rng.standard_normal((S, HKV, D)).astype(np.float16)
    o = kv.decode_attention(q, K, V, HKV).astype(np.float64)
    for h in range(H):
        g = h // 2
        sc = [sum(float(q[h, d]) * float(K[t, g, d]) for d in range(D)) / math.sqrt(D) for t in range(S)]
        m = max(sc)
        w = [math.exp(v - m) for v in sc]
        tot = sum(w)
        for d in range(0, D, 17):
            ref = sum(w[t] * float(V[t, g, d]) for t in range(S)) / tot
            assert abs(o[h, d] - ref) <= 2.0 ** -11 * abs(ref) + 1e-7


# ---------------------------------------------------------------------------
# SmoothAttention (R20)
# ---------------------------------------------------------------------------
def _keys_with_outliers(rng, n=200, h_kv=2, D=128):
    k = rng.standard_normal((n, h_kv, D)).astype(np.float32)
    k[:, :, [5, 70, 100]] *= 10.0                            # fixed outlier channels per head
    return k.astype(np.float16)


def test_smooth_lambda_pairs_and_closed_form():
    """lambda_i = lambda_{i+D/2} = sqrt(max(max|K_i|, max|K_{i+D/2}|)), computed here
    by hand from the samples with Python floats."""
    rng = np.random.default_rng(20)
    k = _keys_with_outliers(rng)
    lam = kv.smooth_attention_lambda(k, 0.5)
    D = k.shape[2]
    assert np.array_equal(lam[:, : D // 2], lam[:, D // 2:])
    for g in range(k.shape[1]):
        for i in (0, 5, 37, 63):
            a = max(abs(float(x)) for x in k[:, g, i])
            b = max(abs(float(x)) for x in k[:, g, i + D // 2])
            want = np.float32(math.sqrt(max(a, b)))               # sqrt of an fp32 value, rounded to fp32
            assert lam[g, i] == want and lam[g, i + D // 2] == want


def test_smooth_lambda_alpha_zero_and_zero_channels():
    rng = np.random.default_rng(21)
    k = _keys_with_outliers(rng)
    assert np.all(kv.smooth_attention_lambda(k, 0.0) == 1.0)
    k[:, 0, 3] = 0
    k[:, 0, 3 + 64] = 0
    lam = kv.smooth_attention_lambda(k, 0.5)
    assert lam[0, 3] == 1.0 and lam[0, 67] == 1.0            # a pair that never leaves 0


def test_smooth_fold_preserves_scores_and_flattens_keys():
    """(q Lambda) . (k Lambda^-1) = q . k: scores from the folded projections equal
    the unfolded ones up to the fp16 rounding of the folded weights; the smoothed
    keys' channel maxima are max|K_i| / lambda_i <= lambda_i, so the largest is the
    square root of the largest raw maximum (outliers compressed)."""
    rng = np.random.default_rng(22)
    h, h_kv, D, dm = 4, 2, 128, 64
    wq = (rng.standard_normal((h * D, dm)) * 0.05).astype(np.float16)
    wk = (rng.standard_normal((h_kv * D, dm)) * 0.05).astype(np.float16)
    wk[[5, 70, D + 100]] *= 10                               # key outlier channels from the weights
    x = rng.standard_normal((300, dm)).astype(np.float16)
    k = (x.astype(np.float64) @ wk.astype(np.float64).T).reshape(300, h_kv, D).astype(np.float16)
    lam = kv.smooth_attention_lambda(k, 0.5)
    wq2, wk2 = kv.smooth_attention_fold(wq, wk, lam, h, h_kv)
    q = x.astype(np.float64) @ wq.astype(np.float64).T
    kk = x.astype(np.float64) @ wk.astype(np.float64).T
    q2 = x.astype(np.float64) @ wq2.astype(np.float64).T
    k2 = x.astype(np.float64) @ wk2.astype(np.float64).T
    for hq in range(h):
        g = hq // (h // h_kv)
        s1 = q[:, hq * D:(hq + 1) * D] @ kk[:, g * D:(g + 1) * D].T
        s2 = q2[:, hq * D:(hq + 1) * D] @ k2[:, g * D:(g + 1) * D].T
        scale = np.abs(q[:, hq * D:(hq + 1) * D]) @ np.abs(kk[:, g * D:(g + 1) * D]).T
        assert np.all(np.abs(s2 - s1) <= 2.0 ** -9 * scale + 1e-12)   # two fp16 roundings of weights
    kmax = np.abs(k.astype(np.float32)).max(axis=0)
    smoothed = kmax / lam
    assert np.all(smoothed <= lam * (1 + 2.0 ** -20))
    assert np.isclose(smoothed.max(), math.sqrt(kmax.max()), rtol=2.0 ** -20)


def test_smooth_reduces_kv4_attention_error():
    """The method's purpose on keys with outlier channels: KV4 attention over
    smoothed keys (queries scaled back) is closer to the unquantized attention."""
    rng = np.random.default_rng(23)
    n, h_kv, h, D = 256, 2, 4, 128
    k = _keys_with_outliers(rng, n, h_kv, D)
    v = rng.standard_normal((n, h_kv, D)).astype(np.float16)
    q = rng.standard_normal((h, D)).astype(np.float16)
    exact = kv.decode_attention(q, k, v, h_kv).astype(np.float64)
    plain = kv.attention_reference(q, k, v, h_kv).astype(np.float64)
    lam = kv.smooth_attention_lambda(k, 0.5)
    ks = (k.astype(np.float32) / lam[None]).astype(np.float16)
    qs = (q.astype(np.float32) * np.repeat(lam, h // h_kv, axis=0)).astype(np.float16)
    smooth = kv.attention_reference(qs, ks, v, h_kv).astype(np.float64)
    assert np.abs(smooth - exact).mean() < 0.5 * np.abs(plain - exact).mean()
