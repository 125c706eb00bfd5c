"""Pins of the fused-producer oracle (oracle/fused_quant_oracle.py): RMSNorm +
quantization and SiLU(gate) * up + quantization.  Each check reaches the value by a
route other than the oracle's own code: exact rational arithmetic with explicit
IEEE rounding (tests/exact_float.py), closed forms, invariances and identities."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import fused_quant_oracle as fq
from oracle import qoq_oracle as o
from tests.exact_float import FP16, FP32, round_float


def _sqrt_rn32(v: Fraction) -> Fraction:
    """Correctly rounded fp32 square root of a positive rational, by bracketing."""
    r = Fraction(float(np.float32(np.sqrt(float(v)))))
    for _ in range(4):                       # walk to the fp32 whose half-ulp interval holds sqrt(v)
        e = r.numerator.bit_length() - r.denominator.bit_length()
        while Fraction(2) ** e > r:
            e -= 1
        ulp = Fraction(2) ** (e - 23)
        lo, hi = r - ulp / 2, r + ulp / 2
        if lo * lo > v:
            r = round_float(r - ulp, FP32)
        elif hi * hi < v:
            r = round_float(r + ulp, FP32)
        else:
            return r
    raise AssertionError("no bracket")


def _rmsnorm_exact(x16, g16, eps):
    """R14 by rationals: mean = RN32(sum x^2 / K), inv = RN32(1 / RN32(sqrt(RN32(mean
    + eps)))), y = RN16(RN32(RN32(x * inv) * gamma))."""
    M, K = x16.shape
    eps32 = Fraction(float(np.float32(eps)))
    out = np.empty((M, K), np.float16)
    for m in range(M):
        xs = [Fraction(float(v)) for v in x16[m]]
        mean = round_float(sum(v * v for v in xs) / K, FP32)
        root = _sqrt_rn32(round_float(mean + eps32, FP32))
        inv = round_float(1 / root, FP32)
        for k in range(K):
            t = round_float(xs[k] * inv, FP32)
            out[m, k] = np.float16(float(round_float(round_float(t * Fraction(float(g16[k])), FP32), FP16)))
    return out


@pytest.mark.parametrize("K", [8, 24, 136])
def test_rmsnorm_matches_exact_rationals(K):
    rng = np.random.default_rng(K)
    x = (rng.standard_normal((4, K)) * rng.choice([0.01, 1.0, 30.0], (4, 1))).astype(np.float16)
    g = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    want = _rmsnorm_exact(x, g, 1e-5)
    got = fq.rmsnorm_fp16(x, g, 1e-5)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_rmsnorm_constant_row_gives_gamma():
    """x = 2 everywhere: mean = 4, 4 + 2^-24 rounds to 4 in fp32, inv = 1/2 exactly,
    so y = gamma bit for bit."""
    rng = np.random.default_rng(3)
    g = rng.standard_normal(256).astype(np.float16)
    x = np.full((2, 256), 2.0, np.float16)
    y = fq.rmsnorm_fp16(x, g, 2.0 ** -24)
    assert np.array_equal(y[0].view(np.uint16), g.view(np.uint16))
    assert np.array_equal(y[1].view(np.uint16), g.view(np.uint16))


@pytest.mark.parametrize("j", [-4, 3])
def test_rmsnorm_power_of_two_invariance(j):
    """With eps below half an ulp of the mean, scaling x by 2^j scales the mean by
    4^j exactly and leaves y unchanged."""
    rng = np.random.default_rng(j + 10)
    x = rng.uniform(1.0, 1.9, (3, 64)).astype(np.float16)        # mean of squares in [1, 4)
    g = rng.standard_normal(64).astype(np.float16)
    y1 = fq.rmsnorm_fp16(x, g, 2.0 ** -30)
    y2 = fq.rmsnorm_fp16((x.astype(np.float32) * 2.0 ** j).astype(np.float16), g, 2.0 ** -30)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_rmsnorm_unit_rms():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 4096)) * 7).astype(np.float16)
    y = fq.rmsnorm_fp16(x, np.ones(4096, np.float16), 1e-5).astype(np.float64)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=2e-3)


def test_rmsnorm_zero_row_quantizes_to_zero():
    x = np.zeros((2, 128), np.float16)
    x[1, 5] = 3.0
    q, s, t = fq.rmsnorm_quantize(x, np.ones(128, np.float16), 1e-5)
    assert s[0] == 0 and not q[0].any() and t[0] == 0
    assert q[1, 5] == 127 and int(np.count_nonzero(q[1])) == 1 and t[1] == 127


def test_rmsnorm_quantize_hand_codes():
    """Constant x with eps 2^-24 gives y = gamma (above); with gamma = (n + 1/2) / 8,
    n = -127 .. 126, and one entry 15.875, the scale is exactly 1/8 and every code
    is a tie: rounded to even."""
    n = np.arange(-127, 127)
    g = np.zeros(512, np.float32)
    g[:254] = (n + 0.5) / 8
    g[300] = 15.875
    g16 = g.astype(np.float16)
    q, s, t = fq.rmsnorm_quantize(np.full((1, 512), 2.0, np.float16), g16, 2.0 ** -24)
    assert float(s[0]) == 0.125
    want = np.zeros(512, np.int64)
    want[:254] = np.where(n % 2 == 0, n, n + 1)                 # n + 1/2, ties to even
    want[300] = 127
    assert np.array_equal(q[0].astype(np.int64), want)
    assert int(t[0]) == int(want.sum())


def test_silu_symmetry_identity():
    """sigma(g) + sigma(-g) = 1, so SiLU(g) - SiLU(-g) = g (u = 1), in fp64."""
    g = np.linspace(-12, 12, 97).astype(np.float16)
    one = np.ones_like(g)
    d = fq.silu_mul_f64(g, one) - fq.silu_mul_f64(-g, one)
    assert np.allclose(d, g.astype(np.float64), rtol=0, atol=1e-13)


def test_silu_special_values():
    g = np.array([0.0, 30.0, -30.0, 4.0, -65504.0], np.float16)
    u = np.array([5.0, 0.5, 2.0, 0.0, 1.0], np.float16)
    h = fq.silu_mul_fp16(g, u).astype(np.float64)
    assert h[0] == 0.0                                   # SiLU(0) = 0
    assert h[1] == 15.0                                  # sigma(30) = 1 - 9.4e-14: g * u, rounded
    assert abs(h[2]) < 2.0 ** -24 * 8                    # -30 * 2 * sigma(-30) ~ -5.6e-12 -> fp16 0
    assert h[3] == 0.0                                   # u = 0
    assert h[4] == 0.0                                   # exp overflow: -65504 / inf -> -0


def test_silu_matches_logistic_form():
    """SiLU(g) u = g u sigma(g) with sigma(g) = 1 / (1 + exp(-g)) written other ways:
    (1 + tanh(g / 2)) / 2 for g >= 0 and exp(g) / (1 + exp(g)) for g < 0 (each free
    of cancellation there); fp64, then one fp16 rounding."""
    rng = np.random.default_rng(6)
    g = (rng.standard_normal(2000) * 3).astype(np.float16)
    u = (rng.standard_normal(2000) * 2).astype(np.float16)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    e = np.exp(np.minimum(g64, 0))
    sig = np.where(g64 >= 0, 0.5 + 0.5 * np.tanh(g64 / 2), e / (1 + e))
    alt = g64 * u64 * sig
    h = fq.silu_mul_f64(g, u)
    assert np.allclose(h, alt, rtol=1e-14, atol=1e-300)
    mism = np.count_nonzero(fq.silu_mul_fp16(g, u).view(np.uint16) != alt.astype(np.float16).view(np.uint16))
    assert mism <= 1                                      # only an fp16 near-tie may round apart


def test_silu_mul_quantize_is_quantizer_of_h():
    rng = np.random.default_rng(7)
    g = (rng.standard_normal((3, 256)) * 2).astype(np.float16)
    u = (rng.standard_normal((3, 256)) * 2).astype(np.float16)
    q, s, t = fq.silu_mul_quantize(g, u)
    h = fq.silu_mul_fp16(g, u).astype(np.float64)
    absmax = np.max(np.abs(h), axis=1)
    assert np.array_equal(s, (absmax / 127).astype(np.float32).astype(np.float16))
    assert np.array_equal(t, q.astype(np.int64).sum(axis=1))
    assert np.all(np.abs(q.astype(np.int64)) <= 127) and np.all(np.max(np.abs(q), axis=1) == 127)
