"""Inputs that cover every finite fp16 value (test helper, no arithmetic of the
method): rows for the exhaustive activation-quantizer tests."""
import numpy as np


def _finite_fp16():
    """Every finite fp16 value (both zeros included), in bit-pattern order."""
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return v[np.isfinite(v)]


# absmax values of the exhaustive rows: the fp16 maximum (every finite value is in
# range), ordinary scales, two whose quotients fall on exact half-integers (s = 1/8
# and s = 3/128: the reciprocal path must defer to the IEEE divide there), a normal
# value near the subnormal boundary, and two subnormal ones (the scale rounds to the
# smallest fp16 subnormal, then to zero)
EXHAUSTIVE_ABSMAX = [65504.0, 1.0, 3.3e-3, 15.875, 2.9765625, 6.2e-5, 2.0 ** -17, 2.0 ** -19]


def exhaustive_rows(absmax, K=4096):
    """Rows of K fp16 values holding every finite fp16 value of magnitude <= absmax
    exactly once (zeros as padding), each row led by absmax so that every row has
    that scale."""
    a = np.float16(absmax)
    v = _finite_fp16()
    v = v[np.abs(v.astype(np.float32)) <= np.float32(a)]
    per = K - 1
    n = -(-len(v) // per)
    body = np.zeros(n * per, np.float16)
    body[:len(v)] = v
    return np.concatenate([np.full((n, 1), a, np.float16), body.reshape(n, per)], axis=1)
