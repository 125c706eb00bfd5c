"""Host-side check of the bound the activation quantizer's fast path relies on
(quant_chunk8 in csrc/qoq_device.h): with s = fp16(absmax / 127) and rcp = fp32(1 / s),
q = fp32(x * rcp) takes the same round-to-nearest-even integer as the correctly
rounded fp32 quotient x / s whenever q is at least 2^-12 away from a half-integer;
the kernel divides exactly inside that band.  numpy's float32 multiply and divide
are IEEE round-to-nearest, as the GPU's are.  Checked on every fp16 x in
[-absmax, absmax] for absmax values spread over the whole fp16 range (normal and
subnormal), plus how close to the band the fast path ever gets."""
import numpy as np


def _fp16_positive():
    bits = np.arange(1, 0x7c00, dtype=np.uint16)            # every positive finite fp16
    return bits.view(np.float16)


def test_fast_quotient_decides_like_ieee_divide():
    pos = _fp16_positive()
    rng = np.random.default_rng(0)
    picks = np.unique(np.r_[pos[:64], pos[-64:], rng.choice(pos, 600, replace=False),
                            np.float16(15.875), np.float16(2.9765625)])
    worst = 0.0
    for a in picks:
        s = np.float16(np.float32(a) / np.float32(127.0))
        if s == 0:
            continue
        s32 = np.float32(s)
        rcp = np.float32(1.0) / s32
        xs = pos[pos <= a].astype(np.float32)
        xs = np.r_[xs, -xs]
        exact = np.rint(xs / s32)                             # fp32 IEEE divide, then RNE
        q = xs * rcp
        f = q - np.floor(q)
        fast = np.abs(f - np.float32(0.5)) >= np.float32(2.0 ** -12)
        assert np.array_equal(np.rint(q[fast]), exact[fast]), float(a)
        worst = max(worst, float(np.max(np.abs(q.astype(np.float64) - (xs / s32).astype(np.float64)))))
    assert worst < 2.0 ** -14                                   # far inside the 2^-12 band
