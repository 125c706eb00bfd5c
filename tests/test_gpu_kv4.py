"""GPU parity of the KV4 path against the CPU oracle (oracle/kv4_oracle.py).

KV write: codes, fp16 scales and zeros read back from the pages (their layout undone
on the host from its documented definition, include/qoq.h and csrc/qoq_kv4.hip) are
compared bit for bit with the oracle's quantization, for tokens written one at a
time and many at once, on shuffled page tables.

Decode attention: the output against the oracle's fp64 attention over the same
dequantized cache, within |err| <= 2^-10 (max|V_hat| + |ref|).  The kernel's
arithmetic: FP16 products with FP32 accumulation (exact dequantized inputs), FP32
softmax, probabilities rounded to FP16 for the second product (relative 2^-11 per
weight, so at most 2^-11 max|V_hat| on the output), FP16 output (2^-11 |o|); the
score accumulation and the exponentials add terms of relative order 2^-20 and
below.  The bound leaves a margin of about 2 over these.
"""
import numpy as np
import pytest
import torch

from oracle import kv4_oracle as kv
from tests.kv4_layout import layout_index as _layout_index
from w4a8_mixed_precision_amd import qoq

pytestmark = pytest.mark.gpu

D = 128
P = 64


def say(msg):
    print(f"[case] {msg}", flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def read_pages(pool, page_ids, h_kv, ntok):
    """Host decode of the first ntok slots of the given pages (in sequence order):
    (k codes, k s, k z, v codes, v s, v z) as [ntok, h_kv, D] / [ntok, h_kv]."""
    pb = qoq.kv4_page_bytes(h_kv) // h_kv
    kb, ksh, vb, vsh = _layout_index()
    out = [np.zeros((ntok, h_kv, D), np.uint8), np.zeros((ntok, h_kv), np.float16),
           np.zeros((ntok, h_kv), np.float16), np.zeros((ntok, h_kv, D), np.uint8),
           np.zeros((ntok, h_kv), np.float16), np.zeros((ntok, h_kv), np.float16)]
    for i in range(ntok):
        page, slot = page_ids[i // P], i % P
        for g in range(h_kv):
            sec = pool[(page * h_kv + g) * pb:(page * h_kv + g + 1) * pb]
            out[0][i, g] = (sec[kb[slot]] >> ksh[slot]) & 0xF
            out[3][i, g] = (sec[vb[slot]] >> vsh[slot]) & 0xF
            kst = sec[8192 + 4 * slot:8192 + 4 * slot + 4].view(np.float16)
            vst = sec[8448 + 16 * (slot // 4):8448 + 16 * (slot // 4) + 16].view(np.float16)
            out[1][i, g], out[2][i, g] = kst[0], kst[1]
            out[4][i, g], out[5][i, g] = vst[slot % 4], vst[4 + slot % 4]
    return out


def _pages(rng, B, max_pages, spare=3):
    ids = rng.permutation(B * max_pages + spare)[: B * max_pages].astype(np.int32)
    return ids.reshape(B, max_pages)


def _kv(rng, n, h_kv, scale=1.0):
    x = (rng.standard_normal((n, h_kv, D)) * scale).astype(np.float32)
    x[:, :, rng.choice(D, 3, replace=False)] *= 8           # a few outlier channels per head
    return x.astype(np.float16)


def test_kv4_write_bit_exact(gpu):
    rng = np.random.default_rng(1)
    h_kv, B, max_pages = 4, 3, 3
    pt = _pages(rng, B, max_pages)
    npages = B * max_pages + 3
    pool = torch.zeros(npages * qoq.kv4_page_bytes(h_kv), dtype=torch.uint8, device=gpu)
    n_tot = 150
    k = _kv(rng, B * n_tot, h_kv).reshape(B, n_tot, h_kv, D)
    v = _kv(rng, B * n_tot, h_kv, 0.3).reshape(B, n_tot, h_kv, D)
    k[0, 5] = 0                                             # an all-zero vector
    v[1, 7] = np.abs(v[1, 7]) + np.float16(2)               # one-signed, away from 0: z < 0
    v[1, 8] = -v[1, 7]                                      # all negative: z > 15
    k[1, 11] = np.float16(3.25)                             # constant: widened range
    k[0, 12] = (np.float16(40) + k[0, 12] * np.float16(0.01)).astype(np.float16)   # narrow, far: widened
    k[0, 13] = (np.float16(2) + np.abs(k[0, 13]) * np.float16(0.3)).astype(np.float16)
    halves = (np.arange(D) % 31 / 2).astype(np.float16)       # 0 .. 15 in steps of 1/2: s = 1, z = 0,
    for t in (9, 40):                                       # every odd value an exact tie x / s
        k[2, t, 1] = halves
        v[2, t, 3] = halves[::-1]
    # tokens 0..36 at once (block kernel), one at a time up to 52 and three at once
    # (per-token kernel), five at once inside one block, then 61..149 at once (block
    # kernel, partial first and last blocks merged with what is there)
    spans = [(0, 37)] + [(i, i + 1) for i in range(37, 53)] + [(53, 56), (56, 61), (61, n_tot)]
    dpt = to_dev(pt, gpu)
    for a, e in spans:
        say(f"kv4_write tokens {a}..{e - 1}")
        qoq.kv4_write(to_dev(k[:, a:e], gpu), to_dev(v[:, a:e], gpu), to_dev(np.full(B, a, np.int32), gpu), dpt, pool)
    poolh = host(pool)
    for b in range(B):
        kc, ks, kz, vc, vs, vz = read_pages(poolh, pt[b], h_kv, n_tot)
        wq, ws, wz = kv.kv_quantize(k[b])
        assert np.array_equal(kc, wq) and np.array_equal(ks.view(np.uint16), ws.view(np.uint16))
        assert np.array_equal(kz.view(np.uint16), wz.view(np.uint16))
        wq, ws, wz = kv.kv_quantize(v[b])
        assert np.array_equal(vc, wq) and np.array_equal(vs.view(np.uint16), ws.view(np.uint16))
        assert np.array_equal(vz.view(np.uint16), wz.view(np.uint16))


def test_kv4_prefill_write_full_shape(gpu):
    """The prefill write of the throughput measurement's Llama-3-8B decode shape (64
    sequences x 1024 tokens x 8 KV heads in one call, the same seeded inputs) on a
    shuffled page table: three sampled sequences read back bit for bit."""
    from w4a8_mixed_precision_amd import workloads as wl
    S = wl.find_kv("llama3_8b_b64_l1024")
    pt = _pages(np.random.default_rng(12), S.B, S.seq_len // P)
    pool = torch.zeros((pt.size + 3) * qoq.kv4_page_bytes(S.h_kv), dtype=torch.uint8, device=gpu)
    k = np.stack([wl.kv_fp16(S, b, S.seq_len, 0) for b in range(S.B)])
    v = np.stack([wl.kv_fp16(S, b, S.seq_len, 1) for b in range(S.B)])
    say(f"kv4_write prefill {S.name}")
    qoq.kv4_write(to_dev(k, gpu), to_dev(v, gpu), to_dev(np.zeros(S.B, np.int32), gpu), to_dev(pt, gpu), pool)
    poolh = host(pool)
    for b in (0, 29, S.B - 1):
        kc, ks, kz, vc, vs, vz = read_pages(poolh, pt[b], S.h_kv, S.seq_len)
        for codes, sc, zp, x in ((kc, ks, kz, k[b]), (vc, vs, vz, v[b])):
            wq, ws, wz = kv.kv_quantize(x)
            assert np.array_equal(codes, wq), b
            assert np.array_equal(sc.view(np.uint16), ws.view(np.uint16)), b
            assert np.array_equal(zp.view(np.uint16), wz.view(np.uint16)), b


def _run_attention(gpu, rng, lens, h, h_kv, kscale=1.0, vscale=1.0):
    B = len(lens)
    max_len = max(lens)
    max_pages = (max_len + P - 1) // P
    pt = _pages(rng, B, max_pages)
    pool = torch.empty((pt.size + 3) * qoq.kv4_page_bytes(h_kv), dtype=torch.uint8, device=gpu)
    pool.fill_(0xA5)                                        # unwritten slots hold garbage
    dpt = to_dev(pt, gpu)
    ks, vs = [], []
    for b, n in enumerate(lens):
        k = _kv(rng, n, h_kv, kscale)
        v = _kv(rng, n, h_kv, vscale)
        ks.append(k)
        vs.append(v)
        qoq.kv4_write(to_dev(k[None], gpu), to_dev(v[None], gpu), to_dev(np.zeros(1, np.int32), gpu), dpt[b:b + 1],
                      pool)
    q = (rng.standard_normal((B, h, D)) * 1.0).astype(np.float16)
    o = host(qoq.kv4_decode_attention(to_dev(q, gpu), pool, dpt, to_dev(np.array(lens, np.int32), gpu), h_kv,
                                      max_len))
    worst = 0.0
    for b in range(B):
        ref = kv.attention_reference(q[b], ks[b], vs[b], h_kv).astype(np.float64)
        vq, vs_, vz = kv.kv_quantize(vs[b])
        vmax = np.abs(kv.kv_dequantize(vq, vs_, vz).astype(np.float64)).max()
        err = np.abs(o[b].astype(np.float64) - ref)
        bound = 2.0 ** -10 * (vmax + np.abs(ref))
        assert np.all(err <= bound), (b, lens[b], float(err.max()), float(vmax))
        worst = max(worst, float((err / bound).max()))
    say(f"largest error / bound: {worst:.3f}")


@pytest.mark.parametrize("lens,h,h_kv", [([1, 17, 64, 300], 32, 8), ([1000, 65], 64, 8), ([16, 15, 33], 8, 8),
                                         ([4096], 32, 8), ([129] * 16, 32, 8),
                                         ([4096, 5, 100, 2000], 32, 8),    # splits, some empty for short rows
                                         ([64, 128, 1, 48], 16, 1),        # 16 heads on one KV head
                                         ([1000, 777], 32, 32),            # no grouping
                                         ([32768], 32, 8)])                # the long single sequence
def test_kv4_decode_attention(gpu, lens, h, h_kv):
    say(f"kv4 attention lens={lens[:4]}{'...' if len(lens) > 4 else ''} h={h} h_kv={h_kv} "
        f"splits={qoq.kv4_attention_workspace_bytes(len(lens), h, h_kv, max(lens)) > 0}")
    _run_attention(gpu, np.random.default_rng(sum(lens) + h), lens, h, h_kv)


def test_kv4_decode_attention_peaked_scores(gpu):
    """Large keys: softmax dominated by a few tokens (scores of order 100)."""
    say("kv4 attention peaked")
    _run_attention(gpu, np.random.default_rng(9), [200, 70], 32, 8, kscale=6.0, vscale=3.0)


def test_kv4_decode_attention_batch64(gpu):
    """The decode shape of the throughput measurement, sampled sequences checked."""
    rng = np.random.default_rng(10)
    say("kv4 attention batch 64 x 1024")
    _run_attention(gpu, rng, [1024] * 64, 32, 8)


def test_kv4_attention_clamps_lengths(gpu):
    """Sequence lengths are device data the host cannot check: 0 attends over the
    first token, a length past max_len over max_len tokens (the documented clamp to
    [1, max_len]); nothing outside the page table or the pool is read."""
    rng = np.random.default_rng(21)
    h, h_kv, n, max_len = 32, 8, 100, 100
    max_pages = (max_len + P - 1) // P
    pt = _pages(rng, 2, max_pages)
    pool = torch.empty((pt.size + 3) * qoq.kv4_page_bytes(h_kv), dtype=torch.uint8, device=gpu)
    pool.fill_(0xA5)
    dpt = to_dev(pt, gpu)
    ks = [_kv(rng, n, h_kv) for _ in range(2)]
    vs = [_kv(rng, n, h_kv) for _ in range(2)]
    for b in range(2):
        qoq.kv4_write(to_dev(ks[b][None], gpu), to_dev(vs[b][None], gpu), to_dev(np.zeros(1, np.int32), gpu),
                      dpt[b:b + 1], pool)
    q = rng.standard_normal((2, h, D)).astype(np.float16)
    say("kv4 attention lengths 0 and 1000 against max_len 100")
    o = host(qoq.kv4_decode_attention(to_dev(q, gpu), pool, dpt, to_dev(np.array([0, 1000], np.int32), gpu), h_kv,
                                      max_len))
    for b, used in ((0, 1), (1, max_len)):
        ref = kv.attention_reference(q[b], ks[b][:used], vs[b][:used], h_kv).astype(np.float64)
        vq, vs_, vz = kv.kv_quantize(vs[b][:used])
        vmax = np.abs(kv.kv_dequantize(vq, vs_, vz).astype(np.float64)).max()
        err = np.abs(o[b].astype(np.float64) - ref)
        assert np.all(err <= 2.0 ** -10 * (vmax + np.abs(ref))), (b, float(err.max()))


def test_kv4_write_guards(gpu):
    """Positions past the page table and page ids outside the pool are skipped by the
    write kernel (its own bounds checks): the pool is left as it was."""
    h_kv = 2
    pool = torch.full((4 * qoq.kv4_page_bytes(h_kv),), 0x5A, dtype=torch.uint8, device=gpu)
    before = host(pool).copy()
    pt = to_dev(np.array([[7, -1], [2, 3]], np.int32), gpu)          # 7 and -1: not pages of a 4-page pool
    rng = np.random.default_rng(3)
    k = to_dev(_kv(rng, 2, h_kv).reshape(2, 1, h_kv, D), gpu)
    v = to_dev(_kv(rng, 2, h_kv).reshape(2, 1, h_kv, D), gpu)
    say("kv4_write guards")
    qoq.kv4_write(k, v, to_dev(np.array([5, 128], np.int32), gpu), pt, pool)   # row 1: position past 2 pages
    qoq.kv4_write(k, v, to_dev(np.array([70, -3], np.int32), gpu), pt, pool)   # row 0 -> page -1; row 1 negative
    assert np.array_equal(host(pool), before)


# ---------------------------------------------------------------------------
# SmoothAttention (offline scales and folding)
# ---------------------------------------------------------------------------
def _key_samples(rng, n, h_kv):
    k = rng.standard_normal((n, h_kv, D)).astype(np.float32)
    k[:, :, rng.choice(D, 4, replace=False)] *= 12.0
    k[:, 1 % h_kv, [9, 9 + D // 2]] = 0.0                   # a pair that is always 0
    return k.astype(np.float16)


@pytest.mark.parametrize("n,h_kv", [(1, 1), (37, 2), (4096, 8), (65536, 8)])
def test_smooth_lambda_exact(gpu, n, h_kv):
    rng = np.random.default_rng(n + h_kv)
    k = _key_samples(rng, n, h_kv)
    dk = to_dev(k, gpu)
    say(f"smooth lambda n={n} h_kv={h_kv}")
    for alpha in (0.5, 0.0):
        got = host(qoq.smooth_attention_lambda(dk, alpha))
        assert np.array_equal(got.view(np.uint32), kv.smooth_attention_lambda(k, alpha).view(np.uint32))
    got = host(qoq.smooth_attention_lambda(dk, 0.3)).astype(np.float64)
    want = kv.smooth_attention_lambda(k, 0.3).astype(np.float64)
    assert np.all(np.abs(got - want) <= 2.0 ** -23 * want)  # the double power rounded to fp32: one ulp


@pytest.mark.parametrize("h,h_kv,dm", [(32, 8, 4096), (8, 8, 640), (16, 1, 1152)])
def test_smooth_fold_exact(gpu, h, h_kv, dm):
    rng = np.random.default_rng(h * 7 + dm)
    wq = (rng.standard_normal((h * D, dm)) * 0.05).astype(np.float16)
    wk = (rng.standard_normal((h_kv * D, dm)) * 0.05).astype(np.float16)
    lam = kv.smooth_attention_lambda(_key_samples(rng, 300, h_kv), 0.5)
    say(f"smooth fold h={h} h_kv={h_kv} d_model={dm}")
    want_q, want_k = kv.smooth_attention_fold(wq, wk, lam, h, h_kv)
    dq, dk, dl = to_dev(wq, gpu), to_dev(wk, gpu), to_dev(lam, gpu)
    gq, gk = qoq.smooth_attention_fold(dq, dk, dl, h, h_kv)
    assert np.array_equal(host(gq).view(np.uint16), want_q.view(np.uint16))
    assert np.array_equal(host(gk).view(np.uint16), want_k.view(np.uint16))
    qoq.smooth_attention_fold(dq, dk, dl, h, h_kv, inplace=True)
    assert np.array_equal(host(dq).view(np.uint16), want_q.view(np.uint16))
    assert np.array_equal(host(dk).view(np.uint16), want_k.view(np.uint16))
