"""GPU parity of the fused activation producers (RMSNorm + quantization, SiLU(gate) *
up + quantization) against the CPU oracle (oracle/fused_quant_oracle.py): codes,
token scales and code sums bit for bit, row-major and tiled, every workgroup split
the launcher can pick, ragged and degenerate rows, full-size layer rows."""
import numpy as np
import pytest
import torch

from oracle import fused_quant_oracle as fq
from w4a8_mixed_precision_amd import qoq
from w4a8_mixed_precision_amd import workloads as wl

pytestmark = pytest.mark.gpu

EPS = 1e-5


def say(msg):
    print(f"[case] {msg}", flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def untile(qt, M, K):
    Mp = (M + 15) // 16 * 16
    a = qt[: Mp * K].reshape(Mp // 16, K // 64, 4, 16, 16)
    return a.transpose(0, 3, 1, 2, 4).reshape(Mp, K)[:M]


def _check(got, want, M, K, tiled):
    q, s, t = got
    wq, ws, wt = want
    q = host(q)
    q = untile(q, M, K) if tiled else q
    assert np.array_equal(q, wq)
    assert np.array_equal(host(s).view(np.uint16), ws.view(np.uint16))
    if t is not None:
        assert np.array_equal(host(t).astype(np.int64), wt.astype(np.int64))


def _rows(M, K, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * scale).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    if M > 2:
        x[1] = 0.0                                    # all-zero token
    if M > 3:
        x[2] *= 1e-3
    return x.astype(np.float16)


SHAPES = [(1, 64), (1, 4096), (3, 136), (5, 640), (16, 4096), (17, 1152), (33, 8192), (64, 4096), (2, 14336),
          (1, 29568), (1, 32768), (70, 1024), (300, 512)]


# many short rows (prompt tokens)
RMS_SHAPES = SHAPES + [(1027, 136), (1500, 4096)]


@pytest.mark.parametrize("M,K", RMS_SHAPES)
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("rowsum", [False, True])
def test_rmsnorm_quantize_exact(gpu, M, K, tiled, rowsum):
    if tiled and (M > 64 or K % 64):
        pytest.skip("tiled layout: M <= 64, K % 64 == 0")
    say(f"rmsnorm_quantize M={M} K={K} tiled={tiled} rowsum={rowsum}")
    x = _rows(M, K, M * 13 + K, 3.0)
    gamma = (1.0 + 0.2 * np.random.default_rng(K).standard_normal(K)).astype(np.float16)
    got = qoq.rmsnorm_quantize(to_dev(x, gpu), to_dev(gamma, gpu), EPS, tiled=tiled, rowsum=rowsum)
    _check(got, fq.rmsnorm_quantize(x, gamma, EPS), M, K, tiled)


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("rowsum", [False, True])
def test_silu_mul_quantize_exact(gpu, M, K, tiled, rowsum):
    if tiled and (M > 64 or K % 64):
        pytest.skip("tiled layout: M <= 64, K % 64 == 0")
    say(f"silu_mul_quantize M={M} K={K} tiled={tiled} rowsum={rowsum}")
    gu = np.concatenate([_rows(M, K, M * 7 + K, 2.0), _rows(M, K, M * 7 + K + 1, 1.5)], axis=1)
    d = to_dev(gu, gpu)
    got = qoq.silu_mul_quantize(d[:, :K], d[:, K:], tiled=tiled, rowsum=rowsum)
    _check(got, fq.silu_mul_quantize(gu[:, :K], gu[:, K:]), M, K, tiled)


def test_silu_extreme_gates(gpu):
    """Gates where exp(-g) overflows or vanishes, subnormal products, exact zeros."""
    K = 512
    g = np.zeros((4, K), np.float32)
    u = np.ones((4, K), np.float32)
    g[0] = np.linspace(-65504, 65504, K)
    g[1] = np.linspace(-20, 20, K)
    u[1] = np.linspace(-3, 3, K)
    g[2, ::2] = -17.0                                     # tiny SiLU values next to zeros
    u[2] = 1e-3
    g[3] = np.linspace(-1e-3, 1e-3, K)
    u[3] = 6e-5                                           # products in the fp16 subnormal range
    g16, u16 = g.astype(np.float16), u.astype(np.float16)
    say("silu extremes")
    for M_rep in (1, 4):
        gg, uu = np.repeat(g16, M_rep, 0), np.repeat(u16, M_rep, 0)
        got = qoq.silu_mul_quantize(to_dev(gg, gpu), to_dev(uu, gpu), rowsum=True)
        _check(got, fq.silu_mul_quantize(gg, uu), gg.shape[0], K, False)


@pytest.mark.parametrize("name,M", [("llama3_8b_qkv", 64), ("qwen72b_qkv", 1), ("llama3_8b_down", 64),
                                    ("llama3_8b_down_prefill", 2048), ("llama3_8b_gate_up_prefill", 4096)])
def test_fused_layer_rows_sampled(gpu, name, M):
    """Layer sizes: RMSNorm on the QKV / gate+up input (K = hidden), SiLU * up on
    the down projection's input (K = intermediate); sampled rows vs the oracle."""
    L = wl.find(name)
    say(f"fused producers {name} M={M} K={L.K}")
    x = wl.activations_fp16(L, M)
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, min(M, 6))])
    if name.endswith("qkv") or "gate_up" in name:      # RMSNorm output feeds QKV and gate+up
        gamma = (1.0 + 0.1 * np.random.default_rng(1).standard_normal(L.K)).astype(np.float16)
        q, s, t = qoq.rmsnorm_quantize(to_dev(x, gpu), to_dev(gamma, gpu), EPS, rowsum=True)
        wq, ws, wt = fq.rmsnorm_quantize(x[rows], gamma, EPS)
    else:
        up = wl.activations_fp16(L, M)[:, ::-1].copy()
        q, s, t = qoq.silu_mul_quantize(to_dev(x, gpu), to_dev(up, gpu), rowsum=True)
        wq, ws, wt = fq.silu_mul_quantize(x[rows], up[rows])
    assert np.array_equal(host(q)[rows], wq)
    assert np.array_equal(host(s)[rows].view(np.uint16), ws.view(np.uint16))
    assert np.array_equal(host(t)[rows].astype(np.int64), wt.astype(np.int64))


def _all_finite_fp16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("u", [1.0, -0.3701171875, 3.125, 0.00099945068359375])
def test_silu_mul_every_fp16_gate(gpu, u):
    """The fp16 value of SiLU(gate) * up for every finite fp16 gate (63488 values),
    bit for bit against the oracle's single rounding of the fp64 expression: pins
    the fast fp32 path, its 2^-20 error band and the fp64 decision between the two
    candidates."""
    g = _all_finite_fp16()
    K = 4096
    n = (g.size + K - 1) // K * K
    gg = np.zeros(n, np.float16)
    gg[: g.size] = g
    gg = gg.reshape(-1, K)
    uu = np.full(gg.shape, u, np.float16)
    say(f"silu_mul every fp16 gate, up={u}")
    h = host(qoq.silu_mul(to_dev(gg, gpu), to_dev(uu, gpu)))
    want = fq.silu_mul_fp16(gg, uu)
    assert np.array_equal(h.view(np.uint16), want.view(np.uint16))


def test_rmsnorm_fp16_values(gpu):
    """The normalization's fp16 output itself, bit for bit, on rows of every scale."""
    rng = np.random.default_rng(12)
    for M, K in [(7, 4096), (3, 14336), (2, 29568), (5, 136)]:
        x = (rng.standard_normal((M, K)) * rng.choice([1e-3, 1.0, 50.0], (M, 1))).astype(np.float16)
        gamma = (1.0 + 0.3 * rng.standard_normal(K)).astype(np.float16)
        say(f"rmsnorm fp16 M={M} K={K}")
        y = host(qoq.rmsnorm(to_dev(x, gpu), to_dev(gamma, gpu), EPS))
        assert np.array_equal(y.view(np.uint16), fq.rmsnorm_fp16(x, gamma, EPS).view(np.uint16))


@pytest.mark.parametrize("M,K", [(1, 29568), (1, 14336), (3, 2056), (16, 14336), (64, 14336), (7, 32768)])
@pytest.mark.parametrize("tiled", [False, True])
def test_silu_split_matches_one_pass(gpu, M, K, tiled):
    """The two-pass split entry point gives the one-pass kernel's codes and scales bit
    for bit, and both match the oracle."""
    if tiled and K % 64:
        pytest.skip("tiled layout: K % 64 == 0")
    say(f"silu split M={M} K={K} tiled={tiled}")
    gu = np.concatenate([_rows(M, K, M * 11 + K, 2.0), _rows(M, K, M * 11 + K + 1, 1.5)], axis=1)
    d = to_dev(gu, gpu)
    assert qoq.silu_mul_quantize_workspace_bytes(M, K) > 0
    a = qoq.silu_mul_quantize(d[:, :K], d[:, K:], tiled=tiled, split=True)
    b = qoq.silu_mul_quantize(d[:, :K], d[:, K:], tiled=tiled, split=False)
    qa, qb = host(a[0]), host(b[0])
    if tiled:                                              # rows past M are padding, never written
        qa, qb = untile(qa, M, K), untile(qb, M, K)
    assert np.array_equal(qa, qb) and np.array_equal(host(a[1]).view(np.uint16), host(b[1]).view(np.uint16))
    _check(a, fq.silu_mul_quantize(gu[:, :K], gu[:, K:]), M, K, tiled)
