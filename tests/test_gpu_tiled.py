"""GPU parity of the tiled activation path (up to 64 tokens) against the CPU oracle.

qoq_quantize_activations_tiled writes the per-token INT8 codes in the tiled layout
the few-token GEMM reads (include/qoq.h); here the layout is undone on the host from
its documented definition and the codes compared bit for bit with the oracle's
row-major codes.  qoq_w4a8_gemm_tiled: exact INT32 accumulators and the fp16
epilogue against the oracle, for every few-token configuration forced on ragged
shapes and for the full-size layer shapes (sampled columns).
"""
import functools
import os

import numpy as np
import pytest
import torch

from oracle import qoq_oracle as o
from w4a8_mixed_precision_amd import qoq
from w4a8_mixed_precision_amd import workloads as wl

from fp16_sweep import EXHAUSTIVE_ABSMAX, exhaustive_rows

pytestmark = pytest.mark.gpu

RTOL = 1e-3
ATOL = 2.0 ** -24


def say(msg):
    print(f"[case] {msg}", flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def untile(qt, M, K):
    """Row-major [M, K] view of tiled codes: block (rb, kb) = 1 KB at
    (rb * K/64 + kb) * 1024; inside it, row r's bytes k = 16 q .. +15 at (16 q + r) * 16."""
    Mp = (M + 15) // 16 * 16
    a = qt[: Mp * K].reshape(Mp // 16, K // 64, 4, 16, 16)        # rb, kb, q, r, byte
    return a.transpose(0, 3, 1, 2, 4).reshape(Mp, K)[:M]


def check_fp16(out16, acc, s_x, s_w):
    ref32 = o.epilogue_fp32(acc, s_x, s_w)
    err = np.abs(out16.astype(np.float32) - ref32)
    assert np.all(err <= np.maximum(RTOL * np.abs(ref32), ATOL))
    assert int(np.sum(out16.view(np.uint16) != ref32.astype(np.float16).view(np.uint16))) == 0


def test_untile_is_a_permutation():
    """The host-side inverse covers every byte of the blocks exactly once."""
    M, K = 19, 192
    Mp = 32
    qt = np.arange(Mp * K, dtype=np.int64)
    full = untile(qt, Mp, K)
    assert np.array_equal(np.sort(full.ravel()), qt)
    # row 17, k = 64 + 16 + 3: block (1, 1), q = 1, r = 1, byte 3
    assert full[17, 83] == ((1 * (K // 64) + 1) * 64 + 16 + 1) * 16 + 3


def _tiled_act_cases():
    rng = np.random.default_rng(11)
    for M, K in [(1, 64), (1, 4096), (5, 640), (16, 4096), (17, 128), (33, 1152), (64, 4096), (2, 29568)]:
        x = (rng.standard_normal((M, K)) * 2).astype(np.float16)
        x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
        if M > 2:
            x[1] = 0
        yield f"M{M}_K{K}", x


@pytest.mark.parametrize("name,x", list(_tiled_act_cases()), ids=lambda v: v if isinstance(v, str) else "")
def test_quantize_tiled_bit_exact(gpu, name, x):
    M, K = x.shape
    say(f"quantize_activations_tiled {name}")
    qt, sx = qoq.quantize_activations_tiled(to_dev(x, gpu))
    want_q, want_s = o.quantize_activations(x)
    assert np.array_equal(untile(host(qt), M, K), want_q)
    assert np.array_equal(host(sx).view(np.uint16), want_s.view(np.uint16))


def _tiled_gemm(dev, x16, packed, meta, s_w, N, config=None):
    with qoq.plan_override(config=config):
        M, K = x16.shape
        qt, sx = qoq.quantize_activations_tiled(to_dev(x16, dev))
        acc = qoq.w4a8_gemm_tiled_i32(qt, packed, meta, M, N, K)
        out = qoq.w4a8_gemm_tiled(qt, sx, packed, meta, s_w, M, N, K)
        return host(acc), host(out)


@pytest.mark.parametrize("absmax", EXHAUSTIVE_ABSMAX)
def test_quantize_tiled_every_fp16(gpu, absmax):
    """Every finite fp16 input through the tiled quantizer (and its code-sum form),
    at each absmax of the row-major exhaustive test: codes, scales and code sums
    bit-exact against the oracle."""
    x = exhaustive_rows(absmax)
    M, K = x.shape
    assert M <= qoq.TILED_MAX_M
    say(f"quantize_activations_tiled every fp16 <= {absmax}: {x.shape}")
    want_q, want_s = o.quantize_activations(x)
    qt, sx = qoq.quantize_activations_tiled(to_dev(x, gpu))
    assert np.array_equal(untile(host(qt), M, K), want_q)
    assert np.array_equal(host(sx).view(np.uint16), want_s.view(np.uint16))
    qt, sx, t = qoq.quantize_activations_rowsum_tiled(to_dev(x, gpu))
    assert np.array_equal(untile(host(qt), M, K), want_q)
    assert np.array_equal(host(sx).view(np.uint16), want_s.view(np.uint16))
    assert np.array_equal(host(t), o.activation_row_sums(want_q))


def _skinny_configs():
    try:
        return [c for c in qoq.gemm_configs() if c.startswith("skinny")]
    except Exception:
        return []


@pytest.mark.parametrize("config", _skinny_configs())
def test_tiled_every_config_exact(gpu, config):
    for (M, N, K) in [(1, 16, 128), (21, 80, 1152), (64, 272, 896), (33, 48, 640), (50, 160, 384)]:
        say(f"gemm_tiled config={config} M={M} N={N} K={K}")
        rng = np.random.default_rng(M * 3 + N + K)
        x16 = (rng.standard_normal((M, K)) * 2).astype(np.float16)
        w16 = (rng.standard_normal((N, K)) * 0.03).astype(np.float16)
        r = o.w4a8_reference(x16, w16)
        packed, meta, s_w = qoq.quantize_pack_weights(to_dev(w16, gpu))
        acc, out = _tiled_gemm(gpu, x16, packed, meta, s_w, N, config)
        assert np.array_equal(acc, r["acc"])
        check_fp16(out, r["acc"], r["s_x"], r["s_w"])


def test_tiled_empty_batch(gpu):
    L = wl.find("tiny")
    w16 = wl.weights_fp16(L)
    packed, meta, s_w = qoq.quantize_pack_weights(to_dev(w16, gpu))
    qt = torch.empty(0, dtype=torch.int8, device=gpu)
    s_x = torch.empty(0, dtype=torch.float16, device=gpu)
    out = qoq.w4a8_gemm_tiled(qt, s_x, packed, meta, s_w, 0, L.N, L.K)
    assert out.shape == (0, L.N)


_CASES = [("llama3_8b_qkv", 1), ("llama3_8b_qkv", 16), ("llama3_8b_qkv", 64), ("llama3_8b_gate_up", 64),
          ("llama3_8b_down", 64), ("qwen72b_down", 1), ("qwen72b_gate_up", 1)]


@functools.lru_cache(maxsize=1)
def _layer_weights(name):
    return wl.weights_fp16(wl.find(name))


@pytest.mark.parametrize("name,M", _CASES)
def test_tiled_layers_sampled(gpu, name, M):
    """Full-size layers in the configuration the library picks for tiled codes;
    the oracle recomputes every row on sampled columns (first / last strips)."""
    L = wl.find(name)
    say(f"gemm_tiled {name} M={M} plan={qoq.gemm_tiled_plan(M, L.N, L.K)}")
    w16 = _layer_weights(name)
    x16 = wl.activations_fp16(L, M)
    packed, meta, s_w = qoq.quantize_pack_weights(to_dev(w16, gpu))
    acc, out = _tiled_gemm(gpu, x16, packed, meta, s_w, L.N)
    rng = np.random.default_rng(M + 1)
    cols = np.unique(np.r_[0:16, L.N - 16:L.N, rng.integers(0, L.N, 160)])
    q0, sw = o.quantize_weights_level0(w16[cols])
    q, z, s = o.quantize_weights_level1(q0)
    qx, sx = o.quantize_activations(x16)
    want = o.contract(qx, o.dequantize_level1(q, z, s))
    assert np.array_equal(acc[:, cols], want)
    check_fp16(out[:, cols], want, sx, sw)
