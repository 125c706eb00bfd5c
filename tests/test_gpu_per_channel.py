"""GPU parity of the per-channel W4A8 variant against the CPU oracle.

Bit-exact: packed codes, zeros, channel scales, activation codes / scales / code
sums, INT32 accumulators (sum_k qx (q - z), which the kernels reach as
sum_k qx q - z t).  FP16 output: within max(1e-3 |ref|, 2^-24) of the oracle's fp32
epilogue and bit-equal to its fp16 result.
"""
import functools
import os

import numpy as np
import pytest
import torch

from oracle import qoq_oracle as o
from w4a8_mixed_precision_amd import qoq
from w4a8_mixed_precision_amd import workloads as wl

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


def check_fp16(out16, acc, s_x, s_w):
    ref32 = o.epilogue_fp32(acc, s_x, s_w)
    err = np.abs(out16.astype(np.float32) - ref32)
    assert np.all(err <= np.maximum(RTOL * np.abs(ref32), ATOL))
    assert int(np.sum(out16.view(np.uint16) != ref32.astype(np.float16).view(np.uint16))) == 0


def _check_pack(dev, w16):
    packed, zeros, s_w = qoq.quantize_pack_weights(to_dev(w16, dev), group=0)
    q, z, s = o.quantize_weights_per_channel(w16)
    assert np.array_equal(host(s_w).view(np.uint16), s.view(np.uint16))
    assert np.array_equal(host(zeros), z)
    assert np.array_equal(host(packed), o.pack_codes(q))
    return packed, zeros, s_w


def test_pc_pack_edge_rows(gpu):
    say("per-channel pack edge rows")
    rng = np.random.default_rng(1)
    N, K = 64, 640
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    w[0] = 0                                                   # s = 0: codes and zero 0
    w[1] = np.abs(w[1])                                        # z = 0
    w[2] = -np.abs(w[2])                                       # z = 15
    w[3] = (rng.standard_normal(K) * 3e-6).astype(np.float16)  # subnormal scale
    w[4] = np.float16(65504) * np.sign(rng.standard_normal(K)).astype(np.float16)
    w[5] = ((rng.integers(0, 16, K) - 7) * 2.0 ** -6).astype(np.float16)   # lossless grid
    w[6, :] = np.float16(1e-3); w[6, 0] = np.float16(-2.0)    # one outlier
    _check_pack(gpu, w)


@pytest.mark.parametrize("name", ["tiny", "llama3_8b_qkv"])
def test_pc_pack_layers(gpu, name):
    L = wl.find(name)
    say(f"per-channel pack {name} N={L.N} K={L.K}")
    _check_pack(gpu, wl.weights_fp16(L))


@pytest.mark.parametrize("M,K", [(1, 128), (7, 4096), (33, 1152), (64, 8192), (1027, 136), (2048, 4096)])
def test_rowsum_bit_exact(gpu, M, K):
    say(f"activation row sums M={M} K={K}")
    rng = np.random.default_rng(M + K)
    x16 = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    x16[0, : K // 2] = np.float16(60000)
    if M > 2:
        x16[2] = 0
    qx, sx, t = qoq.quantize_activations_rowsum(to_dev(x16, gpu))
    qo, so = o.quantize_activations(x16)
    assert np.array_equal(host(qx), qo)
    assert np.array_equal(host(sx).view(np.uint16), so.view(np.uint16))
    assert np.array_equal(host(t), o.activation_row_sums(qo))


def _pc_full(dev, x16, w16, regime=None, config=None, splits=None):
    with qoq.plan_override(config=config, splits=splits or 0, regime=regime):
        N = w16.shape[0]
        packed, zeros, s_w = qoq.quantize_pack_weights(to_dev(w16, dev), group=0)
        qx, s_x, t = qoq.quantize_activations_rowsum(to_dev(x16, dev))
        acc = qoq.w4a8_gemm_pc_i32(qx, t, packed, zeros, N)
        out = qoq.w4a8_gemm_pc(qx, s_x, t, packed, zeros, s_w, N)
        return host(acc), host(out)


SHAPES = [(1, 16, 128), (8, 512, 512), (3, 48, 256), (17, 64, 384), (65, 144, 256), (100, 272, 512),
          (129, 256, 384), (300, 528, 768)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("regime", ["auto", "skinny", "tiled"])
def test_pc_gemm_small_exact(gpu, M, N, K, regime):
    say(f"per-channel gemm M={M} N={N} K={K} regime={regime}")
    rng = np.random.default_rng(M * 5 + N + K)
    x16 = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    w16 = (rng.standard_normal((N, K)) * 0.03).astype(np.float16)
    w16[:, :2] += np.float16(0.2)                              # asymmetric rows: zeros away from 8
    r = o.w4a8_pc_reference(x16, w16)
    acc, out = _pc_full(gpu, x16, w16, None if regime == "auto" else regime)
    assert np.array_equal(acc, r["acc"])
    check_fp16(out, r["acc"], r["s_x"], r["s_w"])


def _configs():
    try:
        return qoq.gemm_configs()
    except Exception:
        return []


@pytest.mark.parametrize("config", _configs())
def test_pc_every_config_exact(gpu, config):
    """Every kernel configuration forced, with split-K forced on the tile kernels."""
    splits = [None] if config.startswith("skinny") else [None, 3]
    for sp in splits:
        for (M, N, K) in [(1, 16, 128), (21, 80, 1152), (70, 272, 896), (130, 160, 384)]:
            say(f"per-channel gemm config={config} splits={sp} M={M} N={N} K={K}")
            rng = np.random.default_rng(M + N + K)
            x16 = (rng.standard_normal((M, K)) * 2).astype(np.float16)
            w16 = (rng.standard_normal((N, K)) * 0.03).astype(np.float16)
            r = o.w4a8_pc_reference(x16, w16)
            acc, out = _pc_full(gpu, x16, w16, config=config, splits=sp)
            assert np.array_equal(acc, r["acc"])
            check_fp16(out, r["acc"], r["s_x"], r["s_w"])


@functools.lru_cache(maxsize=1)
def _layer_weights(name):
    return wl.weights_fp16(wl.find(name))


@pytest.mark.parametrize("name,M", [("llama3_8b_qkv", 1), ("llama3_8b_qkv", 64), ("llama3_8b_down", 256),
                                    ("llama3_8b_gate_up", 1024), ("llama3_8b_down_prefill", 4096)])
def test_pc_layers_sampled(gpu, name, M):
    """Full-size layers in the launch configuration the library picks (skinny, split
    K, 128x256 and 256x256 tiles); sampled rows x columns against the oracle."""
    L = wl.find(name)
    say(f"per-channel gemm {name} M={M} plan={qoq.gemm_plan(M, L.N, L.K)} splits={qoq.gemm_plan_splits(M, L.N, L.K)}")
    w16 = _layer_weights(name)
    x16 = wl.activations_fp16(L, M)
    acc, out = _pc_full(gpu, x16, w16)
    rng = np.random.default_rng(M)
    rows = np.unique(np.r_[0, M - 1, rng.integers(0, M, min(M, 24))])
    cols = np.unique(np.r_[0:16, L.N - 16:L.N, rng.integers(0, L.N, 200)])
    q, z, sw = o.quantize_weights_per_channel(w16[cols])
    qx, sx = o.quantize_activations(x16[rows])
    want = o.contract(qx, o.dequantize_per_channel(q, z))
    assert np.array_equal(acc[np.ix_(rows, cols)], want)
    check_fp16(out[np.ix_(rows, cols)], want, sx, sw)


# ---------------------------------------------------------------------------
# Tiled activation codes (M <= 64): the quantizer with code sums writing the tiled
# layout, and the per-channel few-token kernels reading it
# ---------------------------------------------------------------------------
def untile(qt, M, K):
    """Row-major [M, K] view of tiled codes: block (rb, kb) = 1 KB at
    (rb * K/64 + kb) * 1024; inside it, row r's bytes k = 16 q .. +15 at (16 q + r) * 16."""
    Mp = (M + 15) // 16 * 16
    a = qt[: Mp * K].reshape(Mp // 16, K // 64, 4, 16, 16)        # rb, kb, q, r, byte
    return a.transpose(0, 3, 1, 2, 4).reshape(Mp, K)[:M]


@pytest.mark.parametrize("M,K", [(1, 128), (7, 4096), (33, 1152), (64, 8192)])
def test_rowsum_tiled_bit_exact(gpu, M, K):
    say(f"tiled activation codes with row sums M={M} K={K}")
    rng = np.random.default_rng(M * 3 + K)
    x16 = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    x16[0, : K // 2] = np.float16(60000)
    if M > 2:
        x16[2] = 0
    qt, sx, t = qoq.quantize_activations_rowsum_tiled(to_dev(x16, gpu))
    qo, so = o.quantize_activations(x16)
    assert np.array_equal(untile(host(qt), M, K), qo)
    assert np.array_equal(host(sx).view(np.uint16), so.view(np.uint16))
    assert np.array_equal(host(t), o.activation_row_sums(qo))


def _pc_tiled(dev, x16, w16, config=None):
    with qoq.plan_override(config=config):
        M, K = x16.shape
        N = w16.shape[0]
        packed, zeros, s_w = qoq.quantize_pack_weights(to_dev(w16, dev), group=0)
        qt, s_x, t = qoq.quantize_activations_rowsum_tiled(to_dev(x16, dev))
        acc = qoq.w4a8_gemm_pc_tiled_i32(qt, t, packed, zeros, M, N, K)
        out = qoq.w4a8_gemm_pc_tiled(qt, s_x, t, packed, zeros, s_w, M, N, K)
        return host(acc), host(out)


TILED_SHAPES = [(1, 16, 128), (3, 48, 256), (17, 64, 384), (37, 144, 1152), (64, 272, 512)]


@pytest.mark.parametrize("M,N,K", TILED_SHAPES)
def test_pc_tiled_exact(gpu, M, N, K):
    say(f"per-channel gemm on tiled codes M={M} N={N} K={K} plan={qoq.gemm_tiled_plan(M, N, K)}")
    rng = np.random.default_rng(M * 7 + N + K)
    x16 = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    w16 = (rng.standard_normal((N, K)) * 0.03).astype(np.float16)
    w16[:, :2] += np.float16(0.2)                              # asymmetric rows: zeros away from 8
    r = o.w4a8_pc_reference(x16, w16)
    acc, out = _pc_tiled(gpu, x16, w16)
    assert np.array_equal(acc, r["acc"])
    check_fp16(out, r["acc"], r["s_x"], r["s_w"])


@pytest.mark.parametrize("config", [c for c in _configs() if c.startswith("skinny")])
def test_pc_tiled_every_config_exact(gpu, config):
    """Every few-token configuration forced on tiled codes (ragged row blocks, strips
    past the end of the grid, waves without groups on the short K)."""
    for (M, N, K) in [(1, 16, 128), (21, 80, 1152), (64, 272, 896), (50, 48, 512)]:
        say(f"per-channel tiled gemm config={config} M={M} N={N} K={K}")
        rng = np.random.default_rng(M + N + K + 1)
        x16 = (rng.standard_normal((M, K)) * 2).astype(np.float16)
        w16 = (rng.standard_normal((N, K)) * 0.03).astype(np.float16)
        r = o.w4a8_pc_reference(x16, w16)
        acc, out = _pc_tiled(gpu, x16, w16, config=config)
        assert np.array_equal(acc, r["acc"])
        check_fp16(out, r["acc"], r["s_x"], r["s_w"])


@pytest.mark.parametrize("M", [1, 16, 64])
def test_pc_tiled_layer_sampled(gpu, M):
    """Llama-3-8B fused QKV at the decode batch sizes, full size, in the planner's
    configuration; sampled rows x columns against the oracle."""
    name = "llama3_8b_qkv"
    L = wl.find(name)
    say(f"per-channel tiled gemm {name} M={M} plan={qoq.gemm_tiled_plan(M, L.N, L.K)}")
    w16 = _layer_weights(name)
    x16 = wl.activations_fp16(L, M)
    acc, out = _pc_tiled(gpu, x16, w16)
    rng = np.random.default_rng(M + 1)
    rows = np.unique(np.r_[0, M - 1, rng.integers(0, M, min(M, 24))])
    cols = np.unique(np.r_[0:16, L.N - 16:L.N, rng.integers(0, L.N, 200)])
    q, z, sw = o.quantize_weights_per_channel(w16[cols])
    qx, sx = o.quantize_activations(x16[rows])
    want = o.contract(qx, o.dequantize_per_channel(q, z))
    assert np.array_equal(acc[np.ix_(rows, cols)], want)
    check_fp16(out[np.ix_(rows, cols)], want, sx, sw)
