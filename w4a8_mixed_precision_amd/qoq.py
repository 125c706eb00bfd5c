"""Thin Python binding over the C ABI of ``libqoq.so`` (declared in include/qoq.h).

Argument marshalling only: every step of the path runs in the HIP kernels of the
library.  PyTorch supplies device memory and the current HIP stream.  There is no
fallback: a missing library, a CPU tensor or a non-zero status raises.

The functions carry the C names without the ``qoq_`` prefix and take torch tensors;
``lib()`` exposes the raw ctypes handle for callers that work with pointers.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libqoq.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "qoq.h")

GROUP = 128

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t

_SIGNATURES = {
    "qoq_version": ([], ctypes.c_int),
    "qoq_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "qoq_weight_buffer_sizes": ([_c_i64, _c_i64, _c_i32, ctypes.POINTER(_c_sz), ctypes.POINTER(_c_sz),
                                 ctypes.POINTER(_c_sz)], ctypes.c_int),
    "qoq_quantize_pack_weights": ([_c_vp, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "qoq_quantize_activations": ([_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "qoq_gemm_workspace_bytes": ([_c_i64, _c_i64, _c_i64, _c_i32, ctypes.POINTER(_c_sz)], ctypes.c_int),
    "qoq_w4a8_gemm": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_vp, _c_sz,
                       _c_vp], ctypes.c_int),
    "qoq_w4a8_gemm_i32": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_vp, _c_sz, _c_vp],
                          ctypes.c_int),
    "qoq_gemm_plan": ([_c_i64, _c_i64, _c_i64], ctypes.c_char_p),
    "qoq_quantize_activations_tiled": ([_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "qoq_w4a8_gemm_tiled": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp],
                            ctypes.c_int),
    "qoq_w4a8_gemm_tiled_i32": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp], ctypes.c_int),
    "qoq_gemm_tiled_plan": ([_c_i64, _c_i64, _c_i64], ctypes.c_char_p),
    "qoq_rmsnorm_quantize": ([_c_vp, _c_vp, ctypes.c_float, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp],
                             ctypes.c_int),
    "qoq_silu_mul_quantize": ([_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp],
                              ctypes.c_int),
    "qoq_rmsnorm": ([_c_vp, _c_vp, ctypes.c_float, _c_i64, _c_i64, _c_vp, _c_vp], ctypes.c_int),
    "qoq_silu_mul": ([_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp], ctypes.c_int),
    "qoq_silu_mul_quantize_workspace_bytes": ([_c_i64, _c_i64, ctypes.POINTER(_c_sz)], ctypes.c_int),
    "qoq_silu_mul_quantize_ws": ([_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp],
                                 ctypes.c_int),
    "qoq_kv4_page_bytes": ([_c_i64, _c_i64, ctypes.POINTER(_c_sz)], ctypes.c_int),
    "qoq_kv4_write": ([_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp],
                      ctypes.c_int),
    "qoq_smooth_attention_lambda": ([_c_vp, _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_vp, _c_vp], ctypes.c_int),
    "qoq_smooth_attention_fold": ([_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp],
                                  ctypes.c_int),
    "qoq_kv4_attention_workspace_bytes": ([_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_sz)],
                                          ctypes.c_int),
    "qoq_kv4_decode_attention": ([_c_vp, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                  _c_i64, _c_vp, _c_vp, _c_sz, _c_vp], ctypes.c_int),
    "qoq_quantize_activations_rowsum": ([_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "qoq_quantize_activations_rowsum_tiled": ([_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "qoq_w4a8_gemm_pc_tiled": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp],
                               ctypes.c_int),
    "qoq_w4a8_gemm_pc_tiled_i32": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp], ctypes.c_int),
    "qoq_w4a8_gemm_pc": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_sz,
                          _c_vp], ctypes.c_int),
    "qoq_w4a8_gemm_pc_i32": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_sz, _c_vp],
                             ctypes.c_int),
    "qoq_linear_workspace_bytes": ([_c_i64, _c_i64, _c_i64, _c_i32, ctypes.POINTER(_c_sz)], ctypes.c_int),
    "qoq_w4a8_linear": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_vp, _c_sz,
                         _c_vp], ctypes.c_int),
    "qoq_linear_plan": ([_c_i64, _c_i64, _c_i64], ctypes.c_char_p),
    "qoq_w4a8_linear_noalloc": ([_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_vp],
                                ctypes.c_int),
    "qoq_linear_config_name": ([ctypes.c_int], ctypes.c_char_p),
    "qoq_gemm_plan_splits": ([_c_i64, _c_i64, _c_i64], ctypes.c_int),
    "qoq_gemm_config_name": ([ctypes.c_int], ctypes.c_char_p),
    "qoq_set_plan_override": ([ctypes.c_char_p, _c_i32, ctypes.c_char_p, ctypes.c_char_p], ctypes.c_int),
    "qoq_dequantize_packed": ([_c_vp, _c_vp, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp], ctypes.c_int),
    "qoq_stream_copy": ([_c_vp, _c_vp, _c_sz, _c_vp], ctypes.c_int),
    "qoq_mfma_probe": ([_c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "qoq_mfma_probe32": ([_c_vp, _c_vp, _c_vp, _c_vp], ctypes.c_int),
    "qoq_mfma_peak": ([ctypes.c_int, ctypes.c_int, _c_vp, _c_vp], ctypes.c_int),
    "qoq_mfma_peak_operands": ([_c_vp, _c_sz, _c_vp, _c_sz, ctypes.c_int, ctypes.c_int, _c_vp, _c_vp],
                               ctypes.c_int),
    "qoq_stream_read": ([_c_vp, _c_sz, _c_vp, ctypes.c_int, ctypes.c_int, _c_vp], ctypes.c_int),
}

_lib = None


class QoQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def header_symbols() -> list:
    """Names of the functions include/qoq.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(qoq_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().qoq_status_string(int(status)).decode()


def version() -> int:
    return int(lib().qoq_version())


def _check(fn: str, status: int):
    if status != 0:
        raise QoQError(fn, status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a HIP device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t, name: str):
    _dev(t, name)
    return t


# Host-side size checks: the library sees only pointers, so a buffer that is too
# small for (M, N, K) would be read or written past its end on the device.
def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_bytes(t, name: str, need: int):
    if isinstance(t, torch.Tensor) and _nbytes(t) < need:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, {need} needed")


def _check_weights(packed, meta, s_w, N: int, K: int, per_channel: bool = False):
    """Packed codes N*K/2 bytes; group metadata 2 bytes per (column, group of 128)
    (per-channel: one zero byte per column); N fp16 channel scales."""
    if N <= 0 or K <= 0:
        return                      # the library rejects the shape itself
    _check_bytes(packed, "packed", N * K // 2)
    if per_channel:
        _check_bytes(meta, "zeros", N)
    else:
        _check_bytes(meta, "meta", 2 * N * (K // GROUP))
    _check_bytes(s_w, "s_w", 2 * N)


def _check_rows(t, name: str, M: int, elem: int):
    """A per-token vector (s_x fp16, t int32) must hold M entries."""
    _check_bytes(t, name, elem * M)


def _check_out(out, M: int, N: int):
    if not isinstance(out, torch.Tensor) or tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape ({M}, {N}), got {getattr(out, 'shape', None)}")


# ---------------------------------------------------------------------------
# sizes
# ---------------------------------------------------------------------------
def weight_buffer_sizes(N: int, K: int, group: int = GROUP) -> dict:
    a, b, c = _c_sz(), _c_sz(), _c_sz()
    _check("qoq_weight_buffer_sizes",
           lib().qoq_weight_buffer_sizes(N, K, group, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return {"packed_w": a.value, "group_meta": b.value, "s_w": c.value}


def gemm_workspace_bytes(M: int, N: int, K: int, group: int = GROUP) -> int:
    v = _c_sz()
    _check("qoq_gemm_workspace_bytes", lib().qoq_gemm_workspace_bytes(M, N, K, group, ctypes.byref(v)))
    return v.value


def gemm_plan(M: int, N: int, K: int) -> str:
    return lib().qoq_gemm_plan(M, N, K).decode()


def gemm_plan_splits(M: int, N: int, K: int) -> int:
    v = lib().qoq_gemm_plan_splits(M, N, K)
    if v < 0:
        raise QoQError("qoq_gemm_plan_splits", v)
    return v


_override = {"config": None, "splits": 0, "regime": None, "linear": None}


def set_plan_override(config=None, splits: int = 0, regime=None, linear=None):
    """Replace the planner overrides (qoq_set_plan_override): a configuration forced
    for every GEMM shape, a split-K factor, "skinny" / "tiled", a linear
    configuration or "unfused".  All None / 0 clears them."""
    enc = lambda v: None if v is None else str(v).encode()
    _check("qoq_set_plan_override", lib().qoq_set_plan_override(enc(config), int(splits), enc(regime), enc(linear)))
    _override.update(config=config, splits=int(splits), regime=regime, linear=linear)


class plan_override:
    """Context manager: the given overrides for the body, the previous ones after."""

    def __init__(self, config=None, splits: int = 0, regime=None, linear=None):
        self.new = dict(config=config, splits=splits, regime=regime, linear=linear)

    def __enter__(self):
        self.old = dict(_override)
        set_plan_override(**self.new)
        return self

    def __exit__(self, *exc):
        set_plan_override(**self.old)
        return False


def gemm_configs() -> list:
    """Names of every kernel configuration in the library."""
    out, i = [], 0
    while True:
        n = lib().qoq_gemm_config_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


# ---------------------------------------------------------------------------
# offline weight quantization + packing
# ---------------------------------------------------------------------------
def quantize_pack_weights(w: torch.Tensor, group: int = GROUP, out=None):
    """W fp16 [N, K] -> (packed uint8 [N*K/2], meta, s_w fp16 [N]).
    group 128: meta int16 [N*K/128] (uint16 bits); group 0 (per-channel): meta =
    the zeros, uint8 [N]."""
    N, K = w.shape
    sizes = weight_buffer_sizes(N, K, group)
    mdt = torch.uint8 if group == 0 else torch.int16
    if out is None:
        packed = torch.empty(sizes["packed_w"], dtype=torch.uint8, device=w.device)
        meta = torch.empty(sizes["group_meta"] // (1 if group == 0 else 2), dtype=mdt, device=w.device)
        s_w = torch.empty(N, dtype=torch.float16, device=w.device)
    else:
        packed, meta, s_w = out
    _check("qoq_quantize_pack_weights",
           lib().qoq_quantize_pack_weights(_dev(w, "w", torch.float16), N, K, group,
                                           _dev(packed, "packed", torch.uint8), _dev(meta, "meta", mdt),
                                           _dev(s_w, "s_w", torch.float16), _stream(w)))
    return packed, meta, s_w


# ---------------------------------------------------------------------------
# per-token activation quantization
# ---------------------------------------------------------------------------
def quantize_activations(x: torch.Tensor, out=None):
    """X fp16 [M, K] -> (qx int8 [M, K], s_x fp16 [M])."""
    M, K = x.shape
    if out is None:
        qx = torch.empty((M, K), dtype=torch.int8, device=x.device)
        s_x = torch.empty(M, dtype=torch.float16, device=x.device)
    else:
        qx, s_x = out
    _check("qoq_quantize_activations",
           lib().qoq_quantize_activations(_dev(x, "x", torch.float16), M, K, _dev(qx, "qx", torch.int8),
                                          _dev(s_x, "s_x", torch.float16), _stream(x)))
    return qx, s_x


TILED_MAX_M = 64


def tiled_bytes(M: int, K: int) -> int:
    """Bytes of the tiled activation codes of M tokens (whole 16-row blocks)."""
    return (M + 15) // 16 * 16 * K


def quantize_activations_tiled(x: torch.Tensor, out=None):
    """X fp16 [M, K] (M <= 64) -> (qx_tiled int8 [round_up(M, 16) * K] in the layout of
    qoq_quantize_activations_tiled, s_x fp16 [M])."""
    M, K = x.shape
    if out is None:
        qx = torch.empty(tiled_bytes(M, K), dtype=torch.int8, device=x.device)
        s_x = torch.empty(M, dtype=torch.float16, device=x.device)
    else:
        qx, s_x = out
    if qx.numel() < tiled_bytes(M, K):
        raise ValueError(f"qx_tiled holds {qx.numel()} bytes, {tiled_bytes(M, K)} needed")
    _check("qoq_quantize_activations_tiled",
           lib().qoq_quantize_activations_tiled(_dev(x, "x", torch.float16), M, K, _dev(qx, "qx", torch.int8),
                                                _dev(s_x, "s_x", torch.float16), _stream(x)))
    return qx, s_x


def _fused_outputs(M, K, dev, tiled, rowsum, out):
    if out is not None:
        return out
    qx = torch.empty(tiled_bytes(M, K) if tiled else (M, K), dtype=torch.int8, device=dev)
    s_x = torch.empty(M, dtype=torch.float16, device=dev)
    t = torch.empty(M, dtype=torch.int32, device=dev) if rowsum else None
    return qx, s_x, t


def rmsnorm_quantize(x: torch.Tensor, gamma: torch.Tensor, eps: float, tiled: bool = False, rowsum: bool = False,
                     out=None):
    """RMSNorm + per-token INT8 quantization in one kernel: X fp16 [M, K], gamma fp16
    [K] -> (qx, s_x fp16 [M], t int32 [M] or None); qx row-major [M, K] or tiled."""
    M, K = x.shape
    qx, s_x, t = _fused_outputs(M, K, x.device, tiled, rowsum, out)
    _check("qoq_rmsnorm_quantize",
           lib().qoq_rmsnorm_quantize(_dev(x, "x", torch.float16), _dev(gamma, "gamma", torch.float16), float(eps),
                                      M, K, 1 if tiled else 0, _dev(qx, "qx", torch.int8),
                                      _dev(s_x, "s_x", torch.float16),
                                      None if t is None else _dev(t, "t", torch.int32), _stream(x)))
    return qx, s_x, t


def silu_mul_quantize(gate: torch.Tensor, up: torch.Tensor, tiled: bool = False, rowsum: bool = False, out=None,
                      split: bool = True, workspace=None):
    """SiLU(gate) * up + per-token INT8 quantization.  gate, up: fp16 [M, K] views with
    the same row stride (e.g. the halves of a gate+up output).  Without code sums, a
    few long rows take the two-pass split entry point (split=False forces the one-pass
    kernel); workspace: None = the cached one of this device and stream."""
    M, K = gate.shape
    if up.shape != gate.shape or gate.stride(1) != 1 or up.stride(1) != 1 or gate.stride(0) != up.stride(0):
        raise ValueError("gate and up must be [M, K] views with unit column stride and the same row stride")
    qx, s_x, t = _fused_outputs(M, K, gate.device, tiled, rowsum, out)
    for t_, n_ in ((gate, "gate"), (up, "up")):
        if not isinstance(t_, torch.Tensor) or t_.device.type != "cuda" or t_.dtype != torch.float16:
            raise TypeError(f"{n_} must be an fp16 HIP device tensor")
    if not rowsum and split:
        need = silu_mul_quantize_workspace_bytes(M, K)
        if need:
            ws = workspace if workspace is not None else _silu_workspace(gate, need)
            _check("qoq_silu_mul_quantize_ws",
                   lib().qoq_silu_mul_quantize_ws(ctypes.c_void_p(gate.data_ptr()), ctypes.c_void_p(up.data_ptr()),
                                                  gate.stride(0), M, K, 1 if tiled else 0,
                                                  _dev(qx, "qx", torch.int8), _dev(s_x, "s_x", torch.float16),
                                                  _dev(ws, "workspace"), ws.numel() * ws.element_size(),
                                                  _stream(gate)))
            return qx, s_x, t
    _check("qoq_silu_mul_quantize",
           lib().qoq_silu_mul_quantize(ctypes.c_void_p(gate.data_ptr()), ctypes.c_void_p(up.data_ptr()),
                                       gate.stride(0), M, K, 1 if tiled else 0, _dev(qx, "qx", torch.int8),
                                       _dev(s_x, "s_x", torch.float16),
                                       None if t is None else _dev(t, "t", torch.int32), _stream(gate)))
    return qx, s_x, t


def silu_mul_quantize_workspace_bytes(M: int, K: int) -> int:
    b = _c_sz(0)
    _check("qoq_silu_mul_quantize_workspace_bytes", lib().qoq_silu_mul_quantize_workspace_bytes(M, K, ctypes.byref(b)))
    return int(b.value)


_silu_workspaces = {}


def _silu_workspace(t: torch.Tensor, need: int):
    """The cached two-pass SwiGLU workspace of t's device and current stream."""
    key = (t.device.index, torch.cuda.current_stream(t.device).cuda_stream)
    ws = _silu_workspaces.get(key)
    if ws is None or ws.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the SwiGLU workspace for this shape does not exist yet and cannot be allocated "
                               "during graph capture: call once before capturing or pass workspace=")
        ws = torch.empty(max(need, 2 * ws.numel() if ws is not None else 0), dtype=torch.uint8, device=t.device)
        _silu_workspaces[key] = ws
    return ws


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, out=None):
    """The normalization alone: fp16 [M, K] (the value rmsnorm_quantize quantizes)."""
    M, K = x.shape
    y = torch.empty((M, K), dtype=torch.float16, device=x.device) if out is None else out
    _check("qoq_rmsnorm", lib().qoq_rmsnorm(_dev(x, "x", torch.float16), _dev(gamma, "gamma", torch.float16),
                                            float(eps), M, K, _dev(y, "y", torch.float16), _stream(x)))
    return y


def silu_mul(gate: torch.Tensor, up: torch.Tensor, out=None):
    """SiLU(gate) * up alone: fp16 [M, K] (the value silu_mul_quantize quantizes)."""
    M, K = gate.shape
    if up.shape != gate.shape or gate.stride(1) != 1 or up.stride(1) != 1 or gate.stride(0) != up.stride(0):
        raise ValueError("gate and up must be [M, K] views with unit column stride and the same row stride")
    for t_, n_ in ((gate, "gate"), (up, "up")):
        if not isinstance(t_, torch.Tensor) or t_.device.type != "cuda" or t_.dtype != torch.float16:
            raise TypeError(f"{n_} must be an fp16 HIP device tensor")
    h = torch.empty((M, K), dtype=torch.float16, device=gate.device) if out is None else out
    _check("qoq_silu_mul", lib().qoq_silu_mul(ctypes.c_void_p(gate.data_ptr()), ctypes.c_void_p(up.data_ptr()),
                                              gate.stride(0), M, K, _dev(h, "h", torch.float16), _stream(gate)))
    return h


# ---------------------------------------------------------------------------
# KV4 cache
# ---------------------------------------------------------------------------
KV4_PAGE_TOKENS = 64
KV4_HEAD_DIM = 128


def kv4_page_bytes(h_kv: int) -> int:
    b = _c_sz(0)
    _check("qoq_kv4_page_bytes", lib().qoq_kv4_page_bytes(h_kv, KV4_HEAD_DIM, ctypes.byref(b)))
    return int(b.value)


def _kv4_pool_pages(pool: torch.Tensor, h_kv: int) -> int:
    pb = kv4_page_bytes(h_kv)
    if pool.numel() % pb or pool.numel() == 0:
        raise ValueError(f"kv4 pool: {pool.numel()} bytes is not a whole number of {pb}-byte pages")
    return pool.numel() // pb


def kv4_write(k_new: torch.Tensor, v_new: torch.Tensor, positions: torch.Tensor, page_table: torch.Tensor,
              pool: torch.Tensor):
    """k_new, v_new fp16 [B, n_new, h_kv, 128]; positions int32 [B]; page_table int32
    [B, max_pages]; pool uint8 [num_pages * kv4_page_bytes(h_kv)]."""
    B, n_new, h_kv, D = k_new.shape
    if v_new.shape != k_new.shape or positions.numel() != B or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("kv4_write: shapes of k_new, v_new, positions, page_table disagree")
    num_pages = _kv4_pool_pages(pool, h_kv)
    _check("qoq_kv4_write",
           lib().qoq_kv4_write(_dev(k_new, "k_new", torch.float16), _dev(v_new, "v_new", torch.float16), B, n_new,
                               h_kv, D, _dev(positions, "positions", torch.int32),
                               _dev(page_table, "page_table", torch.int32), page_table.shape[1],
                               _dev(pool, "pool", torch.uint8), num_pages, _stream(k_new)))


def smooth_attention_lambda(k_samples: torch.Tensor, alpha: float = 0.5, out=None):
    """k_samples fp16 [n, h_kv, 128] -> lambda fp32 [h_kv, 128]."""
    n, h_kv, D = k_samples.shape
    lam = torch.empty((h_kv, D), dtype=torch.float32, device=k_samples.device) if out is None else out
    _check("qoq_smooth_attention_lambda",
           lib().qoq_smooth_attention_lambda(_dev(k_samples, "k_samples", torch.float16), n, h_kv, D, float(alpha),
                                             _dev(lam, "lambda", torch.float32), _stream(k_samples)))
    return lam


def smooth_attention_fold(w_q: torch.Tensor, w_k: torch.Tensor, lam: torch.Tensor, h: int, h_kv: int,
                          inplace: bool = False):
    """w_q fp16 [h*128, d_model], w_k fp16 [h_kv*128, d_model], lambda fp32 [h_kv, 128]
    -> (w_q', w_k') with Lambda folded in."""
    if w_q.dim() != 2 or w_k.dim() != 2 or w_q.shape[1] != w_k.shape[1] or w_q.shape[0] != h * KV4_HEAD_DIM \
            or w_k.shape[0] != h_kv * KV4_HEAD_DIM or tuple(lam.shape) != (h_kv, KV4_HEAD_DIM):
        raise ValueError("smooth_attention_fold: shapes of w_q, w_k, lambda disagree with h, h_kv")
    qo = w_q if inplace else torch.empty_like(w_q)
    ko = w_k if inplace else torch.empty_like(w_k)
    _check("qoq_smooth_attention_fold",
           lib().qoq_smooth_attention_fold(_dev(w_q, "w_q", torch.float16), _dev(w_k, "w_k", torch.float16),
                                           _dev(lam, "lambda", torch.float32), h, h_kv, KV4_HEAD_DIM, w_q.shape[1],
                                           _dev(qo, "w_q_out", torch.float16), _dev(ko, "w_k_out", torch.float16),
                                           _stream(w_q)))
    return qo, ko


def kv4_attention_workspace_bytes(B: int, h: int, h_kv: int, max_len: int) -> int:
    b = _c_sz(0)
    _check("qoq_kv4_attention_workspace_bytes",
           lib().qoq_kv4_attention_workspace_bytes(B, h, h_kv, KV4_HEAD_DIM, max_len, ctypes.byref(b)))
    return int(b.value)


def kv4_decode_attention(q: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                         h_kv: int, max_len: int, out=None, workspace=None):
    """q fp16 [B, h, 128] -> o fp16 [B, h, 128] over the cached tokens."""
    B, h, D = q.shape
    if seq_lens.numel() != B or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("kv4_decode_attention: shapes of q, seq_lens, page_table disagree")
    num_pages = _kv4_pool_pages(pool, h_kv)
    if out is None:
        out = torch.empty_like(q)
    if not isinstance(out, torch.Tensor) or tuple(out.shape) != (B, h, D):
        raise ValueError(f"out must have shape ({B}, {h}, {D}), got {getattr(out, 'shape', None)}")
    need = kv4_attention_workspace_bytes(B, h, h_kv, max_len)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws = _dev(workspace, "workspace") if need else None
    _check("qoq_kv4_decode_attention",
           lib().qoq_kv4_decode_attention(_dev(q, "q", torch.float16), _dev(pool, "pool", torch.uint8), num_pages,
                                          _dev(page_table, "page_table", torch.int32), page_table.shape[1],
                                          _dev(seq_lens, "seq_lens", torch.int32), B, h, h_kv, D, max_len,
                                          _dev(out, "out", torch.float16), ws, workspace.numel() if need else 0,
                                          _stream(q)))
    return out


def quantize_activations_rowsum(x: torch.Tensor, out=None):
    """X fp16 [M, K] -> (qx int8 [M, K], s_x fp16 [M], t int32 [M] = sum_k qx)."""
    M, K = x.shape
    if out is None:
        qx = torch.empty((M, K), dtype=torch.int8, device=x.device)
        s_x = torch.empty(M, dtype=torch.float16, device=x.device)
        t = torch.empty(M, dtype=torch.int32, device=x.device)
    else:
        qx, s_x, t = out
    _check("qoq_quantize_activations_rowsum",
           lib().qoq_quantize_activations_rowsum(_dev(x, "x", torch.float16), M, K, _dev(qx, "qx", torch.int8),
                                                 _dev(s_x, "s_x", torch.float16), _dev(t, "t", torch.int32),
                                                 _stream(x)))
    return qx, s_x, t


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def w4a8_gemm_pc(qx, s_x, t, packed, zeros, s_w, N: int, out=None, workspace=None):
    """Per-channel weights: out fp16 [M, N] = fp16((sum qx q - z t) * (s_x * s_w))."""
    M, K = qx.shape
    _check_weights(packed, zeros, s_w, N, K, per_channel=True)
    _check_rows(s_x, "s_x", M, 2)
    _check_rows(t, "t", M, 4)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=qx.device)
    _check_out(out, M, N)
    ws_ptr, ws_bytes = _workspace_args(workspace, _dev_tensor(qx, "qx"), M, N, K, GROUP)
    _check("qoq_w4a8_gemm_pc",
           lib().qoq_w4a8_gemm_pc(_dev(qx, "qx", torch.int8), _dev(s_x, "s_x", torch.float16),
                                  _dev(t, "t", torch.int32), _dev(packed, "packed", torch.uint8),
                                  _dev(zeros, "zeros", torch.uint8), _dev(s_w, "s_w", torch.float16),
                                  _dev(out, "out", torch.float16), M, N, K, ws_ptr, ws_bytes, _stream(qx)))
    return out


def w4a8_gemm_pc_i32(qx, t, packed, zeros, N: int, out=None, workspace=None):
    """Per-channel weights: acc int32 [M, N] = sum_k qx (q - z), exact."""
    M, K = qx.shape
    _check_bytes(packed, "packed", N * K // 2 if N > 0 else 0)
    _check_bytes(zeros, "zeros", max(N, 0))
    _check_rows(t, "t", M, 4)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=qx.device)
    _check_out(out, M, N)
    ws_ptr, ws_bytes = _workspace_args(workspace, _dev_tensor(qx, "qx"), M, N, K, GROUP)
    _check("qoq_w4a8_gemm_pc_i32",
           lib().qoq_w4a8_gemm_pc_i32(_dev(qx, "qx", torch.int8), _dev(t, "t", torch.int32),
                                      _dev(packed, "packed", torch.uint8), _dev(zeros, "zeros", torch.uint8),
                                      _dev(out, "acc", torch.int32), M, N, K, ws_ptr, ws_bytes, _stream(qx)))
    return out


# Split-K workspaces, one per (device, stream), grown when a shape needs more.
_workspaces = {}


def workspace_for(qx: torch.Tensor, M: int, N: int, K: int, group: int = GROUP):
    """The cached workspace of qx's device and current stream, sized for (M, N, K)
    (None when the plan needs none)."""
    need = gemm_workspace_bytes(M, N, K, group)
    if need == 0:
        return None
    key = (qx.device.index, torch.cuda.current_stream(qx.device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the split-K workspace for this shape does not exist yet and cannot be "
                               "allocated during graph capture: call once before capturing or pass workspace=")
        ws = torch.empty(max(need, 2 * ws.numel() if ws is not None else 0), dtype=torch.uint8, device=qx.device)
        _workspaces[key] = ws
    return ws


def _workspace_args(workspace, qx, M, N, K, group):
    if workspace is None:
        workspace = workspace_for(qx, M, N, K, group)
    if workspace is None:
        return ctypes.c_void_p(0), 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def w4a8_gemm(qx, s_x, packed, meta, s_w, N: int, out=None, group: int = GROUP, workspace=None):
    """out fp16 [M, N] = fp16(acc * (s_x[m] * s_w[n])).  workspace: None = the cached
    one of this device and stream (see qoq_gemm_workspace_bytes for the contract)."""
    M, K = qx.shape
    _check_weights(packed, meta, s_w, N, K)
    _check_rows(s_x, "s_x", M, 2)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=qx.device)
    _check_out(out, M, N)
    ws_ptr, ws_bytes = _workspace_args(workspace, _dev_tensor(qx, "qx"), M, N, K, group)
    _check("qoq_w4a8_gemm",
           lib().qoq_w4a8_gemm(_dev(qx, "qx", torch.int8), _dev(s_x, "s_x", torch.float16),
                               _dev(packed, "packed", torch.uint8), _dev(meta, "meta", torch.int16),
                               _dev(s_w, "s_w", torch.float16), _dev(out, "out", torch.float16), M, N, K, group,
                               ws_ptr, ws_bytes, _stream(qx)))
    return out


def w4a8_gemm_i32(qx, packed, meta, N: int, out=None, group: int = GROUP, workspace=None):
    """acc int32 [M, N]: the exact integer accumulators of the same main loop."""
    M, K = qx.shape
    _check_bytes(packed, "packed", N * K // 2 if N > 0 else 0)
    _check_bytes(meta, "meta", 2 * N * (K // GROUP) if N > 0 else 0)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=qx.device)
    _check_out(out, M, N)
    ws_ptr, ws_bytes = _workspace_args(workspace, _dev_tensor(qx, "qx"), M, N, K, group)
    _check("qoq_w4a8_gemm_i32",
           lib().qoq_w4a8_gemm_i32(_dev(qx, "qx", torch.int8), _dev(packed, "packed", torch.uint8),
                                   _dev(meta, "meta", torch.int16), _dev(out, "acc", torch.int32), M, N, K, group,
                                   ws_ptr, ws_bytes, _stream(qx)))
    return out


def _check_tiled(qx, M, K):
    if qx.numel() < tiled_bytes(M, K):
        raise ValueError(f"qx_tiled holds {qx.numel()} bytes, {tiled_bytes(M, K)} needed")


def w4a8_gemm_tiled(qx_tiled, s_x, packed, meta, s_w, M: int, N: int, K: int, out=None):
    """qoq_w4a8_gemm on tiled activation codes (M <= 64): out fp16 [M, N]."""
    _check_tiled(qx_tiled, M, K)
    _check_weights(packed, meta, s_w, N, K)
    _check_rows(s_x, "s_x", M, 2)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=qx_tiled.device)
    _check_out(out, M, N)
    _check("qoq_w4a8_gemm_tiled",
           lib().qoq_w4a8_gemm_tiled(_dev(qx_tiled, "qx_tiled", torch.int8), _dev(s_x, "s_x", torch.float16),
                                     _dev(packed, "packed", torch.uint8), _dev(meta, "meta", torch.int16),
                                     _dev(s_w, "s_w", torch.float16), _dev(out, "out", torch.float16), M, N, K,
                                     _stream(qx_tiled)))
    return out


def w4a8_gemm_tiled_i32(qx_tiled, packed, meta, M: int, N: int, K: int, out=None):
    """Exact INT32 accumulators from tiled activation codes (M <= 64)."""
    _check_tiled(qx_tiled, M, K)
    _check_bytes(packed, "packed", N * K // 2 if N > 0 else 0)
    _check_bytes(meta, "meta", 2 * N * (K // GROUP) if N > 0 else 0)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=qx_tiled.device)
    _check_out(out, M, N)
    _check("qoq_w4a8_gemm_tiled_i32",
           lib().qoq_w4a8_gemm_tiled_i32(_dev(qx_tiled, "qx_tiled", torch.int8), _dev(packed, "packed", torch.uint8),
                                         _dev(meta, "meta", torch.int16), _dev(out, "acc", torch.int32), M, N, K,
                                         _stream(qx_tiled)))
    return out


def quantize_activations_rowsum_tiled(x: torch.Tensor, out=None):
    """X fp16 [M, K] (M <= 64) -> (qx_tiled int8 [round_up(M, 16) * K], s_x fp16 [M],
    t int32 [M] = sum_k qx): the inputs of w4a8_gemm_pc_tiled."""
    M, K = x.shape
    if out is None:
        qx = torch.empty(tiled_bytes(M, K), dtype=torch.int8, device=x.device)
        s_x = torch.empty(M, dtype=torch.float16, device=x.device)
        t = torch.empty(M, dtype=torch.int32, device=x.device)
    else:
        qx, s_x, t = out
    if qx.numel() < tiled_bytes(M, K):
        raise ValueError(f"qx_tiled holds {qx.numel()} bytes, {tiled_bytes(M, K)} needed")
    _check("qoq_quantize_activations_rowsum_tiled",
           lib().qoq_quantize_activations_rowsum_tiled(_dev(x, "x", torch.float16), M, K, _dev(qx, "qx", torch.int8),
                                                       _dev(s_x, "s_x", torch.float16), _dev(t, "t", torch.int32),
                                                       _stream(x)))
    return qx, s_x, t


def w4a8_gemm_pc_tiled(qx_tiled, s_x, t, packed, zeros, s_w, M: int, N: int, K: int, out=None):
    """w4a8_gemm_pc on tiled activation codes (M <= 64): out fp16 [M, N]."""
    _check_tiled(qx_tiled, M, K)
    _check_weights(packed, zeros, s_w, N, K, per_channel=True)
    _check_rows(s_x, "s_x", M, 2)
    _check_rows(t, "t", M, 4)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=qx_tiled.device)
    _check_out(out, M, N)
    _check("qoq_w4a8_gemm_pc_tiled",
           lib().qoq_w4a8_gemm_pc_tiled(_dev(qx_tiled, "qx_tiled", torch.int8), _dev(s_x, "s_x", torch.float16),
                                        _dev(t, "t", torch.int32), _dev(packed, "packed", torch.uint8),
                                        _dev(zeros, "zeros", torch.uint8), _dev(s_w, "s_w", torch.float16),
                                        _dev(out, "out", torch.float16), M, N, K, _stream(qx_tiled)))
    return out


def w4a8_gemm_pc_tiled_i32(qx_tiled, t, packed, zeros, M: int, N: int, K: int, out=None):
    """Exact INT32 accumulators of the per-channel GEMM from tiled codes (M <= 64)."""
    _check_tiled(qx_tiled, M, K)
    _check_bytes(packed, "packed", N * K // 2 if N > 0 else 0)
    _check_bytes(zeros, "zeros", max(N, 0))
    _check_rows(t, "t", M, 4)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=qx_tiled.device)
    _check_out(out, M, N)
    _check("qoq_w4a8_gemm_pc_tiled_i32",
           lib().qoq_w4a8_gemm_pc_tiled_i32(_dev(qx_tiled, "qx_tiled", torch.int8), _dev(t, "t", torch.int32),
                                            _dev(packed, "packed", torch.uint8), _dev(zeros, "zeros", torch.uint8),
                                            _dev(out, "acc", torch.int32), M, N, K, _stream(qx_tiled)))
    return out


def gemm_tiled_plan(M: int, N: int, K: int) -> str:
    return lib().qoq_gemm_tiled_plan(M, N, K).decode()


# ---------------------------------------------------------------------------
# diagnostics
# ---------------------------------------------------------------------------
def dequantize_packed(packed, meta, N: int, K: int, group: int = GROUP, out=None):
    _check_bytes(packed, "packed", N * K // 2 if N > 0 else 0)
    _check_bytes(meta, "meta", 2 * N * (K // GROUP) if N > 0 else 0)
    if out is None:
        out = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _check_bytes(out, "w_i8", N * K if N > 0 else 0)
    _check("qoq_dequantize_packed",
           lib().qoq_dequantize_packed(_dev(packed, "packed", torch.uint8), _dev(meta, "meta", torch.int16), N, K,
                                       group, _dev(out, "w_i8", torch.int8), _stream(packed)))
    return out


def stream_copy(src: torch.Tensor, dst: torch.Tensor):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _check("qoq_stream_copy", lib().qoq_stream_copy(_dev(src, "src"), _dev(dst, "dst"), nbytes, _stream(src)))
    return dst


def stream_read(src: torch.Tensor, sink: torch.Tensor, unroll: int = 4, blocks: int = 2048):
    nbytes = src.numel() * src.element_size()
    _check("qoq_stream_read", lib().qoq_stream_read(_dev(src, "src"), nbytes, _dev(sink, "sink"), unroll, blocks,
                                                    _stream(src)))


def mfma_peak(iters: int, blocks: int, sink: torch.Tensor):
    _check("qoq_mfma_peak", lib().qoq_mfma_peak(iters, blocks, _dev(sink, "sink"), _stream(sink)))


def mfma_peak_operands(a: torch.Tensor, b: torch.Tensor, iters: int, blocks: int, sink: torch.Tensor):
    """qoq_mfma_peak_operands: the MFMA loop on fragments read from a and b."""
    _check("qoq_mfma_peak_operands",
           lib().qoq_mfma_peak_operands(_dev(a, "a"), _nbytes(a), _dev(b, "b"), _nbytes(b), iters, blocks,
                                        _dev(sink, "sink"), _stream(a)))


def mfma_probe(a: torch.Tensor, b: torch.Tensor):
    """a, b int8 [64, 16] per-lane operand bytes -> d int32 [64, 4] per-lane results."""
    if a.shape != (64, 16) or b.shape != (64, 16):
        raise ValueError("a and b must be int8 [64, 16]")
    d = torch.empty((64, 4), dtype=torch.int32, device=a.device)
    _check("qoq_mfma_probe", lib().qoq_mfma_probe(_dev(a, "a", torch.int8), _dev(b, "b", torch.int8),
                                                  _dev(d, "d", torch.int32), _stream(a)))
    return d


def mfma_probe32(a: torch.Tensor, b: torch.Tensor):
    """a, b int8 [64, 16] per-lane operand bytes -> d int32 [64, 16] per-lane results."""
    if a.shape != (64, 16) or b.shape != (64, 16):
        raise ValueError("a and b must be int8 [64, 16]")
    d = torch.empty((64, 16), dtype=torch.int32, device=a.device)
    _check("qoq_mfma_probe32", lib().qoq_mfma_probe32(_dev(a, "a", torch.int8), _dev(b, "b", torch.int8),
                                                      _dev(d, "d", torch.int32), _stream(a)))
    return d


# ---------------------------------------------------------------------------
# the runtime step in one call: quantize + GEMM (one fused kernel for few tokens)
# ---------------------------------------------------------------------------
def linear_workspace_bytes(M: int, N: int, K: int, group: int = GROUP) -> int:
    v = _c_sz()
    _check("qoq_linear_workspace_bytes", lib().qoq_linear_workspace_bytes(M, N, K, group, ctypes.byref(v)))
    return v.value


def linear_plan(M: int, N: int, K: int) -> str:
    return lib().qoq_linear_plan(M, N, K).decode()


def linear_configs() -> list:
    """Names of the fused linear configurations."""
    out, i = [], 0
    while True:
        n = lib().qoq_linear_config_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


_linear_workspaces = {}


def linear_workspace_for(x: torch.Tensor, M: int, N: int, K: int, group: int = GROUP):
    """Cached workspace of x's device and current stream for (M, N, K), or None."""
    need = linear_workspace_bytes(M, N, K, group)
    if need == 0:
        return None
    key = (x.device.index, torch.cuda.current_stream(x.device).cuda_stream)
    ws = _linear_workspaces.get(key)
    if ws is None or ws.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the linear workspace for this shape does not exist yet and cannot be "
                               "allocated during graph capture: call once before capturing or pass workspace=")
        ws = torch.empty(max(need, 2 * ws.numel() if ws is not None else 0), dtype=torch.uint8, device=x.device)
        _linear_workspaces[key] = ws
    return ws


def w4a8_linear(x: torch.Tensor, packed, meta, s_w, N: int, out=None, s_x=None, group: int = GROUP,
                workspace=None):
    """out fp16 [M, N] = quantize(x) then the W4A8 GEMM, in one library call.
    s_x: optional fp16 [M] tensor that receives the token scales."""
    M, K = x.shape
    _check_weights(packed, meta, s_w, N, K)
    if s_x is not None:
        _check_rows(s_x, "s_x", M, 2)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check_out(out, M, N)
    if workspace is None:
        workspace = linear_workspace_for(_dev_tensor(x, "x"), M, N, K, group)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    sx_ptr = _dev(s_x, "s_x", torch.float16) if s_x is not None else ctypes.c_void_p(0)
    _check("qoq_w4a8_linear",
           lib().qoq_w4a8_linear(_dev(x, "x", torch.float16), _dev(packed, "packed", torch.uint8),
                                 _dev(meta, "meta", torch.int16), _dev(s_w, "s_w", torch.float16),
                                 _dev(out, "out", torch.float16), sx_ptr, M, N, K, group, ws_ptr, ws_bytes,
                                 _stream(x)))
    return out


SCRATCH_BYTES = 64 << 20        # QOQ_SCRATCH_BYTES


def w4a8_linear_noalloc(x: torch.Tensor, packed, meta, s_w, N: int, out=None, s_x=None, group: int = GROUP):
    """qoq_w4a8_linear_noalloc: w4a8_linear without a workspace (the library's static
    scratch array instead); pass `out` to make the whole call allocation-free."""
    M, K = x.shape
    _check_weights(packed, meta, s_w, N, K)
    if s_x is not None:
        _check_rows(s_x, "s_x", M, 2)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check_out(out, M, N)
    sx_ptr = _dev(s_x, "s_x", torch.float16) if s_x is not None else ctypes.c_void_p(0)
    _check("qoq_w4a8_linear_noalloc",
           lib().qoq_w4a8_linear_noalloc(_dev(x, "x", torch.float16), _dev(packed, "packed", torch.uint8),
                                         _dev(meta, "meta", torch.int16), _dev(s_w, "s_w", torch.float16),
                                         _dev(out, "out", torch.float16), sx_ptr, M, N, K, group, _stream(x)))
    return out
