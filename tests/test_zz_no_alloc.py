"""qoq_w4a8_linear_noalloc (the entry point that allocates nothing) against
qoq_w4a8_linear: the same kernels with the library's static scratch array in place
of the caller's workspace, so the fp16 outputs and token scales must be bit-equal.
Two calls in a row share the array, the second with a smaller input (the first
call's contents are still there); a shape beyond the array's size is refused before
anything is launched; the fused few-token path needs no scratch at all."""
import numpy as np
import pytest
import torch

from w4a8_mixed_precision_amd import qoq
from w4a8_mixed_precision_amd import workloads as wl

pytestmark = pytest.mark.gpu

SCRATCH = -6


def say(msg):
    print(f"[case] {msg}", flush=True)


def _packed(N, K, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w = (torch.randn((N, K), generator=g, device=dev) * 0.02).half()
    return qoq.quantize_pack_weights(w)


def _x(M, K, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, device=dev).half()
    x[:, :: max(1, K // 40)] *= 20                      # outlier channels
    if M > 3:
        x[2] = 0                                         # an all-zero token
    return x


def _compare(x, packed, meta, s_w, N):
    M, K = x.shape
    need = qoq.linear_workspace_bytes(M, N, K)
    ws = torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device=x.device)
    sx_ref = torch.empty(M, dtype=torch.float16, device=x.device)
    ref = qoq.w4a8_linear(x, packed, meta, s_w, N, s_x=sx_ref, workspace=ws if need else None)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=x.device)
    sx = torch.empty(M, dtype=torch.float16, device=x.device)
    qoq.w4a8_linear_noalloc(x, packed, meta, s_w, N, out=out, s_x=sx)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(sx.view(torch.int16), sx_ref.view(torch.int16))
    return need


def test_noalloc_two_calls_second_smaller(gpu):
    L = wl.find("llama3_8b_down")
    packed, meta, s_w = _packed(L.N, L.K, gpu, 7)
    for M in (256, 70, 17):                # split-K partials + row-major codes; row-major; tiled codes
        say(f"linear_noalloc {L.name} M={M} plan={qoq.linear_plan(M, L.N, L.K)} "
            f"splits={qoq.gemm_plan_splits(M, L.N, L.K)} scratch={qoq.linear_workspace_bytes(M, L.N, L.K)}")
        need = _compare(_x(M, L.K, gpu, M), packed, meta, s_w, L.N)
        assert 0 < need <= qoq.SCRATCH_BYTES


def test_noalloc_after_other_shapes(gpu):
    """A different layer after the previous test's calls, then the fused path
    (no scratch), then a ragged shape."""
    for name, M in (("llama3_8b_gate_up", 1024), ("llama3_8b_qkv", 1), ("llama3_8b_qkv", 33)):
        L = wl.find(name)
        packed, meta, s_w = _packed(L.N, L.K, gpu, M)
        say(f"linear_noalloc {name} M={M} plan={qoq.linear_plan(M, L.N, L.K)}")
        _compare(_x(M, L.K, gpu, M + 1), packed, meta, s_w, L.N)
    packed, meta, s_w = _packed(144, 256, gpu, 3)
    say("linear_noalloc ragged M=65 N=144 K=256")
    _compare(_x(65, 256, gpu, 65), packed, meta, s_w, 144)


def test_noalloc_rejects_shapes_beyond_scratch(gpu):
    L = wl.find("llama3_8b_down_prefill")
    M = 8192
    assert qoq.linear_workspace_bytes(M, L.N, L.K) > qoq.SCRATCH_BYTES
    say(f"linear_noalloc beyond the scratch: {L.name} M={M}")
    packed = torch.empty(L.N * L.K // 2, dtype=torch.uint8, device=gpu)
    meta = torch.empty(L.N * L.K // 128, dtype=torch.int16, device=gpu)
    s_w = torch.empty(L.N, dtype=torch.float16, device=gpu)
    x = torch.zeros((M, L.K), dtype=torch.float16, device=gpu)
    out = torch.full((M, L.N), 3.0, dtype=torch.float16, device=gpu)
    with pytest.raises(qoq.QoQError) as e:
        qoq.w4a8_linear_noalloc(x, packed, meta, s_w, L.N, out=out)
    assert e.value.status == SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())                      # nothing was launched
