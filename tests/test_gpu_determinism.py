"""Repeat-run determinism of every kernel the planner selects, at full size.

For every layer shape and batch size of the workloads, in the launch configuration
the library picks: the GEMM on row-major codes (INT32 and fp16 epilogues, split-K
plans included) and the linear entry point (the fused few-token kernel, the tiled
few-token kernels or the quantizer + GEMM plan) run twice on the same inputs and
must agree bit for bit.  Every reduction in the library has a fixed order (LDS
sums across waves, split-K slices summed by a second kernel), so nothing may
depend on timing.  Inputs are drawn on the device from a seeded generator: the
comparison is between two runs, not against the oracle (the parity tests do that).
"""
import pytest
import torch

from w4a8_mixed_precision_amd import qoq
from w4a8_mixed_precision_amd import workloads as wl

pytestmark = pytest.mark.gpu

_CASES = [(L.name, M) for L in wl.LAYERS for M in L.Ms]


def say(msg):
    print(f"[case] {msg}", flush=True)


_weights = {}


def _packed(name, dev):
    """Packed weights of a random fp16 matrix of the layer's shape (one layer kept)."""
    if name not in _weights:
        _weights.clear()
        torch.cuda.empty_cache()
        L = wl.find(name)
        g = torch.Generator(device=dev)
        g.manual_seed(L.cfg * 100 + L.layer)
        w = (torch.randn((L.N, L.K), generator=g, device=dev) * 0.02).half()
        _weights[name] = qoq.quantize_pack_weights(w)
        del w
    return _weights[name]


@pytest.mark.parametrize("name,M", _CASES)
def test_planned_kernels_repeat_bit_for_bit(gpu, name, M):
    L = wl.find(name)
    N, K = L.N, L.K
    say(f"determinism {name} M={M} gemm={qoq.gemm_plan(M, N, K)} splits={qoq.gemm_plan_splits(M, N, K)} "
        f"linear={qoq.linear_plan(M, N, K)}")
    packed, meta, s_w = _packed(name, gpu)
    g = torch.Generator(device=gpu)
    g.manual_seed(M)
    x = torch.randn((M, K), generator=g, device=gpu).half()
    qx, s_x = qoq.quantize_activations(x)
    runs = []
    for _ in range(2):
        acc = qoq.w4a8_gemm_i32(qx, packed, meta, N)
        out = qoq.w4a8_gemm(qx, s_x, packed, meta, s_w, N)
        lin = qoq.w4a8_linear(x, packed, meta, s_w, N)
        runs.append((acc, out, lin))
    torch.cuda.synchronize()
    (a1, o1, l1), (a2, o2, l2) = runs
    assert torch.equal(a1, a2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int16), l2.view(torch.int16))
    # the linear entry point and the two-step path give the same fp16 values
    assert torch.equal(l1.view(torch.int16), o1.view(torch.int16))
