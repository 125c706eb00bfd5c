"""C-ABI checks that need no GPU: the library loads, exports every function
include/qoq.h declares, and rejects bad arguments with the documented status
before anything is launched (no call here reaches the HIP runtime)."""
import ctypes

import pytest

from w4a8_mixed_precision_amd import qoq

OK, INVALID, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIPERR, SCRATCH = 0, -1, -2, -3, -4, -5, -6
FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x10001)        # misaligned
NUL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def L():
    return qoq.lib()


def test_exports_every_declared_symbol(L):
    names = qoq.header_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert qoq.version() >= 1
    for s in (OK, INVALID, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIPERR, SCRATCH):
        assert qoq.status_string(s)
    assert qoq.status_string(12345) == "unknown status"


def test_weight_buffer_sizes():
    s = qoq.weight_buffer_sizes(6144, 4096)
    assert s == {"packed_w": 6144 * 4096 // 2, "group_meta": 6144 * 32 * 2, "s_w": 6144 * 2}
    with pytest.raises(qoq.QoQError) as e:
        qoq.weight_buffer_sizes(6144, 4096, group=64)
    assert e.value.status == UNSUPPORTED
    for N, K in [(0, 128), (17, 128), (16, 100), (16, -128)]:
        with pytest.raises(qoq.QoQError) as e:
            qoq.weight_buffer_sizes(N, K)
        assert e.value.status == INVALID
    with pytest.raises(qoq.QoQError) as e:
        qoq.weight_buffer_sizes(16, 139648 + 128)
    assert e.value.status == UNSUPPORTED


def test_config_names():
    names = qoq.gemm_configs()
    assert len(names) >= 4 and len(set(names)) == len(names)
    assert any(n.startswith("skinny") for n in names) and any(n.startswith("dma2") for n in names)
    assert qoq.gemm_plan(1, 6144, 4096) in names


@pytest.mark.parametrize("regime", [None, "skinny", "tiled"])
def test_plan_defined_for_every_shape(regime):
    """The planner (host code) returns a real configuration for every batch size,
    also under the measurement overrides."""
    names = set(qoq.gemm_configs())
    with qoq.plan_override(regime=regime):
        for (N, K) in [(16, 128), (6144, 4096), (4096, 14336), (59136, 8192), (8192, 29568)]:
            for M in list(range(1, 300)) + [511, 512, 1023, 4096, 8192, 100000]:
                assert qoq.gemm_plan(M, N, K) in names, (M, N, K, regime)
    for name in names:
        with qoq.plan_override(config=name):
            assert qoq.gemm_plan(77, 6144, 4096) == name


def test_plan_override_rejects_unknown_names():
    """Unknown names and negative split factors are refused and change nothing."""
    before = qoq.gemm_plan(300, 6144, 4096)
    for kw in ({"config": "no_such_config"}, {"regime": "sideways"}, {"linear": "nothing"}, {"splits": -1}):
        with pytest.raises(qoq.QoQError) as e:
            qoq.set_plan_override(**kw)
        assert e.value.status == INVALID
    assert qoq.gemm_plan(300, 6144, 4096) == before


def _table_rows():
    """Rows of the measured dispatch table as compiled into the library."""
    import os
    import re
    path = os.path.join(os.path.dirname(qoq.LIB_PATH), "..", "csrc", "qoq_plan_table.inc")
    rows = re.findall(r'QOQ_PLAN_ROW\((\d+), (\d+), (\d), (\d+), "([^"]+)", (\d+)\)', open(path).read())
    return [(int(n), int(k), int(t), int(m), c, int(sp)) for n, k, t, m, c, sp in rows]


def test_plan_table_rows():
    """The planner takes the table's configuration (and split factor) at every
    profiled point, and between two points the row of the nearer M (in ratio); the
    table covers every (N, K) of the workloads in both code layouts."""
    rows = _table_rows()
    assert len(rows) >= 200
    for (N, K, t, M, cfg, sp) in rows:
        plan = qoq.gemm_tiled_plan(M, N, K) if t else qoq.gemm_plan(M, N, K)
        assert plan == cfg, (N, K, t, M, plan, cfg)
        if not t and not cfg.startswith("skinny"):
            assert qoq.gemm_plan_splits(M, N, K) == min(sp, K // 128)
    from w4a8_mixed_precision_amd import workloads as wl
    for L in wl.LAYERS:
        for t in (0, 1):
            assert any((N, K, tt) == (L.N, L.K, t) for (N, K, tt, *_r) in rows), (L.name, t)
    # nearest in ratio: 1536 lies between 1024 and 2048 (ratio 1.5 vs 1.33 -> 2048)
    by_m = {M: cfg for (N, K, t, M, cfg, sp) in rows if (N, K, t) == (28672, 4096, 0)}
    assert qoq.gemm_plan(1400, 28672, 4096) == by_m[1536]
    assert qoq.gemm_plan(100000, 28672, 4096) == by_m[8192]


def test_every_config_is_in_the_table():
    """Every configuration compiled into the library is the table's choice at some
    profiled point (the rest were dropped from the build)."""
    used = {r[4] for r in _table_rows()}
    names = qoq.gemm_configs()
    assert set(names) == used, (set(names) - used, used - set(names))


def _linear_rows():
    """Rows of the measured linear table as compiled into the library."""
    import os
    import re
    path = os.path.join(os.path.dirname(qoq.LIB_PATH), "..", "csrc", "qoq_linear_table.inc")
    rows = re.findall(r'QOQ_LINEAR_ROW\((\d+), (\d+), (\d+), "([^"]+)"\)', open(path).read())
    return [(int(n), int(k), int(m), c) for n, k, m, c in rows]


def test_linear_table_rows():
    """The linear entry point takes the table's choice at every profiled point: the
    named fused kernel, or the quantizer + GEMM pair (then the GEMM plan of the
    tiled codes); every fused configuration in the build except the rule's default
    is the table's choice somewhere; beyond the largest profiled M the pair."""
    rows = _linear_rows()
    fused = qoq.linear_configs()
    assert rows and all(c in fused or c == "unfused" for (_n, _k, _m, c) in rows)
    for (N, K, M, cfg) in rows:
        plan = qoq.linear_plan(M, N, K)
        if cfg == "unfused":
            assert plan == qoq.gemm_tiled_plan(M, N, K), (N, K, M, plan)
        else:
            assert plan == cfg, (N, K, M, plan, cfg)
    used = {c for (_n, _k, _m, c) in rows}
    assert set(fused[1:]) <= used, set(fused[1:]) - used
    N, K, _m, _c = rows[-1]
    assert qoq.linear_plan(16, N, K) == qoq.gemm_tiled_plan(16, N, K)
    # outside the table the rule: the first fused configuration up to two tokens
    assert qoq.linear_plan(1, 4096, 1024) == fused[0]
    assert qoq.linear_plan(3, 4096, 1024) == qoq.gemm_tiled_plan(3, 4096, 1024)


def test_plan_rules_outside_the_table():
    """Shapes the table does not cover get a configuration from the rules."""
    names = set(qoq.gemm_configs())
    for (N, K) in [(1024, 2048), (12288, 5120), (2048, 33280)]:
        for M in (1, 16, 40, 64, 100, 300, 1000, 5000):
            assert qoq.gemm_plan(M, N, K) in names
            assert qoq.gemm_tiled_plan(min(M, 64), N, K) in names
    # the rules' own picks (each a configuration of the build, not the fallback):
    # few-token kernels up to 16 tokens, 32-row blocks to 64, the shared-dequantization
    # kernel for the largest tile counts, the copy-engine tile kernel for few tiles
    assert qoq.gemm_plan(1, 12288, 5120) == "skinny_mt1_nb1_w8_u2_nt"     # wide, short K
    assert qoq.gemm_plan(1, 2048, 33280) == "skinny_mt1_nb2_w16_u2_nt"
    assert qoq.gemm_plan(8, 1024, 2048) == "skinny_mt1_nb1_w8_u2_nt"
    assert qoq.gemm_plan(40, 12288, 5120) == "skinny32_mt2_np2_w8_u1_r2_nt"
    assert qoq.gemm_plan(5000, 12288, 5120) == "sd_as3"
    assert qoq.gemm_plan(300, 1024, 2048) == "dma2_tm4_tn1"


def test_split_plan_and_workspace():
    """Split-K plans: factor, workspace size (splits x M x N INT32 partial sums),
    and the override."""
    split_rows = [r for r in _table_rows() if r[2] == 0 and r[5] > 1]
    assert split_rows
    N, K, _t, M, cfg, sp = split_rows[0]
    assert qoq.gemm_plan(M, N, K) == cfg and qoq.gemm_plan_splits(M, N, K) == sp
    assert qoq.gemm_workspace_bytes(M, N, K) == sp * M * N * 4
    assert qoq.gemm_plan_splits(1, 6144, 4096) == 1 and qoq.gemm_workspace_bytes(1, 6144, 4096) == 0
    assert qoq.gemm_workspace_bytes(0, 6144, 4096) == 0
    tile = [n for n in qoq.gemm_configs() if n.startswith("dma2")][0]   # a split-K capable tile kernel
    for want, K in [(3, 4096), (16, 4096), (2, 256), (1, 128)]:
        with qoq.plan_override(config=tile, splits=want):
            assert qoq.gemm_plan_splits(300, 1024, K) == min(want, K // 128)
    with qoq.plan_override(config=tile, splits=1):
        assert qoq.gemm_workspace_bytes(300, 1024, 4096) == 0
    skinny = [n for n in qoq.gemm_configs() if n.startswith("skinny")][0]
    with qoq.plan_override(config=skinny, splits=8):               # no split-K support
        assert qoq.gemm_plan_splits(300, 1024, 4096) == 1
    with pytest.raises(qoq.QoQError):
        qoq.gemm_plan_splits(0, 1024, 4096)


def test_workspace_validation(L):
    """Shapes whose plan splits K need the workspace: NULL or short -> WORKSPACE,
    not 16-byte aligned -> ALIGNMENT (checked before any launch)."""
    N, K, _t, M, _c, _s = [r for r in _table_rows() if r[2] == 0 and r[5] > 1][0]
    need = qoq.gemm_workspace_bytes(M, N, K)
    assert need > 0
    f = L.qoq_w4a8_gemm
    a = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, 128)
    assert f(*a, NUL, 0, NUL) == WORKSPACE
    assert f(*a, FAKE, need - 1, NUL) == WORKSPACE
    assert f(*a, ctypes.c_void_p(0x10008), need, NUL) == ALIGNMENT
    g = L.qoq_w4a8_gemm_i32
    assert g(FAKE, FAKE, FAKE, FAKE, M, N, K, 128, NUL, 0, NUL) == WORKSPACE


def test_workspace_and_plan():
    assert qoq.gemm_workspace_bytes(16, 6144, 4096) == 0
    assert qoq.gemm_plan(1, 6144, 4096).startswith("skinny")
    assert qoq.gemm_plan(4096, 28672, 4096).startswith(("dma2", "sd", "wide2"))
    assert qoq.gemm_plan(1, 17, 4096) == "invalid"
    assert qoq.gemm_plan(0, 16, 128) == "invalid"


def test_pack_validation(L):
    f = L.qoq_quantize_pack_weights
    assert f(FAKE, 32, 256, 64, FAKE, FAKE, FAKE, NUL) == UNSUPPORTED
    assert f(FAKE, 33, 256, 128, FAKE, FAKE, FAKE, NUL) == INVALID
    assert f(FAKE, 32, 200, 128, FAKE, FAKE, FAKE, NUL) == INVALID
    assert f(NUL, 32, 256, 128, FAKE, FAKE, FAKE, NUL) == INVALID
    assert f(ODD, 32, 256, 128, FAKE, FAKE, FAKE, NUL) == ALIGNMENT
    assert f(FAKE, 32, 256, 128, ODD, FAKE, FAKE, NUL) == ALIGNMENT


def test_activation_validation(L):
    f = L.qoq_quantize_activations
    assert f(FAKE, -1, 256, FAKE, FAKE, NUL) == INVALID
    assert f(FAKE, 4, 12, FAKE, FAKE, NUL) == INVALID
    assert f(FAKE, 4, 0, FAKE, FAKE, NUL) == INVALID
    assert f(NUL, 0, 256, NUL, NUL, NUL) == OK          # empty batch: nothing to do
    assert f(NUL, 4, 256, FAKE, FAKE, NUL) == INVALID
    assert f(ODD, 4, 256, FAKE, FAKE, NUL) == ALIGNMENT


def test_gemm_validation(L):
    f = L.qoq_w4a8_gemm
    args = lambda qx=FAKE, sx=FAKE, pw=FAKE, md=FAKE, sw=FAKE, out=FAKE, M=4, N=32, K=256, g=128: (
        qx, sx, pw, md, sw, out, M, N, K, g, NUL, 0, NUL)
    assert f(*args(g=32)) == UNSUPPORTED
    assert f(*args(N=40)) == INVALID
    assert f(*args(K=192)) == INVALID
    assert f(*args(M=-1)) == INVALID
    assert f(*args(M=0, qx=NUL, out=NUL)) == OK
    assert f(*args(qx=NUL)) == INVALID
    assert f(*args(sx=NUL)) == INVALID
    assert f(*args(qx=ODD)) == ALIGNMENT
    assert f(*args(pw=ODD)) == ALIGNMENT
    assert f(*args(md=ctypes.c_void_p(0x10002))) == ALIGNMENT
    assert f(*args(out=ODD)) == ALIGNMENT
    assert f(*args(out=ctypes.c_void_p(0x10008))) == ALIGNMENT
    assert f(*args(K=139648 + 128)) == UNSUPPORTED
    g = L.qoq_w4a8_gemm_i32
    assert g(FAKE, FAKE, FAKE, NUL, 4, 32, 256, 128, NUL, 0, NUL) == INVALID
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 32, 256, 96, NUL, 0, NUL) == UNSUPPORTED


def test_diag_validation(L):
    assert L.qoq_stream_copy(FAKE, FAKE, 17, NUL) == INVALID
    assert L.qoq_stream_copy(ODD, FAKE, 32, NUL) == ALIGNMENT
    assert L.qoq_stream_copy(FAKE, FAKE, 0, NUL) == OK
    assert L.qoq_stream_read(FAKE, 32, NUL, 4, 8, NUL) == INVALID
    assert L.qoq_stream_read(FAKE, 17, FAKE, 4, 8, NUL) == INVALID
    assert L.qoq_stream_read(ODD, 32, FAKE, 4, 8, NUL) == ALIGNMENT
    assert L.qoq_mfma_peak(0, 8, FAKE, NUL) == INVALID
    assert L.qoq_mfma_peak(8, 8, ODD, NUL) == ALIGNMENT
    f = L.qoq_mfma_peak_operands
    assert f(NUL, 64, FAKE, 64, 8, 8, FAKE, NUL) == INVALID
    assert f(FAKE, 8, FAKE, 64, 8, 8, FAKE, NUL) == INVALID        # fewer than one fragment
    assert f(FAKE, 64, FAKE, 64, 0, 8, FAKE, NUL) == INVALID
    assert f(FAKE, 64, FAKE, 64, 8, 0, FAKE, NUL) == INVALID
    assert f(ODD, 64, FAKE, 64, 8, 8, FAKE, NUL) == ALIGNMENT
    assert f(FAKE, 64, FAKE, 64, 8, 8, ODD, NUL) == ALIGNMENT
    assert L.qoq_mfma_probe(NUL, FAKE, FAKE, NUL) == INVALID
    assert L.qoq_mfma_probe32(FAKE, NUL, FAKE, NUL) == INVALID
    assert L.qoq_mfma_probe32(FAKE, FAKE, ODD, NUL) == ALIGNMENT
    assert L.qoq_mfma_probe(ODD, FAKE, FAKE, NUL) == ALIGNMENT
    assert L.qoq_dequantize_packed(FAKE, FAKE, 32, 100, 128, FAKE, NUL) == INVALID
    assert L.qoq_dequantize_packed(ODD, FAKE, 32, 256, 128, FAKE, NUL) == ALIGNMENT


def test_binding_size_checks():
    """The binding compares every buffer with (M, N, K) before the library sees a
    pointer: packed codes, group metadata (or per-channel zeros), channel scales,
    token scales, code sums and the output shape (ValueError, nothing launched)."""
    import torch
    M, N, K = 4, 64, 256
    i8 = lambda *sh: torch.zeros(sh, dtype=torch.int8)
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)
    f16 = lambda *sh: torch.zeros(sh, dtype=torch.float16)
    i16 = lambda n: torch.zeros(n, dtype=torch.int16)
    i32 = lambda *sh: torch.zeros(sh, dtype=torch.int32)
    qx, sx, t = i8(M, K), f16(M), i32(M)
    good = dict(packed=u8(N * K // 2), meta=i16(N * K // 128), s_w=f16(N))
    bad = [dict(good, packed=u8(N * K // 2 - 16)), dict(good, meta=i16(N * K // 128 - 1)), dict(good, s_w=f16(N - 1))]
    for b in bad:
        with pytest.raises(ValueError):
            qoq.w4a8_gemm(qx, sx, b["packed"], b["meta"], b["s_w"], N)
        with pytest.raises(ValueError):
            qoq.w4a8_linear(f16(M, K), b["packed"], b["meta"], b["s_w"], N)
        with pytest.raises(ValueError):
            qoq.w4a8_gemm_tiled(i8(16 * K), sx, b["packed"], b["meta"], b["s_w"], M, N, K)
    for b in bad[:2]:
        with pytest.raises(ValueError):
            qoq.w4a8_gemm_i32(qx, b["packed"], b["meta"], N)
        with pytest.raises(ValueError):
            qoq.dequantize_packed(b["packed"], b["meta"], N, K)
    with pytest.raises(ValueError):                                     # token scales
        qoq.w4a8_gemm(qx, f16(M - 1), good["packed"], good["meta"], good["s_w"], N)
    with pytest.raises(ValueError):
        qoq.w4a8_linear(f16(M, K), good["packed"], good["meta"], good["s_w"], N, s_x=f16(M - 1))
    with pytest.raises(ValueError):                                     # output shape
        qoq.w4a8_gemm(qx, sx, good["packed"], good["meta"], good["s_w"], N, out=f16(M, N - 16))
    with pytest.raises(ValueError):
        qoq.w4a8_gemm_i32(qx, good["packed"], good["meta"], N, out=i32(M + 1, N))
    with pytest.raises(ValueError):
        qoq.w4a8_linear(f16(M, K), good["packed"], good["meta"], good["s_w"], N, out=f16(N, M))
    # per-channel: one zero byte per column, code sums per token
    with pytest.raises(ValueError):
        qoq.w4a8_gemm_pc(qx, sx, t, good["packed"], u8(N - 1), good["s_w"], N)
    with pytest.raises(ValueError):
        qoq.w4a8_gemm_pc(qx, sx, i32(M - 1), good["packed"], u8(N), good["s_w"], N)
    with pytest.raises(ValueError):
        qoq.w4a8_gemm_pc_i32(qx, t, u8(N * K // 2 - 1), u8(N), N)
    with pytest.raises(ValueError):
        qoq.w4a8_gemm_pc_tiled(i8(16 * K), sx, t, good["packed"], u8(N - 1), good["s_w"], M, N, K)
    with pytest.raises(ValueError):
        qoq.w4a8_gemm_pc_tiled_i32(i8(16 * K), t, good["packed"], u8(N), M, N, K, out=i32(M, N + 16))
    with pytest.raises(ValueError):                                     # attention output shape
        qoq.kv4_decode_attention(f16(2, 8, 128), u8(8704), i32(2, 1), i32(2), 1, 64, out=f16(2, 8, 64))


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((4, 256), dtype=torch.float16)
    with pytest.raises(TypeError):
        qoq.quantize_activations(x)


def test_linear_plan_and_workspace():
    """Fused linear for a few tokens and K <= 8192 (no workspace); two kernels
    otherwise: tiled codes (whole 16-row blocks) and s_X up to 64 tokens, row-major
    codes, s_X and the GEMM's own workspace beyond."""
    fused = qoq.linear_configs()
    assert len(fused) >= 1
    assert qoq.linear_plan(1, 6144, 4096) in fused
    assert qoq.linear_plan(2, 512, 512) in fused
    assert qoq.linear_plan(1, 59136, 8192) == qoq.gemm_tiled_plan(1, 59136, 8192)   # measured: the pair
    assert qoq.linear_workspace_bytes(1, 6144, 4096) == 0
    assert qoq.linear_plan(3, 6144, 4096) == qoq.gemm_tiled_plan(3, 6144, 4096)
    assert qoq.linear_plan(2, 131072, 8192) == qoq.gemm_tiled_plan(2, 131072, 8192)   # too much repeated work
    assert qoq.linear_plan(16, 6144, 4096) == qoq.gemm_tiled_plan(16, 6144, 4096)
    assert qoq.linear_plan(17, 6144, 4096) == qoq.gemm_tiled_plan(17, 6144, 4096)
    assert qoq.linear_plan(64, 28672, 4096) == qoq.gemm_tiled_plan(64, 28672, 4096)
    assert qoq.linear_plan(65, 6144, 4096) == qoq.gemm_plan(65, 6144, 4096)
    assert qoq.linear_plan(1, 4096, 20480) == qoq.gemm_tiled_plan(1, 4096, 20480)   # outside the table: K > 8192
    r256 = lambda v: (v + 255) // 256 * 256
    for M, N, K in [(17, 6144, 4096), (1, 4096, 20480), (64, 28672, 4096)]:
        assert qoq.linear_workspace_bytes(M, N, K) == r256((M + 15) // 16 * 16 * K) + r256(2 * M)
    for M, N, K in [(65, 6144, 4096), (256, 4096, 14336)]:
        assert qoq.linear_workspace_bytes(M, N, K) == r256(M * K) + r256(2 * M) + qoq.gemm_workspace_bytes(M, N, K)
    assert qoq.linear_workspace_bytes(0, 6144, 4096) == 0
    assert qoq.linear_plan(0, 6144, 4096) == "invalid"
    with qoq.plan_override(linear="unfused"):
        assert qoq.linear_plan(1, 6144, 4096) == qoq.gemm_tiled_plan(1, 6144, 4096)
        assert qoq.linear_workspace_bytes(1, 6144, 4096) == 16 * 4096 + 256
    for name in fused:                             # forced: any shape the kernel can hold
        with qoq.plan_override(linear=name):
            assert qoq.linear_plan(4, 6144, 4096) == name
            assert qoq.linear_plan(8, 6144, 2048) == name
            assert qoq.linear_plan(1, 59136, 8192) == name
            assert qoq.linear_plan(17, 6144, 4096) == qoq.gemm_tiled_plan(17, 6144, 4096)


def test_tiled_plans_and_validation(L):
    """The tiled-code GEMM runs few-token kernels only, up to 64 tokens."""
    for M, N, K in [(1, 6144, 4096), (16, 6144, 4096), (64, 6144, 4096), (64, 28672, 4096), (33, 4096, 14336)]:
        assert qoq.gemm_tiled_plan(M, N, K).startswith("skinny")
    assert qoq.gemm_tiled_plan(65, 6144, 4096) == "invalid"
    assert qoq.gemm_tiled_plan(0, 6144, 4096) == "invalid"
    assert qoq.tiled_bytes(1, 4096) == 16 * 4096 and qoq.tiled_bytes(17, 128) == 32 * 128
    q = L.qoq_quantize_activations_tiled
    assert q(FAKE, 65, 4096, FAKE, FAKE, NUL) == UNSUPPORTED
    assert q(FAKE, 4, 96, FAKE, FAKE, NUL) == INVALID              # K % 64
    assert q(FAKE, 0, 4096, NUL, NUL, NUL) == OK
    assert q(FAKE, 4, 4096, NUL, FAKE, NUL) == INVALID
    assert q(ODD, 4, 4096, FAKE, FAKE, NUL) == ALIGNMENT
    g = L.qoq_w4a8_gemm_tiled
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65, 6144, 4096, NUL) == UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 6144, 4000, NUL) == INVALID
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 6144, 4096, NUL) == OK
    assert g(FAKE, NUL, FAKE, FAKE, FAKE, FAKE, 4, 6144, 4096, NUL) == INVALID
    assert g(ODD, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 6144, 4096, NUL) == ALIGNMENT
    gi = L.qoq_w4a8_gemm_tiled_i32
    assert gi(FAKE, FAKE, FAKE, FAKE, 65, 6144, 4096, NUL) == UNSUPPORTED
    assert gi(FAKE, FAKE, FAKE, ODD, 4, 6144, 4096, NUL) == ALIGNMENT
    # per-channel weights on tiled codes
    qr = L.qoq_quantize_activations_rowsum_tiled
    assert qr(FAKE, 65, 4096, FAKE, FAKE, FAKE, NUL) == UNSUPPORTED
    assert qr(FAKE, 4, 96, FAKE, FAKE, FAKE, NUL) == INVALID              # K % 64
    assert qr(FAKE, 0, 4096, NUL, NUL, NUL, NUL) == OK
    assert qr(FAKE, 4, 4096, FAKE, FAKE, NUL, NUL) == INVALID             # no code sums
    assert qr(FAKE, 4, 4096, FAKE, FAKE, ctypes.c_void_p(0x10002), NUL) == ALIGNMENT
    gp = L.qoq_w4a8_gemm_pc_tiled
    assert gp(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65, 6144, 4096, NUL) == UNSUPPORTED
    assert gp(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 6144, 4000, NUL) == INVALID
    assert gp(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 6144, 4096, NUL) == OK
    assert gp(FAKE, FAKE, NUL, FAKE, FAKE, FAKE, FAKE, 4, 6144, 4096, NUL) == INVALID   # t_x
    assert gp(FAKE, FAKE, FAKE, FAKE, NUL, FAKE, FAKE, 4, 6144, 4096, NUL) == INVALID   # zeros
    assert gp(ODD, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 6144, 4096, NUL) == ALIGNMENT
    gpi = L.qoq_w4a8_gemm_pc_tiled_i32
    assert gpi(FAKE, FAKE, FAKE, FAKE, FAKE, 65, 6144, 4096, NUL) == UNSUPPORTED
    assert gpi(FAKE, FAKE, FAKE, FAKE, ODD, 4, 6144, 4096, NUL) == ALIGNMENT


def test_linear_validation(L):
    f = L.qoq_w4a8_linear
    a = lambda x=FAKE, pw=FAKE, md=FAKE, sw=FAKE, out=FAKE, sx=NUL, M=4, N=32, K=256, g=128, ws=NUL, wb=0: (
        x, pw, md, sw, out, sx, M, N, K, g, ws, wb, NUL)
    assert f(*a(g=64)) == UNSUPPORTED
    assert f(*a(N=40)) == INVALID
    assert f(*a(K=200)) == INVALID
    assert f(*a(M=-1)) == INVALID
    assert f(*a(M=0, x=NUL, out=NUL)) == OK
    assert f(*a(x=NUL)) == INVALID
    assert f(*a(sw=NUL)) == INVALID
    assert f(*a(x=ODD)) == ALIGNMENT
    assert f(*a(out=ctypes.c_void_p(0x10008))) == ALIGNMENT
    assert f(*a(sx=ODD)) == ALIGNMENT
    M, N, K = 64, 6144, 4096                      # two kernels: needs the workspace
    need = qoq.linear_workspace_bytes(M, N, K)
    assert f(*a(M=M, N=N, K=K)) == WORKSPACE
    assert f(*a(M=M, N=N, K=K, ws=FAKE, wb=need - 1)) == WORKSPACE
    assert f(*a(M=M, N=N, K=K, ws=ctypes.c_void_p(0x10010), wb=need)) == ALIGNMENT


def test_per_channel_sizes_and_validation(L):
    s = qoq.weight_buffer_sizes(6144, 4096, group=0)
    assert s == {"packed_w": 6144 * 4096 // 2, "group_meta": 6144, "s_w": 6144 * 2}
    f = L.qoq_quantize_pack_weights
    assert f(FAKE, 32, 256, 0, FAKE, ODD, FAKE, NUL) != ALIGNMENT    # zeros: bytes, any address
    r = L.qoq_quantize_activations_rowsum
    assert r(FAKE, 4, 256, FAKE, FAKE, NUL, NUL) == INVALID
    assert r(FAKE, 4, 256, FAKE, FAKE, ctypes.c_void_p(0x10002), NUL) == ALIGNMENT
    assert r(NUL, 0, 256, NUL, NUL, NUL, NUL) == OK
    g = L.qoq_w4a8_gemm_pc
    a = lambda qx=FAKE, sx=FAKE, t=FAKE, pw=FAKE, z=FAKE, sw=FAKE, out=FAKE, M=4, N=32, K=256: (
        qx, sx, t, pw, z, sw, out, M, N, K, NUL, 0, NUL)
    assert g(*a(t=NUL)) == INVALID
    assert g(*a(z=NUL)) == INVALID
    assert g(*a(t=ctypes.c_void_p(0x10002))) == ALIGNMENT
    assert g(*a(N=40)) == INVALID
    assert g(*a(M=0, qx=NUL, out=NUL)) == OK
    M, N, K = 256, 4096, 14336                    # split-K plan: needs the workspace
    assert g(*a(M=M, N=N, K=K)) == WORKSPACE
    h = L.qoq_w4a8_gemm_pc_i32
    assert h(FAKE, FAKE, FAKE, NUL, FAKE, 4, 32, 256, NUL, 0, NUL) == INVALID
    assert qoq.gemm_workspace_bytes(M, N, K, group=0) == qoq.gemm_workspace_bytes(M, N, K)


def test_fused_producer_validation(L):
    """RMSNorm / SiLU*up + quantization: argument checks before any launch."""
    r = L.qoq_rmsnorm_quantize
    ok = dict(x=FAKE, g=FAKE, eps=1e-5, M=4, K=4096, lay=0, q=FAKE, s=FAKE, t=NUL)
    call = lambda **kw: r(*[{**ok, **kw}[k] for k in ("x", "g", "eps", "M", "K", "lay", "q", "s", "t")], NUL)
    assert call(M=0) == OK
    assert call(eps=0.0) == INVALID and call(eps=-1.0) == INVALID
    assert call(K=100) == INVALID                               # K % 8
    assert call(K=32776) == UNSUPPORTED                         # one row in registers
    assert call(lay=2) == INVALID
    assert call(lay=1, K=4104) == INVALID                       # tiled: K % 64
    assert call(lay=1, M=65) == UNSUPPORTED
    assert call(x=NUL) == INVALID and call(q=NUL) == INVALID and call(s=NUL) == INVALID
    assert call(x=ODD) == ALIGNMENT and call(g=ODD) == ALIGNMENT and call(q=ODD) == ALIGNMENT
    assert call(t=ODD) == ALIGNMENT
    f = L.qoq_silu_mul_quantize
    ok2 = dict(gt=FAKE, up=FAKE, ld=8192, M=4, K=4096, lay=0, q=FAKE, s=FAKE, t=NUL)
    call2 = lambda **kw: f(*[{**ok2, **kw}[k] for k in ("gt", "up", "ld", "M", "K", "lay", "q", "s", "t")], NUL)
    assert call2(M=0) == OK
    assert call2(ld=4000) == INVALID                            # ld < K
    assert call2(ld=8196) == INVALID                            # ld % 8
    assert call2(K=40000, ld=40000) == UNSUPPORTED
    assert call2(lay=1, M=65) == UNSUPPORTED
    assert call2(gt=NUL) == INVALID and call2(up=NUL) == INVALID
    assert call2(gt=ODD) == ALIGNMENT and call2(up=ODD) == ALIGNMENT and call2(q=ODD) == ALIGNMENT


def test_kv4_validation(L):
    """KV4 cache entry points: sizes, splits and argument checks before any launch."""
    assert qoq.kv4_page_bytes(8) == 8 * 8704
    with pytest.raises(qoq.QoQError) as e:
        b = ctypes.c_size_t(0)
        qoq._check("qoq_kv4_page_bytes", L.qoq_kv4_page_bytes(8, 64, ctypes.byref(b)))
    assert e.value.status == UNSUPPORTED
    assert qoq.kv4_attention_workspace_bytes(64, 32, 8, 1024) == 0          # 512 workgroups already
    w = qoq.kv4_attention_workspace_bytes(1, 32, 8, 4096)                   # split over the sequence
    assert w > 0 and w % (32 * 130 * 4) == 0 and w // (32 * 130 * 4) <= 64
    wr = L.qoq_kv4_write
    assert wr(FAKE, FAKE, 2, 1, 8, 64, FAKE, FAKE, 4, FAKE, 16, NUL) == UNSUPPORTED       # head dim
    assert wr(FAKE, FAKE, 0, 1, 8, 128, FAKE, FAKE, 4, FAKE, 16, NUL) == OK
    assert wr(NUL, FAKE, 2, 1, 8, 128, FAKE, FAKE, 4, FAKE, 16, NUL) == INVALID
    assert wr(FAKE, FAKE, 2, 1, 8, 128, FAKE, FAKE, 4, ODD, 16, NUL) == ALIGNMENT
    assert wr(ctypes.c_void_p(0x10004), FAKE, 2, 1, 8, 128, FAKE, FAKE, 4, FAKE, 16, NUL) == ALIGNMENT   # 16-byte loads
    at = L.qoq_kv4_decode_attention
    args = lambda **kw: [kw.get(k, v) for k, v in dict(q=FAKE, pool=FAKE, np_=16, pt=FAKE, mp=4, sl=FAKE, B=2, h=32, hkv=8,
                                                           hd=128, ml=256, out=FAKE, ws=NUL, wb=0, st=NUL).items()]
    assert at(*args(h=30)) == INVALID                                       # h % h_kv
    assert at(*args(h=256, hkv=8)) == UNSUPPORTED                           # group of 32 heads
    assert at(*args(ml=257)) == INVALID                                     # beyond the page table
    assert at(*args(hd=64)) == UNSUPPORTED
    assert at(*args(B=0)) == OK
    assert at(*args(out=ODD)) == ALIGNMENT
    assert at(*args(B=1, ml=4096, mp=64)) == WORKSPACE                      # needs split partials
    assert at(*args(np_=0)) == INVALID and wr(FAKE, FAKE, 2, 1, 8, 128, FAKE, FAKE, 4, FAKE, 0, NUL) == INVALID


def test_smooth_attention_validation(L):
    lam = L.qoq_smooth_attention_lambda
    assert lam(FAKE, 0, 8, 128, ctypes.c_float(0.5), FAKE, NUL) == INVALID
    assert lam(FAKE, 10, 8, 128, ctypes.c_float(1.5), FAKE, NUL) == INVALID
    assert lam(FAKE, 10, 8, 64, ctypes.c_float(0.5), FAKE, NUL) == UNSUPPORTED
    assert lam(ODD, 10, 8, 128, ctypes.c_float(0.5), FAKE, NUL) == ALIGNMENT
    fold = L.qoq_smooth_attention_fold
    assert fold(FAKE, FAKE, FAKE, 30, 8, 128, 4096, FAKE, FAKE, NUL) == INVALID      # h % h_kv
    assert fold(FAKE, FAKE, FAKE, 32, 8, 64, 4096, FAKE, FAKE, NUL) == UNSUPPORTED
    assert fold(FAKE, FAKE, NUL, 32, 8, 128, 4096, FAKE, FAKE, NUL) == INVALID
    assert fold(FAKE, FAKE, ODD, 32, 8, 128, 4096, FAKE, FAKE, NUL) == ALIGNMENT


def test_silu_split_validation(L):
    b = ctypes.c_size_t(0)
    assert L.qoq_silu_mul_quantize_workspace_bytes(1, 29568, ctypes.byref(b)) == OK and b.value == 4 * 15
    assert L.qoq_silu_mul_quantize_workspace_bytes(65, 29568, ctypes.byref(b)) == OK and b.value == 0
    assert L.qoq_silu_mul_quantize_workspace_bytes(1, 12, ctypes.byref(b)) == INVALID
    f = L.qoq_silu_mul_quantize_ws
    assert f(FAKE, FAKE, 29568, 1, 29568, 0, FAKE, FAKE, NUL, 0, NUL) == WORKSPACE
    assert f(FAKE, FAKE, 29568, 1, 29568, 0, FAKE, FAKE, FAKE, 59, NUL) == WORKSPACE
    assert f(FAKE, FAKE, 29568, 1, 29568, 0, FAKE, FAKE, ODD, 60, NUL) == ALIGNMENT
    assert f(FAKE, FAKE, 100, 1, 29568, 0, FAKE, FAKE, FAKE, 60, NUL) == INVALID        # ld < K
    assert f(FAKE, FAKE, 29568, 0, 29568, 0, FAKE, FAKE, NUL, 0, NUL) == OK             # M = 0



def test_linear_noalloc_validation(L):
    """Argument checks of the allocation-free linear entry point, all before the
    scratch array is looked up or anything is launched: shapes, pointers, alignment,
    and shapes whose workspace would exceed QOQ_SCRATCH_BYTES."""
    f = L.qoq_w4a8_linear_noalloc
    assert qoq.SCRATCH_BYTES == 64 << 20
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, NUL, 0, 6144, 4096, 128, NUL) == OK          # nothing to do
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, NUL, 4, 6144, 4096, 64, NUL) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, NUL, 4, 6150, 4096, 128, NUL) == INVALID
    assert f(NUL, FAKE, FAKE, FAKE, FAKE, NUL, 4, 6144, 4096, 128, NUL) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, NUL, NUL, 4, 6144, 4096, 128, NUL) == INVALID
    assert f(ODD, FAKE, FAKE, FAKE, FAKE, NUL, 4, 6144, 4096, 128, NUL) == ALIGNMENT
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, ODD, 4, 6144, 4096, 128, NUL) == ALIGNMENT
    for M, N, K in [(8192, 4096, 14336), (4096, 4096, 29568)]:
        assert qoq.linear_workspace_bytes(M, N, K) > qoq.SCRATCH_BYTES
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, NUL, M, N, K, 128, NUL) == SCRATCH
