"""Benchmark of the W4A8 per-group GEMM path on one MI355X.

Default workload: the Llama-3-8B fused QKV projection (K=4096, N=6144, group 128)
at decode batches M = 1, 16 and 64.  One step = for each M, the per-token INT8
activation quantizer followed by the W4A8 GEMM with its fp16 epilogue, on inputs
already resident in HBM; the weights are packed once, offline, before timing (the
method quantizes and reorders weights offline).  Weight buffers are rotated over
copies totalling >= 1 GiB so that the 256 MB MALL and the L2 do not serve them.

Prints ONE JSON line (rank 0) with the throughput, the roofline fraction of the
dominant kernel (timed with HIP events on the stream the kernels run on), the CPU
oracle timed on the host cores and, as context, the KV4 decode attention of
Llama-3-8B at 64 sequences x 1024 cached tokens (kv4_attention; --no-kv4 skips it).

--sweep runs every layer shape / batch size of the workload registry and writes a
table to gpurun_out/sweep.json (not the headline line); with --format channel it
measures the per-channel weight format instead (gpurun_out/sweep_channel.json).
--kv4 measures the INT4 KV cache path instead (decode attention and the KV write on
the decode shapes of the registry, gpurun_out/kv4.json).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A8 GEMM TOPS and weight GB/s vs MI355X roofline, M=1..4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic_llama3_8b_qkv.md")
GEMM_SOURCES = [os.path.join(ROOT, "w4a8_mixed_precision_amd", "csrc", f)
                for f in ("qoq_gemm.hip", "qoq_device.h")]
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layer", default="llama3_8b_qkv")
    ap.add_argument("--ms", default="")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-launches", type=int, default=200)
    ap.add_argument("--kv4", action="store_true", help="measure the KV4 decode attention and KV write")
    ap.add_argument("--no-kv4", action="store_true", help="skip the KV4 attention figure of the headline line")
    ap.add_argument("--format", choices=("group", "channel"), default="group",
                    help="weight format: per-group g128 (default) or the per-channel variant")
    return ap.parse_args()


class Case:
    """Resident, rotated buffers for one (layer, M)."""

    def __init__(self, L, M, dev, packed_sets, per_channel=False):
        import torch
        from w4a8_mixed_precision_amd import workloads as wl
        self.L, self.M = L, M
        self.pc = per_channel
        self.sets = packed_sets
        x16 = wl.activations_fp16(L, M)
        self.x = torch.from_numpy(x16).to(dev)
        self.qx = torch.empty((M, L.K), dtype=torch.int8, device=dev)
        self.sx = torch.empty(M, dtype=torch.float16, device=dev)
        self.tx = torch.empty(M, dtype=torch.int32, device=dev)
        self.out = torch.empty((M, L.N), dtype=torch.float16, device=dev)
        # up to 64 tokens the step feeds the GEMM tiled codes (both weight formats);
        # the GEMM and quantizer timings below use the same kernels
        from w4a8_mixed_precision_amd import qoq
        self.tiled = M <= qoq.TILED_MAX_M
        self.qt = torch.empty(qoq.tiled_bytes(M, L.K), dtype=torch.int8, device=dev) if self.tiled else None
        self.ops = wl.algorithmic_ops(M, L.N, L.K)
        self.bytes = wl.algorithmic_bytes(M, L.N, L.K, per_channel)
        self.ws = None
        self.lws = None
        self.prod = None
        self.sws = None
        self.i = 0

    def workspace(self, q):
        """The split-K workspace this case's plan needs (grown outside graph capture:
        capture() runs fn once before capturing)."""
        need = q.gemm_workspace_bytes(self.M, self.L.N, self.L.K)
        if need and (self.ws is None or self.ws.numel() < need):
            import torch
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.x.device)
        return self.ws if need else None

    def linear_workspace(self, q):
        need = q.linear_workspace_bytes(self.M, self.L.N, self.L.K)
        if need and (self.lws is None or self.lws.numel() < need):
            import torch
            self.lws = torch.empty(need, dtype=torch.uint8, device=self.x.device)
        return self.lws if need else None

    def step(self, q):
        """The runtime path: quantize + GEMM in one library call (one fused kernel
        for few tokens, else the quantizer and the GEMM plan)."""
        if self.pc:
            # per-channel format: the quantizer (with code sums) and the GEMM
            self.quant_only(q)
            self.gemm_only(q)
            return
        p, m, s = self.sets[self.i % len(self.sets)]
        self.i += 1
        q.w4a8_linear(self.x, p, m, s, self.L.N, out=self.out, workspace=self.linear_workspace(q))

    def gemm_only(self, q):
        p, m, s = self.sets[self.i % len(self.sets)]
        self.i += 1
        if self.pc and self.tiled:
            q.w4a8_gemm_pc_tiled(self.qt, self.sx, self.tx, p, m, s, self.M, self.L.N, self.L.K, out=self.out)
        elif self.pc:
            q.w4a8_gemm_pc(self.qx, self.sx, self.tx, p, m, s, self.L.N, out=self.out,
                           workspace=self.workspace(q))
        elif self.tiled:
            q.w4a8_gemm_tiled(self.qt, self.sx, p, m, s, self.M, self.L.N, self.L.K, out=self.out)
        else:
            q.w4a8_gemm(self.qx, self.sx, p, m, s, self.L.N, out=self.out, workspace=self.workspace(q))

    def producer(self, q):
        """The kernel that would feed this GEMM with the quantization fused in: RMSNorm
        + quantization before QKV / gate+up (K = hidden size), SiLU(gate) * up +
        quantization before the down projection (K = intermediate size); same code
        layout as the linear step."""
        import torch
        if self.prod is None:
            if self.L.name.startswith(("llama3_8b_down", "qwen72b_down")):
                gu = torch.cat([self.x, self.x.flip(1)], dim=1).contiguous()
                self.prod = ("silu", gu)
            else:
                g = torch.ones(self.L.K, dtype=torch.float16, device=self.x.device)
                self.prod = ("norm", g)
        kind, t = self.prod
        out = (self.qt if self.tiled else self.qx, self.sx, None)
        if kind == "silu":
            need = q.silu_mul_quantize_workspace_bytes(self.M, self.L.K)
            if need and (self.sws is None or self.sws.numel() < need):
                self.sws = torch.empty(need, dtype=torch.uint8, device=self.x.device)
            q.silu_mul_quantize(t[:, :self.L.K], t[:, self.L.K:], tiled=self.tiled, out=out,
                                workspace=self.sws if need else None)
        else:
            q.rmsnorm_quantize(self.x, t, 1e-5, tiled=self.tiled, out=out)

    def producer_bytes(self):
        M, K = self.M, self.L.K
        if self.prod is not None and self.prod[0] == "silu":
            return 4 * M * K + M * K + 2 * M
        return 2 * M * K + 2 * K + M * K + 2 * M

    def quant_only(self, q):
        if self.pc and self.tiled:
            q.quantize_activations_rowsum_tiled(self.x, out=(self.qt, self.sx, self.tx))
        elif self.pc:
            q.quantize_activations_rowsum(self.x, out=(self.qx, self.sx, self.tx))
        elif self.tiled:
            q.quantize_activations_tiled(self.x, out=(self.qt, self.sx))
        else:
            q.quantize_activations(self.x, out=(self.qx, self.sx))


def packed_sets_for(L, dev, q, max_sets=128, per_channel=False):
    """Pack the layer's weights once, then clone the packed buffers until the
    rotation covers ROTATE_BYTES (at least 2 sets).  Per-channel format: the second
    buffer holds one zero byte per channel instead of the group metadata."""
    import torch
    from w4a8_mixed_precision_amd import workloads as wl
    w = torch.from_numpy(wl.weights_fp16(L)).to(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    p, m, s = q.quantize_pack_weights(w, group=0 if per_channel else 128)
    torch.cuda.synchronize()
    pack_s = time.perf_counter() - t0
    del w
    wbytes = p.numel() + m.numel() * m.element_size() + s.numel() * 2
    n = max(2, min(max_sets, -(-ROTATE_BYTES // wbytes)))
    sets = [(p, m, s)] + [(p.clone(), m.clone(), s.clone()) for _ in range(n - 1)]
    torch.cuda.synchronize()
    return sets, pack_s


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(plan: str, M: int, N: int, K: int):
    """HBM bytes per launch of this GEMM from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the factor the same counter shows for a
    copy kernel of known size), or None when the summary is absent, covers another
    shape, or was taken with different GEMM sources."""
    import re
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != gemm_source_hash():
        return None
    for k in rec.get("kernels", []):
        if k["plan"] == plan and (k["M"], k["N"], k["K"]) == (M, N, K):
            return k["fetch_bytes"] + k["write_bytes"]
    return None


def capture(fn, n, torch):
    """HIP graph of n back-to-back calls of fn.  The library launches on torch's
    current stream, which is the capture stream inside torch.cuda.graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps, torch):
    """Seconds per replay of graph g, from HIP events recorded on the current stream
    (graph replays run on it)."""
    st = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def time_launches(fn, n, torch, reps=3):
    """Average duration per launch of fn: n launches captured in one HIP graph
    (host launch overhead removed), replayed reps times, timed with HIP events."""
    g = capture(fn, n, torch)
    return time_graph(g, reps, torch) / n


def cpu_baseline(L, Ms, seconds):
    """The CPU oracle (unchanged) over the same step: activation quantization,
    dequantization of the stored codes, exact contraction, fp32 epilogue."""
    import numpy as np
    from oracle import qoq_oracle as o
    from w4a8_mixed_precision_amd import workloads as wl
    w16 = wl.weights_fp16(L)
    q0, s_w = o.quantize_weights_level0(w16)
    q_u4, z, s_u8 = o.quantize_weights_level1(q0)
    xs = {M: wl.activations_fp16(L, M) for M in Ms}
    ops = sum(wl.algorithmic_ops(M, L.N, L.K) for M in Ms)
    t0 = time.perf_counter()
    steps = 0
    while True:
        for M in Ms:
            qx, s_x = o.quantize_activations(xs[M])
            w_hat = o.dequantize_level1(q_u4, z, s_u8)
            acc = o.contract(qx, w_hat)
            o.epilogue(acc, s_x, s_w)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_step = el / steps
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    return {
        "value": ops / per_step / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
        "sample": f"{steps} full step(s) of {L.name} M={list(Ms)} (activation quant + dequant + exact "
                  f"fp64 contraction + epilogue), {el:.1f} s, host cpu_count={os.cpu_count()}",
        "s_per_step": per_step,
    }


def run_case_metrics(c, q, torch, launches):
    g = time_launches(lambda: c.gemm_only(q), launches, torch)
    a = time_launches(lambda: c.quant_only(q), launches, torch)
    s = time_launches(lambda: c.step(q), launches, torch)
    pr = None
    if not c.pc and c.L.K <= 32768:
        c.producer(q)
        pr = time_launches(lambda: c.producer(q), launches, torch)
    b = c.bytes
    return {
        "M": c.M, "K": c.L.K, "N": c.L.N,
        "plan": q.gemm_tiled_plan(c.M, c.L.N, c.L.K) + ":tiled" if c.tiled else q.gemm_plan(c.M, c.L.N, c.L.K),
        "linear_plan": (("quant_rowsum_tiled+gemm_pc_tiled" if c.tiled else "quant_rowsum+gemm_pc") if c.pc
                        else q.linear_plan(c.M, c.L.N, c.L.K)),
        "linear_us": s * 1e6, "format": "channel" if c.pc else "group",
        "gemm_us": g * 1e6, "quant_us": a * 1e6,
        "TOPS": c.ops / g / 1e12,
        "weight_GBps": b["weight"] / g / 1e9,
        "total_GBps": b["total"] / g / 1e9,
        "hbm_frac": b["total"] / g / 1e9 / HBM_PEAK_GBPS,
        "mfma_frac": c.ops / g / 1e12 / INT8_PEAK_TOPS,
        "roofline_frac": max(b["total"] / (HBM_PEAK_GBPS * 1e9), c.ops / (INT8_PEAK_TOPS * 1e12)) / g,
        "quant_GBps": (3 * c.M * c.L.K + 2 * c.M) / a / 1e9,
        "producer": None if pr is None else (c.prod[0] + "_quant"),
        "producer_us": None if pr is None else pr * 1e6,
        "producer_GBps": None if pr is None else c.producer_bytes() / pr / 1e9,
        "rotation_sets": len(c.sets),
    }


class KvCase:
    """Resident KV4 cache for one decode shape, copied into disjoint page ranges until
    the rotation covers ROTATE_BYTES (so the MALL and L2 do not serve the cache); each
    call attends over the next copy."""

    def __init__(self, S, dev, q):
        import numpy as np
        import torch
        from w4a8_mixed_precision_amd import workloads as wl
        self.S = S
        P = wl.KV_PAGE_TOKENS
        mp = -(-S.seq_len // P)
        pb = q.kv4_page_bytes(S.h_kv)
        set_pages = S.B * mp
        set_bytes = set_pages * pb
        self.nsets = max(2, -(-ROTATE_BYTES // set_bytes))
        self.pool = torch.empty(self.nsets * set_bytes, dtype=torch.uint8, device=dev)
        perm = np.random.default_rng(S.B * 7 + S.seq_len).permutation(set_pages).astype(np.int32).reshape(S.B, mp)
        self.tables = [torch.from_numpy(perm + i * set_pages).to(dev) for i in range(self.nsets)]
        base = self.pool[:set_bytes]
        self.zero = torch.zeros(S.B, dtype=torch.int32, device=dev)
        # the whole cache written in one call (the prefill write), kept for timing it
        self.k_all = torch.from_numpy(np.stack([wl.kv_fp16(S, b, S.seq_len, 0) for b in range(S.B)])).to(dev)
        self.v_all = torch.from_numpy(np.stack([wl.kv_fp16(S, b, S.seq_len, 1) for b in range(S.B)])).to(dev)
        q.kv4_write(self.k_all, self.v_all, self.zero, self.tables[0], base)
        for i in range(1, self.nsets):
            self.pool[i * set_bytes:(i + 1) * set_bytes].copy_(base)
        self.q = torch.from_numpy(wl.kv_queries_fp16(S)).to(dev)
        self.lens = torch.full((S.B,), S.seq_len, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        need = q.kv4_attention_workspace_bytes(S.B, S.h, S.h_kv, S.seq_len)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        # the decode-step write: one new token per sequence at position seq_len - 1
        self.k1 = torch.from_numpy(np.stack([wl.kv_fp16(S, b, 1, 0)[0] for b in range(S.B)])[:, None]).to(dev)
        self.v1 = torch.from_numpy(np.stack([wl.kv_fp16(S, b, 1, 1)[0] for b in range(S.B)])[:, None]).to(dev)
        self.pos = torch.full((S.B,), S.seq_len - 1, dtype=torch.int32, device=dev)
        self.bytes = wl.kv_attention_bytes(S.B, S.seq_len, S.h, S.h_kv)
        self.flops = wl.kv_attention_flops(S.B, S.seq_len, S.h)
        self.splits = need // (S.B * S.h * (wl.KV_HEAD_DIM + 2) * 4) if need else 1
        self.i = 0

    def attend(self, q):
        t = self.tables[self.i % self.nsets]
        self.i += 1
        q.kv4_decode_attention(self.q, self.pool, t, self.lens, self.S.h_kv, self.S.seq_len, out=self.out,
                               workspace=self.ws)

    def write(self, q):
        t = self.tables[self.i % self.nsets]
        self.i += 1
        q.kv4_write(self.k1, self.v1, self.pos, t, self.pool)

    def write_all(self, q):
        """The prefill write: every cached token of every sequence in one call."""
        t = self.tables[self.i % self.nsets]
        self.i += 1
        q.kv4_write(self.k_all, self.v_all, self.zero, t, self.pool)


def kv4_case_metrics(S, q, torch, dev, launches):
    from w4a8_mixed_precision_amd import workloads as wl
    c = KvCase(S, dev, q)
    for _ in range(3):
        c.attend(q)
    torch.cuda.synchronize()
    ta = time_launches(lambda: c.attend(q), launches, torch)
    tw = time_launches(lambda: c.write(q), launches, torch)
    tp = time_launches(lambda: c.write_all(q), max(2, launches // 20), torch)
    r = {"shape": S.name, "B": S.B, "seq_len": S.seq_len, "h": S.h, "h_kv": S.h_kv, "splits": c.splits,
         "attention_us": ta * 1e6, "bytes_per_launch": c.bytes, "GBps": c.bytes / ta / 1e9,
         "hbm_frac": c.bytes / ta / 1e9 / HBM_PEAK_GBPS, "TFLOPs": c.flops / ta / 1e12,
         "tokens_per_s": S.B * S.seq_len / ta,
         "write_us": tw * 1e6, "write_bytes": S.B * S.h_kv * (4 * wl.KV_HEAD_DIM + wl.KV_TOKEN_HEAD_BYTES),
         "prefill_write_us": tp * 1e6,
         "prefill_write_GBps": S.B * S.seq_len * S.h_kv * (4 * wl.KV_HEAD_DIM + wl.KV_TOKEN_HEAD_BYTES) / tp / 1e9,
         "rotation_sets": c.nsets}
    del c
    torch.cuda.empty_cache()
    return r


def kv4_bench(q, torch, dev, launches):
    from w4a8_mixed_precision_amd import workloads as wl
    rows = []
    for S in wl.KV_SHAPES:
        r = kv4_case_metrics(S, q, torch, dev, launches)
        rows.append(r)
        print(json.dumps(r), flush=True)
    os.makedirs(os.path.join(ROOT, "gpurun_out"), exist_ok=True)
    with open(os.path.join(ROOT, "gpurun_out", "kv4.json"), "w") as f:
        json.dump(rows, f, indent=1)
    return rows


def copy_ceiling(q, torch, dev, nbytes=1 << 30, reps=10):
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    q.stream_copy(src, dst)
    t = time_launches(lambda: q.stream_copy(src, dst), reps, torch, reps=1)
    del src, dst
    return {"bytes_per_launch": 2 * nbytes, "us": t * 1e6, "GBps": 2 * nbytes / t / 1e9}


class ReadCeiling:
    """The library's streaming-read kernel over the same byte count as a case, on
    slices of one 1 GiB buffer taken in rotation (so the MALL and L2 do not serve
    them): the practical HBM read ceiling at that size."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(ROTATE_BYTES + (64 << 20), dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(16, dtype=torch.uint8, device=dev)
        self.i = 0

    def gbps(self, q, torch, nbytes, launches):
        nbytes = (nbytes + 4095) // 4096 * 4096
        nsl = max(2, ROTATE_BYTES // nbytes)

        def one():
            off = (self.i % nsl) * nbytes
            self.i += 1
            q.stream_read(self.buf[off:off + nbytes], self.sink)
        one()
        torch.cuda.synchronize()
        return nbytes / time_launches(one, launches, torch) / 1e9


def mfma_ceiling(q, torch, dev, iters=2000, blocks=2048):
    """INT8 ops/s of the library's register-only MFMA loop (practical matrix-core
    ceiling): blocks x 4 waves x iters x 4 MFMAs x 65536 ops."""
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    q.mfma_peak(iters, blocks, sink)
    t = time_launches(lambda: q.mfma_peak(iters, blocks, sink), 3, torch, reps=3)
    return blocks * 4 * iters * 4 * 65536 / t / 1e12


def oracle_case(L, M, per_channel=False, cols=256):
    """Seconds of the CPU oracle (unchanged) for one case, by stage: activation
    quantization over the whole [M, K]; weight quantization, dequantization,
    contraction (fp64, exact) and epilogue on `cols` output columns, scaled by N / cols
    (every stage is linear in N)."""
    import numpy as np
    from oracle import qoq_oracle as o
    from w4a8_mixed_precision_amd import workloads as wl
    ns = min(cols, L.N)
    w16 = wl.weights_fp16(L, N=ns)            # the first ns rows of the layer's W
    x16 = wl.activations_fp16(L, M)
    t = {}
    t0 = time.perf_counter()
    qx, s_x = o.quantize_activations(x16)
    t["act_quant_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    q0, s_w = o.quantize_weights_level0(w16)
    q_u4, z, s_u8 = o.quantize_weights_level1(q0)
    t["pack_s"] = (time.perf_counter() - t0) * L.N / ns
    t0 = time.perf_counter()
    w_hat = o.dequantize_level1(q_u4, z, s_u8)
    acc = o.contract(qx, w_hat)
    t["contract_s"] = (time.perf_counter() - t0) * L.N / ns
    t0 = time.perf_counter()
    o.epilogue(acc, s_x, s_w)
    t["epilogue_s"] = (time.perf_counter() - t0) * L.N / ns
    t["step_s"] = t["act_quant_s"] + t["contract_s"] + t["epilogue_s"]
    t["sample"] = f"{ns} of {L.N} columns, scaled"
    return {k: (round(v, 6) if isinstance(v, float) else v) for k, v in t.items()}


def sweep(q, torch, dev, launches, per_channel=False, with_oracle=True):
    from w4a8_mixed_precision_amd import workloads as wl
    rows = []
    ceil = ReadCeiling(torch, dev)
    mfma_tops = mfma_ceiling(q, torch, dev)
    print(json.dumps({"mfma_ceiling_TOPS": mfma_tops}), flush=True)
    for L in wl.LAYERS:
        sets, pack_s = packed_sets_for(L, dev, q, per_channel=per_channel)
        for M in L.Ms:
            c = Case(L, M, dev, sets, per_channel)
            for _ in range(3):
                c.step(q)
            torch.cuda.synchronize()
            r = run_case_metrics(c, q, torch, launches)
            r.update({"layer": L.name, "pack_ms": pack_s * 1e3})
            rc = ceil.gbps(q, torch, c.bytes["total"], launches)
            r.update({"read_ceiling_GBps": rc, "hbm_frac_of_ceiling": r["total_GBps"] / rc,
                      "mfma_ceiling_TOPS": mfma_tops, "mfma_frac_of_ceiling": r["TOPS"] / mfma_tops})
            if with_oracle:
                r["oracle"] = oracle_case(L, M, per_channel)
            rows.append(r)
            print(json.dumps(r), flush=True)
            del c
        del sets
        torch.cuda.empty_cache()
    os.makedirs(os.path.join(ROOT, "gpurun_out"), exist_ok=True)
    name = "sweep_channel.json" if per_channel else "sweep.json"
    with open(os.path.join(ROOT, "gpurun_out", name), "w") as f:
        json.dump(rows, f, indent=1)
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path's sharding is "
              f"described in DESIGN.md and is not measured here", file=sys.stderr)
        sys.exit(2)
    import torch
    from w4a8_mixed_precision_amd import qoq
    from w4a8_mixed_precision_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    qoq.lib()

    if args.kv4:
        kv4_bench(qoq, torch, dev, args.kernel_launches)
        return
    if args.sweep:
        sweep(qoq, torch, dev, args.kernel_launches, args.format == "channel", not args.no_cpu_baseline)
        return
    if args.format != "group":
        print("the headline line measures the per-group format; use --format channel with --sweep",
              file=sys.stderr)
        sys.exit(2)

    L = wl.find(args.layer)
    Ms = tuple(int(m) for m in args.ms.split(",")) if args.ms else L.Ms
    sets, pack_s = packed_sets_for(L, dev, qoq)
    cases = [Case(L, M, dev, sets) for M in Ms]

    def step():
        for c in cases:
            c.step(qoq)

    # warmup steps run eagerly; the K timed steps are one HIP graph of exactly K steps
    # (each step rotates to the next packed-weight copy), replayed once between a
    # synchronize on both sides and timed with HIP events on the replay stream.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    g_steps = capture(step, args.steps, torch)
    g_steps.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_host0 = time.perf_counter()
    e0.record(st)
    g_steps.replay()
    e1.record(st)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    step_s = e0.elapsed_time(e1) * 1e-3 / args.steps

    per_case = [run_case_metrics(c, qoq, torch, args.kernel_launches) for c in cases]
    ops = sum(c.ops for c in cases)
    wbytes = sum(c.bytes["weight"] for c in cases)
    # dominant kernel: the GEMM launch with the largest time in the step; its bound
    # is whichever of HBM bytes and INT8 MFMA ops takes longer at the published peaks
    dom = max(per_case, key=lambda r: r["gemm_us"])
    dom_case = cases[per_case.index(dom)]
    t_launch = dom["gemm_us"] * 1e-6
    if dom_case.ops / (INT8_PEAK_TOPS * 1e12) > dom_case.bytes["total"] / (HBM_PEAK_GBPS * 1e9):
        bound, unit, peak, achieved = "mfma", "TOPS", INT8_PEAK_TOPS, dom_case.ops / t_launch / 1e12
    else:
        bound, unit, peak, achieved = "hbm", "GB/s", HBM_PEAK_GBPS, dom_case.bytes["total"] / t_launch / 1e9
    result = {
        "metric": METRIC,
        "value": ops / step_s / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{L.name}: W4A8 g128 GEMM K={L.K} N={L.N}, M in {list(Ms)}, "
                               f"per-token INT8 activation quant + GEMM + fp16 epilogue per M "
                               f"(one qoq_w4a8_linear call per M)",
                   "K": L.K, "N": L.N, "M": list(Ms), "group": 128},
        "weight_GBps_step": wbytes / step_s / 1e9,
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak,
                     "traffic": measured_traffic(dom["plan"], dom["M"], L.N, L.K),
                     "kernel": dom["plan"], "M": dom["M"],
                     "bytes_per_launch": dom_case.bytes["total"], "launch_us": dom["gemm_us"]},
        "cases": per_case,
        "offline_pack_ms": pack_s * 1e3,
        "copy_ceiling": copy_ceiling(qoq, torch, dev),
        "kv4_attention": None if args.no_kv4 else kv4_case_metrics(wl.find_kv("llama3_8b_b64_l1024"), qoq, torch, dev,
                                                                    args.kernel_launches),
        "host_wall_s": t_host,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(L, Ms, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
