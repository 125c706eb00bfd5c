"""Benchmark of the W4A8 per-group GEMM path on one MI355X.

Default workload: the metric's range M = 1 .. 4096 in one step, group 128:
  Llama-3-8B fused QKV (K=4096, N=6144) at decode batches M = 1, 16, 64;
  Qwen-72B-class gate+up (K=8192, N=59136) and down (K=29568, N=8192) at M = 1
  (the largest weight streams: the bandwidth-bound regime);
  Llama-3-8B gate+up (K=4096, N=28672) and down (K=14336, N=4096) at M = 4096
  prompt tokens (the INT8 matrix-core-bound regime).
One step = for each case, the per-token INT8 activation quantization followed by
the W4A8 GEMM with its fp16 epilogue (one qoq_w4a8_linear call), on inputs already
resident in HBM; the weights are packed once, offline, before timing (the method
quantizes and reorders weights offline).  Weight buffers are rotated over copies
totalling >= 1 GiB per layer so that the 256 MB MALL and the L2 do not serve them.

Prints ONE JSON line (rank 0) with the throughput, the roofline fraction of the
dominant kernel (timed with HIP events on the stream the kernels run on), one
roofline block per regime (HBM: Qwen-72B gate+up at M = 1; MFMA: Llama-3-8B gate+up
at M = 4096), the CPU oracle timed on the host cores on a column sample of the same
step and, as context, the KV4 decode attention of Llama-3-8B at 64 sequences x 1024
cached tokens (kv4_attention; --no-kv4 skips it).  --layer / --ms time one layer
instead of the default step.

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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic_step.md")
GEMM_SOURCES = [os.path.join(ROOT, "w4a8_mixed_precision_amd", "csrc", f)
                for f in ("qoq_gemm.hip", "qoq_device.h")]
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
ROTATE_BYTES = 1 << 30

# the default step: (layer, batch sizes); the regime blocks of the line
STEP = (("llama3_8b_qkv", (1, 16, 64)), ("qwen72b_gate_up", (1,)), ("qwen72b_down", (1,)),
        ("llama3_8b_gate_up_prefill", (4096,)), ("llama3_8b_down_prefill", (4096,)))
REGIMES = {"hbm": ("qwen72b_gate_up", 1), "mfma": ("llama3_8b_gate_up_prefill", 4096)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layer", default="", help="time this layer alone (default: the mixed step)")
    ap.add_argument("--ms", default="")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-launches", type=int, default=200)
    ap.add_argument("--kv4", action="store_true", help="measure the KV4 decode attention and KV write")
    ap.add_argument("--no-kv4", action="store_true", help="skip the KV4 attention figure of the headline line")
    ap.add_argument("--profile-plan", action="store_true",
                    help="time every configuration (and split-K factor) on the workloads' layer shapes over a grid "
                         "of M and write the fastest per point as the dispatch table "
                         "(gpurun_out/qoq_plan_table.inc, gpurun_out/plan_profile.json)")
    ap.add_argument("--profile-layers", default="",
                    help="with --profile-plan: only these layers' (N, K) (comma-separated names); the results go "
                         "to gpurun_out/plan_profile_<names>.json for --profile-merge")
    ap.add_argument("--profile-merge", nargs="*", default=None,
                    help="merge profile files into the dispatch table and the committed profile (no GPU)")
    ap.add_argument("--check-plan", action="store_true",
                    help="time the planner's choice against the best configurations of the committed profile")
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


def cpu_baseline_step(plan, seconds, cols=256):
    """The CPU oracle (unchanged) over a column sample of the step: per case the
    activation quantization over the whole [M, K], then dequantization of the stored
    codes, exact fp64 contraction and fp32 epilogue on the first `cols` output
    columns, scaled by N / cols (those stages are linear in N); whole sampled steps
    are repeated until `seconds` have passed."""
    import numpy as np
    from oracle import qoq_oracle as o
    from w4a8_mixed_precision_amd import workloads as wl
    prep = []
    for name, Ms in plan:
        L = wl.find(name)
        ns = min(cols, L.N)
        q0, s_w = o.quantize_weights_level0(wl.weights_fp16(L, N=ns))
        q_u4, z, s_u8 = o.quantize_weights_level1(q0)
        for M in Ms:
            prep.append((L, M, ns, wl.activations_fp16(L, M), q_u4, z, s_u8, s_w))
    ops = sum(wl.algorithmic_ops(M, L.N, L.K) for (L, M, *_rest) in prep)
    t_begin = time.perf_counter()
    per_step = []
    while True:
        t_step = 0.0
        for (L, M, ns, x16, q_u4, z, s_u8, s_w) in prep:
            t0 = time.perf_counter()
            qx, s_x = o.quantize_activations(x16)
            t1 = time.perf_counter()
            acc = o.contract(qx, o.dequantize_level1(q_u4, z, s_u8))
            o.epilogue(acc, s_x, s_w)
            t2 = time.perf_counter()
            t_step += (t1 - t0) + (t2 - t1) * L.N / ns
        per_step.append(t_step)
        el = time.perf_counter() - t_begin
        if el >= seconds:
            break
    s_step = float(np.median(per_step))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    return {
        "value": ops / s_step / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
        "sample": f"{len(per_step)} column-sampled step(s) of the same cases ({cols} output columns per layer, "
                  f"dequant + exact fp64 contraction + epilogue scaled by N/{cols}; activation quant over the "
                  f"whole [M, K]), median {s_step:.2f} s per full step, {el:.1f} s of CPU work, "
                  f"host cpu_count={os.cpu_count()}",
        "s_per_step": s_step,
    }


def roofline_of(r, c):
    """Roofline object of one case's GEMM launch: the bound with the longer time at
    the published peaks, achieved = algorithmic bytes (or ops) / measured launch."""
    t = r["gemm_us"] * 1e-6
    if c.ops / (INT8_PEAK_TOPS * 1e12) > c.bytes["total"] / (HBM_PEAK_GBPS * 1e9):
        bound, unit, peak, achieved = "mfma", "TOPS", INT8_PEAK_TOPS, c.ops / t / 1e12
    else:
        bound, unit, peak, achieved = "hbm", "GB/s", HBM_PEAK_GBPS, c.bytes["total"] / t / 1e9
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": measured_traffic(r["plan"], r["M"], r["N"], r["K"]),
            "kernel": r["plan"], "layer": c.L.name, "M": r["M"], "N": r["N"], "K": r["K"],
            "bytes_per_launch": c.bytes["total"], "ops_per_launch": c.ops, "launch_us": r["gemm_us"]}


def run_case_metrics(c, q, torch, launches):
    # the GEMM-only timing reads the codes the quantizer writes: write them from the
    # case's activations first (codes never written are zeros or stale memory, and
    # zero operands draw less power, which lets the matrix cores clock higher)
    c.quant_only(q)
    torch.cuda.synchronize()
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


def mfma_ceiling_data(q, torch, c, iters=1000, blocks=2048):
    """INT8 ops/s of the same register-only MFMA loop fed with this case's own
    operands (its activation codes and its dequantized weights): the matrix-core
    ceiling for the data the GEMM multiplies (the clock under MFMA load depends on
    the operands' toggling).  blocks x 4 waves x iters x 8 MFMAs x 65536 ops."""
    p, m, _s = c.sets[0]
    w = q.dequantize_packed(p, m, c.L.N, c.L.K)
    c.quant_only(q)
    sink = torch.zeros(16, dtype=torch.int32, device=w.device)
    q.mfma_peak_operands(c.qx, w, iters, blocks, sink)
    t = time_launches(lambda: q.mfma_peak_operands(c.qx, w, iters, blocks, sink), 3, torch, reps=3)
    del w
    torch.cuda.empty_cache()
    return blocks * 4 * iters * 8 * 65536 / t / 1e12


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


# M grids of the profiling sweep: tiled activation codes (the linear entry point up
# to 64 tokens) and row-major codes (the GEMM entry point, and the linear one beyond)
PROFILE_M_TILED = (1, 2, 4, 8, 12, 16, 24, 32, 40, 48, 56, 64)
PROFILE_M_ROW = (1, 8, 16, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192)
PROFILE_SPLITS = (1, 2, 3, 4, 6, 8, 12, 16)
PROFILE_M_LINEAR = (1, 2, 4, 8)
PROFILE_FILE = os.path.join(ROOT, "profiles", "plan_profile_mi355x.json")
PLAN_TABLE = os.path.join(ROOT, "w4a8_mixed_precision_amd", "csrc", "qoq_plan_table.inc")
LINEAR_TABLE = os.path.join(ROOT, "w4a8_mixed_precision_amd", "csrc", "qoq_linear_table.inc")


def warm_up(fn, torch, seconds=0.03):
    """Run fn back to back for about `seconds` of GPU time before timing: after the
    host has left the GPU idle (building a case's inputs), the clock takes a few
    milliseconds to come back up, and the first configuration timed would pay for it."""
    t = time_launches(fn, 2, torch, reps=1)
    g = capture(fn, int(max(2, min(256, seconds / max(t, 1e-7)))), torch)
    g.replay()
    torch.cuda.synchronize()
    del g


def time_adaptive(fn, torch, target_s=2e-3):
    """Seconds per launch of fn: one short graph to estimate, then a graph of about
    target_s, best of two replays."""
    t0 = time_launches(fn, 2, torch, reps=1)
    n = int(max(2, min(64, target_s / max(t0, 1e-7))))
    g = capture(fn, n, torch)
    best = min(time_graph(g, 1, torch) for _ in range(2)) / n
    del g
    return best


def profile_candidates(q, M, N, tiled):
    """(config, splits) pairs worth timing at M: few-token kernels (the only ones
    on tiled codes) up to 128 tokens, tile kernels from 16 tokens with every split
    factor whose INT32 partial sums stay within 512 MiB."""
    out = []
    for name in q.gemm_configs():
        few = name.startswith("skinny")
        if tiled and not few:
            continue
        if few and M > 128:
            continue
        if few:
            out.append((name, 0))
        elif M >= 16:
            out += [(name, sp) for sp in PROFILE_SPLITS if sp == 1 or sp * M * N * 4 <= 512 << 20]
    return out


def profile_plan(q, torch, dev, only=""):
    """The measured dispatch table: for every (N, K) of the workloads and every M of
    the grids, each candidate configuration timed on real codes with the weights
    rotated; the fastest per point becomes a table row."""
    from w4a8_mixed_precision_amd import workloads as wl
    shapes = []
    for L in wl.LAYERS:
        if only and L.name not in only.split(","):
            continue
        if (L.N, L.K) not in [(x.N, x.K) for x in shapes]:
            shapes.append(L)
    points = []
    for L in shapes:
        sets, _ = packed_sets_for(L, dev, q, max_sets=64)
        for tiled, grid in ((1, PROFILE_M_TILED), (0, PROFILE_M_ROW)):
            for M in grid:
                c = Case(L, M, dev, sets)
                c.tiled = bool(tiled)
                c.quant_only(q)
                torch.cuda.synchronize()
                warm_up(lambda: c.gemm_only(q), torch)
                res = []
                for cfg, sp in profile_candidates(q, M, L.N, tiled):
                    with q.plan_override(config=cfg, splits=sp):
                        c.workspace(q)
                        try:
                            t = time_adaptive(lambda: c.gemm_only(q), torch)
                        except Exception as ex:        # a configuration the shape cannot take
                            print(json.dumps({"skip": cfg, "splits": sp, "err": str(ex)[:80]}), file=sys.stderr)
                            continue
                    res.append((t, cfg, sp))
                res.sort()
                t_best, cfg, sp = res[0]
                pt = {"N": L.N, "K": L.K, "tiled": tiled, "M": M, "best": cfg, "splits": sp,
                      "best_us": t_best * 1e6,
                      "top": [{"config": c_, "splits": s_, "us": round(t_ * 1e6, 3)} for t_, c_, s_ in res[:8]]}
                points.append(pt)
                print(json.dumps({k: pt[k] for k in ("N", "K", "tiled", "M", "best", "splits", "best_us")}),
                      flush=True)
                del c
        del sets
        torch.cuda.empty_cache()
    linear_points = profile_linear(q, torch, dev, shapes)
    os.makedirs(os.path.join(ROOT, "gpurun_out"), exist_ok=True)
    tag = only.replace(",", "+") if only else "all"
    path = os.path.join(ROOT, "gpurun_out", f"plan_profile_{tag}.json")
    with open(path, "w") as f:
        json.dump({"points": points, "linear_points": linear_points, "M_tiled": PROFILE_M_TILED,
                   "M_row": PROFILE_M_ROW, "M_linear": PROFILE_M_LINEAR, "splits": PROFILE_SPLITS}, f, indent=1)
    profile_merge([path])


def profile_linear(q, torch, dev, shapes):
    """The linear entry point at a few tokens: the pair (quantizer + the GEMM
    plan, "unfused") and every fused configuration that takes the shape, timed as
    the whole call on the same rotated weights."""
    points = []
    for L in shapes:
        sets, _ = packed_sets_for(L, dev, q, max_sets=64)
        for M in PROFILE_M_LINEAR:
            c = Case(L, M, dev, sets)
            torch.cuda.synchronize()
            warm_up(lambda: c.step(q), torch)
            res = []
            for cfg in ["unfused"] + q.linear_configs():
                with q.plan_override(linear=cfg):
                    if cfg != "unfused" and q.linear_plan(M, L.N, L.K) != cfg:
                        continue                      # the fused kernel does not take this shape
                    res.append((time_adaptive(lambda: c.step(q), torch), cfg))
            res.sort()
            pt = {"N": L.N, "K": L.K, "M": M, "best": res[0][1], "best_us": res[0][0] * 1e6,
                  "top": [{"config": c_, "us": round(t_ * 1e6, 3)} for t_, c_ in res[:8]]}
            points.append(pt)
            print(json.dumps({k: pt[k] for k in ("N", "K", "M", "best", "best_us")}), flush=True)
            del c
        del sets
        torch.cuda.empty_cache()
    return points


COVER_TOL = 0.03       # run-to-run spread of one configuration is about this


def cover_configs(points, tol=COVER_TOL):
    """The fewest configurations such that at every profiled point one of them is
    within tol of the fastest (greedy set cover: repeatedly keep the configuration
    that is near-best at the most points not yet covered).  Configurations that win
    only by noise drop out of the table."""
    near = []
    for p in points:
        best = p["top"][0]["us"]
        near.append({t["config"] for t in p["top"] if t["us"] <= best * (1 + tol)})
    keep, todo = set(), set(range(len(points)))
    while todo:
        count = {}
        for i in todo:
            for c in near[i]:
                count[c] = count.get(c, 0) + 1
        c = max(sorted(count), key=lambda k: count[k])
        keep.add(c)
        todo = {i for i in todo if c not in near[i]}
    return keep


def profile_merge(paths):
    """Profile files -> the committed profile (profiles/) and the dispatch table
    (the fastest configuration per point)."""
    points = []
    for pth in paths:
        with open(pth) as f:
            points += json.load(f)["points"]
    points.sort(key=lambda p: (p["N"], p["K"], p["tiled"], p["M"]))
    keep = cover_configs(points)
    lpoints = []
    for pth in paths:
        with open(pth) as f:
            lpoints += json.load(f).get("linear_points", [])
    lpoints.sort(key=lambda p: (p["N"], p["K"], p["M"]))
    lkeep = cover_configs(lpoints)
    lrows = []
    for p in lpoints:
        alt = [t for t in p["top"] if t["config"] in lkeep]
        pick = min(alt, key=lambda t: t["us"])
        p["table"] = {"config": pick["config"], "us": pick["us"]}
        lrows.append((p["N"], p["K"], p["M"], pick["config"]))
    rows = []
    for p in points:
        alt = [t for t in p["top"] if t["config"] in keep]
        pick = min(alt, key=lambda t: t["us"])
        p["table"] = {"config": pick["config"], "splits": pick["splits"], "us": pick["us"]}
        rows.append((p["N"], p["K"], p["tiled"], p["M"], pick["config"], max(pick["splits"], 1)))
    compact = [{"N": p["N"], "K": p["K"], "tiled": p["tiled"], "M": p["M"], "best": p["best"],
                "splits": p["splits"], "best_us": round(p["best_us"], 3), "table": p["table"],
                "top": p["top"][:4]} for p in points]
    lcompact = [{"N": p["N"], "K": p["K"], "M": p["M"], "best": p["best"], "best_us": round(p["best_us"], 3),
                 "table": p["table"], "top": p["top"][:4]} for p in lpoints]
    with open(PROFILE_FILE, "w") as f:
        json.dump({"command": "python -m w4a8_mixed_precision_amd.build --all-configs; python bench.py "
                              "--profile-plan [--profile-layers ...]; python bench.py --profile-merge <files>",
                   "kept_configs": sorted(keep), "kept_linear_configs": sorted(lkeep), "cover_tolerance": COVER_TOL,
                   "M_tiled": PROFILE_M_TILED, "M_row": PROFILE_M_ROW, "M_linear": PROFILE_M_LINEAR,
                   "splits": PROFILE_SPLITS, "points": compact, "linear_points": lcompact}, f, separators=(",", ":"))
    with open(LINEAR_TABLE, "w") as f:
        f.write("// The measured linear table: QOQ_LINEAR_ROW(N, K, M, configuration), the fastest of\n"
                "// the fused quantize + GEMM configurations and the quantizer + GEMM pair (\"unfused\")\n"
                "// per point of the profiling sweep on MI355X (python bench.py --profile-plan).\n")
        for r in lrows:
            f.write('QOQ_LINEAR_ROW(%d, %d, %d, "%s")\n' % r)
    with open(PLAN_TABLE, "w") as f:
        f.write("// The measured dispatch table: QOQ_PLAN_ROW(N, K, tiled codes, M, configuration,\n"
                "// split-K factor), the fastest configuration per point of the profiling sweep on\n"
                "// MI355X (python bench.py --profile-plan; real activation codes, weights rotated over\n"
                "// >= 1 GiB, graph-timed).  Rows of one (N, K, layout) are sorted by M.\n")
        for r in rows:
            f.write('QOQ_PLAN_ROW(%d, %d, %d, %d, "%s", %d)\n' % r)
    print(f"wrote {PLAN_TABLE} ({len(rows)} rows), {LINEAR_TABLE} ({len(lrows)} rows) and {PROFILE_FILE}",
          flush=True)


def check_plan(q, torch, dev, tol=0.05):
    """The planner's choice against the best configurations of the committed
    profile, timed side by side at every profiled point: the ratio of the
    planner's time to the best of them."""
    from w4a8_mixed_precision_amd import workloads as wl
    with open(PROFILE_FILE) as f:
        prof = json.load(f)
    by_shape = {}
    for pt in prof["points"]:
        by_shape.setdefault((pt["N"], pt["K"]), []).append(pt)
    out = []
    for (N, K), pts in by_shape.items():
        L = next(x for x in wl.LAYERS if (x.N, x.K) == (N, K))
        sets, _ = packed_sets_for(L, dev, q, max_sets=64)
        for pt in pts:
            M, tiled = pt["M"], pt["tiled"]
            c = Case(L, M, dev, sets)
            c.tiled = bool(tiled)
            c.quant_only(q)
            torch.cuda.synchronize()
            plan = q.gemm_tiled_plan(M, N, K) if tiled else q.gemm_plan(M, N, K)
            plan_sp = 0 if plan.startswith("skinny") else q.gemm_plan_splits(M, N, K)
            c.workspace(q)
            warm_up(lambda: c.gemm_only(q), torch)
            # the fastest configurations of the profile that the library still holds
            # (the others were dropped from the build) other than the plan itself,
            # timed beside it in two alternating rounds, the better of each kept
            kept = set(q.gemm_configs())
            alts = [(a["config"], a["splits"]) for a in pt["top"] if a["config"] in kept]
            alts = [a for a in alts if not (a[0] == plan.split(":")[0] and max(a[1], 1) == max(plan_sp, 1))][:3]
            t_plan, t_alt = float("inf"), [float("inf")] * len(alts)
            for _ in range(2):
                c.workspace(q)
                t_plan = min(t_plan, time_adaptive(lambda: c.gemm_only(q), torch))
                for i, (cfg, sp) in enumerate(alts):
                    with q.plan_override(config=cfg, splits=sp):
                        c.workspace(q)
                        t_alt[i] = min(t_alt[i], time_adaptive(lambda: c.gemm_only(q), torch))
            t_alt = [t_plan] + t_alt
            r = {"N": N, "K": K, "tiled": tiled, "M": M, "plan": plan, "plan_us": t_plan * 1e6,
                 "best_now_us": min(t_alt) * 1e6, "ratio": t_plan / min(t_alt),
                 "profile_best": pt["best"], "profile_best_us": pt["best_us"],
                 "ratio_to_profile_best": t_plan * 1e6 / pt["best_us"]}
            out.append(r)
            print(json.dumps(r), flush=True)
            del c
        del sets
        torch.cuda.empty_cache()
    # the linear entry point at a few tokens: the planner's choice (fused or the
    # pair) against the profile's fastest alternatives that the library holds
    lout = []
    lby = {}
    for pt in prof.get("linear_points", []):
        lby.setdefault((pt["N"], pt["K"]), []).append(pt)
    for (N, K), pts in lby.items():
        L = next(x for x in wl.LAYERS if (x.N, x.K) == (N, K))
        sets, _ = packed_sets_for(L, dev, q, max_sets=64)
        for pt in pts:
            M = pt["M"]
            c = Case(L, M, dev, sets)
            torch.cuda.synchronize()
            plan = q.linear_plan(M, N, K)
            warm_up(lambda: c.step(q), torch)
            kept = set(q.linear_configs()) | {"unfused"}
            fused_plan = plan in kept
            alts = [a["config"] for a in pt["top"] if a["config"] in kept]
            alts = [a for a in alts if a != (plan if fused_plan else "unfused")][:3]
            t_plan, t_alt = float("inf"), [float("inf")] * len(alts)
            for _ in range(2):
                t_plan = min(t_plan, time_adaptive(lambda: c.step(q), torch))
                for i, cfg in enumerate(alts):
                    with q.plan_override(linear=cfg):
                        t_alt[i] = min(t_alt[i], time_adaptive(lambda: c.step(q), torch))
            t_alt = [t_plan] + t_alt
            r = {"N": N, "K": K, "M": M, "plan": plan, "plan_us": t_plan * 1e6, "best_now_us": min(t_alt) * 1e6,
                 "ratio": t_plan / min(t_alt), "profile_best": pt["best"], "profile_best_us": pt["best_us"]}
            lout.append(r)
            print(json.dumps(r), flush=True)
            del c
        del sets
        torch.cuda.empty_cache()
    worst = max(r["ratio"] for r in out)
    summary = {"points": len(out), "worst_ratio": worst, "within_tol": sum(r["ratio"] <= 1 + tol for r in out),
               "tol": tol, "median_ratio_to_profile_best": sorted(r["ratio_to_profile_best"] for r in out)[len(out) // 2],
               "worst_ratio_to_profile_best": max(r["ratio_to_profile_best"] for r in out),
               "linear_points": len(lout), "linear_within_tol": sum(r["ratio"] <= 1 + tol for r in lout),
               "linear_worst_ratio": max((r["ratio"] for r in lout), default=None)}
    with open(os.path.join(ROOT, "gpurun_out", "plan_check.json"), "w") as f:
        json.dump({"summary": summary, "points": out, "linear_points": lout}, f, indent=1)
    with open(os.path.join(ROOT, "gpurun_out", "plan_check.md"), "w") as f:
        f.write("# Dispatch table check (MI355X)\n\nCommand: `python bench.py --check-plan` (the planner's choice "
                "timed beside the fastest other configurations of the committed profile that the library holds, at "
                "every profiled point, in two alternating rounds, the better time of each kept; real codes, weights "
                "rotated, graph-timed after a warm-up).\n\n")
        f.write(f"Points: {summary['points']}; within {tol:.0%} of the best timed beside it: "
                f"{summary['within_tol']}; worst ratio {summary['worst_ratio']:.3f}; median ratio to the "
                f"profile's best (all 41 candidates, other run) {summary['median_ratio_to_profile_best']:.3f}, "
                f"worst {summary['worst_ratio_to_profile_best']:.3f}.\n\n")
        f.write("| N | K | codes | M | plan | plan us | best now us | ratio | profile best | profile us |\n"
                "|---|---|---|---|---|---|---|---|---|---|\n")
        for r in out:
            f.write(f"| {r['N']} | {r['K']} | {'tiled' if r['tiled'] else 'row'} | {r['M']} | {r['plan']} | "
                    f"{r['plan_us']:.2f} | {r['best_now_us']:.2f} | {r['ratio']:.3f} | {r['profile_best']} | "
                    f"{r['profile_best_us']:.2f} |\n")
        if lout:
            f.write(f"\nLinear entry point (quantize + GEMM in one call) at a few tokens: {summary['linear_points']} "
                    f"points, within {tol:.0%}: {summary['linear_within_tol']}, worst ratio "
                    f"{summary['linear_worst_ratio']:.3f}.\n\n")
            f.write("| N | K | M | plan | plan us | best now us | ratio | profile best | profile us |\n"
                    "|---|---|---|---|---|---|---|---|---|\n")
            for r in lout:
                f.write(f"| {r['N']} | {r['K']} | {r['M']} | {r['plan']} | {r['plan_us']:.2f} | "
                        f"{r['best_now_us']:.2f} | {r['ratio']:.3f} | {r['profile_best']} | "
                        f"{r['profile_best_us']:.2f} |\n")
    print(json.dumps(summary), flush=True)


def main():
    args = parse()
    if args.profile_merge is not None:
        profile_merge(args.profile_merge)
        return
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
    if args.profile_plan:
        profile_plan(qoq, torch, dev, args.profile_layers)
        return
    if args.check_plan:
        check_plan(qoq, torch, dev)
        return
    if args.sweep:
        sweep(qoq, torch, dev, args.kernel_launches, args.format == "channel", not args.no_cpu_baseline)
        return
    if args.format != "group":
        print("the headline line measures the per-group format; use --format channel with --sweep",
              file=sys.stderr)
        sys.exit(2)

    plan = ((args.layer, tuple(int(m) for m in args.ms.split(",")) if args.ms else wl.find(args.layer).Ms),) \
        if args.layer else STEP
    cases, pack_ms = [], {}
    for name, Ms in plan:
        L = wl.find(name)
        sets, pack_s = packed_sets_for(L, dev, qoq)
        pack_ms[name] = pack_s * 1e3
        cases += [Case(L, M, dev, sets) for M in Ms]

    def step():
        for c in cases:
            c.step(qoq)

    # warmup steps run eagerly; the K timed steps are one HIP graph of exactly K steps
    # (each step rotates to the next packed-weight copy of every layer), replayed once
    # between a synchronize on both sides and timed with HIP events on the replay stream.
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
    del g_steps

    per_case = []
    for c in cases:
        r = run_case_metrics(c, qoq, torch, args.kernel_launches)
        r["layer"] = c.L.name
        per_case.append(r)
        print(json.dumps({"case": r["layer"], "M": r["M"], "gemm_us": round(r["gemm_us"], 2),
                          "linear_us": round(r["linear_us"], 2), "roofline_frac": round(r["roofline_frac"], 3)}),
              file=sys.stderr, flush=True)
    ops = sum(c.ops for c in cases)
    wbytes = sum(c.bytes["weight"] for c in cases)
    # dominant kernel: the GEMM launch with the largest time in the step
    dom = max(per_case, key=lambda r: r["gemm_us"])
    regimes = {}
    for k, (name, M) in REGIMES.items():
        for r, c in zip(per_case, cases):
            if (r["layer"], r["M"]) == (name, M):
                regimes[k] = roofline_of(r, c)
    if "mfma" in regimes:
        c = cases[[(r["layer"], r["M"]) for r in per_case].index(REGIMES["mfma"])]
        data_tops = mfma_ceiling_data(qoq, torch, c)
        const_tops = mfma_ceiling(qoq, torch, dev)
        regimes["mfma"].update({"ceiling_TOPS_same_data": data_tops,
                                "frac_of_ceiling_same_data": regimes["mfma"]["achieved"] / data_tops,
                                "ceiling_TOPS_constant_operands": const_tops})
    workload = "; ".join(f"{name} M={','.join(str(m) for m in Ms)} (K={wl.find(name).K} N={wl.find(name).N})"
                         for name, Ms in plan)
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
        "config": {"workload": "W4A8 g128 linear per case (per-token INT8 activation quant + GEMM + fp16 "
                               "epilogue, one qoq_w4a8_linear call): " + workload,
                   "cases": [{"layer": name, "K": wl.find(name).K, "N": wl.find(name).N, "M": list(Ms)}
                             for name, Ms in plan],
                   "group": 128},
        "weight_GBps_step": wbytes / step_s / 1e9,
        "roofline": roofline_of(dom, cases[per_case.index(dom)]),
        "regimes": regimes,
        "cases": per_case,
        "offline_pack_ms": pack_ms,
        "copy_ceiling": copy_ceiling(qoq, torch, dev),
        "kv4_attention": None if args.no_kv4 else kv4_case_metrics(wl.find_kv("llama3_8b_b64_l1024"), qoq, torch, dev,
                                                                    args.kernel_launches),
        "host_wall_s": t_host,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_step(plan, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
