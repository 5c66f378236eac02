#!/usr/bin/env python3
"""Benchmark of the MXFP8 Linear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic, seeded
input that is already resident in HBM: the MXFP8 quantize kernels that
produce the GEMM operands from bf16, then the MXFP8 GEMM(s) with their
epilogues.  The default workload is the large square forward GEMM:
rowwise and columnwise MXFP8 quantize of both 8192 x 8192 bf16 inputs, then
the 8192^3 E4M3 GEMM (bf16 out).  Other workloads (--workload decoder_fwd,
hybrid_bwd, moe_grouped, tiny) print the same kind of line for their step.

One JSON line is printed.  `value` is the whole-step throughput: the GEMM
flops of a step divided by the measured wall time of a step (quantize time
included).  Per-kernel averages come from HIP events recorded between the
launches on the launch stream inside the timed region; `roofline` reports
the dominant kernel against MI355X's published peak (HIP-event timing),
and beside it, when summaries taken on the current kernel sources are
committed under profiles/, that kernel's rocprofv3 average duration and
its counter-measured HBM traffic (both looked up, and labelled so);
`targets` says which headline targets apply to the workload and whether
this run meets them; `kernels` lists every kernel, `cpu_baseline` the CPU
oracle timed on a bounded sample.

Bandwidth measurements rotate over several copies of every bf16 input and
quantize output (more than the 256 MB last-level cache), so a kernel's
reads come from HBM rather than from a cache warmed by the previous step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # dense FP8 / MXFP8 MFMA, MI355X
PEAK_HBM_GBS = 8000.0         # HBM3E, MI355X
METRIC = "MXFP8 GEMM TFLOP/s + % of MI355X FP8 MFMA peak; quantize GB/s % of HBM"
ROTATE = 4                     # copies of each bandwidth-bound input / output
# kernels each kind of op launches, in order (names as the profiler reports
# them; "a|b": the library picks one of the two by size)
KERNELS = {"quantize_row": ["quantize_rowwise_kernel"], "quantize_col": ["quantize_colwise_kernel"],
           "gemm": ["mx_gemm_kernel|mx_gemm4_kernel"], "grouped": ["mx_grouped_gemm_kernel"],
           "cast": ["amax_partial_kernel", "cast_current_kernel"],
           "quantize_bgrad": ["quantize_both128_kernel|quantize_colwise_kernel", "bgrad_final_kernel"],
           "cast_delayed": ["cast_amax_kernel", "delayed_update_kernel"],
           "quantize_block1d": ["block_quantize_1d_kernel"], "quantize_block2d": ["block_quantize_2d_kernel"],
           "gemm_block_e8m0": ["mx_gemm_kernel"], "gemm_block_fp32": ["mx_gemm_kernel"]}
ATTR_RUNS = 7                  # timed runs of each op's back-to-back launches (per-op mean, median, p10, p90)
CALIBRATION_BYTES = 512 << 20  # one device-to-device copy of this many bytes reads and writes it once


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--workload", default="square_8192",
                   choices=["square_8192", "decoder_fwd", "decoder_fwd_mx", "decoder_fwd_delayed", "hybrid_bwd",
                            "hybrid_bwd_fused", "moe_grouped", "block_e8m0_square_8192", "block_fp32_square_8192",
                            "tiny"])
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed region, copy a 512 MiB buffer 3 times (counter calibration)")
    p.add_argument("--record-ops", metavar="PATH",
                   help="write the op / kernel launch order and this run's line to PATH (for profile summaries)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/")
    p.add_argument("--stats-from", metavar="DIR",
                   help="no GPU: turn a rocprofv3 --kernel-trace --stats run into profiles/")
    p.add_argument("--mfma-from", metavar="DIR",
                   help="no GPU: turn a rocprofv3 --pmc run of the MFMA and clock counters into profiles/")
    p.add_argument("--command", default="", help="the profiling command, recorded with --stats-from / --mfma-from")
    p.add_argument("--no-graph", action="store_true",
                   help="launch every op from Python instead of replaying captured HIP graphs")
    return p.parse_args()


# ----------------------------------------------------------------- the step

class Step:
    """A list of kernel launches over resident buffers, with per-op accounting."""

    def __init__(self, name):
        self.name = name
        self.ops = []      # (label, kind, fn(rot), flops, bytes)
        self.kernels = []  # per op: names of the kernels it launches, in launch order

    def add(self, label, kind, fn, flops=0.0, nbytes=0.0, kernels=None):
        self.ops.append((label, kind, fn, flops, nbytes))
        self.kernels.append(list(kernels or KERNELS[kind]))

    @property
    def flops(self):
        return sum(o[3] for o in self.ops)


def percentile(sorted_vals, q):
    """Linear-interpolation percentile of an ascending list."""
    if len(sorted_vals) == 1:
        return sorted_vals[0]
    x = (len(sorted_vals) - 1) * q / 100.0
    i = int(x)
    j = min(i + 1, len(sorted_vals) - 1)
    return sorted_vals[i] + (sorted_vals[j] - sorted_vals[i]) * (x - i)


def q_bytes(rows, cols):
    return rows * cols * (2 + 1 + 1 / 32)


def gemm_bytes(M, N, K, epi, grouped_experts=0, mx_out=False):
    b = M * K * (1 + 1 / 32) + N * K * (1 + 1 / 32) * max(1, grouped_experts) + M * N * (1 + 1 / 32 if mx_out else 2)
    if epi == "bias_gelu_aux":
        b += M * N * 2
    if epi != "none":
        b += N * 2 * max(1, grouped_experts)
    return b


def build_step(workload, torch, te, workloads):
    """Allocate resident inputs and outputs; return a Step whose ops take the rotation index."""
    dev = torch.device("cuda:0")

    def upload(bits):
        return torch.from_numpy(bits.view("int16")).to(dev)

    def rotated(bits):
        t = upload(bits)
        return [t] + [t.clone() for _ in range(ROTATE - 1)]

    def qbufs(rows, cols, direction):
        out = []
        for _ in range(ROTATE):
            if direction == "row":
                out.append((torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                            torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)))
            else:
                out.append((torch.empty((cols, rows), dtype=torch.uint8, device=dev),
                            torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)))
        return out

    step = Step(workload)
    w = workloads.ALL[workload]()
    quantized = {}  # (tensor spec, dir) -> rotating (q, s)

    def add_quantize(spec, fmt, direction, label):
        key = (spec, direction, fmt)
        if key in quantized:
            return quantized[key]
        src = rotated(spec.make())
        rows, cols = spec.shape
        bufs = qbufs(rows, cols, direction)

        def fn(r, src=src, bufs=bufs, fmt=fmt, direction=direction):
            q, s = bufs[r]
            if direction == "row":
                te.te_mxfp8_quantize(src[r], fmt, "row", q, s, None, None)
            else:
                te.te_mxfp8_quantize(src[r], fmt, "col", None, None, q, s)
        step.add(label, "quantize", fn, 0.0, q_bytes(rows, cols), KERNELS["quantize_" + direction])
        quantized[key] = bufs
        return bufs

    for spec, fmt, direction in w.quantize:
        add_quantize(spec, fmt, direction, f"quantize_{direction}_{spec.shape[0]}x{spec.shape[1]}_t{spec.tensor_id}")

    for spec, fmt in w.fused_bgrad:
        src = rotated(spec.make())
        rows, cols = spec.shape
        rbufs, cbufs = qbufs(rows, cols, "row"), qbufs(rows, cols, "col")
        bgrads = [torch.empty(cols, dtype=torch.float32, device=dev) for _ in range(ROTATE)]
        ws = torch.empty(te.te_mxfp8_quantize_bgrad_workspace_size(rows, cols), dtype=torch.uint8, device=dev)

        def fn(r, src=src, rbufs=rbufs, cbufs=cbufs, bgrads=bgrads, ws=ws, fmt=fmt):
            te.te_mxfp8_quantize_bgrad(src[r], fmt, rbufs[r][0], rbufs[r][1], cbufs[r][0], cbufs[r][1], bgrads[r], ws)
        # read bf16 once; write both copies, their scales and the fp32 column sums
        nbytes = rows * cols * (2 + 2 + 2 / 32) + 4 * cols
        step.add(f"quantize_both_bgrad_{rows}x{cols}", "quantize", fn, 0.0, nbytes, KERNELS["quantize_bgrad"])
        quantized[(spec, "row", fmt)] = rbufs
        quantized[(spec, "col", fmt)] = cbufs

    def add_delayed_cast(spec, fmt, label):
        # one tensor's delayed-scaling state (scale, amax history) and its rotating casts
        src = rotated(spec.make())
        n = spec.shape[0] * spec.shape[1]
        scale = torch.ones(1, dtype=torch.float32, device=dev)
        hist = torch.zeros(16, dtype=torch.float32, device=dev)
        ws = torch.empty(te.te_amax_workspace_size(n), dtype=torch.uint8, device=dev)
        outs = [(torch.empty(spec.shape, dtype=torch.uint8, device=dev), torch.empty(1, dtype=torch.float32, device=dev))
                for _ in range(ROTATE)]

        def fn(r, src=src, outs=outs, scale=scale, hist=hist, ws=ws, fmt=fmt):
            te.te_fp8_cast_delayed_scaling(src[r], fmt, outs[r][0], outs[r][1], scale, hist, ws, "max", 0)
        step.add(label, "cast", fn, 0.0, n * (2 + 1), KERNELS["cast_delayed"])
        return outs

    def add_block_quantize(spec, fmt, block_2d, label):
        src = rotated(spec.make())
        rows, cols = spec.shape
        srows = (rows + 127) // 128 if block_2d else rows
        outs = [(torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                 torch.empty((srows, cols // 128), dtype=torch.float32, device=dev)) for _ in range(ROTATE)]

        def fn(r, src=src, outs=outs, fmt=fmt, block_2d=block_2d):
            te.te_fp8_block_quantize(src[r], fmt, block_2d, outs[r][0], outs[r][1])
        step.add(label, "quantize", fn, 0.0, rows * cols * 3 + srows * (cols // 128) * 4,
                 KERNELS["quantize_block2d" if block_2d else "quantize_block1d"])
        return outs

    mx_outputs = {}  # GEMM name -> rotating (codes, scales) of its MXFP8 output
    for g in w.gemms:
        if g.scaling.startswith("block_"):
            mode = g.scaling[len("block_"):]
            qa = add_block_quantize(g.a_src, g.fmt_a, False, f"quantize_block1d_{g.name}_A")
            qb = add_block_quantize(g.b_src, g.fmt_b, True, f"quantize_block2d_{g.name}_B")
            bias = upload(g.bias.make()) if g.bias is not None else None
            d = torch.empty((g.M, g.N), dtype=torch.bfloat16, device=dev)
            aux = torch.empty((g.M, g.N), dtype=torch.bfloat16, device=dev) if g.epilogue == "bias_gelu_aux" else None
            wsb = te.te_fp8_block_gemm_workspace_size(g.M, g.N, g.K, mode)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

            def fn(r, g=g, qa=qa, qb=qb, bias=bias, d=d, aux=aux, ws=ws, mode=mode):
                te.te_fp8_block_gemm(qa[r][0], qa[r][1], g.fmt_a, qb[r][0], qb[r][1], g.fmt_b, True, d, g.epilogue,
                                     bias, aux, mode, ws)
            # algorithmic bytes: 1 B per operand element, the fp32 scales (one per 128 elements of A, per
            # 128 x 128 of B) and the output
            nbytes = gemm_bytes(g.M, g.N, g.K, g.epilogue) - (g.M + g.N) * g.K / 32 + g.M * g.K / 32 + \
                ((g.N + 127) // 128) * g.K / 32
            step.add(f"gemm_block_{mode}_{g.name}_{g.M}x{g.N}x{g.K}", "gemm", fn, g.flops, nbytes,
                     KERNELS["gemm_block_" + mode])
            continue
        if g.scaling == "delayed":
            ca = add_delayed_cast(g.a_src, g.fmt_a, f"cast_delayed_{g.name}_A")
            cb = add_delayed_cast(g.b_src, g.fmt_b, f"cast_delayed_{g.name}_B")
            bias = upload(g.bias.make()) if g.bias is not None else None
            d = torch.empty((g.M, g.N), dtype=torch.bfloat16, device=dev)
            aux = torch.empty((g.M, g.N), dtype=torch.bfloat16, device=dev) if g.epilogue == "bias_gelu_aux" else None

            def fn(r, g=g, ca=ca, cb=cb, bias=bias, d=d, aux=aux):
                te.te_fp8_gemm(ca[r][0], ca[r][1], g.fmt_a, cb[r][0], cb[r][1], g.fmt_b, d, g.epilogue, bias, aux)
            # per-tensor operands: 1 B per element, no block scales
            nbytes = gemm_bytes(g.M, g.N, g.K, g.epilogue) - (g.M + g.N) * g.K / 32
            step.add(f"gemm_fp8_{g.name}_{g.M}x{g.N}x{g.K}", "gemm", fn, g.flops, nbytes)
            continue
        if g.a_from is not None:
            qa = mx_outputs[g.a_from]
        else:
            qa = add_quantize(g.a_src, g.fmt_a, g.a_dir, f"quantize_{g.a_dir}_{g.name}_A")
        qb = add_quantize(g.b_src, g.fmt_b, g.b_dir, f"quantize_{g.b_dir}_{g.name}_B")
        bias = upload(g.bias.make()) if g.bias is not None else None
        aux = torch.empty((g.M, g.N), dtype=torch.bfloat16, device=dev) if g.epilogue == "bias_gelu_aux" else None
        # the GEMM's workspace (allocated here, outside the timed region): with it the 4-wave kernel
        # runs, after a small kernel that rearranges the operands' scales into it
        ws = te.gemm_workspace(g.M, g.N, g.K, dev)
        gemm_kernels = ["scale_blocks_kernel", "mx_gemm4_kernel"] if ws is not None else ["mx_gemm_kernel"]
        if g.mx_out:
            outs = qbufs(g.M, g.N, "row")
            mx_outputs[g.name] = outs

            def fn(r, g=g, qa=qa, qb=qb, bias=bias, outs=outs, aux=aux, ws=ws):
                te.te_mxfp8_gemm_mxout(qa[r][0], qa[r][1], g.fmt_a, qb[r][0], qb[r][1], g.fmt_b, outs[r][0],
                                       outs[r][1], "e4m3", g.epilogue, bias, aux, ws)
            step.add(f"gemm_{g.name}_mxout_{g.M}x{g.N}x{g.K}", "gemm", fn, g.flops,
                     gemm_bytes(g.M, g.N, g.K, g.epilogue, mx_out=True), gemm_kernels)
            continue
        d = torch.empty((g.M, g.N), dtype=torch.bfloat16, device=dev)

        def fn(r, g=g, qa=qa, qb=qb, bias=bias, d=d, aux=aux, ws=ws):
            te.te_mxfp8_gemm(qa[r][0], qa[r][1], g.fmt_a, qb[r][0], qb[r][1], g.fmt_b, d, g.epilogue, bias, aux,
                             ws)
        step.add(f"gemm_{g.name}_{g.M}x{g.N}x{g.K}", "gemm", fn, g.flops, gemm_bytes(g.M, g.N, g.K, g.epilogue),
                 gemm_kernels)

    for g in w.grouped:
        qa = add_quantize(g.a_src, g.fmt_a, "row", f"quantize_row_{g.name}_A")
        qb = add_quantize(g.b_src, g.fmt_b, "row", f"quantize_row_{g.name}_B")
        bias = upload(g.bias.make()) if g.bias is not None else None
        counts = workloads.moe_counts(g.total_m, g.experts)
        splits = torch.tensor(counts, dtype=torch.int32, device=dev)
        d = torch.empty((g.total_m, g.N), dtype=torch.bfloat16, device=dev)
        aux = torch.empty((g.total_m, g.N), dtype=torch.bfloat16, device=dev) if g.epilogue == "bias_gelu_aux" else None

        def fn(r, g=g, qa=qa, qb=qb, bias=bias, d=d, aux=aux, splits=splits):
            te.te_mxfp8_grouped_gemm(splits, qa[r][0], qa[r][1], g.fmt_a, qb[r][0], qb[r][1], g.fmt_b, g.N, d,
                                     g.epilogue, bias, aux)
        flops = 2.0 * g.total_m * g.N * g.K
        step.add(f"grouped_gemm_{g.name}_{g.experts}x{g.N}x{g.K}", "gemm", fn, flops,
                 gemm_bytes(g.total_m, g.N, g.K, g.epilogue, g.experts), KERNELS["grouped"])

    for spec, fmt in w.current_scaling:
        src = rotated(spec.make())
        n = spec.shape[0] * spec.shape[1]
        ws = torch.empty(te.te_amax_workspace_size(n), dtype=torch.uint8, device=dev)
        outs = [(torch.empty(spec.shape, dtype=torch.uint8, device=dev),
                 *(torch.empty(1, dtype=torch.float32, device=dev) for _ in range(3))) for _ in range(ROTATE)]

        def fn(r, src=src, outs=outs, ws=ws, fmt=fmt):
            q, a, s, si = outs[r]
            te.te_fp8_cast_current_scaling(src[r], fmt, q, a, s, si, ws)
        step.add(f"current_scaling_cast_{spec.shape[0]}x{spec.shape[1]}", "cast", fn, 0.0, n * (2 + 3))
    return step


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(workload, workloads):
    """Time the oracle on a bounded sample of the step and scale it to the full step.

    Sample: the oracle's step restricted to the first rows of every operand
    (up to 4096, fewer where one sampled GEMM block would exceed 2.5e11
    flop): the quantizes of those rows and the GEMM block they produce; about
    10-20 s of host work.  The full-step time is estimated as
    quantize_time * (full quantize elements / sampled ones) +
    gemm_time * (full GEMM flops / sampled ones).
    """
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl absent
        threads = 1
    w = workloads.ALL[workload]()
    q_time = q_elems_s = q_elems_full = 0.0
    g_time = g_flops_s = g_flops_full = 0.0
    S = 4096
    gemms = list(w.gemms)
    for g in gemms:
        a, b = g.a_src.make(), g.b_src.make()
        sm, sn = min(S, g.M), min(S, g.N)
        while 2.0 * sm * sn * g.K > 2.5e11:
            if sm >= sn:
                sm //= 2
            else:
                sn //= 2
        fa, fb = oracle.format_by_name(g.fmt_a), oracle.format_by_name(g.fmt_b)
        bias = g.bias.make()[:sn] if g.bias is not None else None
        if g.scaling.startswith("block_"):
            sn = max(128, sn // 128 * 128)  # whole 128-row blocks of B
            t0 = time.perf_counter()
            qa, sa = oracle.quantize_1d(a[:sm], fa)
            qb, sb = oracle.quantize_2d(b[:sn], fb)
            t1 = time.perf_counter()
            if g.scaling == "block_e8m0":
                sa, sb = oracle.pow2_at_least(sa), oracle.pow2_at_least(sb)
            oracle.block_gemm(qa, sa, fa, qb, sb, fb, True, bias, g.epilogue)
            t2 = time.perf_counter()
        elif g.scaling == "delayed":
            t0 = time.perf_counter()
            h0 = np.zeros(16, np.float32)
            qa, ia, _, _, _ = oracle.delayed_scaling_step(a[:sm], fa, h0, np.float32(1.0))
            qb, ib, _, _, _ = oracle.delayed_scaling_step(b[:sn], fb, h0, np.float32(1.0))
            t1 = time.perf_counter()
            oracle.fp8_gemm_per_tensor(qa, ia, fa, qb, ib, fb, bias, g.epilogue)
            t2 = time.perf_counter()
        else:
            t0 = time.perf_counter()
            qa, sa = (oracle.quantize_rowwise(a[:sm], fa) if g.a_dir == "row"
                      else oracle.quantize_colwise(np.ascontiguousarray(a[:, :sm]), fa))
            qb, sb = (oracle.quantize_rowwise(b[:sn], fb) if g.b_dir == "row"
                      else oracle.quantize_colwise(np.ascontiguousarray(b[:, :sn]), fb))
            t1 = time.perf_counter()
            oracle.mx_gemm(qa, sa, fa, qb, sb, fb, bias, g.epilogue)
            t2 = time.perf_counter()
        q_time += t1 - t0
        q_elems_s += (sm + sn) * g.K
        q_elems_full += (g.M + g.N) * g.K
        g_time += t2 - t1
        g_flops_s += 2.0 * sm * sn * g.K
        g_flops_full += 2.0 * g.M * g.N * g.K
    for spec, fmt, direction in w.quantize:
        if any(spec in (g.a_src, g.b_src) for g in gemms):
            q_elems_full += spec.shape[0] * spec.shape[1]  # the other direction of an operand already timed
    b_time = b_elems_s = b_elems_full = 0.0
    for spec, fmt in w.fused_bgrad:
        x = spec.make()
        sr = min(S, spec.shape[0])
        t0 = time.perf_counter()
        oracle.column_sums(x[:sr])
        b_time += time.perf_counter() - t0
        b_elems_s += sr * spec.shape[1]
        b_elems_full += spec.shape[0] * spec.shape[1]
    for g in w.grouped:
        counts = workloads.moe_counts(g.total_m, g.experts)
        a = g.a_src.make()
        b = g.b_src.make()
        sm = min(256, int(counts[0]))
        fa = oracle.format_by_name(g.fmt_a)
        t0 = time.perf_counter()
        qa, sa = oracle.quantize_rowwise(a[:sm], fa)
        qb, sb = oracle.quantize_rowwise(b[:g.N], fa)
        t1 = time.perf_counter()
        bias = g.bias.make()[0] if g.bias is not None else None
        oracle.mx_gemm(qa, sa, fa, qb, sb, fa, bias, g.epilogue)
        t2 = time.perf_counter()
        q_time += t1 - t0
        q_elems_s += (sm + g.N) * g.K
        q_elems_full += (g.total_m + g.experts * g.N) * g.K
        g_time += t2 - t1
        g_flops_s += 2.0 * sm * g.N * g.K
        g_flops_full += 2.0 * g.total_m * g.N * g.K
    est = q_time * (q_elems_full / max(q_elems_s, 1)) + g_time * (g_flops_full / max(g_flops_s, 1))
    est += b_time * (b_elems_full / max(b_elems_s, 1))
    return {"value": g_flops_full / est / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"oracle (numpy fp64) on the first rows of each operand (up to {S}): quantize "
                       f"{q_elems_s:.3g} elements in {q_time:.2f} s (1 thread), GEMM {g_flops_s:.3g} flop in "
                       f"{g_time:.2f} s ({threads} BLAS threads); full step estimated at {est:.1f} s by scaling "
                       f"each part to the full step's elements / flops"),
            "host_cpus": os.cpu_count()}


# ------------------------------------------------------------------ traffic

TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp8_mixed_precision_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, label):
    """HBM bytes per launch of one op from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_JSON) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("sources_hash") != kernel_sources_hash():
        return None
    entry = data.get("workloads", {}).get(workload, {}).get("ops", {}).get(label)
    return None if entry is None else entry["bytes_per_launch"]


def _read_counters(csv_path, counter):
    """Dispatches of one rocprofv3 --pmc CSV: [(kernel name, value in KiB)] in dispatch order."""
    import csv
    with open(csv_path) as fh:
        rows = [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]


def _per_op(dispatches, record):
    """Average the counter over each op's launches (an op's kernels summed).

    The library's dispatches come in the order bench.py made them: the
    (pre + warmup + steps) passes over the step's ops, then, op by op, its
    attribution launches."""
    ours = [(n, v) for n, v in dispatches if "temx::" in n]
    order = []
    for _ in range(record.get("pre", 0) + record["warmup"] + record["steps"]):
        order += [op for op in record["ops"]]
    for op, n in zip(record["ops"], record.get("attr_launches", [1 + record["steps"]] * len(record["ops"]))):
        order += [op] * n
    expected = sum(len(op["kernels"]) for op in order)
    if len(ours) != expected:
        raise SystemExit(f"expected {expected} library dispatches, found {len(ours)}")
    totals = {op["label"]: 0.0 for op in record["ops"]}
    launches = {op["label"]: 0 for op in record["ops"]}
    i = 0
    for op in order:
        for kern in op["kernels"]:
            name, v = ours[i]
            if not any(k in name for k in kern.split("|")):
                raise SystemExit(f"dispatch {i}: expected {kern}, found {name[:80]}")
            totals[op["label"]] += v
            i += 1
        launches[op["label"]] += 1
    return {k: totals[k] / launches[k] for k in totals}


def _calibration(dispatches, record):
    """KiB the counter reads for one copy of CALIBRATION_BYTES (the copies bench.py makes last)."""
    copies = [v for n, v in dispatches if "copyBuffer" in n][-record["calibration_copies"]:]
    return sum(copies) / len(copies)


def traffic_from(fetch_dir, write_dir):
    """Write the per-op HBM traffic of two counter runs into the committed summary."""
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        with open(os.path.join(d, "ops.json")) as fh:
            record = json.load(fh)
        csvs = [os.path.join(r, f) for r, _, fs in os.walk(d) for f in fs if f.endswith("counter_collection.csv")]
        disp = _read_counters(csvs[0], counter)
        copy_kib = _calibration(disp, record)
        factor = CALIBRATION_BYTES / (copy_kib * 1024.0)
        out[counter] = (record, copy_kib, factor, _per_op(disp, record))
    record = out["FETCH_SIZE"][0]
    wl = record["workload"]
    try:
        with open(TRAFFIC_JSON) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    if data.get("sources_hash") != kernel_sources_hash():
        data = {"sources_hash": kernel_sources_hash(), "workloads": {}}
    ops = {}
    for op in record["ops"]:
        lab = op["label"]
        fb = out["FETCH_SIZE"][3][lab] * 1024.0 * out["FETCH_SIZE"][2]
        wb = out["WRITE_SIZE"][3][lab] * 1024.0 * out["WRITE_SIZE"][2]
        ops[lab] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                    "algorithmic_bytes": round(op["bytes"]) if op["bytes"] else None}
    data["workloads"][wl] = {
        "calibration": {"copy_bytes": CALIBRATION_BYTES,
                        "fetch_kib_per_copy": out["FETCH_SIZE"][1], "fetch_factor": round(out["FETCH_SIZE"][2], 4),
                        "write_kib_per_copy": out["WRITE_SIZE"][1], "write_factor": round(out["WRITE_SIZE"][2], 4)},
        "commands": [out[c][0]["command"].replace("PMC", c) for c in ("FETCH_SIZE", "WRITE_SIZE")],
        "ops": ops}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(data, fh, indent=1)
    md = [f"# HBM traffic per launch, workload {wl}", "",
          "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), one rocprofv3 --pmc run each, scaled by",
          f"what the same counter reads for a device-to-device copy of {CALIBRATION_BYTES >> 20} MiB made in the "
          "same run:", ""]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        md.append(f"- {c}: {out[c][1]:.1f} KiB per copy -> factor {out[c][2]:.4f}")
    md += ["", "Commands (from the repository root):", ""]
    md += ["    " + c for c in data["workloads"][wl]["commands"]]
    md += ["", "| op | fetch MB | write MB | total MB | algorithmic MB | total / algorithmic |",
           "|---|---:|---:|---:|---:|---:|"]
    for lab, e in ops.items():
        alg = e["algorithmic_bytes"]
        md.append(f"| {lab} | {e['fetch_bytes'] / 1e6:.2f} | {e['write_bytes'] / 1e6:.2f} | "
                  f"{e['bytes_per_launch'] / 1e6:.2f} | {alg / 1e6 if alg else float('nan'):.2f} | "
                  f"{e['bytes_per_launch'] / alg if alg else float('nan'):.3f} |")
    md += ["", f"Kernel sources hash: {data['sources_hash']}", ""]
    path = os.path.join(ROOT, "profiles", f"{wl}_traffic.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md))
    print(f"wrote {TRAFFIC_JSON} and {path}")


KERNEL_TIME_JSON = os.path.join(ROOT, "profiles", "kernel_time.json")


def _read_trace(csv_path):
    """Dispatches of one rocprofv3 kernel-trace CSV: [(kernel name, duration in us)] in dispatch order."""
    import csv
    with open(csv_path) as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]


def rocprof_kernel_time(workload, label):
    """rocprofv3 average duration (us) of one op's kernels from the committed kernel-trace summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(KERNEL_TIME_JSON) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("sources_hash") != kernel_sources_hash():
        return None
    return data.get("workloads", {}).get(workload, {}).get("ops_avg_us", {}).get(label)


def stats_from(stats_dir, command):
    """Summarise a rocprofv3 --kernel-trace --stats run next to the bench line it profiled: the
    per-kernel statistics, and each op's average kernel duration from the trace (its kernels summed,
    over every launch of the run), which also goes into profiles/kernel_time.json."""
    import csv
    files = [os.path.join(r, f) for r, _, fs in os.walk(stats_dir) for f in fs]
    with open([f for f in files if f.endswith("kernel_stats.csv")][0]) as fh:
        rows = list(csv.DictReader(fh))
    with open(os.path.join(stats_dir, "ops.json")) as fh:
        record = json.load(fh)
    wl = record["workload"]
    per_op = _per_op(_read_trace([f for f in files if f.endswith("kernel_trace.csv")][0]), record)
    try:
        with open(KERNEL_TIME_JSON) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    if data.get("sources_hash") != kernel_sources_hash():
        data = {"sources_hash": kernel_sources_hash(), "workloads": {}}
    data["workloads"][wl] = {"command": command, "ops_avg_us": {k: round(v, 3) for k, v in per_op.items()}}
    with open(KERNEL_TIME_JSON, "w") as fh:
        json.dump(data, fh, indent=1)
    md = [f"# Kernel time, workload {wl}", "", "Command (from the repository root):", "",
          "    " + command, "", "rocprofv3 kernel statistics:", "",
          "| kernel | calls | avg us | min us | max us | total % |", "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        short = name.replace("void ", "").replace("temx::(anonymous namespace)::", "").split("(")[0]
        md.append(f"| `{short[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    ops = {o["label"]: o for o in record["ops"]}
    events = {k["name"]: k["avg_ms"] * 1e3 for k in (record.get("bench_line") or {}).get("kernels", [])}
    md += ["", "Per op: the average duration of its kernels in the trace above (every launch of the run), and",
           "the HIP-event average of the same run (bench.py, back-to-back launches after the timed region):", "",
           "| op | rocprof avg us | HIP events avg us | rocprof TFLOP/s | rocprof GB/s |", "|---|---:|---:|---:|---:|"]
    for lab, us in per_op.items():
        o = ops[lab]
        tf = f"{o['flops'] / (us * 1e-6) / 1e12:.1f}" if o.get("flops") else ""
        gb = f"{o['bytes'] / (us * 1e-6) / 1e9:.1f}" if o.get("bytes") else ""
        ev = f"{events[lab]:.2f}" if lab in events else ""
        md.append(f"| {lab} | {us:.2f} | {ev} | {tf} | {gb} |")
    if record.get("bench_line"):
        md += ["", "bench.py line of this run:", "", "    " + json.dumps(record["bench_line"]["summary"])]
    md += ["", f"Kernel sources hash: {kernel_sources_hash()}", ""]
    path = os.path.join(ROOT, "profiles", f"{wl}_kernel_stats.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md))
    print(f"wrote {path}")


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE GRBM_COUNT"


def mfma_from(pmc_dir, command):
    """Summarise a rocprofv3 --pmc run of MFMA_COUNTERS: per MFMA kernel, the FP8 MFMA work the counters
    saw against the op's algorithmic flops, and the MFMA-busy share of the SIMDs' active cycles."""
    import csv
    import statistics
    csvs = [os.path.join(r, f) for r, _, fs in os.walk(pmc_dir) for f in fs if f.endswith("counter_collection.csv")]
    with open(csvs[0]) as fh:
        rows = list(csv.DictReader(fh))
    with open(os.path.join(pmc_dir, "ops.json")) as fh:
        record = json.load(fh)
    by, name, dur = {}, {}, {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        by.setdefault(d, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        name[d] = r["Kernel_Name"].replace("void ", "").replace("temx::(anonymous namespace)::", "").split("(")[0]
        dur[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    xcc, simds = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
    gemm_flops = sorted({o["flops"] for o in record["ops"] if o.get("flops")})
    wl = record["workload"]
    md = [f"# MFMA utilisation, workload {wl}", "", "Command (from the repository root):", "",
          "    " + command, "",
          "Per dispatch of each kernel that issues FP8 MFMAs (medians over the run's dispatches):", "",
          "- MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 (the counter counts multiply and add operations / 512);",
          "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): the share of the",
          "  SIMDs' active cycles in which the matrix unit is busy;",
          "- GRBM cycles per ns = GRBM_GUI_ACTIVE / 8 over the dispatch's counter-run duration (a relative clock:",
          "  compare it with the HBM-bound kernels of the same run, which run at the full clock).", "",
          "| kernel | dispatches | MFMA flops | algorithmic flops | ratio | MFMA busy | GRBM cycles per ns |",
          "|---|---:|---:|---:|---:|---:|---:|"]
    kernels = sorted({name[d] for d in by})
    other = []
    for k in kernels:
        ds = [d for d in by if name[d] == k]
        f = statistics.median([by[d].get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) * 512 for d in ds])
        clk = statistics.median([by[d]["GRBM_GUI_ACTIVE"] / xcc / max(dur[d], 1) for d in ds])
        if f <= 0:
            other.append((k, len(ds), clk))
            continue
        busy = statistics.median([by[d]["SQ_VALU_MFMA_BUSY_CYCLES"] / (by[d]["GRBM_GUI_ACTIVE"] / xcc * simds)
                                  for d in ds])
        alg = min(gemm_flops, key=lambda x: abs(x - f)) if gemm_flops else 0.0
        md.append(f"| `{k[:80]}` | {len(ds)} | {f:.4g} | {alg:.4g} | {f / alg if alg else 0:.4f} | "
                  f"{100 * busy:.1f}% | {clk:.3f} |")
    md += ["", "Kernels without MFMA work in the same run:", "", "| kernel | dispatches | GRBM cycles per ns |",
           "|---|---:|---:|"]
    md += [f"| `{k[:80]}` | {n} | {c:.3f} |" for k, n, c in other]
    md += ["", f"Kernel sources hash: {kernel_sources_hash()}", ""]
    path = os.path.join(ROOT, "profiles", f"{wl}_mfma_util.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md))
    print(f"wrote {path}")


# --------------------------------------------------------------------- main

TARGET_QUANTIZE_FRAC_HBM = 0.70   # every MXFP8 quantize kernel, of MI355X's HBM peak
TARGET_GEMM_8192_FRAC = 0.60      # the 8192^3 MXFP8 GEMM, of the dense FP8 MFMA peak, per rocprof


def targets(w, kernels, roof):
    """The headline targets that apply to this workload, each with what this run measured and whether it
    is met (the GEMM target by the rocprof figure when one is committed for these sources)."""
    out = {}
    q = [k["frac_hbm_peak"] for k in kernels if k["kind"] == "quantize" and "frac_hbm_peak" in k]
    if q:
        out["quantize_frac_hbm"] = {"target": TARGET_QUANTIZE_FRAC_HBM, "min_measured": min(q),
                                    "met": min(q) >= TARGET_QUANTIZE_FRAC_HBM}
    if w.name == "square_8192":
        by = roof["rocprof"]["frac"] if roof.get("rocprof") else roof["frac"]
        out["gemm_8192_frac_fp8_peak"] = {"target": TARGET_GEMM_8192_FRAC, "events": roof["frac"],
                                          "rocprof": roof["rocprof"]["frac"] if roof.get("rocprof") else None,
                                          "met": by >= TARGET_GEMM_8192_FRAC}
    return out


def arithmetic(w):
    kinds = {g.scaling for g in w.gemms} or {"mx"}
    text = {"mx": "MXFP8 (E4M3/E5M2 codes, E8M0 scales per 32 elements)",
            "delayed": "per-tensor FP8 (E4M3/E5M2 codes, one FP32 scale per tensor, delayed scaling)",
            "block_e8m0": "blockwise FP8 (E4M3/E5M2 codes, FP32 scales per 1x128 / 128x128 block, cast to E8M0)",
            "block_fp32": "blockwise FP8 (E4M3/E5M2 codes, FP32 scales per 1x128 / 128x128 block, applied in fp32)"}
    return "; ".join(text[k] for k in sorted(kinds)) + " products, fp32 accumulate"


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.stats_from:
        stats_from(args.stats_from, args.command)
        return
    if args.mfma_from:
        mfma_from(args.mfma_from, args.command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MXFP8 Linear path is built and measured on a single MI355X "
              "(multi-GPU sharding is described, not run). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import mxfp8_mixed_precision_amd as te
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    step = build_step(args.workload, torch, te, workloads)
    stream = torch.cuda.current_stream()
    nops = len(step.ops)

    def run_eager(i):
        r = i % ROTATE
        for _, _, fn, _, _ in step.ops:
            fn(r)

    # Eager steps first (the library's cached device queries happen here),
    # then, unless --no-graph, HIP graphs of the step's launches: one per
    # buffer rotation, and one of all ROTATE rotations in order.  Replaying
    # them removes the host-side launch cost from the timed region, which
    # matters for the small kernels; a graph replay itself costs a few us
    # (measured: ~1.2 us per kernel with 4-kernel graphs, none with 48), so
    # whole rotation cycles replay as one graph.
    pre = 2 * ROTATE
    for i in range(pre):
        run_eager(i)
    torch.cuda.synchronize()
    graphs = None
    graph_cycle = None
    if not args.no_graph:
        graphs = []
        for r in range(ROTATE):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _, _, fn, _, _ in step.ops:
                    fn(r)
            graphs.append(g)
        graph_cycle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_cycle):
            for r in range(ROTATE):
                for _, _, fn, _, _ in step.ops:
                    fn(r)

    def run_steps(first, n):
        # exactly n steps, the i-th on buffer rotation i % ROTATE
        i = first
        while i < first + n:
            if graphs is None:
                run_eager(i)
                i += 1
            elif i % ROTATE == 0 and first + n - i >= ROTATE:
                graph_cycle.replay()
                i += ROTATE
            else:
                graphs[i % ROTATE].replay()
                i += 1

    run_steps(0, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.warmup, args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Per-op attribution, right after the timed region on the same stream: each
    # op launched back to back over the rotating buffers (one captured graph of
    # all its timed launches, replayed once to warm up and then ATTR_RUNS times,
    # each replay bracketed by two HIP events, so no marker sits between its
    # launches).
    reps = max(1, args.steps // ROTATE)
    kernels = []
    attr_launches = []
    for label, kind, fn, flops, nbytes in step.ops:
        # ATTR_RUNS timed runs of the op's reps * ROTATE back-to-back launches: the mean over all of them, and
        # the median, p10 and p90 of the per-run averages
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ATTR_RUNS)]
        if graphs is None:
            fn(0)
            for e0, e1 in evs:
                e0.record(stream)
                for i in range(reps * ROTATE):
                    fn(i % ROTATE)
                e1.record(stream)
            attr_launches.append(1 + ATTR_RUNS * reps * ROTATE)
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps * ROTATE):
                    fn(i % ROTATE)
            g.replay()
            for e0, e1 in evs:
                e0.record(stream)
                g.replay()
                e1.record(stream)
            attr_launches.append((1 + ATTR_RUNS) * reps * ROTATE)
        torch.cuda.synchronize()
        runs = sorted(e0.elapsed_time(e1) / (reps * ROTATE) for e0, e1 in evs)
        ms = sum(runs) / len(runs)
        ent = {"name": label, "kind": kind, "avg_ms": round(ms, 5), "median_ms": round(percentile(runs, 50), 5),
               "p10_ms": round(percentile(runs, 10), 5), "p90_ms": round(percentile(runs, 90), 5)}
        if flops:
            ent["tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
            ent["frac_fp8_peak"] = round(ent["tflops"] / PEAK_FP8_TFLOPS, 4)
            if nbytes:  # the roofline's attainable rate at this op's arithmetic intensity (HBM-limited below the ridge)
                attainable = min(PEAK_FP8_TFLOPS, flops / nbytes * PEAK_HBM_GBS / 1e3)
                ent["frac_attainable"] = round(ent["tflops"] / attainable, 4)
        if nbytes:
            ent["gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            ent["frac_hbm_peak"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
        kernels.append(ent)

    dom = max(range(nops), key=lambda k: kernels[k]["avg_ms"])
    dlabel, dkind, _, dflops, dbytes = step.ops[dom]
    dms = kernels[dom]["avg_ms"]
    if dkind == "gemm":
        roof = {"bound": "mfma", "achieved": round(dflops / (dms * 1e-3) / 1e12, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(dbytes / (dms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    w = workloads.ALL[args.workload]()
    roof["kernel"] = dlabel
    roof["timing"] = "HIP events on the launch stream, the op's launches back to back after the timed region"
    # the same kernel's rocprofv3 average, looked up from the committed kernel-trace summary
    r_us = rocprof_kernel_time(w.name, dlabel)
    if r_us is not None:
        r_ach = (dflops / (r_us * 1e-6) / 1e12) if dkind == "gemm" else (dbytes / (r_us * 1e-6) / 1e9)
        roof["rocprof"] = {"avg_us": r_us, "achieved": round(r_ach, 1), "frac": round(r_ach / roof["peak"], 4),
                           "source": f"profiles/{w.name}_kernel_stats.md (rocprofv3 --kernel-trace on these kernel "
                                     f"sources, {kernel_sources_hash()}; looked up, not measured in this run)"}
    else:
        roof["rocprof"] = None
    roof["traffic"] = measured_traffic(w.name, dlabel)
    roof["traffic_source"] = (
        f"profiles/{w.name}_traffic.md (rocprofv3 FETCH_SIZE and WRITE_SIZE runs on these kernel sources, "
        f"{kernel_sources_hash()}; looked up, not measured in this run)" if roof["traffic"] is not None else
        "no counter summary taken on the current kernel sources")

    value = step.flops / (ms_per_step * 1e-3) / 1e12
    qk = [k for k in kernels if k["kind"] == "quantize"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded N(0, sigma) bf16, outlier columns per config)",
        "config": {"workload": w.name, "gemm_flops_per_step": step.flops, "parallelism": "single GPU",
                   "launch": "eager" if graphs is None else "HIP graph replay (a graph per cycle of the 4 buffer rotations)",
                   "arithmetic": arithmetic(w),
                   "rotating_buffers": ROTATE},
        "roofline": roof,
        "quantize_gbs_min": min((k["gbs"] for k in qk), default=None),
        "quantize_frac_hbm_min": min((k["frac_hbm_peak"] for k in qk), default=None),
        "targets": targets(w, kernels, roof),
        "kernels": kernels,
    }
    if args.copy_calibration:
        src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, workloads)
    if args.record_ops:
        summary = {k: v for k, v in out.items() if k != "kernels"}
        rdir = os.path.relpath(os.path.dirname(os.path.abspath(args.record_ops)), ROOT)
        rec = {"workload": w.name, "pre": pre, "warmup": args.warmup, "steps": args.steps,
               "attr_launches": attr_launches,
               "calibration_copies": 3 if args.copy_calibration else 0,
               "command": f"timeout -s KILL 170 rocprofv3 --pmc PMC --output-format csv -d {rdir} -o run -- "
                          f"python bench.py --workload {args.workload} --steps {args.steps} "
                          f"--warmup {args.warmup} --no-cpu-baseline --copy-calibration "
                          f"--record-ops {os.path.relpath(os.path.abspath(args.record_ops), ROOT)}",
               "ops": [{"label": o[0], "kind": o[1], "bytes": o[4], "flops": o[3], "kernels": k}
                       for o, k in zip(step.ops, step.kernels)],
               "bench_line": {"kernels": kernels, "summary": summary}}
        os.makedirs(os.path.dirname(os.path.abspath(args.record_ops)), exist_ok=True)
        with open(args.record_ops, "w") as fh:
            json.dump(rec, fh)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
