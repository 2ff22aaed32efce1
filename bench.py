#!/usr/bin/env python3
"""Benchmark of the MX quantize / block-Hadamard / MX-GEMM hot path on one MI355X.

One step runs the three Llama-3.1-8B linear-layer workloads back to back on
seeded synthetic inputs already resident in device memory:
  QKV Fprop, MXFP8:     quantize X [8192x4096] and W [6144x4096] to E4M3,
                        Y[8192x6144] = X W^T, bf16 out;
  gate+up Fprop, MXFP4: quantize X [8192x4096] and W [28672x4096] to E2M1,
                        Y[8192x28672] = X W^T, bf16 out;
  down-proj Wgrad, MXFP4 with the fixed block-Hadamard rotation:
                        rotate-and-transpose-quantize dY [8192x14336] and
                        X [8192x4096] along tokens to E2M1,
                        dW[14336x4096] = dY^T X, fp32 out.
The pages quote their gains on Llama-3.1-8B pre-training on MI355X
(FP4-training article on hzrcw.cc, section 03); these are that model's
linear-layer shapes.  `value` is the step's GEMM work divided by the whole
step time (quantizers included), in TFLOP/s.  Each kernel is also timed with
HIP events on the stream it runs on and reported against its roofline, both
inside the step and alone after a clean fill of the last-level cache.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

# MI355X published peaks (dense)
PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "bf16": 2500.0}
CONFIGS = (1, 2, 3)  # the three Llama-3.1-8B workloads
WORKLOAD = "llama31_8b_linear_set"
PROFILE_COMMANDS = (
    "rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/prof_trace -o trace -- "
    "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --no-extra --iso-reps 5",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/prof_fetch -o fetch -- "
    "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-extra --iso-reps 5 --calibrate-copy",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/prof_write -o write -- "
    "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-extra --iso-reps 5 --calibrate-copy",
    "rocprofv3 --pmc GRBM_GUI_ACTIVE --output-format csv -d rocprof_out/prof_clock -o clock -- "
    "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --no-extra --iso-reps 5",
    "rocprofv3 --pmc MfmaUtil --output-format csv -d rocprof_out/prof_mfma -o mfma -- "
    "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --no-extra --iso-reps 5",
    "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE --output-format csv -d rocprof_out/prof_lds -o lds -- "
    "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --no-extra --iso-reps 5",
)
XCDS = 8          # MI355X: GRBM_GUI_ACTIVE sums the busy cycles of the 8 accelerator dies
PEAK_SCLK_GHZ = 2.4
MIN_CLOCK_US = 100  # shortest kernel whose counted busy cycles give a clock


def quant_bytes(rows: int, cols: int, fmt: str) -> float:
    """algorithmic HBM bytes of one quantize call: bf16 in, codes + scales out"""
    return rows * cols * (2.0 + (0.5 if fmt == "e2m1" else 1.0) + 1.0 / 32)


def spread(samples) -> list:
    """10th and 90th percentile of a list of times"""
    return [round(float(np.percentile(samples, 10)), 4), round(float(np.percentile(samples, 90)), 4)]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "precision_block_amax_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _profile_summary():
    """the committed rocprofv3 counter summary, if it was taken on the current
    kernel sources; else None"""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    return data if data.get("source_sha") == kernel_source_sha() else None


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None"""
    data = _profile_summary()
    k = None if data is None else data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def measured_mfma_util(kernel: str):
    """MFMA busy cycles as % of the SIMDs' cycles (rocprofv3 MfmaUtil) over the kernel's timed
    step launches, from the committed counter summary, or None"""
    data = _profile_summary()
    return None if data is None else data.get("mfma_util_pct", {}).get(kernel)


def measured_clock(kernel: str):
    """sustained shader clock (GHz) of the kernel's timed step launches from the
    committed counter summary, or None"""
    data = _profile_summary()
    return None if data is None else data.get("sclk_ghz", {}).get(kernel)


def pair_layout(qs, shapes):
    """How a GEMM's quantize calls run: (pair, panels).  Both operands go in one
    mx_quantize_pair launch when they share mode, format and sign mask; a
    transposed or rotated pair writes its codes in the K-panel layout when both
    tensors' rows are whole panels (256 elements for E2M1, 128 for FP8), and the
    GEMM then reads that layout in place (mx_gemm_layout)."""
    pair = len(qs) == 2 and len({(q.kind, q.fmt, q.sign_mask) for q in qs}) == 1
    panels = pair and qs[0].kind != "row" and all(
        shp[0] % (256 if q.fmt == "e2m1" else 128) == 0 for q, shp in zip(qs, shapes))
    return pair, panels


class Step:
    """device buffers and the ordered kernel launches of one step"""

    def __init__(self, mx, torch, seed: int):
        self.mx, self.torch = mx, torch
        self.launches = []  # (name, kind, work, fn)
        dev = torch.device("cuda", 0)

        def bf16(cfg, name):
            bits = workloads.draw_tensor(cfg, name, seed=seed)
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        for ci in CONFIGS:
            cfg = workloads.config(ci)
            tens = {t.name: bf16(cfg, t.name) for t in cfg.tensors}
            qs = cfg.quants
            pair, panels = pair_layout(qs, [tuple(tens[q.tensor].shape) for q in qs])
            ops = {}
            for q in cfg.quants:
                x = tens[q.tensor]
                rows, cols = x.shape
                out_rows, k = (rows, cols) if q.kind == "row" else (cols, rows)
                cshape = ((mx.code_cols(k, q.fmt) // 128, out_rows, 128) if panels
                          else (out_rows, mx.code_cols(k, q.fmt)))
                codes = torch.empty(cshape, dtype=torch.uint8, device=dev)
                scales = torch.empty((out_rows, k // 32), dtype=torch.uint8, device=dev)
                ops[q.name] = (codes, scales, q.fmt)
            if pair:
                # both operands of the GEMM in one launch (mx_quantize_pair)
                q0, q1 = qs
                x0, x1 = tens[q0.tensor], tens[q1.tensor]
                mode = q0.kind + ("_panels" if panels else "")
                fn = (lambda mode=mode, q0=q0, x0=x0, x1=x1, o0=ops[q0.name][:2], o1=ops[q1.name][:2]:
                      mx.quantize_pair(mode, x0, x1, q0.fmt, q0.sign_mask, out0=o0, out1=o1))
                self.launches.append(("%s/%s+%s mx_quantize_pair %s %s" % (cfg.name, q0.name, q1.name, mode, q0.fmt),
                                      "quant", quant_bytes(*x0.shape, q0.fmt) + quant_bytes(*x1.shape, q1.fmt), fn))
            else:
                for q in qs:
                    x = tens[q.tensor]
                    codes, scales = ops[q.name][:2]
                    fn = {"row": lambda x=x, q=q, c=codes, s=scales: mx.quantize(x, q.fmt, out=(c, s)),
                          "transpose": lambda x=x, q=q, c=codes, s=scales: mx.quantize_transpose(x, q.fmt, out=(c, s)),
                          "hadamard": lambda x=x, q=q, c=codes, s=scales: mx.hadamard32_quantize(
                              x, q.fmt, q.sign_mask, out=(c, s))}[q.kind]
                    kname = {"row": "mx_quantize", "transpose": "mx_quantize_transpose",
                             "hadamard": "mx_hadamard32_quantize"}[q.kind]
                    self.launches.append(("%s/%s %s %s" % (cfg.name, q.name, kname, q.fmt), "quant",
                                          quant_bytes(*x.shape, q.fmt), fn))
            for gm in cfg.gemms:
                a, b = ops[gm.a], ops[gm.b]
                out = torch.empty((gm.M, gm.N), dtype=torch.bfloat16 if gm.out == "bf16" else torch.float32,
                                  device=dev)
                fn = (lambda a=a, b=b, out=out: mx.gemm(a[0], a[1], a[2], b[0], b[1], b[2],
                                                        out_dtype=out.dtype, out=out))
                arith = "fp4" if a[2] == "e2m1" and b[2] == "e2m1" else "bf16"
                entry = "mx_gemm_layout" if a[0].dim() == 3 or b[0].dim() == 3 else "mx_gemm"
                self.launches.append(("%s/%s %s %sx%s" % (cfg.name, gm.name, entry, a[2], b[2]), "gemm:" + arith,
                                      2.0 * gm.M * gm.N * gm.K, fn))
        self.flops = sum(w for _, kind, w, _ in self.launches if kind.startswith("gemm"))

    def run(self, events=None, only=None):
        """one step; `events[i]` brackets launch i, or `only` = (i, pair) brackets launch i alone"""
        for i, (_, _, _, fn) in enumerate(self.launches):
            ev = events[i] if events is not None else (only[1] if only is not None and only[0] == i else None)
            if ev is not None:
                ev[0].record()
            fn()
            if ev is not None:
                ev[1].record()


def cpu_model() -> str:
    """the host CPU's model name"""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(seed: int, step_flops: float, launches=None, kernels=None) -> dict:
    """the oracle on a bounded sample of the same step, extrapolated to the
    step; rows per quantize and rows of A per GEMM are sampled.  Per kernel:
    the oracle's extrapolated time and rate, and the GPU kernel's speed-up
    over it (in-step GPU time)."""
    import oracle
    # GEMM rows 128 and 512: enough that the fp64 product, not the operands' dequantization, sets the slope
    qrows, grow_a, grow_b = 512, 128, 512
    t_total = 0.0
    parts, part_s, per_kernel = [], {}, []
    for ci in CONFIGS:
        cfg = workloads.config(ci)
        for q in cfg.quants:
            spec = cfg.tensor(q.tensor)
            x = workloads.draw_tensor(cfg, q.tensor, seed=seed, rows=(0, qrows))
            fn = {"row": lambda: oracle.quantize(x, q.fmt),
                  "transpose": lambda: oracle.quantize_transpose(x, q.fmt),
                  "hadamard": lambda: oracle.hadamard32_quantize(x, q.fmt, q.sign_mask)}[q.kind]
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            t_full = dt * spec.rows / qrows
            t_total += t_full
            part_s[(cfg.name, q.name)] = t_full
            parts.append("%s/%s: %d of %d rows" % (cfg.name, q.name, qrows, spec.rows))
            per_kernel.append({"kernel": "%s/%s %s %s" % (cfg.name, q.name, q.kind, q.fmt), "oracle_s": round(t_full, 4),
                               "oracle_GBps": round(quant_bytes(spec.rows, spec.cols, q.fmt) / t_full / 1e9, 3)})
        for gm in cfg.gemms:
            qa, qb = cfg.quant(gm.a), cfg.quant(gm.b)
            # operands from the oracle's own quantizers (full tensors: the GEMM needs all of B)
            def operand(q):
                x = workloads.draw_tensor(cfg, q.tensor, seed=seed)
                if q.kind == "row":
                    return oracle.quantize(x, q.fmt)
                if q.kind == "transpose":
                    return oracle.quantize_transpose(x, q.fmt)
                return oracle.hadamard32_quantize(x, q.fmt, q.sign_mask)
            A, B = operand(qa), operand(qb)
            times = []
            for r in (grow_a, grow_b):
                t0 = time.perf_counter()
                oracle.gemm(A[0], A[1], qa.fmt, B[0], B[1], qb.fmt, rows=np.arange(r))
                times.append(time.perf_counter() - t0)
            per_row = max(times[1] - times[0], 0.0) / (grow_b - grow_a)
            fixed = max(times[0] - per_row * grow_a, 0.0)
            t_g = fixed + per_row * gm.M
            t_total += t_g
            part_s[(cfg.name, gm.name)] = t_g
            parts.append("%s/%s: GEMM rows %d and %d of %d, linear fit" % (cfg.name, gm.name, grow_a, grow_b, gm.M))
            per_kernel.append({"kernel": "%s/%s gemm %dx%dx%d" % (cfg.name, gm.name, gm.M, gm.N, gm.K),
                               "oracle_s": round(t_g, 3),
                               "oracle_GFLOPs": round(2.0 * gm.M * gm.N * gm.K / t_g / 1e9, 2)})
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    speedups = []
    if launches is not None and kernels is not None:
        # each GPU launch against the oracle time of the quantize calls or GEMM it performs
        for (name, _, _, _), k in zip(launches, kernels):
            cfg_name, rest = name.split("/", 1)
            names = rest.split()[0].split("+")
            t = sum(part_s.get((cfg_name, nm), 0.0) for nm in names)
            if t > 0:
                speedups.append({"kernel": name, "oracle_s": round(t, 4), "gpu_ms": round(k["ms"], 4),
                                 "gpu_over_oracle": round(t / (k["ms"] * 1e-3), 1)})
    return {"value": step_flops / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "; ".join(parts) + "; per-step time extrapolated to %.1f s" % t_total,
            "kernels": per_kernel, "gpu_over_oracle": speedups}


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _time_sequence(torch, launches, reps):
    """median over `reps` passes of each launch's event time and of the whole pass
    (launches run back to back on the current stream; no cache flush in between)"""
    per = [[] for _ in launches]
    whole = []
    for _ in range(reps):
        evs = [_events(torch) for _ in launches]
        w0, w1 = _events(torch)
        w0.record()
        for (_, fn), e in zip(launches, evs):
            e[0].record()
            fn()
            e[1].record()
        w1.record()
        torch.cuda.synchronize()
        for k, e in enumerate(evs):
            per[k].append(e[0].elapsed_time(e[1]))
        whole.append(w0.elapsed_time(w1))
    seq = []
    for _ in range(reps):  # the same pass without per-launch events, for the pass time alone
        w0, w1 = _events(torch)
        w0.record()
        for _, fn in launches:
            fn()
        w1.record()
        torch.cuda.synchronize()
        seq.append(w0.elapsed_time(w1))
    return [float(np.median(p)) for p in per], float(np.median(seq))


def linear_layer(mx, torch, seed: int, reps: int) -> dict:
    """One whole Llama-3.1-8B gate+up linear layer in the MXFP4 recipe (FP4-training
    article on hzrcw.cc, section 02): X, W and dY each quantized once by the
    dual-direction quantizer (row form + transposed or rotated form from one read),
    then Fprop, Dgrad and Wgrad.  The same layer with the six single-direction
    quantize calls is timed beside it; the difference is what the fused quantizer
    saves where it applies.  Passes run back to back (median of `reps`)."""
    cfg = workloads.config(5)
    dev = {t.name: torch.from_numpy(workloads.draw_tensor(cfg, t.name, seed=seed).view(np.int16)).view(
        torch.bfloat16).to("cuda") for t in cfg.tensors}
    ops = {}
    for q in cfg.quants:
        x = dev[q.tensor]
        rows, k = (x.shape[0], x.shape[1]) if q.kind == "row" else (x.shape[1], x.shape[0])
        ops[q.name] = (torch.empty((rows, mx.code_cols(k, q.fmt)), dtype=torch.uint8, device="cuda"),
                       torch.empty((rows, k // 32), dtype=torch.uint8, device="cuda"), q.fmt)
    outs = {g.name: torch.empty((g.M, g.N), dtype=torch.bfloat16 if g.out == "bf16" else torch.float32,
                                device="cuda") for g in cfg.gemms}

    def gemm_launch(g):
        a, b = ops[g.a], ops[g.b]
        return ("%s %dx%dx%d %sx%s" % (g.name, g.M, g.N, g.K, a[2], b[2]),
                lambda: mx.gemm(a[0], a[1], a[2], b[0], b[1], b[2], out_dtype=outs[g.name].dtype, out=outs[g.name]))

    duals, singles, work = [], [], {}
    for src, q_row, q_t in workloads.LAYER_DUALS:
        qr, qt = cfg.quant(q_row), cfg.quant(q_t)
        x = dev[src]
        rot = qt.kind == "hadamard"
        o = ops[q_row][:2] + ops[q_t][:2]
        name = "dual %s %dx%d: %s row + %s %s" % (src, x.shape[0], x.shape[1], qr.fmt, qt.fmt,
                                                   "rotated" if rot else "transposed")
        duals.append((name, lambda x=x, qr=qr, qt=qt, rot=rot, o=o: mx.quantize_dual(
            x, qr.fmt, qt.fmt, rot, 0, out=o)))
        n_el = x.numel()
        work[name] = n_el * (2.0 + (0.5 if qr.fmt == "e2m1" else 1.0) + (0.5 if qt.fmt == "e2m1" else 1.0) + 2 / 32)
        for q in (qr, qt):
            c, sc, _ = ops[q.name]
            fn = {"row": lambda x=x, q=q, c=c, sc=sc: mx.quantize(x, q.fmt, out=(c, sc)),
                  "transpose": lambda x=x, q=q, c=c, sc=sc: mx.quantize_transpose(x, q.fmt, out=(c, sc)),
                  "hadamard": lambda x=x, q=q, c=c, sc=sc: mx.hadamard32_quantize(x, q.fmt, 0, out=(c, sc))}[q.kind]
            nm = "%s %s %s" % (q.name, q.kind, q.fmt)
            singles.append((nm, fn))
            work[nm] = quant_bytes(x.shape[0], x.shape[1], q.fmt)
    gemms = [gemm_launch(g) for g in cfg.gemms]
    for g, (nm, _) in zip(cfg.gemms, gemms):
        work[nm] = 2.0 * g.M * g.N * g.K
    for _ in range(2):  # warm-up
        for _, fn in duals + singles + gemms:
            fn()
    torch.cuda.synchronize()
    t_dual, layer_dual = _time_sequence(torch, duals + gemms, reps)
    t_single, layer_single = _time_sequence(torch, singles + gemms, reps)
    flops = sum(2.0 * g.M * g.N * g.K for g in cfg.gemms)

    def row(name, ms):
        w = work[name]
        if name.startswith(("fprop", "dgrad", "wgrad")):
            tf = w / (ms * 1e-3) / 1e12
            return {"launch": name, "ms": round(ms, 4), "TFLOPs": round(tf, 1), "frac_of_fp4_peak": round(
                tf / PEAK_TFLOPS["fp4"], 4)}
        gb = w / (ms * 1e-3) / 1e9
        return {"launch": name, "ms": round(ms, 4), "GBps": round(gb, 1), "frac_of_hbm_peak": round(gb / PEAK_HBM_GBPS, 4)}

    return {
        "layer": "Llama-3.1-8B gate+up: X [8192x4096], W [28672x4096], dY [8192x28672]; MXFP4 Fprop, Dgrad, "
                 "rotated Wgrad",
        "layer_ms_dual_quantize": round(layer_dual, 4), "layer_ms_single_quantizes": round(layer_single, 4),
        "layer_TFLOPs_dual": round(flops / (layer_dual * 1e-3) / 1e12, 1),
        "quantize_ms_dual": round(sum(t_dual[:len(duals)]), 4),
        "quantize_ms_single": round(sum(t_single[:len(singles)]), 4),
        "launches_dual": [row(n, t) for (n, _), t in zip(duals + gemms, t_dual)],
        "launches_single": [row(n, t) for (n, _), t in zip(singles, t_single)],
        "how": "median of %d back-to-back passes; per-launch figures from event pairs around each launch, "
               "pass times from passes without them" % reps,
    }


def _device_tensor(torch, spec, gen):
    """a bf16 tensor of the recipe's shape and distribution drawn on the device
    (timing input only: the 70B set's host-seeded bytes would take the host
    minutes to draw)"""
    out = torch.empty((spec.rows, spec.cols), dtype=torch.bfloat16, device="cuda")
    chan = None
    if spec.outlier_channels > 0:
        n_out = int(round(spec.outlier_channels * spec.cols))
        chan = torch.randperm(spec.cols, generator=gen, device="cuda")[:n_out]
    for r0 in range(0, spec.rows, 2048):
        r1 = min(spec.rows, r0 + 2048)
        shape = (r1 - r0, spec.cols)
        v = torch.randn(shape, generator=gen, device="cuda")
        if spec.dist == "t3":  # Student-t, 3 degrees of freedom: z / sqrt(chi2_3 / 3)
            chi = sum(torch.randn(shape, generator=gen, device="cuda") ** 2 for _ in range(3))
            v = v / torch.sqrt(chi / 3.0)
        v *= spec.scale
        if chan is not None:
            v[:, chan] *= spec.outlier_factor
        out[r0:r1] = v.to(torch.bfloat16)
    return out


def llama70b_set(mx, torch, seed: int, reps: int = 3) -> dict:
    """The Llama-3.1-70B single-layer linear set at 8192 tokens: each GEMM's
    quantize launches (one pair launch where both operands share a mode, as in
    the step; else two calls) and the GEMM, back to back, per launch (median of
    `reps` passes).  Eight of the nine GEMMs have FP8 operands and run on the bf16
    carrier; they are reported against the bf16 matrix peak it runs on and
    against MXFP8's."""
    cfg = workloads.config(4)
    gen = torch.Generator(device="cuda").manual_seed(seed + 70)
    dev = {t.name: _device_tensor(torch, t, gen) for t in cfg.tensors}
    out, total_ms, total_flops, quant_ms, quant_bytes_ = [], 0.0, 0.0, 0.0, 0.0
    for g in cfg.gemms:
        launches, ops = [], {}
        qs = (cfg.quant(g.a), cfg.quant(g.b))
        pair, panels = pair_layout(qs, [tuple(dev[q.tensor].shape) for q in qs])
        for q in qs:
            x = dev[q.tensor]
            rows, k = (x.shape[0], x.shape[1]) if q.kind == "row" else (x.shape[1], x.shape[0])
            shape = (mx.code_cols(k, q.fmt) // 128, rows, 128) if panels else (rows, mx.code_cols(k, q.fmt))
            c = torch.empty(shape, dtype=torch.uint8, device="cuda")
            sc = torch.empty((rows, k // 32), dtype=torch.uint8, device="cuda")
            ops[q.name] = (c, sc, q.fmt)
            if not pair:
                fn = {"row": lambda x=x, q=q, c=c, sc=sc: mx.quantize(x, q.fmt, out=(c, sc)),
                      "transpose": lambda x=x, q=q, c=c, sc=sc: mx.quantize_transpose(x, q.fmt, out=(c, sc)),
                      "hadamard": lambda x=x, q=q, c=c, sc=sc: mx.hadamard32_quantize(
                          x, q.fmt, q.sign_mask, out=(c, sc))}[q.kind]
                launches.append(("%s %s %s" % (q.name, q.kind, q.fmt), fn, quant_bytes(x.shape[0], x.shape[1], q.fmt)))
        if pair:
            q0, q1 = qs
            mode = q0.kind + ("_panels" if panels else "")
            fn = (lambda mode=mode, q0=q0, x0=dev[q0.tensor], x1=dev[q1.tensor], o0=ops[q0.name][:2],
                  o1=ops[q1.name][:2]: mx.quantize_pair(mode, x0, x1, q0.fmt, q0.sign_mask, out0=o0, out1=o1))
            launches.append(("%s+%s pair %s %s" % (q0.name, q1.name, mode, q0.fmt), fn,
                             sum(quant_bytes(*dev[q.tensor].shape, q.fmt) for q in qs)))
        a, b = ops[g.a], ops[g.b]
        cbuf = torch.empty((g.M, g.N), dtype=torch.bfloat16 if g.out == "bf16" else torch.float32, device="cuda")
        launches.append(("%s gemm" % g.name, lambda a=a, b=b, cbuf=cbuf: mx.gemm(
            a[0], a[1], a[2], b[0], b[1], b[2], out_dtype=cbuf.dtype, out=cbuf), 2.0 * g.M * g.N * g.K))
        for _, fn, _ in launches:
            fn()
        torch.cuda.synchronize()
        t, _ = _time_sequence(torch, [(n, fn) for n, fn, _ in launches], reps)
        gi = len(launches) - 1  # the GEMM; the quantize launches before it
        arith = "fp4" if a[2] == "e2m1" and b[2] == "e2m1" else "bf16"
        tf = launches[gi][2] / (t[gi] * 1e-3) / 1e12
        r = {"gemm": g.name, "M": g.M, "N": g.N, "K": g.K, "formats": "%sx%s" % (a[2], b[2]), "ms": round(t[gi], 4),
             "TFLOPs": round(tf, 1), "arith": arith, "frac": round(tf / PEAK_TFLOPS[arith], 4),
             "quantize": [{"call": launches[k][0], "ms": round(t[k], 4),
                           "GBps": round(launches[k][2] / (t[k] * 1e-3) / 1e9, 1),
                           "frac_of_hbm_peak": round(launches[k][2] / (t[k] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
                          for k in range(gi)]}
        if arith == "bf16":
            r["frac_of_mxfp8_peak"] = round(tf / PEAK_TFLOPS["fp8"], 4)
        out.append(r)
        total_ms += t[gi]
        total_flops += launches[gi][2]
        quant_ms += sum(t[:gi])
        quant_bytes_ += sum(w for _, _, w in launches[:gi])
        del launches, ops, cbuf, a, b
    return {"gemms": out, "gemm_ms_total": round(total_ms, 3),
            "gemm_TFLOPs_aggregate": round(total_flops / (total_ms * 1e-3) / 1e12, 1),
            "quantize_ms_total": round(quant_ms, 3),
            "quantize_GBps_aggregate": round(quant_bytes_ / (quant_ms * 1e-3) / 1e9, 1),
            "inputs": "drawn on the device with the recipe's shapes and distributions (timing only; the parity "
                      "tests use the seeded host draws)",
            "how": "each GEMM after its operands' quantize launches (one pair launch where both share a "
                   "mode), back to back; median of %d passes" % reps}


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError("%s/*%s" % (d, suffix))


def summarize_profiles(trace_dir: str, fetch_dir: str, write_dir: str, clock_dir: str, command: str,
                       out_dir: str = os.path.join(ROOT, "profiles"), mfma_dir: str = None,
                       lds_dir: str = None) -> None:
    """Turn rocprofv3 CSV output (kernel trace with stats; FETCH_SIZE and
    WRITE_SIZE counter passes with --calibrate-copy) into the short summaries
    kept under profiles/: per-kernel average durations, and HBM bytes per
    launch scaled by what the counters read for the 256 MiB copy."""
    stats = _read_csv(_find(trace_dir, "kernel_stats.csv"))
    fetch = _read_csv(_find(fetch_dir, "counter_collection.csv"))
    write = _read_csv(_find(write_dir, "counter_collection.csv"))

    def per_kernel(rows):
        # the step's own launches (before the first cache-filling reduction) where the kernel has
        # any: the extra records after them run some kernels at other shapes
        rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
        first = next((int(r["Dispatch_Id"]) for r in rows if "reduce" in r["Kernel_Name"].lower()), None)
        step, rest = {}, {}
        for r in rows:
            in_step = first is not None and int(r["Dispatch_Id"]) < first
            (step if in_step else rest).setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        out = {k: sum(v) / len(v) for k, v in rest.items()}
        out.update({k: sum(v) / len(v) for k, v in step.items()})
        return out

    f_kib, w_kib = per_kernel(fetch), per_kernel(write)
    copy = [k for k in f_kib if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        raise RuntimeError("no copy kernel in the counter passes (run bench.py with --calibrate-copy)")

    def largest_copy(rows):
        # the 256 MiB calibration copies run last, after every library kernel (earlier copies
        # include dtype conversions of other sizes)
        last_mx = max(int(r["Dispatch_Id"]) for r in rows if "mx::" in r["Kernel_Name"])
        per = {}
        for r in rows:
            if r["Kernel_Name"] in copy and int(r["Dispatch_Id"]) > last_mx:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not per:
            raise RuntimeError("no calibration copy after the library's kernels (run bench.py with --calibrate-copy)")
        return max(per.values())

    known_kib = 256 * 1024.0
    f_copy, w_copy = largest_copy(fetch), largest_copy(write)
    f_scale, w_scale = known_kib / f_copy, known_kib / w_copy
    os.makedirs(out_dir, exist_ok=True)
    lines = ["# rocprofv3 kernel trace: %s" % WORKLOAD, "",
             "Command (run from the repository root on an MI355X):", "", "    " + command[0], "",
             "The library's kernels only (torch's kernels that fill the cache before each lone launch, "
             "and its copies, are left out; share is of the library's kernel time). Calls count the "
             "launches inside the step and the lone launches after a clean cache fill.", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    mine = [r for r in stats if "mx::" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in mine) or 1.0
    for r in sorted(mine, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
            r["Name"], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, 100.0 * float(r["TotalDurationNs"]) / total))
    # The same dispatches split by phase: every library launch before the first
    # cache-filling reduction belongs to the warm-up, instrumented and timed
    # steps (each kernel's last `steps` of them are the timed ones); the rest
    # are the lone launches and the extra records.
    trace = sorted(_read_csv(_find(trace_dir, "kernel_trace.csv")), key=lambda r: int(r["Dispatch_Id"]))
    first_flush = next((int(r["Dispatch_Id"]) for r in trace if "reduce" in r["Kernel_Name"].lower()), None)
    steps, warmup = (int(a) for a in re.search(r"--steps (\d+) --warmup (\d+)", command[0]).groups())
    step_calls = {}
    for r in trace:
        if "mx::" in r["Kernel_Name"] and (first_flush is None or int(r["Dispatch_Id"]) < first_flush):
            step_calls.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "Inside the steps only (each kernel's last %d launches before the first cache fill: "
              "bench.py runs %d warm-up steps, %d steps per launch with events around that launch alone, "
              "the %d timed steps, then %d steps each bracketed by one event pair, whose launches these "
              "are):" % (steps, warmup, steps, steps, steps), "",
              "| kernel | timed calls | average (us) |", "|---|---|---|"]
    for k, d in sorted(step_calls.items(), key=lambda kv: -sum(kv[1])):
        timed = d[-steps:]
        lines.append("| `%s` | %d | %.1f |" % (k, len(timed), sum(timed) / len(timed)))
    with open(os.path.join(out_dir, "kernel_trace_%s.md" % WORKLOAD), "w") as f:
        f.write("\n".join(lines) + "\n")

    kern = {}
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE): %s" % WORKLOAD, "",
             "Commands (run from the repository root on an MI355X), one counter per run:", "",
             "    " + command[1], "    " + command[2], "",
             "Calibration: a plain 256 MiB device copy (`%s`) reads FETCH_SIZE = %.0f KiB and "
             "WRITE_SIZE = %.0f KiB per dispatch for 262144 KiB read and written, so counter KiB are "
             "scaled by %.4f (fetch) and %.4f (write). Each kernel's figure is the mean over its launches "
             "inside the step (for a kernel the step runs at several sizes, such as the row quantizers, "
             "the mean over those); kernels only the extra records run are averaged over their calls." % (
                 copy[0], f_copy, w_copy, f_scale, w_scale),
             "", "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (MB) | written (MB) |", "|---|---|---|---|---|"]
    for k in f_kib:
        if k in copy or "mx::" not in k:
            continue
        rd, wr = f_kib[k] * f_scale * 1024, w_kib.get(k, 0.0) * w_scale * 1024
        kern[k] = {"read_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr}
        lines.append("| `%s` | %.0f | %.0f | %.1f | %.1f |" % (k, f_kib[k], w_kib.get(k, 0.0), rd / 1e6, wr / 1e6))
    with open(os.path.join(out_dir, "hbm_traffic_%s.md" % WORKLOAD), "w") as f:
        f.write("\n".join(lines) + "\n")
    # sustained shader clock of each library kernel over its timed step launches (dispatches
    # before the first cache-filling reduction, after the warm-up share): busy cycles summed over
    # the dies / (dies x dispatch time)
    rows = sorted(_read_csv(_find(clock_dir, "counter_collection.csv")), key=lambda r: int(r["Dispatch_Id"]))
    first_flush_c = next((int(r["Dispatch_Id"]) for r in rows if "reduce" in r["Kernel_Name"].lower()), None)
    csteps = int(re.search(r"--steps (\d+)", command[3]).group(1))
    per = {}
    for r in rows:
        if r["Counter_Name"] != "GRBM_GUI_ACTIVE" or "mx::" not in r["Kernel_Name"]:
            continue
        if first_flush_c is not None and int(r["Dispatch_Id"]) >= first_flush_c:
            continue
        dt = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if dt > 0:
            per.setdefault(r["Kernel_Name"], []).append((float(r["Counter_Value"]) / (XCDS * dt), dt))
    sclk = {}
    lines = ["# Sustained shader clock per kernel (rocprofv3 GRBM_GUI_ACTIVE): %s" % WORKLOAD, "",
             "Command (run from the repository root on an MI355X):", "", "    " + command[3], "",
             "GRBM_GUI_ACTIVE sums the busy cycles of the %d dies; clock = value / (%d x dispatch time), "
             "averaged over the timed step launches (each kernel's last %d before the first cache fill). "
             "The dense peaks assume %.1f GHz. Kernels whose launches average under %d us are left out: "
             "their counts include busy cycles outside the dispatch window (they read above the %.1f GHz "
             "maximum)." % (XCDS, XCDS, csteps, PEAK_SCLK_GHZ, MIN_CLOCK_US, PEAK_SCLK_GHZ), "",
             "| kernel | timed launches | average (us) | clock (GHz) |", "|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: kv[0]):
        timed = v[-csteps:]
        us = sum(t for _, t in timed) / len(timed) / 1e3
        if us < MIN_CLOCK_US:
            continue
        sclk[k] = sum(c for c, _ in timed) / len(timed)
        lines.append("| `%s` | %d | %.1f | %.2f |" % (k, len(timed), us, sclk[k]))
    with open(os.path.join(out_dir, "sclk_%s.md" % WORKLOAD), "w") as f:
        f.write("\n".join(lines) + "\n")
    # MFMA busy %: rocprofv3's MfmaUtil, the MFMA busy cycles summed over the SIMDs over
    # (busy cycles of the busiest die x SIMDs), averaged over the kernel's timed step launches
    mfma = {}
    if mfma_dir is not None:
        rows = sorted(_read_csv(_find(mfma_dir, "counter_collection.csv")), key=lambda r: int(r["Dispatch_Id"]))
        first_m = next((int(r["Dispatch_Id"]) for r in rows if "reduce" in r["Kernel_Name"].lower()), None)
        msteps = int(re.search(r"--steps (\d+)", command[4]).group(1))
        perm = {}
        for r in rows:
            if r["Counter_Name"] != "MfmaUtil" or "mx::" not in r["Kernel_Name"]:
                continue
            if first_m is not None and int(r["Dispatch_Id"]) >= first_m:
                continue
            perm.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        lines = ["# MFMA busy per kernel (rocprofv3 MfmaUtil): %s" % WORKLOAD, "",
                 "Command (run from the repository root on an MI355X):", "", "    " + command[4], "",
                 "MfmaUtil = MFMA busy cycles summed over the SIMDs / (busy cycles of the busiest die x SIMD "
                 "count) x 100, averaged over each kernel's timed step launches (its last %d before the first "
                 "cache fill). Kernels without matrix instructions read 0 and are left out." % msteps, "",
                 "| kernel | timed launches | MFMA busy (%) |", "|---|---|---|"]
        for k, v in sorted(perm.items(), key=lambda kv: kv[0]):
            timed = v[-msteps:]
            util = sum(timed) / len(timed)
            if util <= 0.0:
                continue
            mfma[k] = util
            lines.append("| `%s` | %d | %.1f |" % (k, len(timed), util))
        with open(os.path.join(out_dir, "mfma_util_%s.md" % WORKLOAD), "w") as f:
            f.write("\n".join(lines) + "\n")
    # LDS bank conflicts: cycles the LDS stalled on bank conflicts over the cycles it was busy with
    # indexed accesses (both summed over the shader engines), over each kernel's timed step launches
    lds = {}
    if lds_dir is not None:
        rows = sorted(_read_csv(_find(lds_dir, "counter_collection.csv")), key=lambda r: int(r["Dispatch_Id"]))
        first_l = next((int(r["Dispatch_Id"]) for r in rows if "reduce" in r["Kernel_Name"].lower()), None)
        lsteps = int(re.search(r"--steps (\d+)", command[5]).group(1))
        perl = {}
        for r in rows:
            if "mx::" not in r["Kernel_Name"] or (first_l is not None and int(r["Dispatch_Id"]) >= first_l):
                continue
            d = perl.setdefault(r["Kernel_Name"], {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        lines = ["# LDS bank conflicts per kernel (rocprofv3 SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE): %s" % WORKLOAD,
                 "", "Command (run from the repository root on an MI355X):", "", "    " + command[5], "",
                 "Both counters are cycles summed over the shader engines. Conflict share = bank-conflict stall "
                 "cycles / cycles the LDS was busy with indexed accesses, over each kernel's timed step launches "
                 "(its last %d before the first cache fill). Kernels without LDS traffic are left out." % lsteps, "",
                 "| kernel | timed launches | LDS busy (Mcycles per launch) | conflict stalls (Mcycles per launch) "
                 "| conflict share |", "|---|---|---|---|---|"]
        for k, disp in sorted(perl.items(), key=lambda kv: kv[0]):
            timed = [disp[i] for i in sorted(disp)][-lsteps:]
            act = sum(d.get("SQ_LDS_IDX_ACTIVE", 0.0) for d in timed) / len(timed)
            con = sum(d.get("SQ_LDS_BANK_CONFLICT", 0.0) for d in timed) / len(timed)
            if act <= 0:
                continue
            lds[k] = 100.0 * con / act
            lines.append("| `%s` | %d | %.2f | %.3f | %.2f%% |" % (k, len(timed), act / 1e6, con / 1e6, lds[k]))
        with open(os.path.join(out_dir, "lds_bank_conflicts_%s.md" % WORKLOAD), "w") as f:
            f.write("\n".join(lines) + "\n")
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump({"source_sha": kernel_source_sha(), "workload": WORKLOAD, "fetch_scale": f_scale,
                   "write_scale": w_scale, "kernels": kern, "sclk_ghz": sclk, "mfma_util_pct": mfma,
                   "lds_conflict_pct": lds, "commands": command[1:]}, f, indent=1)


def ablation(mx, torch, seed: int) -> dict:
    """Numerical proxy for the weight-gradient recipe (FP4-training article
    on hzrcw.cc, sections 02-03): dW = dY^T X over 8192 tokens with dY
    heavy-tailed (1e-3 * Student-t, nu = 3, as the down-projection gradient)
    and X ~ N(0, 1), through the library's quantizers and GEMM, against the
    fp64 product of the same bf16 inputs.  Relative Frobenius error of:
    MXFP4 without rotation, with the fixed-sign rotation (two masks), with
    random signs drawn anew for each of 8 steps, with stochastic rounding
    (a new seed each step) with and without the fixed rotation, and MXFP8
    without rotation.  For the randomised variants the error of the 8-step
    average dW is given too: it falls below the single-step error only
    where the steps' errors vary and cancel."""
    cfg = workloads.config(3)
    dy = workloads.draw_tensor(cfg, "dY", seed=seed)[:, :1024]
    x = workloads.draw_tensor(cfg, "X", seed=seed)[:, :512]
    f64 = lambda b: workloads.bf16_bits_to_f32(b).astype(np.float64)
    ref = f64(dy).T @ f64(x)
    nref = np.linalg.norm(ref)
    dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to("cuda")
    dyd, xd = dev(dy), dev(x)

    def dw_mat(qa, qb, fmt):
        c = mx.gemm(qa[0], qa[1], fmt, qb[0], qb[1], fmt, out_dtype=torch.float32)
        return c.cpu().numpy().astype(np.float64)

    def dw(qa, qb, fmt):
        return float(np.linalg.norm(dw_mat(qa, qb, fmt) - ref) / nref)

    def steps_of(make, n=8):
        """relative error of each of n steps, and of their average dW (which
        shrinks only where the steps' errors differ and cancel)"""
        mats = [make(i) for i in range(n)]
        errs = [float(np.linalg.norm(m - ref) / nref) for m in mats]
        return {"mean": float(np.mean(errs)), "min": float(np.min(errs)), "max": float(np.max(errs)),
                "error_of_the_%d_step_average" % n: float(np.linalg.norm(np.mean(mats, axis=0) - ref) / nref)}

    out = {"shape": "dW[1024x512] = dY[8192x1024]^T X[8192x512]", "metric": "||dW - dW_fp64||_F / ||dW_fp64||_F"}
    out["mxfp4_no_rotation"] = dw(mx.quantize_transpose(dyd, "e2m1"), mx.quantize_transpose(xd, "e2m1"), "e2m1")
    for mask in (0, 0x9E3779B9):
        out["mxfp4_fixed_rotation_mask_%08x" % mask] = dw(mx.hadamard32_quantize(dyd, "e2m1", mask),
                                                          mx.hadamard32_quantize(xd, "e2m1", mask), "e2m1")
    rng = np.random.default_rng(seed + 1)
    errs = []
    for _ in range(8):
        mask = int(rng.integers(0, 1 << 32))
        errs.append(dw(mx.hadamard32_quantize(dyd, "e2m1", mask), mx.hadamard32_quantize(xd, "e2m1", mask), "e2m1"))
    out["mxfp4_random_sign_rotation_8_steps"] = {"mean": float(np.mean(errs)), "min": float(np.min(errs)),
                                                 "max": float(np.max(errs))}
    # stochastic rounding of both operands, a fresh seed per step (the two operands draw from
    # disjoint parts of the stream through different seeds)
    out["mxfp4_stochastic_rounding_8_steps"] = steps_of(lambda i: dw_mat(
        mx.quantize_transpose_sr(dyd, "e2m1", 2 * i + 1), mx.quantize_transpose_sr(xd, "e2m1", 2 * i + 2), "e2m1"))
    out["mxfp4_fixed_rotation_and_stochastic_rounding_8_steps"] = steps_of(lambda i: dw_mat(
        mx.quantize_transpose_sr(dyd, "e2m1", 2 * i + 1, True, 0),
        mx.quantize_transpose_sr(xd, "e2m1", 2 * i + 2, True, 0), "e2m1"))
    out["mxfp8_e4m3_no_rotation"] = dw(mx.quantize_transpose(dyd, "e4m3"), mx.quantize_transpose(xd, "e4m3"), "e4m3")
    return out


def write_ablation_summary(abl: dict, path: str, seed: int) -> None:
    """the ablation's table as markdown, with the command that made it"""
    lines = ["# Weight-gradient recipe ablation (dW error through the library)", "",
             "Command (run from the repository root on an MI355X):", "",
             "    python3 bench.py --ablation --seed %d --ablation-summary %s" % (seed, os.path.relpath(path, ROOT)), "",
             "%s; metric %s, against the fp64 product of the same bf16 inputs. dY = 1e-3 x Student-t (3 degrees of "
             "freedom), X ~ N(0, 1), seeded synthetic data (a numerical proxy, not training)." % (
                 abl["shape"], abl["metric"]), "",
             "| recipe | relative error, one step | 8 steps: min / max | error of the 8-step average |",
             "|---|---|---|---|"]
    for k, v in abl.items():
        if k in ("shape", "metric"):
            continue
        if isinstance(v, dict):
            avg = next((x for kk, x in v.items() if kk.startswith("error_of")), None)
            lines.append("| %s | %.4f (mean) | %.4f / %.4f | %s |" % (
                k.replace("_", " "), v["mean"], v["min"], v["max"], "%.4f" % avg if avg is not None else "-"))
        else:
            lines.append("| %s | %.4f | - | (same) |" % (k.replace("_", " "), v))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def kernel_symbol(name: str) -> str:
    """the kernel symbol a bench launch name runs (GEMMs; other names are returned as they are)"""
    if "mx_gemm" in name:
        fa, fb = name.split()[-1].split("x")
        code = {"e4m3": 0, "e5m2": 1, "e2m1": 2}
        out = "true" if "/Y " in name else "false"
        mode = 0 if fa == fb == "e2m1" else 1
        return "void mx::(anonymous namespace)::pipe::k_gemm_pipe<%d, %d, %s, %d>(mx::GemmArgs)" % (
            code[fa], code[fb], out, mode)
    return name


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=workloads.DEFAULT_SEED)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave out the whole-layer and Llama-3.1-70B sections (profiling runs)")
    ap.add_argument("--iso-reps", type=int, default=50, help="lone launches per kernel (median)")
    ap.add_argument("--kernels", action="store_true", help="also print the per-kernel table to stderr")
    ap.add_argument("--ablation", action="store_true",
                    help="only the weight-gradient rotation ablation (dW error of the Wgrad recipes)")
    ap.add_argument("--summarize-profiles", nargs="+", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 CSV output (TRACE FETCH WRITE CLOCK [MFMA [LDS]] "
                         "directories) and exit")
    ap.add_argument("--ablation-summary", metavar="PATH",
                    help="with --ablation: also write the table as markdown to PATH")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 256 MiB device copy three times (HBM counter calibration)")
    args = ap.parse_args()
    if args.summarize_profiles:
        if len(args.summarize_profiles) not in (4, 5, 6):
            ap.error("--summarize-profiles takes the TRACE, FETCH, WRITE, CLOCK and optionally MFMA and LDS "
                     "directories")
        d = args.summarize_profiles
        summarize_profiles(*d[:4], command=PROFILE_COMMANDS, mfma_dir=d[4] if len(d) >= 5 else None,
                           lds_dir=d[5] if len(d) == 6 else None)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: the hot path runs on a single MI355X and the library "
              "has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import precision_block_amax_amd as mx
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    mx.lib()
    torch.cuda.set_device(0)

    if args.ablation:
        abl = ablation(mx, torch, args.seed)
        print(json.dumps({"ablation": abl}), flush=True)
        if args.ablation_summary:
            write_ablation_summary(abl, args.ablation_summary, args.seed)
        return 0

    print("bench: building inputs", file=sys.stderr, flush=True)
    step = Step(mx, torch, args.seed)
    torch.cuda.synchronize()
    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # Per-kernel times inside the step: for each launch, `steps` steps in which HIP events
    # (on the stream it runs on: torch's current stream, which the binding passes to the
    # library) bracket that launch alone, so no other launch's events sit in the step.
    # The median names the dominant kernel; the timed steps then bracket it alone.
    n = len(step.launches)
    new_ev = lambda: [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
    in_step = []
    for i in range(n):
        evs = [new_ev() for _ in range(args.steps)]
        for s_ in range(args.steps):
            step.run(only=(i, evs[s_]))
        torch.cuda.synchronize()
        in_step.append([e[0].elapsed_time(e[1]) for e in evs])
    in_step_med = [float(np.median(t)) for t in in_step]
    dom_i = int(np.argmax(in_step_med))
    dom_events = [new_ev() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step.run(only=(dom_i, dom_events[s_]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dom_t = [e[0].elapsed_time(e[1]) for e in dom_events]
    dom_ms = float(np.mean(dom_t))
    print("bench: timed %d steps, %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr, flush=True)
    # the spread of single steps: `steps` more steps, each bracketed by one event pair
    step_events = [new_ev() for _ in range(args.steps)]
    for s_ in range(args.steps):
        step_events[s_][0].record()
        step.run()
        step_events[s_][1].record()
    torch.cuda.synchronize()
    step_t = np.array([e[0].elapsed_time(e[1]) for e in step_events])

    # Each kernel again on its own: the last-level cache (256 MB) is first
    # filled with clean lines by reading a 512 MiB buffer, so the kernel
    # neither finds its inputs cached nor pays for writing back dirty lines
    # left by the previous kernel (inside the step a quantizer that follows a
    # GEMM does, which can halve its read rate).  Median of `iso_reps` calls.
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1, dtype=torch.int64, device="cuda")

    def alone(fn, reps=args.iso_reps):
        ts = []
        for _ in range(reps):
            sink.copy_(flush.view(torch.int64).sum().view(1))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    isolated = [alone(fn) for (_, _, _, fn) in step.launches]

    # The fused dual-direction quantizer (one read, row form + rotated
    # transposed form) on the down-projection output gradient, against the
    # two single-direction calls it replaces; each alone, clean cache.
    cfg3 = workloads.config(3)
    dy = torch.from_numpy(workloads.draw_tensor(cfg3, "dY", seed=args.seed).view(np.int16)).view(
        torch.bfloat16).to("cuda")
    outs = mx.quantize_dual(dy, "e2m1", "e2m1", True, 0)
    r_out, t_out = outs[:2], outs[2:]
    t_dual = alone(lambda: mx.quantize_dual(dy, "e2m1", "e2m1", True, 0, out=outs))
    t_row = alone(lambda: mx.quantize(dy, "e2m1", out=r_out))
    t_rot = alone(lambda: mx.hadamard32_quantize(dy, "e2m1", 0, out=t_out))
    p_outs = mx.quantize_dual(dy, "e2m1", "e2m1", True, 0, layout="panels")
    t_pan = alone(lambda: mx.quantize_dual(dy, "e2m1", "e2m1", True, 0, out=p_outs, layout="panels"))
    n_el = dy.numel()
    dual_bytes = n_el * (2.0 + 2 * (0.5 + 1.0 / 32))
    fused_dual = {"tensor": "%s/dY %dx%d" % (cfg3.name, dy.shape[0], dy.shape[1]), "formats": "e2m1 row + e2m1 rotated",
                  "ms": round(t_dual, 4), "GBps": round(dual_bytes / (t_dual * 1e-3) / 1e9, 1),
                  "frac_of_hbm_peak": round(dual_bytes / (t_dual * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                  "separate_ms": round(t_row + t_rot, 4), "speedup": round((t_row + t_rot) / t_dual, 3),
                  "k_panels": {"ms": round(t_pan, 4),
                               "frac_of_hbm_peak": round(dual_bytes / (t_pan * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                               "how": "mx_quantize_dual_panels: both forms' codes in the K-panel layout"}}
    del dy, outs, r_out, t_out, p_outs

    # The stochastic-rounding variant of the rotated gradient quantizer (the
    # ablation's randomised cast; Philox words generated in the kernel) against
    # the round-to-nearest kernel on the same gradient, each alone.
    dy = torch.from_numpy(workloads.draw_tensor(cfg3, "dY", seed=args.seed).view(np.int16)).view(
        torch.bfloat16).to("cuda")
    sr_out = mx.quantize_transpose_sr(dy, "e2m1", 1, True, 0)
    t_sr = alone(lambda: mx.quantize_transpose_sr(dy, "e2m1", 1, True, 0, out=sr_out))
    t_rn = alone(lambda: mx.hadamard32_quantize(dy, "e2m1", 0, out=sr_out))
    sr_bytes = quant_bytes(dy.shape[0], dy.shape[1], "e2m1")
    stochastic_rounding = {"tensor": "%s/dY %dx%d" % (cfg3.name, dy.shape[0], dy.shape[1]),
                           "format": "e2m1, rotated", "ms": round(t_sr, 4),
                           "GBps": round(sr_bytes / (t_sr * 1e-3) / 1e9, 1),
                           "nearest_rounding_ms": round(t_rn, 4), "slowdown": round(t_sr / t_rn, 3)}
    del dy, sr_out

    # One rank's share of an FSDP2 MXFP8 weight all-gather: quantize its slab
    # of gate/up weight rows (1/8 of dim 0) to E4M3 into its gather-ready
    # payload (rows of [codes | scales], mx_quantize_strided); the payload it
    # contributes to the gather is 1.03 bytes per element instead of bf16's 2.
    # The GEMM on the gathered payload (the whole weight, read in place through
    # mx_gemm_strided) is timed against the same GEMM on dense operands.
    cfg2 = workloads.config(2)
    wfull = workloads.draw_tensor(cfg2, "W", seed=args.seed)
    slab_rows = wfull.shape[0] // 8
    wdev = torch.from_numpy(wfull.view(np.int16)).view(torch.bfloat16).to("cuda")
    del wfull
    slab = wdev[:slab_rows]
    payload = mx.fsdp_payload(slab, "e4m3")
    t_slab = alone(lambda: mx.fsdp_payload(slab, "e4m3", out=payload))
    K2 = slab.shape[1]
    width = mx.payload_width(K2, "e4m3")
    gathered = torch.cat([mx.fsdp_payload(wdev[r * slab_rows:(r + 1) * slab_rows], "e4m3") for r in range(8)])
    pc, ps = mx.payload_views(gathered, K2, "e4m3")
    qw_dense = mx.quantize(wdev, "e4m3")
    xq = mx.quantize(torch.from_numpy(workloads.draw_tensor(cfg2, "X", seed=args.seed).view(np.int16)).view(
        torch.bfloat16).to("cuda"), "e4m3")
    yb = torch.empty((xq[0].shape[0], wdev.shape[0]), dtype=torch.bfloat16, device="cuda")
    t_g_payload = alone(lambda: mx.gemm(xq[0], xq[1], "e4m3", pc, ps, "e4m3", out_dtype=torch.bfloat16, out=yb), 10)
    t_g_dense = alone(lambda: mx.gemm(xq[0], xq[1], "e4m3", qw_dense[0], qw_dense[1], "e4m3",
                                      out_dtype=torch.bfloat16, out=yb), 10)
    nb = slab.numel()
    fsdp_shard = {"slab": "%s/W rows 0..%d of %d (one of 8 ranks)" % (cfg2.name, slab_rows, slab_rows * 8),
                  "format": "e4m3", "layout": "rows of [codes %d B | scales %d B], stride %d B" % (
                      K2, K2 // 32, width),
                  "ms": round(t_slab, 4),
                  "GBps": round(slab_rows * K2 * (2.0 + width / K2) / (t_slab * 1e-3) / 1e9, 1),
                  "gather_bytes": slab_rows * width, "gather_bytes_bf16": nb * 2.0,
                  "gather_ratio": round(width / (2.0 * K2), 4),
                  "gemm_on_gathered_payload_ms": round(t_g_payload, 4), "gemm_on_dense_operands_ms": round(t_g_dense, 4)}
    del slab, payload, gathered, pc, ps, qw_dense, xq, yb, wdev

    # The full MXFP4 recipe and the mixed-format GEMMs at the gate/up layer's
    # shapes, each alone with a clean cache: Dgrad in FP4 (dX = dY W through
    # the transposed weight, K = 28672), FP8 activations x FP4 weights, the
    # E5M2-gradient Dgrad of the MXFP8 recipe, and an FP4 GEMM whose M and N
    # are not multiples of the 256 x 256 tile.  dY here is seeded Gaussian
    # noise of scale 1e-3 drawn on the device (a timing input only).
    gen = torch.Generator(device="cuda").manual_seed(args.seed)
    dy = (torch.randn((8192, 28672), generator=gen, device="cuda") * 1e-3).to(torch.bfloat16)
    xg = torch.from_numpy(workloads.draw_tensor(cfg2, "X", seed=args.seed).view(np.int16)).view(torch.bfloat16).to("cuda")
    wg = torch.from_numpy(workloads.draw_tensor(cfg2, "W", seed=args.seed).view(np.int16)).view(torch.bfloat16).to("cuda")
    recipe = {}

    def rec(name, a, fa, b, fb, out_dtype, peak_key):
        M, N, K = a[0].shape[0], b[0].shape[0], a[1].shape[1] * 32
        c = torch.empty((M, N), dtype=out_dtype, device="cuda")
        t = alone(lambda: mx.gemm(a[0], a[1], fa, b[0], b[1], fb, out_dtype=out_dtype, out=c))
        tf = 2.0 * M * N * K / (t * 1e-3) / 1e12
        r = {"M": M, "N": N, "K": K, "formats": "%sx%s" % (fa, fb), "ms": round(t, 4), "TFLOPs": round(tf, 1),
             "peak": PEAK_TFLOPS[peak_key], "frac": round(tf / PEAK_TFLOPS[peak_key], 4)}
        if peak_key == "bf16":
            r["frac_of_mxfp8_peak"] = round(tf / PEAK_TFLOPS["fp8"], 4)
        recipe[name] = r

    q_dy4 = mx.quantize(dy, "e2m1")
    q_wt4 = mx.quantize_transpose(wg, "e2m1")
    rec("dgrad_fp4 dX = dY W", q_dy4, "e2m1", q_wt4, "e2m1", torch.bfloat16, "fp4")
    del q_dy4
    q_x8 = mx.quantize(xg, "e4m3")
    q_w4 = mx.quantize(wg, "e2m1")
    rec("fprop_e4m3_x_e2m1 Y = X W^T", q_x8, "e4m3", q_w4, "e2m1", torch.bfloat16, "bf16")
    # The carrier's exact per-block path: a tile any of whose rows mixes an
    # all-zero block (scale byte 0) with normal blocks goes to the second
    # kernel.  The same 8192 x 6144 x 4096 E4M3 GEMM once with the workload's
    # activations and once with their first 32 columns zeroed, which puts one
    # all-zero block in every row of X and sends every tile there.
    q_w8 = mx.quantize(wg[:6144], "e4m3")
    rec("fprop_e4m3 8192x6144x4096", q_x8, "e4m3", q_w8, "e4m3", torch.bfloat16, "bf16")
    xz = xg.clone()
    xz[:, :32] = 0
    q_xz = mx.quantize(xz, "e4m3")
    rec("fprop_e4m3 8192x6144x4096, one all-zero block per row of X", q_xz, "e4m3", q_w8, "e4m3",
        torch.bfloat16, "bf16")
    del q_x8, q_w8, q_xz, xz
    q_dy5 = mx.quantize(dy, "e5m2")
    q_wt8 = mx.quantize_transpose(wg, "e4m3")
    rec("dgrad_e5m2_x_e4m3 dX = dY W", q_dy5, "e5m2", q_wt8, "e4m3", torch.bfloat16, "bf16")
    del q_dy5, q_wt8
    q_x4 = mx.quantize(xg, "e2m1")
    rec("fprop_fp4_tails 8000x28000", (q_x4[0][:8000], q_x4[1][:8000]), "e2m1",
        (q_w4[0][:28000], q_w4[1][:28000]), "e2m1", torch.bfloat16, "fp4")
    del q_x4, q_w4, q_wt4, dy, xg, wg

    # Achievable HBM rate for context: a plain device copy, alone with a clean
    # cache, at the size of the 8192 x 4096 activation (64 MiB -> 64 MiB, the
    # small quantizers' volume) and of the 28672 x 4096 weight (224 MiB).
    hbm_copy = {}
    for mib in (64, 224):
        src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        t = alone(lambda: dst.copy_(src))
        gbps = 2.0 * (mib << 20) / (t * 1e-3) / 1e9
        hbm_copy["%dMiB" % mib] = {"ms": round(t, 4), "GBps": round(gbps, 1),
                                   "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        del src, dst
    del flush

    extra = {}
    if not args.no_extra:
        print("bench: whole gate/up linear layer", file=sys.stderr, flush=True)
        extra["llama31_8b_gateup_layer_mxfp4"] = linear_layer(mx, torch, args.seed, args.iso_reps)
        print("bench: Llama-3.1-70B layer set", file=sys.stderr, flush=True)
        extra["llama31_70b_layer_linear_set"] = llama70b_set(mx, torch, args.seed)

    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    kernels = []
    for i, (name, kind, work, _) in enumerate(step.launches):
        # median of the kernel's in-step samples; the dominant kernel: its events in the timed steps
        ms = float(np.median(dom_t)) if i == dom_i else in_step_med[i]
        iso = isolated[i]
        if kind == "quant":
            ach, iach = work / (ms * 1e-3) / 1e9, work / (iso * 1e-3) / 1e9
            kernels.append({"kernel": name, "ms": ms, "bound": "hbm", "achieved": ach, "unit": "GB/s",
                            "peak": PEAK_HBM_GBPS, "frac": ach / PEAK_HBM_GBPS, "work": work,
                            "ms_p10_p90": spread(dom_t if i == dom_i else in_step[i]),
                            "isolated": {"ms": iso, "achieved": iach, "frac": iach / PEAK_HBM_GBPS}})
        else:
            arith = kind.split(":")[1]
            ach, iach = work / (ms * 1e-3) / 1e12, work / (iso * 1e-3) / 1e12
            k = {"kernel": name, "ms": ms, "bound": "mfma", "achieved": ach, "unit": "TFLOP/s",
                 "peak": PEAK_TFLOPS[arith], "frac": ach / PEAK_TFLOPS[arith], "arith": arith, "work": work,
                 "ms_p10_p90": spread(dom_t if i == dom_i else in_step[i]),
                 "isolated": {"ms": iso, "achieved": iach, "frac": iach / PEAK_TFLOPS[arith]}}
            if arith == "bf16":  # MXFP8 operands carried as bf16: also against the MXFP8 peak
                k["frac_of_mxfp8_peak"] = ach / PEAK_TFLOPS["fp8"]
            kernels.append(k)

    dom = kernels[dom_i]
    traffic = measured_traffic(kernel_symbol(dom["kernel"]))
    # achieved: the dominant kernel's algorithmic flops over its AVERAGE event duration in the timed steps
    dom_ach = dom["work"] / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": dom["bound"], "achieved": round(dom_ach, 3), "peak": dom["peak"],
                "unit": dom["unit"], "frac": round(dom_ach / dom["peak"], 4), "traffic": traffic, "kernel": dom["kernel"],
                "launch_ms_mean": round(dom_ms, 4), "launch_ms_median": round(float(np.median(dom_t)), 4),
                "timed_launches": len(dom_t)}
    sclk = measured_clock(kernel_symbol(dom["kernel"]))
    if sclk is not None:  # the profiled run's sustained clock: the peak the kernel could reach at it
        roofline["sclk_ghz"] = round(sclk, 3)
        roofline["frac_of_clock_adjusted_peak"] = round(roofline["frac"] * PEAK_SCLK_GHZ / sclk, 4)
    mfma_util = measured_mfma_util(kernel_symbol(dom["kernel"]))
    if mfma_util is not None:  # the profiled run's MFMA busy share of the SIMD cycles
        roofline["mfma_busy_pct"] = round(mfma_util, 1)
    q = [k for k in kernels if k["bound"] == "hbm"]
    quant_gbps = sum(k["work"] for k in q) / (sum(k["ms"] for k in q) * 1e-3) / 1e9
    quant_gbps_iso = sum(k["work"] for k in q) / (sum(k["isolated"]["ms"] for k in q) * 1e-3) / 1e9

    value = step.flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": "MX-GEMM TFLOPS & quantize GB/s at Llama-3.1-8B shapes, % of MI355X peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "step_ms": {"median": round(float(np.median(step_t)), 4), "p10": round(float(np.percentile(step_t, 10)), 4),
                    "p90": round(float(np.percentile(step_t, 90)), 4), "min": round(float(step_t.min()), 4),
                    "max": round(float(step_t.max()), 4), "steps": int(step_t.size),
                    "how": "a further pass of `steps` steps, each bracketed by one event pair"},
        "dtype": "mxfp8/mxfp4 operands, fp32 accumulate", "data": "synthetic",
        "config": {"workload": WORKLOAD, "global_batch": 8192, "seq_len": 8192, "parallelism": "none",
                   "gemms": [k["kernel"] for k in kernels if k["bound"] == "mfma"]},
        "roofline": roofline,
        "quantize_GBps": round(quant_gbps, 1), "quantize_frac_of_hbm_peak": round(quant_gbps / PEAK_HBM_GBPS, 4),
        "quantize_GBps_isolated": round(quant_gbps_iso, 1),
        "fused_dual": fused_dual,
        "fsdp_shard": fsdp_shard,
        "stochastic_rounding": stochastic_rounding,
        "hbm_copy": hbm_copy,
        "mxfp4_recipe_and_mixed_gemms": recipe,
        **extra,
        "quantize_frac_of_hbm_peak_isolated": round(quant_gbps_iso / PEAK_HBM_GBPS, 4),
        "kernels": [{kk: (round(v, 4) if isinstance(v, float) else
                          {a: round(b, 4) for a, b in v.items()} if isinstance(v, dict) else v)
                     for kk, v in k.items() if kk != "work"} for k in kernels],
        "kernel_timing": ("ms: median over `steps` steps in which events bracket that launch alone (the dominant "
                          "kernel: its events in the timed steps); isolated: median of %d lone launches, each "
                          "after a clean fill of the last-level cache" % args.iso_reps),
    }
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle on a bounded sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.seed, step.flops, step.launches, kernels)
    if args.kernels:
        print("%-70s %21s %7s   %s" % ("kernel", "in the step", "", "alone, clean cache"), file=sys.stderr)
        for k in kernels:
            print("%-70s %8.1f us %9.1f %s %5.1f%%   %8.1f us %5.1f%%" % (
                k["kernel"], k["ms"] * 1e3, k["achieved"], k["unit"], 100 * k["frac"],
                k["isolated"]["ms"] * 1e3, 100 * k["isolated"]["frac"]), file=sys.stderr)
        print("fused dual quantize (%s, %s): %.1f us alone, %.1f%% of HBM (K-panel codes: %.1f us); "
              "the two single calls: %.1f us" % (
                  fused_dual["tensor"], fused_dual["formats"], fused_dual["ms"] * 1e3,
                  100 * fused_dual["frac_of_hbm_peak"], fused_dual["k_panels"]["ms"] * 1e3,
                  fused_dual["separate_ms"] * 1e3), file=sys.stderr)
        print("fsdp2 shard quantize (%s, e4m3): %.1f us alone, %.0f GB/s; gather payload %.3fx of bf16" % (
            fsdp_shard["slab"], fsdp_shard["ms"] * 1e3, fsdp_shard["GBps"], fsdp_shard["gather_ratio"]),
            file=sys.stderr)
        print("stochastic-rounding quantize (%s, %s): %.1f us alone, %.0f GB/s; nearest rounding %.1f us" % (
            stochastic_rounding["tensor"], stochastic_rounding["format"], stochastic_rounding["ms"] * 1e3,
            stochastic_rounding["GBps"], stochastic_rounding["nearest_rounding_ms"] * 1e3), file=sys.stderr)
        for k, v in recipe.items():
            print("%-34s %5dx%5dx%5d %-10s %7.1f us alone, %6.0f TFLOP/s, %4.1f%% of %.0f" % (
                k, v["M"], v["N"], v["K"], v["formats"], v["ms"] * 1e3, v["TFLOPs"], 100 * v["frac"], v["peak"]),
                file=sys.stderr)
        for k, v in hbm_copy.items():
            print("device copy %s -> %s: %.1f us alone, %.0f GB/s (%.1f%% of HBM peak)" % (
                k, k, v["ms"] * 1e3, v["GBps"], 100 * v["frac_of_hbm_peak"]), file=sys.stderr)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
