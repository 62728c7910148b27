#!/usr/bin/env python3
"""Benchmark of the INT4 dequantize-matmul hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rotate R] [--quick]

One *step* is the decode-time product of the Llama-7B workload: y = x . W^T
for x bf16 [1, 4096] against both INT4-packed weights, [4096, 4096] and
[11008, 4096] (group 128, fp16 scales and zero-points), bf16 out.  ``value``
is algorithmic bytes per step (packed codes + scales + zeros + x + y) over
the measured step time, in GB/s.  Weight copies are rotated (R copies, > 1 GB
in total by default) so every step reads its weights from HBM rather than
from the 256 MB Infinity Cache.  Inputs are resident in HBM before timing.

The JSON line also carries:
  roofline      the dominant kernel (the [11008, 4096] decode product) timed
                alone with HIP events on its stream, against 8 TB/s;
  cpu_baseline  the CPU oracle timed on this host on a bounded sample;
  extra         every other step of the path (quantize + pack, dequantize,
                INT8 activations, small-batch sweep, M=2048 prefill, W4A8
                decode and prefill), each with its algorithmic rate.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "int4 dequant-matmul GB/s (% of HBM peak) at M=1; TFLOP/s at M=2048"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
# fp32 vector ALU instruction rate: the 157.3 TFLOP/s fp32-vector peak counts
# an FMA as two flops, so 78.6 T fp32 lane-instructions per second (256 CUs x
# 4 SIMDs x 32 fp32 lanes per cycle x 2.4 GHz)
VALU_PEAK_TOPS = 157.3 / 2
FP64_PEAK_TFLOPS = 78.6          # MI355X float64 vector (and matrix) peak
FP32_MATRIX_PEAK_TFLOPS = 157.3  # MI355X dense float32 matrix peak


# ---------------------------------------------------------------------------
# Algorithmic work (bytes that must cross HBM, flops that must be done)
# ---------------------------------------------------------------------------
def w4a16_bytes(m, n, k, g, x_bytes=2, y_bytes=2, sz_bytes=2):
    return n * k // 2 + 2 * n * (k // g) * sz_bytes + m * k * x_bytes + m * n * y_bytes


def w4a8_bytes(m, n, k, g, y_bytes=2, sz_bytes=2):
    return n * k // 2 + 2 * n * (k // g) * sz_bytes + m * k + 4 * m + m * n * y_bytes


def quant_bytes(n, k, g, w_bytes=2, sz_bytes=2):
    return n * k * w_bytes + n * k // 2 + 2 * n * (k // g) * sz_bytes


# Sources of the kernel that runs the [11008,4096] decode product (and of its
# launch); stored counters and kernel traces are used only while these are unchanged.
DECODE_SOURCES = ("w4_common.h", "gemv_dot2.hip")


def src_hash(files=DECODE_SOURCES):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dequant_gemm_quantize_amd", "csrc")
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=32, help="distinct weight copies cycled through")
    ap.add_argument("--quick", action="store_true", help="skip the extra per-step measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget for the CPU oracle sample")
    ap.add_argument("--kernel", choices=("decode_wb", "decode_m4_wb", "prefill_wb", "w4a8_m1", "w4a8_m512",
                                         "w4a8_shard_m512", "decode_m8_wb", "copy", "gptq", "read", "llama32"),
                    default=None,
                    help="launch only this kernel --launches times, eagerly, for counter runs: "
                         "decode_wb / decode_m4_wb / decode_m8_wb = the [11008,4096] product at 1 / 4 / 8 "
                         "tokens on rotated "
                         "weights, llama32 = the 32-layer decode, --launches tokens (one graph each), "
                         "prefill_wb = the M=2048 product on [11008,4096], "
                         "w4a8_m1 / w4a8_m512 = the W4A8 product on [28672,8192], "
                         "w4a8_shard_m512 = the same at 512 tokens on its first 3584 rows (one GPU's "
                         "8-way column shard; split K over the workspace), "
                         "copy = a plain device copy of --copy-mib MiB (calibrates byte counters), "
                         "read = the streaming-read measurement kernel over the decode product's byte "
                         "count, rotated through a 1 GiB buffer")
    ap.add_argument("--launches", type=int, default=40)
    ap.add_argument("--copy-mib", type=int, default=256)
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dequant_gemm_quantize_amd as w4
    import workloads as WL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w4.load()
    stream = torch.cuda.current_stream(dev)

    def to_dev(t):
        if t.kind == "bf16":
            return torch.from_numpy(t.data.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(t.data).to(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def time_region(fn, iters, per_graph=None):
        """Seconds per call of fn(i), i = 0..iters-1.

        The calls are captured into HIP graphs (per_graph calls each, default
        all of them) and replayed between two HIP events recorded on the
        launch stream, so host-side launch cost does not enter the figure.
        One untimed replay of every graph precedes the timed one.
        """
        per = per_graph or iters
        graphs = []
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        done = 0
        while done < iters:
            cnt = min(per, iters - done)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                for i in range(done, done + cnt):
                    fn(i)
            graphs.append(gr)
            done += cnt
        stream.wait_stream(side)
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for gr in graphs:
            gr.replay()
        e1.record(stream)
        e1.synchronize()
        del graphs
        return e0.elapsed_time(e1) / 1e3 / iters

    if args.kernel is not None:
        return kernel_only(args, w4, WL, torch, dev, to_dev, log, time_region)

    g = 128
    log("generating Llama-7B decode weights")
    wa, wb = WL.weight("Wa"), WL.weight("Wb")
    xa1 = WL.activation(2, 1, 4096)
    x1 = to_dev(xa1)
    data_sha = {name: hashlib.sha256(np.ascontiguousarray(t.data).tobytes()).hexdigest()[:16]
                for name, t in (("Wa", wa), ("Wb", wb), ("x", xa1))}
    shapes = {"Wa": (4096, 4096), "Wb": (11008, 4096)}

    # quantize once on the GPU, then clone R copies of the packed weights
    q = {}
    for name, t in (("Wa", wa), ("Wb", wb)):
        wt = to_dev(t)
        q[name] = w4.quantize_pack_int4(wt, g, torch.float16)
        del wt
    R = max(1, args.rotate)
    copies = {name: [tuple(a.clone() for a in q[name]) for _ in range(R)] for name in q}
    y_out = {name: torch.empty((1, shapes[name][0]), dtype=torch.bfloat16, device=dev) for name in q}
    torch.cuda.synchronize()

    def step(i):
        for name in ("Wa", "Wb"):
            p, s, z = copies[name][i % R]
            w4.w4a16_matmul(x1, p, s, z, g, out=y_out[name])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    sec = time_region(step, args.steps)
    step_bytes = sum(w4a16_bytes(1, n, k, g) for n, k in shapes.values())
    value = step_bytes / sec / 1e9
    log(f"decode step: {sec * 1e6:.2f} us, {value:.1f} GB/s")

    # dominant kernel alone: the [11008, 4096] decode product
    def dom(i):
        p, s, z = copies["Wb"][i % R]
        w4.w4a16_matmul(x1, p, s, z, g, out=y_out["Wb"])

    for i in range(args.warmup):
        dom(i)
    dsec = time_region(dom, args.steps)
    dbytes = w4a16_bytes(1, 11008, 4096, g)
    achieved = dbytes / dsec / 1e9
    roof = {"kernel": "w4a16 decode, W [11008,4096] int4 g128, x bf16 [1,4096]",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "avg_launch_us": round(dsec * 1e6, 3),
            "timing": "HIP events on the launch stream around graph replays of back-to-back launches "
                      "over the rotated weight copies",
            "bytes_per_launch": dbytes, "traffic": None, "kernel_trace": None}
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tr = json.load(fh)
        ent = tr.get("w4a16_decode_Wb")
        if ent and ent.get("src_hash") == src_hash():
            roof["traffic"] = ent.get("bytes_per_launch")
            kt = ent.get("kernel_trace")
            if kt:  # the rocprofv3 kernel trace of this kernel, same sources
                roof["kernel_trace"] = dict(kt, frac_at_median=round(dbytes / kt["median_us"] / 1e3 / HBM_PEAK_GBS, 4))
    log(f"dominant kernel: {dsec * 1e6:.2f} us/launch, {achieved:.1f} GB/s")

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama7b_decode_m1: x bf16 [1,4096] . W^T for W int4 "
                               "[4096,4096] and [11008,4096], group 128, fp16 scales/zeros, bf16 out",
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
                   "rotated_weight_copies": R,
                   "rotated_bytes": int(R * sum(sum(a.numel() * a.element_size() for a in q[nm]) for nm in q)),
                   "hbm_pct": round(100 * value / HBM_PEAK_GBS, 2),
                   "data_sha256_16": data_sha, "numpy": np.__version__},
        "roofline": roof,
    }
    del q

    if not args.quick:
        result["extra"] = extras(args, w4, WL, torch, np, dev, stream, to_dev, time_region, log, copies, x1,
                                 dsec * 1e6)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, WL, np, log, wa, wb)

    print(json.dumps(result), flush=True)
    return 0


def extras(args, w4, WL, torch, np, dev, stream, to_dev, time_region, log, copies, x1, dom_us):
    """Rates of every other step of the path; each is timed with HIP events."""
    out = {}
    g = 128
    R = len(copies["Wa"])
    reps = max(10, min(50, args.steps // 4))

    # small-batch sweep on the Llama-7B shapes (rotated weights)
    sweep = {}
    for m in (1, 2, 4, 8, 16, 32, 64):
        x = to_dev(WL.activation(2 if m == 1 else 3, m, 4096))
        row = {}
        for name, (n, k) in (("Wa", (4096, 4096)), ("Wb", (11008, 4096))):
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            fn = lambda i, name=name, x=x, y=y: w4.w4a16_matmul(x, *copies[name][i % R], g, out=y)
            for i in range(3):
                fn(i)
            sec = time_region(fn, reps)
            b = w4a16_bytes(m, n, k, g)
            row[name] = {"us": round(sec * 1e6, 3), "GB/s": round(b / sec / 1e9, 1),
                         "TFLOP/s": round(2 * m * n * k / sec / 1e12, 3)}
        sweep[f"M={m}"] = row
    out["w4a16_small_batch"] = sweep
    log(f"small-batch sweep: {json.dumps(sweep)}")

    # prefill M=2048 on [11008,4096] and [4096,11008]
    pre = {}
    for name, (n, k) in (("Wb", (11008, 4096)), ("Wd", (4096, 11008))):
        t = WL.weight(name)
        wt = to_dev(t)
        p, s, z = w4.quantize_pack_int4(wt, g, torch.float16)
        # quantize + pack rate on this weight (bf16 in)
        qo = (torch.empty_like(p), torch.empty_like(s), torch.empty_like(z))
        qsec = time_region(lambda i: w4.quantize_pack_int4(wt, g, torch.float16, out=qo), reps)
        out.setdefault("quantize_pack", {})[name] = {
            "us": round(qsec * 1e6, 2), "GB/s": round(quant_bytes(n, k, g) / qsec / 1e9, 1)}
        # the symmetric variant moves the same bytes
        qsec = time_region(lambda i: w4.quantize_pack_int4_sym(wt, g, torch.float16, out=qo), reps)
        out.setdefault("quantize_pack_sym", {})[name] = {
            "us": round(qsec * 1e6, 2), "GB/s": round(quant_bytes(n, k, g) / qsec / 1e9, 1)}
        if name == "Wb":
            # range-clipping calibrators: the percentile (a bitonic sort per
            # group) and the MSE search (1000 candidates, 8.75 fp32 VALU
            # instructions per candidate and weight)
            qsec = time_region(lambda i: w4.quantize_pack_int4_sym_percentile(wt, g, 99.9, torch.float16,
                                                                             out=qo), 5)
            cal = {"percentile_99.9": {"us": round(qsec * 1e6, 1),
                                       "GB/s": round(quant_bytes(n, k, g) / qsec / 1e9, 1)}}
            ncand = 1000
            qsec = time_region(lambda i: w4.quantize_pack_int4_sym_mse(wt, g, ncand, torch.float16, out=qo), 3)
            tops = 8.75 * n * k * ncand / qsec / 1e12
            cal["mse_1000"] = {"us": round(qsec * 1e6, 1), "valu_TOP/s": round(tops, 2),
                               "frac_valu_peak": round(tops / VALU_PEAK_TOPS, 4)}
            out["calibrate_sym_Wb"] = cal
            log(f"calibrators: {json.dumps(cal)}")
        del qo
        if name == "Wb":
            dq = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
            dsec = time_region(lambda i: w4.dequant_int4(p, s, z, g, out=dq), reps)
            out["dequant_int4_bf16"] = {"us": round(dsec * 1e6, 2),
                                        "GB/s": round((n * k // 2 + 4 * n * (k // g) + 2 * n * k) / dsec / 1e9, 1)}
            del dq
        del wt
        if name == "Wd":
            # the down projection [4096,11008] at decode and small-batch sizes
            # (K = 11008 is not a whole number of 512-column slices per wave)
            cpd = [(p, s, z)] + [tuple(a.clone() for a in (p, s, z)) for _ in range(R - 1)]
            down = {}
            for m in (1, 16, 64, 128):
                xd = to_dev(WL.activation(2 if m == 1 else 3, m, k))
                yd = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                fn = lambda i, xd=xd, yd=yd: w4.w4a16_matmul(xd, *cpd[i % R], g, out=yd)
                for i in range(3):
                    fn(i)
                sec = time_region(fn, reps)
                down[f"M={m}"] = {"us": round(sec * 1e6, 3),
                                  "GB/s": round(w4a16_bytes(m, n, k, g) / sec / 1e9, 1),
                                  "TFLOP/s": round(2 * m * n * k / sec / 1e12, 3)}
            out["w4a16_down_proj_4096x11008"] = down
            log(f"down projection: {json.dumps(down)}")
            del cpd
        x = to_dev(WL.activation(4, 2048, k))
        y = torch.empty((2048, n), dtype=torch.bfloat16, device=dev)
        fn = lambda i: w4.w4a16_matmul(x, p, s, z, g, out=y)
        for i in range(3):
            fn(i)
        sec = time_region(fn, reps)
        tf = 2 * 2048 * n * k / sec / 1e12
        pre[name] = {"us": round(sec * 1e6, 2), "TFLOP/s": round(tf, 1),
                     "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
        del x, y, p, s, z
    out["w4a16_prefill_m2048"] = pre
    log(f"prefill: {json.dumps(pre)}")

    # W4A8 on the 70B-class MLP projection
    t = WL.weight("We")
    wt = to_dev(t)
    n, k = 28672, 8192
    p, s, z = w4.quantize_pack_int4(wt, g, torch.float16)
    qo = (torch.empty_like(p), torch.empty_like(s), torch.empty_like(z))
    qsec = time_region(lambda i: w4.quantize_pack_int4(wt, g, torch.float16, out=qo), 5)
    out.setdefault("quantize_pack", {})["We"] = {"us": round(qsec * 1e6, 2),
                                                 "GB/s": round(quant_bytes(n, k, g) / qsec / 1e9, 1)}
    del wt, qo
    cp8 = [(p, s, z)] + [tuple(a.clone() for a in (p, s, z)) for _ in range(3)]
    w8 = {}
    for m in (1, 2, 8, 16, 512):
        xb = to_dev(WL.activation(5, m, 8192))
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xs = torch.empty((m,), dtype=torch.float32, device=dev)
        asec = time_region(lambda i: w4.quantize_act_int8(xb, out=(xq, xs)), reps)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        fn = lambda i: w4.w4a8_matmul(xq, xs, *cp8[i % len(cp8)], g, out=y)
        for i in range(3):
            fn(i)
        sec = time_region(fn, reps)
        b = w4a8_bytes(m, n, k, g)
        w8[f"M={m}"] = {"act_quant_us": round(asec * 1e6, 2), "us": round(sec * 1e6, 2),
                        "GB/s": round(b / sec / 1e9, 1), "TOP/s": round(2 * m * n * k / sec / 1e12, 2),
                        "frac_int8_peak": round(2 * m * n * k / sec / 1e12 / INT8_PEAK_TOPS, 4),
                        "frac_hbm": round(b / sec / 1e9 / HBM_PEAK_GBS, 4)}
    out["w4a8_70b_mlp"] = w8
    log(f"w4a8: {json.dumps(w8)}")
    del cp8

    # One GPU's share of the same projection under 8-way column (N) sharding:
    # rows 0..3583, the same kernels on [3584, 8192]; 24 copies (375 MB) are
    # rotated so that the one-token launches read from HBM, not the 256 MB MALL.
    ns = n // 8
    cps = [tuple(a[:ns].clone() for a in (p, s, z)) for _ in range(24)]
    ws = {}
    for m in (1, 512):
        xb = to_dev(WL.activation(5, m, 8192))
        xq, xs = w4.quantize_act_int8(xb)
        y = torch.empty((m, ns), dtype=torch.bfloat16, device=dev)
        fn = lambda i: w4.w4a8_matmul(xq, xs, *cps[i % len(cps)], g, out=y)
        for i in range(3):
            fn(i)
        sec = time_region(fn, reps)
        b = w4a8_bytes(m, ns, k, g)
        ws[f"M={m}"] = {"us": round(sec * 1e6, 2), "GB/s": round(b / sec / 1e9, 1),
                        "TOP/s": round(2 * m * ns * k / sec / 1e12, 2),
                        "frac_int8_peak": round(2 * m * ns * k / sec / 1e12 / INT8_PEAK_TOPS, 4),
                        "frac_hbm": round(b / sec / 1e9 / HBM_PEAK_GBS, 4)}
    out["w4a8_70b_mlp_tp8_shard_3584x8192"] = ws
    log(f"w4a8 tp8 shard: {json.dumps(ws)}")
    del cps, p, s, z

    # single fp32 layer (latency bound)
    t1 = WL.weight("W1")
    w1 = to_dev(t1)
    p, s, z = w4.quantize_pack_int4(w1, 32, torch.float32)
    x = to_dev(WL.activation(1, 1, 256))
    y = torch.empty((1, 256), dtype=torch.float32, device=dev)
    sec = time_region(lambda i: w4.w4a16_matmul(x, p, s, z, 32, out=y), reps)
    out["single_layer_fp32_256"] = {"us": round(sec * 1e6, 2)}
    del p, s, z, w1

    out["llama7b_decode_32_layers"] = llama_decode(w4, torch, dev, time_region, log, g)
    out["gptq_Wb"] = gptq_bench(w4, torch, np, dev, time_region, log)
    out["measured_peaks"] = measured_peaks(w4, WL, torch, dev, to_dev, time_region, log, copies, x1, out,
                                           dom_us)
    return out


def load_peaks_lib():
    """libw4peaks.so (measurement kernels, built next to libw4.so)."""
    import ctypes
    path = os.path.join(ROOT, "dequant_gemm_quantize_amd", "libw4peaks.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.w4_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.w4_peak_mfma_loop.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]
    return lib


def measured_peaks(w4, WL, torch, dev, to_dev, time_region, log, copies, x1, out, dom_us, g=128):
    """Context for the fractions above, measured in the same process:
    - the decode product with one weight copy (resident in the 256 MB
      Infinity Cache, so not an HBM figure);
    - a plain streaming read of the decode product's byte count with the
      decode kernels' geometry (rotated through a 1 GiB buffer, so from HBM),
      and of 1 GiB: the read bandwidth this GPU sustains for such launches;
    - back-to-back bf16 and int8 matrix instructions (MFMA-only loops): the
      matrix rate this GPU sustains under that load;
    - a 1 GiB device copy, and the dense bf16 library GEMM (torch.matmul on a
      dequantized weight, run as a black box) on the M = 2048 shape."""
    import ctypes
    lib = load_peaks_lib()

    def sid():  # the stream being captured or run on, at call time
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = {}
    y = torch.empty((1, 11008), dtype=torch.bfloat16, device=dev)
    p, s, z = copies["Wb"][0]
    sec = time_region(lambda i: w4.w4a16_matmul(x1, p, s, z, g, out=y), 200)
    res["decode_Wb_warm"] = {"us": round(sec * 1e6, 3), "GB/s": round(w4a16_bytes(1, 11008, 4096, g) / sec / 1e9, 1),
                             "note": "one weight copy, cache-resident: not an HBM figure"}

    # streaming reads
    big = torch.empty(1 << 28, dtype=torch.int32, device=dev).random_()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    dbytes = w4a16_bytes(1, 11008, 4096, g)            # 23,983,616: a multiple of 16
    nreg = (big.numel() * 4) // dbytes
    base = big.data_ptr()

    def rd(i, nbytes=dbytes, lanes=8, stride=dbytes, regions=nreg):
        rc = lib.w4_peak_stream_read(ctypes.c_void_p(base + (i % regions) * stride), nbytes, lanes,
                                     ctypes.c_void_p(sink.data_ptr()), sid())
        if rc != 0:
            raise RuntimeError(f"w4_peak_stream_read failed ({rc})")
    for i in range(5):
        rd(i)
    rsec = time_region(rd, 200)
    res["stream_read_decode_bytes"] = {
        "bytes": dbytes, "us": round(rsec * 1e6, 3), "GB/s": round(dbytes / rsec / 1e9, 1),
        "frac_of_8TBs": round(dbytes / rsec / 1e9 / HBM_PEAK_GBS, 4),
        "decode_Wb_time_over_it": round(dom_us / (rsec * 1e6), 4),
        "note": "the decode product's byte count read once, 732 workgroups of 256 lanes, 8 x 16 B "
                "non-temporal loads per lane (the decode kernels' pattern), rotated over a 1 GiB buffer"}
    gib = big.numel() * 4
    gsec = time_region(lambda i: rd(0, gib, 16, 0, 1), 10)
    res["stream_read_1GiB"] = {"us": round(gsec * 1e6, 2), "GB/s": round(gib / gsec / 1e9, 1),
                               "frac_of_8TBs": round(gib / gsec / 1e9 / HBM_PEAK_GBS, 4)}

    # matrix-instruction loops on random operands
    ops = torch.randn(1024, dtype=torch.float32, device=dev).to(torch.bfloat16)  # 128 x 16 B of bf16
    ops8 = torch.randint(-128, 128, (2048,), dtype=torch.int8, device=dev)
    blocks, iters = 512, 2000
    mout = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    for kind, buf, unit_ops, peak, name in ((0, ops, 32768, BF16_PEAK_TFLOPS, "mfma_loop_bf16"),
                                            (1, ops8, 65536, INT8_PEAK_TOPS, "mfma_loop_i8")):
        def mf(i, kind=kind, buf=buf):
            rc = lib.w4_peak_mfma_loop(kind, ctypes.c_void_p(buf.data_ptr()), blocks, iters,
                                       ctypes.c_void_p(mout.data_ptr()), sid())
            if rc != 0:
                raise RuntimeError(f"w4_peak_mfma_loop failed ({rc})")
        for i in range(3):
            mf(i)
        msec = time_region(mf, 10)
        work = blocks * 4 * iters * 4 * unit_ops
        res[name] = {"us": round(msec * 1e6, 1), "T/s": round(work / msec / 1e12, 1),
                     "frac_of_peak": round(work / msec / 1e12 / peak, 4),
                     "note": f"{blocks} workgroups x 4 waves, {iters} rounds of 4 independent chains"}
    del big, sink, mout

    src = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(1)
    dst = torch.empty_like(src)
    csec = time_region(lambda i: dst.copy_(src), 10)
    copy_gbs = 2 * src.numel() * 4 / csec / 1e9
    del src, dst
    res["hbm_copy_1GiB"] = {"GB/s": round(copy_gbs, 1), "frac_of_8TBs": round(copy_gbs / HBM_PEAK_GBS, 4),
                            "note": "read + write bytes of a plain device-to-device copy"}
    wd = w4.dequant_int4(*w4.quantize_pack_int4(to_dev(WL.weight("Wb")), g, torch.float16), g,
                         out_dtype=torch.bfloat16)
    xm = to_dev(WL.activation(4, 2048, 4096))
    wt = wd.t()
    for _ in range(3):                      # the library GEMM is timed eagerly: it cannot be graph-captured
        torch.matmul(xm, wt)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(xm, wt)
    e1.record()
    e1.synchronize()
    msec = e0.elapsed_time(e1) / 1e3 / 10
    tflops = 2 * 2048 * 11008 * 4096 / msec / 1e12
    ours = out.get("w4a16_prefill_m2048", {}).get("Wb", {}).get("TFLOP/s")
    res["dense_bf16_library_gemm_Wb_m2048"] = {"us": round(msec * 1e6, 1), "TFLOP/s": round(tflops, 1),
                                               "fused_w4a16_frac_of_it": round(ours / tflops, 4) if ours else None}
    log(f"measured peaks: {json.dumps(res)}")
    return res


def gptq_arrays(np, n=11008, k=4096, t=4096):
    """Weight [n, k] from N(0, 0.02) and t calibration rows from N(0, 1)
    (synthetic stand-ins for a layer's weight and its input activations)."""
    rng = np.random.default_rng(77)
    return rng.normal(0, 0.02, (n, k)).astype(np.float32), rng.normal(0, 1, (t, k)).astype(np.float32)


def gptq_setup(torch, np, dev, n=11008, k=4096, t=4096):
    w, x = gptq_arrays(np, n, k, t)
    return torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev)


def gptq_update_flops(n, k, block=128):
    """Algorithmic flops of the sweep's lazy updates: 2 n b (k - b1) per block."""
    return sum(2 * n * min(block, k - b0) * (k - b0 - min(block, k - b0)) for b0 in range(0, k, block))


def gptq_bench(w4, torch, np, dev, time_region, log, n=11008, k=4096, t=4096, g=128):
    """GPTQ on the Llama-7B gate shape: Hessian from t calibration rows, the
    inverse Cholesky factor, and the column sweep, each timed on its own.  The
    factor and sweep timings include a device copy of their input (h: 134 MB,
    w: 180 MB), because both calls use it as working storage."""
    w, x = gptq_setup(torch, np, dev, n, k, t)
    h = torch.empty((k, k), dtype=torch.float64, device=dev)
    hsec = time_region(lambda i: w4.gptq_hessian(x, out=h), 3)
    hw = torch.empty_like(h)
    u = torch.empty_like(h)

    def factor(i):
        hw.copy_(h)
        w4.gptq_inverse_cholesky(hw, out=u, overwrite_h=True, check=False)
    usec = time_region(factor, 3)
    work = torch.empty_like(w)
    outs = (torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
            torch.empty((n, k // g), dtype=torch.float16, device=dev),
            torch.empty((n, k // g), dtype=torch.float16, device=dev))

    def sweep(i):
        work.copy_(w)
        w4.gptq_quantize_pack_int4(work, u, g, False, torch.float16, overwrite_w=True, out=outs)
    ssec = time_region(sweep, 3)
    upd = gptq_update_flops(n, k)
    res = {"shape": [n, k], "calibration_rows": t, "group": g,
           "hessian_ms": round(hsec * 1e3, 3),
           "hessian_fp64_TFLOP/s": round(t * k * k / hsec / 1e12, 2),
           "hessian_frac_fp64_peak": round(t * k * k / hsec / 1e12 / FP64_PEAK_TFLOPS, 4),
           "inverse_cholesky_ms": round(usec * 1e3, 3),
           "sweep_ms": round(ssec * 1e3, 3),
           "sweep_update_TFLOP/s": round(upd / ssec / 1e12, 2),
           "sweep_frac_fp32_matrix_peak": round(upd / ssec / 1e12 / FP32_MATRIX_PEAK_TFLOPS, 4),
           "total_ms": round((hsec + usec + ssec) * 1e3, 3)}
    log(f"gptq: {json.dumps(res)}")
    return res


# One Llama-7B decoder layer's linears with the usual fusions: q, k and v as
# one [12288, 4096] product, gate and up as one [22016, 4096].
LLAMA7B_LINEARS = (("qkv", 12288, 4096), ("o", 4096, 4096), ("gate_up", 22016, 4096), ("down", 4096, 11008))


def llama_decode(w4, torch, dev, time_region, log, g, layers=32, tokens=8):
    """Decode throughput over all 32 layers' linears of a Llama-7B-shaped
    model at one token: 128 products per token, each consuming the previous
    one's output (a slice of it stands in for attention and the MLP
    activation, which are not part of this path).  Weights are synthetic
    N(0, 0.02) bf16 drawn on the GPU, quantized by quantize_pack_int4
    (group 128, fp16 scales); every token's launches are captured in a HIP
    graph, so the figure is GPU time."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    model = []
    nbytes = 0
    for _ in range(layers):
        per = {}
        for name, n, k in LLAMA7B_LINEARS:
            w = (torch.randn((n, k), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            per[name] = w4.quantize_pack_int4(w, g, torch.float16)
            nbytes += w4a16_bytes(1, n, k, g)
            del w
        model.append(per)
    x = (torch.randn((1, 4096), generator=gen, device=dev)).to(torch.bfloat16)
    qkv = torch.empty((1, 12288), dtype=torch.bfloat16, device=dev)
    o = torch.empty((1, 4096), dtype=torch.bfloat16, device=dev)
    gu = torch.empty((1, 22016), dtype=torch.bfloat16, device=dev)
    y = [torch.empty((1, 4096), dtype=torch.bfloat16, device=dev) for _ in range(2)]

    def token(i):
        cur = x
        for li, per in enumerate(model):
            w4.w4a16_matmul(cur, *per["qkv"], g, out=qkv)
            w4.w4a16_matmul(qkv[:, :4096], *per["o"], g, out=o)
            w4.w4a16_matmul(o, *per["gate_up"], g, out=gu)
            w4.w4a16_matmul(gu[:, :11008], *per["down"], g, out=y[li % 2])
            cur = y[li % 2]

    for i in range(2):
        token(i)
    sec = time_region(token, tokens, per_graph=1)
    res = {"ms_per_token": round(sec * 1e3, 4), "tokens_per_s": round(1.0 / sec, 1),
           "weight_bytes_per_token": nbytes, "GB/s": round(nbytes / sec / 1e9, 1),
           "hbm_frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4), "launches_per_token": 4 * layers,
           "us_per_launch": round(sec * 1e6 / (4 * layers), 3)}
    log(f"llama-7b decode, 32 layers: {json.dumps(res)}")
    del model
    torch.cuda.empty_cache()
    return res


def kernel_only(args, w4, WL, torch, dev, to_dev, log, time_region):
    """Eager launches of one kernel and nothing else of note, so a counter
    run's per-dispatch records are easy to pick out."""
    n_launch = max(1, args.launches)
    if args.kernel == "copy":
        nbytes = args.copy_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(n_launch):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"kernel": "copy", "launches": n_launch, "read_bytes": nbytes,
                          "write_bytes": nbytes}), flush=True)
        return 0
    if args.kernel == "read":
        import ctypes
        lib = load_peaks_lib()
        big = torch.empty(1 << 28, dtype=torch.int32, device=dev).random_()
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        nbytes = w4a16_bytes(1, 11008, 4096, 128)
        nreg = (big.numel() * 4) // nbytes
        sid = torch.cuda.current_stream(dev).cuda_stream
        torch.cuda.synchronize()
        for i in range(n_launch):
            rc = lib.w4_peak_stream_read(ctypes.c_void_p(big.data_ptr() + (i % nreg) * nbytes), nbytes, 8,
                                         ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(sid))
            assert rc == 0, rc
        torch.cuda.synchronize()
        print(json.dumps({"kernel": "read", "launches": n_launch, "bytes_per_launch": nbytes}), flush=True)
        return 0
    if args.kernel == "gptq":
        import numpy as np
        w, x = gptq_setup(torch, np, dev)
        torch.cuda.synchronize()
        for _ in range(n_launch):
            u = w4.gptq_inverse_cholesky(w4.gptq_hessian(x), overwrite_h=True)
            w4.gptq_quantize_pack_int4(w, u, 128, False, torch.float16)
        torch.cuda.synchronize()
        print(json.dumps({"kernel": "gptq", "passes": n_launch,
                          "update_flops_per_pass": gptq_update_flops(*w.shape)}), flush=True)
        return 0
    if args.kernel == "prefill_wb":
        g, n, k = 128, 11008, 4096
        wt = to_dev(WL.weight("Wb"))
        p, s, z = w4.quantize_pack_int4(wt, g, torch.float16)
        del wt
        x = to_dev(WL.activation(4, 2048, k))
        y = torch.empty((2048, n), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for i in range(n_launch):
            w4.w4a16_matmul(x, p, s, z, g, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"kernel": "prefill_wb", "launches": n_launch,
                          "flops_per_launch": 2 * 2048 * n * k}), flush=True)
        return 0
    if args.kernel in ("w4a8_m1", "w4a8_m512", "w4a8_shard_m512"):
        g, n, k = 128, 28672, 8192
        m = 1 if args.kernel == "w4a8_m1" else 512
        wt = to_dev(WL.weight("We"))
        q = w4.quantize_pack_int4(wt, g, torch.float16)
        del wt
        if args.kernel == "w4a8_shard_m512":
            n = n // 8
            q = tuple(a[:n].clone() for a in q)
        copies = [q] + [tuple(a.clone() for a in q) for _ in range(3)]
        xq, xs = w4.quantize_act_int8(to_dev(WL.activation(5, m, k)))
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for i in range(n_launch):
            w4.w4a8_matmul(xq, xs, *copies[i % 4], g, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"kernel": args.kernel, "launches": n_launch,
                          "bytes_per_launch": w4a8_bytes(m, n, k, g),
                          "ops_per_launch": 2 * m * n * k}), flush=True)
        return 0
    g, n, k = 128, 11008, 4096
    if args.kernel == "llama32":
        res = llama_decode(w4, torch, dev, time_region, log, g, tokens=n_launch)
        print(json.dumps(dict(res, kernel="llama32")), flush=True)
        return 0
    m = {"decode_m4_wb": 4, "decode_m8_wb": 8}.get(args.kernel, 1)
    wt = to_dev(WL.weight("Wb"))
    q = w4.quantize_pack_int4(wt, g, torch.float16)
    del wt
    R = max(1, args.rotate)
    copies = [tuple(a.clone() for a in q) for _ in range(R)]
    x = to_dev(WL.activation(2 if m == 1 else 3, m, k))
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"{args.kernel}: {n_launch} launches over {R} weight copies")
    for i in range(n_launch):
        w4.w4a16_matmul(x, *copies[i % R], g, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": args.kernel, "launches": n_launch,
                      "bytes_per_launch": w4a16_bytes(m, n, k, g)}), flush=True)
    return 0


def cpu_baseline(args, WL, np, log, wa, wb):
    """The oracle (unchanged) on this host: the same decode step, repeated
    until about --cpu-seconds of CPU work have run."""
    import oracle.w4_oracle as O
    try:
        from threadpoolctl import threadpool_info
    except Exception:  # pragma: no cover
        threadpool_info = None
    g = 128
    qa = O.quantize_pack_int4(wa.data, wa.kind, g, "f16")
    qb = O.quantize_pack_int4(wb.data, wb.kind, g, "f16")
    x = WL.activation(2, 1, 4096).as_f32()
    steps = 0
    t0 = time.perf_counter()
    while True:
        O.matmul_w4a16_f64(x, *qa, g)
        O.matmul_w4a16_f64(x, *qb, g)
        steps += 1
        if time.perf_counter() - t0 > args.cpu_seconds or steps >= 1000:
            break
    sec = (time.perf_counter() - t0) / steps
    step_bytes = w4a16_bytes(1, 4096, 4096, g) + w4a16_bytes(1, 11008, 4096, g)
    blas_threads = 1
    if threadpool_info is not None:
        for info in threadpool_info():
            if info.get("user_api") == "blas":
                blas_threads = max(blas_threads, int(info.get("num_threads", 1)))
    res = {"value": round(step_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": blas_threads,
           "kind": "oracle",
           "sample": f"{steps} full decode steps (W4A16 M=1 on [4096,4096] and [11008,4096]): "
                     f"NumPy unpack/dequantize chunk by chunk in float64 (1 thread) and a BLAS "
                     f"float64 product ({blas_threads} threads); {sec * 1e3:.1f} ms per step",
           "ms_per_step": round(sec * 1e3, 3), "host_cpus": os.cpu_count(),
           "affinity_cpus": len(os.sched_getaffinity(0)), "numpy": np.__version__}
    log(f"cpu baseline: {res['value']} GB/s over {steps} steps")
    res["stages"] = oracle_stages(WL, np, log, wb)
    res["gptq"] = gptq_cpu(np, log)
    return res


def oracle_stages(WL, np, log, wb, g=128, seconds=2.0):
    """The oracle's other stages on this host (NumPy, one thread), each run
    whole and repeated for about `seconds`, as rates on the same algorithmic
    bytes as the GPU figures: quantize + pack of the [11008, 4096] weight
    (bf16 in, fp16 scales), and the per-token INT8 activations of x bf16
    [512, 8192]."""
    import oracle.w4_oracle as O
    out = {}

    def rate(fn, nbytes):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 > seconds:
                break
        sec = (time.perf_counter() - t0) / reps
        return {"ms": round(sec * 1e3, 2), "GB/s": round(nbytes / sec / 1e9, 3), "reps": reps}

    n, k = 11008, 4096
    out["quantize_pack_Wb"] = rate(lambda: O.quantize_pack_int4(wb.data, wb.kind, g, "f16"), quant_bytes(n, k, g))
    x = WL.activation(5, 512, 8192).as_f32()
    out["act_quant_int8_512x8192"] = rate(lambda: O.act_quant_int8(x), 512 * 8192 * (2 + 1) + 4 * 512)
    log(f"oracle stages: {json.dumps(out)}")
    return out


def gptq_cpu(np, log, rows=64, g=128):
    """The GPTQ oracle on the benchmark's [11008, 4096] layer with 4096
    calibration rows: Hessian and factor in full, the sweep on the first
    `rows` weight rows (rows are independent), scaled linearly to all rows.
    The scaled figure is a lower bound: the full sweep's working set no
    longer fits in the host's caches."""
    import oracle.gptq_oracle as G
    w, x = gptq_arrays(np)
    t0 = time.perf_counter()
    h = G.gptq_hessian(x)
    t1 = time.perf_counter()
    u = G.gptq_inverse_cholesky(h)
    t2 = time.perf_counter()
    G.gptq_quantize_pack_int4(w[:rows], "f32", u, g, "f16")
    t3 = time.perf_counter()
    per_row = (t3 - t2) / rows
    res = {"hessian_s": round(t1 - t0, 3), "factor_s": round(t2 - t1, 3),
           "sweep_s_per_row": round(per_row, 5), "sweep_s_all_rows": round(per_row * w.shape[0], 1),
           "total_s": round((t1 - t0) + (t2 - t1) + per_row * w.shape[0], 1),
           "sample": f"Hessian and factor in full; the sweep on {rows} of {w.shape[0]} rows, scaled "
                     f"linearly (a lower bound for the full sweep)"}
    log(f"gptq oracle: {json.dumps(res)}")
    return res


if __name__ == "__main__":
    sys.exit(main())
