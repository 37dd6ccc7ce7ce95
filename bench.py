"""Throughput of the rotate / quantize / W4A4 path on one MI355X.

One step = one fused randomized-Hadamard + int4 quantization pass
(hr_rotate_quant_int4) over bf16 activations of 65536 tokens x 2048 channels,
group 128, fp16 scales -- the workload the headline metric is quoted on.
``value`` is that pass's throughput in GB/s of algorithmic bytes (input read
once + codes and scales written once).  The W4A4 GEMM (4096^3 and M=16) and
the other kernels are timed the same way and reported under ``kernels``.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA peak
METRIC = "fused RHT+int4 quant GB/s (% of HBM peak) at K=2048; W4A4 GEMM int8 TOPS"

ROWS, N, GROUP = 65536, 2048, 128

HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")
CSRC = os.path.join(HERE, "hadamard_rotation_int4_amd", "csrc")
# sources that make up the headline kernel (its counters go stale when they change)
MAIN_KERNEL_SOURCES = ("rht2048_mfma.hip", "mfma2048.h", "fwht2048.h", "hr_device.h", "hr_internal.h")
MAIN_KERNEL_NAME = "rht2048_mfma_kernel<128, true, false, 4, 1>"
TRAFFIC_FILE = os.path.join(PROFILES, "rht_quant_bf16_65536x2048_g128.traffic.json")
COPY_BYTES = 512 * 1024 * 1024       # calibration copy: reads and writes this many bytes


def main_kernel_hash():
    h = hashlib.sha256()
    for name in MAIN_KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter
    summary, or None when it is missing or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != main_kernel_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def rht_alg_bytes(rows, n, group, in_bytes=2, scale_bytes=2):
    return rows * n * in_bytes + rows * n // 2 + rows * (n // group) * scale_bytes


def _timed(fn, steps, warmup, nbuf=1):
    """Run fn(i) warmup + steps times on the current stream; HIP events bracket
    the timed launches.  Returns ms per call."""
    import torch
    for i in range(warmup):
        fn(i % nbuf)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i % nbuf)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def _timed_graph(fn, steps, warmup, per_graph=20):
    """Like _timed, for kernels shorter than a Python call: per_graph calls are
    captured once in a HIP graph, and the timed region replays it, so the
    host's launch cost per call is not what gets measured.  Returns ms per call."""
    import torch
    for i in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn(0)
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / (reps * per_graph)


def cpu_baseline(target_s: float = 15.0):
    """The oracle (fp64, explicit Hadamard matrix) on a bounded sample of the
    same workload, on this host's cores."""
    import hr_inputs
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = os.cpu_count() or 1
    inp = hr_inputs.rht_inputs(rows=ROWS, n=N)
    x = inp.x

    def run(r0, r1):
        y64 = oracle.hadamard.rht(x[r0:r1].float().numpy(), inp.signs)
        codes, scales, _ = oracle.quant.quantize_groups(y64, GROUP, "f16")
        oracle.quant.pack_int4(codes)

    run(0, 512)                       # first call pays one-time costs
    t0 = time.perf_counter()
    run(0, 2048)
    per_row = (time.perf_counter() - t0) / 2048
    rows = int(min(ROWS, max(512, target_s / max(per_row, 1e-9))))
    rows -= rows % 512
    t0 = time.perf_counter()
    for r0 in range(0, rows, 4096):
        run(r0, min(rows, r0 + 4096))
    dt = time.perf_counter() - t0
    gbs = rht_alg_bytes(rows, N, GROUP) / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"first {rows} of {ROWS} rows (bf16 x {N}, G={GROUP}, fp16 scales), "
                      f"{dt:.1f} s wall, dense fp64 Hadamard matrix product + quantization"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="time only the headline kernel")
    ap.add_argument("--profile-gemm", action="store_true",
                    help="run only the 4096^3 W4A4 and W4A8 GEMMs, --steps times each (for counters)")
    ap.add_argument("--profile-mixed", action="store_true",
                    help="run only the bf16 16384x14336 (m = 7) mixed-radix quantization, --steps times "
                         "(for counters)")
    ap.add_argument("--profile-run", action="store_true",
                    help="run the headline kernel and a plain copy (for rocprofv3 --pmc), print nothing")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="turn rocprofv3 outputs under DIR (ktrace/, fetch/, write/) into profiles/")
    args = ap.parse_args(argv)
    if args.summarize_profile:
        return summarize_profile(args.summarize_profile)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only (rows are independent; see DESIGN.md "
              "for how it would shard); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import hr_inputs
    import hadamard_rotation_int4_amd as hr

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- headline workload: 3 buffer sets (>= 1 GB) so consecutive steps do
    # not hit in the 256 MB last-level cache
    inp = hr_inputs.rht_inputs(rows=ROWS, n=N)
    nbuf = 3
    xs = [inp.x.to(dev) for _ in range(nbuf)]
    d = torch.from_numpy(inp.signs).to(dev)
    codes = [torch.empty((ROWS, N // 2), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    scales = [torch.empty((ROWS, N // GROUP), dtype=torch.float16, device=dev) for _ in range(nbuf)]

    def step(i):
        hr.rotate_quant_int4(xs[i], GROUP, d, codes=codes[i], scales=scales[i])

    if args.profile_gemm:
        gi = hr_inputs.gemm_inputs(M=4096)
        g8 = hr_inputs.gemm_w4a8_inputs(M=4096)
        t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
        wd, swd = t(gi.w_codes), t(gi.w_scales)
        cg = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        for call, a_codes, a_scales in ((hr.w4a4_gemm, t(gi.a_codes), t(gi.a_scales)),
                                        (hr.w4a8_gemm, t(g8.a_codes), t(g8.a_scales))):
            for _ in range(args.steps):
                call(a_codes, a_scales, wd, swd, 128, out=cg)
        torch.cuda.synchronize()
        return 0

    if args.profile_mixed:
        mi = hr_inputs.mixed_inputs()
        xm = mi.x.to(dev)
        dm, om = torch.from_numpy(mi.signs).to(dev), torch.from_numpy(mi.block).to(dev)
        cm = torch.empty((mi.rows, mi.m * mi.p // 2), dtype=torch.uint8, device=dev)
        sm = torch.empty((mi.rows, mi.m * mi.p // 128), dtype=torch.float16, device=dev)
        for _ in range(args.steps):
            hr.rotate_quant_int4(xm, 128, dm, om, codes=cm, scales=sm)
        torch.cuda.synchronize()
        return 0

    if args.profile_run:
        for i in range(args.steps):
            step(i % nbuf)
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)         # plain elementwise pass: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        return 0

    ms = _timed(step, args.steps, args.warmup, nbuf)
    alg = rht_alg_bytes(ROWS, N, GROUP)
    gbs = alg / (ms * 1e-3) / 1e9
    kernels = {"rht_quant_bf16_65536x2048_g128": {"ms": ms, "GB/s": gbs,
                                                  "frac_hbm": gbs / HBM_PEAK_GBS, "bytes": alg}}

    if not args.only_main:
        s32 = [torch.empty((ROWS, N // 32), dtype=torch.float16, device=dev) for _ in range(nbuf)]
        ms32 = _timed(lambda i: hr.rotate_quant_int4(xs[i], 32, d, codes=codes[i], scales=s32[i]),
                      args.steps, args.warmup, nbuf)
        b32 = rht_alg_bytes(ROWS, N, 32)
        kernels["rht_quant_bf16_65536x2048_g32"] = {"ms": ms32, "GB/s": b32 / ms32 / 1e6,
                                                    "frac_hbm": b32 / ms32 / 1e6 / HBM_PEAK_GBS,
                                                    "bytes": b32}
        del s32
        # int8 activation codes for the W4A8 GEMM (one byte per code)
        c8 = [torch.empty((ROWS, N), dtype=torch.int8, device=dev) for _ in range(nbuf)]
        ms8 = _timed(lambda i: hr.rotate_quant_int8(xs[i], GROUP, d, codes=c8[i], scales=scales[i]),
                     args.steps, args.warmup, nbuf)
        b8 = ROWS * N * 2 + ROWS * N + ROWS * (N // GROUP) * 2
        kernels["rht_quant_int8_bf16_65536x2048_g128"] = {"ms": ms8, "GB/s": b8 / ms8 / 1e6,
                                                          "frac_hbm": b8 / ms8 / 1e6 / HBM_PEAK_GBS,
                                                          "bytes": b8}
        del c8
        yf = torch.empty((ROWS, N), dtype=torch.float32, device=dev)
        msr = _timed(lambda i: hr.rotate(xs[i], d, out=yf), args.steps, args.warmup, nbuf)
        br = ROWS * N * 2 + ROWS * N * 4
        kernels["rotate_bf16_to_f32_65536x2048"] = {"ms": msr, "GB/s": br / msr / 1e6,
                                                    "frac_hbm": br / msr / 1e6 / HBM_PEAK_GBS,
                                                    "bytes": br}
        del yf
        dq = torch.empty((ROWS, N), dtype=torch.float32, device=dev)
        msd = _timed(lambda i: hr.dequant_int4(codes[i], scales[i], GROUP, out=dq),
                     args.steps, args.warmup, nbuf)
        bd = ROWS * N // 2 + ROWS * (N // GROUP) * 2 + ROWS * N * 4
        kernels["dequant_int4_65536x2048_g128"] = {"ms": msd, "GB/s": bd / msd / 1e6,
                                                   "frac_hbm": bd / msd / 1e6 / HBM_PEAK_GBS,
                                                   "bytes": bd}
        del dq
        del xs, codes, scales

        # mixed radix 16384 x (7*2048), G=128
        mi = hr_inputs.mixed_inputs()
        xm = mi.x.to(dev)
        dm = torch.from_numpy(mi.signs).to(dev)
        om = torch.from_numpy(mi.block).to(dev)
        cm = torch.empty((mi.rows, mi.m * mi.p // 2), dtype=torch.uint8, device=dev)
        sm = torch.empty((mi.rows, mi.m * mi.p // 128), dtype=torch.float16, device=dev)
        msm = _timed(lambda i: hr.rotate_quant_int4(xm, 128, dm, om, codes=cm, scales=sm),
                     max(5, args.steps // 2), 3)
        bm = rht_alg_bytes(mi.rows, mi.m * mi.p, 128)
        kernels["mixed_radix_quant_bf16_16384x14336_g128"] = {
            "ms": msm, "GB/s": bm / msm / 1e6, "frac_hbm": bm / msm / 1e6 / HBM_PEAK_GBS, "bytes": bm}
        del xm, cm, sm

        # butterfly fp32 32768 x 4096 -> fp32, and fused G=64 quantization
        bi = hr_inputs.butterfly_inputs()
        xb = torch.from_numpy(bi.x).to(dev)
        co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(dev), False)
        pb = torch.from_numpy(bi.perm).to(dev)
        yb = torch.empty_like(xb)
        msb = _timed(lambda i: hr.butterfly_apply(xb, co, False, pb, out=yb),
                     max(5, args.steps // 2), 3)
        bb = bi.rows * bi.n * 8
        kernels["butterfly_f32_32768x4096"] = {"ms": msb, "GB/s": bb / msb / 1e6,
                                               "frac_hbm": bb / msb / 1e6 / HBM_PEAK_GBS, "bytes": bb}
        msbq = _timed(lambda i: hr.butterfly_apply(xb, co, False, pb, want_y=False, group=64),
                      max(5, args.steps // 2), 3)
        bbq = bi.rows * bi.n * 4 + bi.rows * bi.n // 2 + bi.rows * (bi.n // 64) * 2
        kernels["butterfly_quant_f32_32768x4096_g64"] = {
            "ms": msbq, "GB/s": bbq / msbq / 1e6, "frac_hbm": bbq / msbq / 1e6 / HBM_PEAK_GBS,
            "bytes": bbq}
        del xb, yb

        # HARP general processor: 4096 rows of d = 5120 = (8, 8, 8, 5, 2)
        hi = hr_inputs.harp_inputs()
        fb = torch.from_numpy(np.concatenate([f.ravel() for f in hi.fallbacks])).to(dev)
        hblk = hr.harp_blocks(hi.radices, torch.from_numpy(hi.theta).to(dev), fb)
        hx = torch.from_numpy(hi.x).to(dev)
        hy = torch.empty_like(hx)
        tab = hblk.numel() * 4                 # the block table, read once
        msh = _timed(lambda i: hr.harp_apply(hx, hi.radices, hblk, out=hy), max(5, args.steps // 2), 3)
        bh = hi.rows * hi.d * 8 + tab
        kernels["harp_f32_4096x5120_r88852"] = {"ms": msh, "GB/s": bh / msh / 1e6,
                                                "frac_hbm": bh / msh / 1e6 / HBM_PEAK_GBS, "bytes": bh}
        mshq = _timed(lambda i: hr.harp_apply(hx, hi.radices, hblk, want_y=False, group=128),
                      max(5, args.steps // 2), 3)
        bhq = hi.rows * (hi.d * 4 + hi.d // 2 + (hi.d // 128) * 2) + tab
        kernels["harp_quant_f32_4096x5120_r88852_g128"] = {
            "ms": mshq, "GB/s": bhq / mshq / 1e6, "frac_hbm": bhq / mshq / 1e6 / HBM_PEAK_GBS,
            "bytes": bhq}
        del hx, hy, hblk

        # W4A4 GEMM 4096^3 and M=16, G=128
        for M in (4096, 16):
            gi = hr_inputs.gemm_inputs(M=M)
            t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
            ad, sad, wd, swd = t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales)
            cg = torch.empty((M, 4096), dtype=torch.float32, device=dev)
            # a decode-sized call is shorter than the Python call that issues it
            timer = _timed if M > 16 else _timed_graph
            msg = timer(lambda i: hr.w4a4_gemm(ad, sad, wd, swd, 128, out=cg), args.steps,
                        args.warmup)
            ops = 2 * M * 4096 * 4096
            byts = M * 2048 + 4096 * 2048 + (M + 4096) * 32 * 2 + M * 4096 * 4
            kernels[f"w4a4_gemm_{M}x4096x4096_g128"] = {
                "ms": msg, "TOPS": ops / msg / 1e9, "frac_int8_peak": ops / msg / 1e9 / INT8_PEAK_TOPS,
                "GB/s": byts / msg / 1e6, "ops": ops, "bytes": byts,
                "timing": "eager launches" if M > 16 else "HIP graph of 20 launches, replayed"}

        # one decode step with online rotation: the 16 activation rows (bf16, K =
        # 4096) are rotated and quantized, then multiplied by the int4 weights;
        # both launches in one graph, against the GEMM alone above
        gi = hr_inputs.gemm_inputs(M=16)
        wd, swd = (torch.from_numpy(gi.w_codes).to(dev), torch.from_numpy(gi.w_scales).to(dev))
        ri = hr_inputs.rht_inputs(rows=16, n=4096, seed=7)
        xa, da = ri.x.to(dev), torch.from_numpy(ri.signs).to(dev)
        ac = torch.empty((16, 2048), dtype=torch.uint8, device=dev)
        asc = torch.empty((16, 32), dtype=torch.float16, device=dev)
        cg = torch.empty((16, 4096), dtype=torch.float32, device=dev)

        def decode_step(i):
            hr.rotate_quant_int4(xa, 128, da, codes=ac, scales=asc)
            hr.w4a4_gemm(ac, asc, wd, swd, 128, out=cg)

        msd = _timed_graph(decode_step, args.steps, args.warmup)
        msg16 = kernels["w4a4_gemm_16x4096x4096_g128"]["ms"]
        kernels["decode_step_rotate_quant_w4a4_16x4096x4096_g128"] = {
            "ms": msd, "gemm_alone_ms": msg16, "rotation_overhead": msd / msg16 - 1.0,
            "timing": "HIP graph of 20 steps (2 launches each), replayed"}

        # W4A8 GEMM: int8 activations, the same int4 weights
        for M in (4096, 16):
            gi = hr_inputs.gemm_w4a8_inputs(M=M)
            t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
            ad, sad, wd, swd = t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales)
            cg = torch.empty((M, 4096), dtype=torch.float32, device=dev)
            timer = _timed if M > 16 else _timed_graph
            msg = timer(lambda i: hr.w4a8_gemm(ad, sad, wd, swd, 128, out=cg), args.steps,
                        args.warmup)
            ops = 2 * M * 4096 * 4096
            byts = M * 4096 + 4096 * 2048 + (M + 4096) * 32 * 2 + M * 4096 * 4
            kernels[f"w4a8_gemm_{M}x4096x4096_g128"] = {
                "ms": msg, "TOPS": ops / msg / 1e9, "frac_int8_peak": ops / msg / 1e9 / INT8_PEAK_TOPS,
                "GB/s": byts / msg / 1e6, "ops": ops, "bytes": byts,
                "timing": "eager launches" if M > 16 else "HIP graph of 20 launches, replayed"}

        # W8A8 GEMM: the W4A4 workload with its codes held one per byte
        g8 = hr_inputs.gemm_i8_inputs(M=4096)
        t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
        ad, sad, wd, swd = t(g8.a_codes), t(g8.a_scales), t(g8.w_codes), t(g8.w_scales)
        cg = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        msg = _timed(lambda i: hr.w8a8_gemm(ad, sad, wd, swd, 128, out=cg), args.steps, args.warmup)
        ops = 2 * 4096 ** 3
        byts = 2 * 4096 * 4096 + 2 * 4096 * 32 * 2 + 4096 * 4096 * 4
        kernels["w8a8_gemm_4096x4096x4096_g128"] = {
            "ms": msg, "TOPS": ops / msg / 1e9, "frac_int8_peak": ops / msg / 1e9 / INT8_PEAK_TOPS,
            "GB/s": byts / msg / 1e6, "ops": ops, "bytes": byts, "timing": "eager launches",
            "codes": "int4 values held in int8 (uniform -7..7)"}

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "rotate_quant_int4: bf16 65536x2048 -> int4 codes + fp16 scales, "
                               "G=128, seeded signs, 0.1% outlier channels x50",
                   "rows": ROWS, "n": N, "group": GROUP},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic()},
    }
    if not args.only_main:
        # a plain elementwise pass over COPY_BYTES (read and write) as the
        # practical HBM ceiling of the box the line was measured on
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        msc = _timed(lambda i: torch.neg(src, out=dst), 20, 5)
        out["practical_ceiling"] = {"kernel": "torch.neg over 512 MiB bf16 (read + write)",
                                    "GB/s": round(2 * COPY_BYTES / msc / 1e6, 1)}
        del src, dst
    g4096 = kernels.get("w4a4_gemm_4096x4096x4096_g128")
    if g4096:
        out["w4a4_gemm_tops"] = round(g4096["TOPS"], 1)
        out["w4a4_gemm_frac_int8_peak"] = round(g4096["frac_int8_peak"], 4)
    out["kernels"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in kernels.items()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


def _read_csv(pattern):
    rows = []
    for path in glob.glob(pattern, recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _counter_per_dispatch(rows, kernel_substr, counter):
    vals = [float(r["Counter_Value"]) for r in rows
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


GEMM_COUNTER_PASSES = (
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES",
    "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY "
    "SQ_ACTIVE_INST_ANY SQ_INSTS_SALU SQ_INSTS_VMEM_RD",
)


def _summarize_counters(d, prefix, kernels, out_name, title, run_flag):
    """Per-dispatch counter averages of the named kernels from the passes under
    d/<prefix>1, d/<prefix>2 (one rocprofv3 --pmc run each)."""
    rows = []
    for i in range(1, len(GEMM_COUNTER_PASSES) + 1):
        rows += _read_csv(os.path.join(d, f"{prefix}{i}", "**", "*counter_collection.csv"))
    if not rows:
        return
    lines = [f"# rocprofv3 --pmc counters, per dispatch, of {title}",
             f"# command, one per pass: rocprofv3 --pmc <pass> -d <dir>/{prefix}<i> -o run --output-format csv "
             f"-- python bench.py {run_flag} --steps 10"]
    for i, pmc in enumerate(GEMM_COUNTER_PASSES, 1):
        lines.append(f"# pass {i}: {pmc}")
    for label, name in kernels:
        vals = {}
        for pmc in " ".join(GEMM_COUNTER_PASSES).split():
            v, n = _counter_per_dispatch(rows, name, pmc)
            if v is not None:
                vals[pmc] = v
        if not vals:
            continue
        lines.append(f"{label} ({name}):")
        for k, v in vals.items():
            lines.append(f"  {k} = {v:.6g}")
        mf, va = vals.get("SQ_INSTS_MFMA"), vals.get("SQ_INSTS_VALU")
        if mf and va:
            lines.append(f"  VALU instructions per MFMA = {va / mf:.2f}")
        bc, al = vals.get("SQ_LDS_BANK_CONFLICT"), vals.get("SQ_ACTIVE_INST_LDS")
        if bc is not None and al:
            lines.append(f"  LDS bank-conflict cycles / LDS-active cycles = {bc / al:.4f}")
        mb, co = vals.get("SQ_VALU_MFMA_BUSY_CYCLES"), vals.get("SQ_VALU_MFMA_COEXEC_CYCLES")
        if mb and co is not None:
            lines.append(f"  VALU co-issued during MFMA-busy cycles = {co / mb:.4f}")
        wv = vals.get("SQ_WAVES")
        if wv and va:
            lines.append(f"  VALU instructions per wave = {va / wv:.1f}")
    with open(os.path.join(PROFILES, out_name), "w") as f:
        f.write("\n".join(lines) + "\n")


def _summarize_gemm_counters(d):
    _summarize_counters(d, "gemm_p", (("W4A4", "w4a4_gemm_tile_kernel<128, true, false, false>"),
                                      ("W4A8", "w4a4_gemm_tile_kernel<128, true, false, true>")),
                        "w4a4_w4a8_gemm_4096_g128.counters.txt",
                        "the 4096^3 G=128 fp16-scale GEMM tile kernels", "--profile-gemm")


def _summarize_mixed_counters(d):
    _summarize_counters(d, "mixed_p", (("mixed radix m = 7", "mixed2048_mfma_kernel<7, 128, true, false, false>"),),
                        "mixed_radix_quant_bf16_16384x14336_g128.counters.txt",
                        "the bf16 16384x14336 (m = 7, O_7 dense) G=128 mixed-radix quantization kernel",
                        "--profile-mixed")


def summarize_profile(d):
    """Write the kernel-duration summary and the HBM-traffic summary of the
    headline kernel from rocprofv3 outputs under d/ktrace, d/fetch, d/write."""
    os.makedirs(PROFILES, exist_ok=True)
    stats = _read_csv(os.path.join(d, "ktrace", "**", "*kernel_stats.csv"))
    lines = ["# rocprofv3 --kernel-trace --stats summary (times in microseconds)",
             "# command: rocprofv3 --kernel-trace --stats -d <dir>/ktrace -o run -- "
             "python bench.py --steps 20 --warmup 5 --no-cpu-baseline",
             "kernel | calls | avg_us | min_us | max_us | total_%"]
    for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        lines.append(" | ".join([r["Name"][:110], r["Calls"],
                                 f"{float(r['AverageNs']) / 1e3:.2f}", f"{float(r['MinNs']) / 1e3:.2f}",
                                 f"{float(r['MaxNs']) / 1e3:.2f}", f"{float(r['Percentage']):.2f}"]))
    with open(os.path.join(PROFILES, "kernel_stats_bench_default.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    fetch = _read_csv(os.path.join(d, "fetch", "**", "*counter_collection.csv"))
    write = _read_csv(os.path.join(d, "write", "**", "*counter_collection.csv"))
    kf, nk = _counter_per_dispatch(fetch, MAIN_KERNEL_NAME, "FETCH_SIZE")
    kw, _ = _counter_per_dispatch(write, MAIN_KERNEL_NAME, "WRITE_SIZE")
    cf = cw = None
    nc = 0
    copy_kernel = None
    for pat in ("neg_kernel",):           # the elementwise negation of COPY_BYTES
        cf, nc = _counter_per_dispatch(fetch, pat, "FETCH_SIZE")
        cw, _ = _counter_per_dispatch(write, pat, "WRITE_SIZE")
        if cf and cw:
            copy_kernel = pat
            break
    out = {"kernel": MAIN_KERNEL_NAME, "workload": "bf16 65536x2048, G=128, fp16 scales",
           "source_hash": main_kernel_hash(),
           "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -d <dir>/fetch -o run -- "
                      "python bench.py --profile-run --steps 20",
           "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": nk,
           "copy_kernel_match": copy_kernel, "copy_bytes": COPY_BYTES, "copy_fetch_kib": cf,
           "copy_write_kib": cw, "copy_dispatches": nc}
    _summarize_gemm_counters(d)
    _summarize_mixed_counters(d)
    if None not in (kf, kw, cf, cw):
        ff = COPY_BYTES / (cf * 1024.0)
        fw = COPY_BYTES / (cw * 1024.0)
        out.update({"fetch_scale": ff, "write_scale": fw,
                    "fetch_bytes_per_launch": kf * 1024.0 * ff,
                    "write_bytes_per_launch": kw * 1024.0 * fw,
                    "traffic_bytes_per_launch": kf * 1024.0 * ff + kw * 1024.0 * fw,
                    "algorithmic_bytes_per_launch": rht_alg_bytes(ROWS, N, GROUP)})
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
