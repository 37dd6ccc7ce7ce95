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
FP6_PEAK_TOPS = 10100.0        # MI355X dense fp6 / fp4 MFMA peak
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


class _Progress(dict):
    """The kernel table; each entry also prints a progress line on stderr
    (stdout carries only the one JSON line)."""

    def __setitem__(self, k, v):
        super().__setitem__(k, v)
        print(f"bench.py: {k} done", file=sys.stderr, flush=True)


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


class Timing(float):
    """ms per call (the mean over the timed region) that also carries the
    per-call median and minimum."""

    def __new__(cls, mean, median, minimum):
        t = super().__new__(cls, mean)
        t.median = median
        t.min = minimum
        return t


def _timed(fn, steps, warmup, nbuf=1):
    """Run fn(i) warmup + steps times on the current stream (the stream the
    library launches on).  HIP events bracket the timed launches: the mean is
    the whole timed region over the number of launches.  The region is cut
    into batches of at least 10 launches by one event each (an event between
    every launch would add about 2 us to each); the median and the minimum are
    over the per-launch means of those batches.  Returns a Timing (ms)."""
    import torch
    for i in range(warmup):
        fn(i % nbuf)
    torch.cuda.synchronize()
    nb = min(20, max(1, steps // 10))
    cuts = [round(k * steps / nb) for k in range(nb + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    ev[0].record()
    for b in range(nb):
        for i in range(cuts[b], cuts[b + 1]):
            fn(i % nbuf)
        ev[b + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[b].elapsed_time(ev[b + 1]) / (cuts[b + 1] - cuts[b]) for b in range(nb)])
    return Timing(ev[0].elapsed_time(ev[nb]) / steps, float(np.median(per)), float(per.min()))


def _timed_graph(fn, steps, warmup, per_graph=20, nbuf=1):
    """Like _timed, for kernels shorter than a Python call: per_graph calls
    (fn(k % nbuf), k < per_graph) are captured once in a HIP graph, and the
    timed region replays it, so the host's launch cost per call is not what
    gets measured.  The warmup steps run as replays of the same graph right
    before the timed ones: the first 10-15 replays after a capture run up to
    30% slower (the headline: 76 us down to 59 us per call), so a warmup done
    before the capture would leave that transient inside the timed region.
    Median and minimum are per replay.  Returns a Timing (ms per call)."""
    import torch
    for i in range(min(warmup, 2 * per_graph)):
        fn(i % nbuf)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(per_graph):
            fn(k % nbuf)
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    for _ in range(max(3, -(-warmup // per_graph))):
        graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        graph.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]) / per_graph
    return Timing(ev[0].elapsed_time(ev[reps]) / (reps * per_graph), float(np.median(per)),
                  float(per.min()))


def _entry(t, **kw):
    """A kernels[] entry: mean ms plus the per-call median and minimum."""
    d = {"ms": float(t), "ms_median": t.median, "ms_min": t.min}
    d.update(kw)
    return d


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
            "cpu_model": cpu_model(),
            "sample": f"first {rows} of {ROWS} rows (bf16 x {N}, G={GROUP}, fp16 scales), "
                      f"{dt:.1f} s wall, dense fp64 Hadamard matrix product + quantization"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def build_cpu_fwht(out_dir=None) -> str:
    """Compile bench_cpu_fwht.c (the fast CPU baseline) for this host."""
    import subprocess
    out_dir = out_dir or os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "bench_cpu_fwht")
    cmd = ["gcc", "-O3", "-march=native", "-fopenmp", os.path.join(HERE, "bench_cpu_fwht.c"), "-o", exe,
           "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def cpu_fast_baseline(reps: int = 5):
    """The fair CPU number: an O(n log n) fast Walsh-Hadamard transform plus
    int4 quantization in C with OpenMP (bench_cpu_fwht.c, written apart from
    the oracle), over the whole headline workload on this host's cores; the
    best of ``reps`` passes (inputs already in memory)."""
    import subprocess
    import tempfile
    import hr_inputs
    exe = build_cpu_fwht()
    inp = hr_inputs.rht_inputs(rows=ROWS, n=N)
    with tempfile.TemporaryDirectory() as td:
        xf, sf = os.path.join(td, "x.bf16"), os.path.join(td, "signs.i8")
        inp.x.view(__import__("torch").int16).numpy().tofile(xf)
        inp.signs.astype(np.int8).tofile(sf)
        r = subprocess.run([exe, xf, sf, str(ROWS), str(N), str(GROUP), str(reps)], check=True,
                           capture_output=True, text=True)
    res = json.loads(r.stdout.strip().splitlines()[-1])
    gbs = rht_alg_bytes(ROWS, N, GROUP) / res["best_s"] / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": res["threads"],
            "kind": "O(n log n) FWHT + int4 quantization in C, OpenMP over rows, gcc -O3 -march=native",
            "cpu_model": cpu_model(),
            "sample": f"all {ROWS} rows (bf16 x {N}, G={GROUP}, fp16 scales), best of {reps} passes "
                      f"({res['best_s'] * 1e3:.1f} ms; mean {res['mean_s'] * 1e3:.1f} ms)"}


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
    ap.add_argument("--profile-butterfly", action="store_true",
                    help="run only the fp32 32768x4096 butterfly, fp32 output and G=64 codes only, --steps "
                         "times each (for counters)")
    ap.add_argument("--profile-harp", action="store_true",
                    help="run only the HARP processor on fp32 4096x5120, (8, 8, 8, 5, 2), fp32 output, "
                         "--steps times (for counters)")
    ap.add_argument("--profile-run", action="store_true",
                    help="run the headline kernel and a plain copy (for rocprofv3 --pmc), print nothing")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="turn rocprofv3 outputs under DIR (ktrace/, fetch/, write/) into profiles/")
    args = ap.parse_args(argv)
    if args.summarize_profile:
        return summarize_profile(args.summarize_profile)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only (rows are independent, so several GPUs "
              "would each take their own rows); run with --gpus 1", file=sys.stderr)
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
        a6, sta = hr.w4a4_to_fp6(t(gi.a_codes), t(gi.a_scales), 128)
        w6, stw = hr.w4a4_to_fp6(wd, swd, 128)
        for _ in range(args.steps):
            hr.w4a4_gemm_fp6(a6, sta, w6, stw, 128, 4096, out=cg)
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

    if args.profile_butterfly:
        bi = hr_inputs.butterfly_inputs()
        xb = torch.from_numpy(bi.x).to(dev)
        co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(dev), False)
        pb = torch.from_numpy(bi.perm).to(dev)
        yb = torch.empty_like(xb)
        for _ in range(args.steps):
            hr.butterfly_apply(xb, co, False, pb, out=yb)
        for _ in range(args.steps):
            hr.butterfly_apply(xb, co, False, pb, want_y=False, group=64)
        torch.cuda.synchronize()
        return 0

    if args.profile_harp:
        hi = hr_inputs.harp_inputs()
        fb = torch.from_numpy(np.concatenate([f.ravel() for f in hi.fallbacks])).to(dev)
        hblk = hr.harp_blocks(hi.radices, torch.from_numpy(hi.theta).to(dev), fb)
        hx = [torch.from_numpy(hi.x).to(dev) for _ in range(2)]
        hy = [torch.empty_like(hx[0]) for _ in range(2)]
        for i in range(args.steps):
            hr.harp_apply(hx[i % 2], hi.radices, hblk, out=hy[i % 2])
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

    # the timed steps are replays of a HIP graph of 20 launches (K a multiple
    # of 20; else of 10, else eager launches): the host then stays far ahead
    # of the GPU, so a pause of the Python process cannot leave the GPU idle
    # inside the timed region
    pg = 20 if args.steps % 20 == 0 else 10 if args.steps % 10 == 0 else 1
    if pg > 1:
        ms = _timed_graph(step, args.steps, args.warmup, per_graph=pg, nbuf=nbuf)
        how = f"HIP graph of {pg} launches over {nbuf} buffer sets, replayed {args.steps // pg} times"
    else:
        ms = _timed(step, args.steps, args.warmup, nbuf)
        how = "eager launches"
    alg = rht_alg_bytes(ROWS, N, GROUP)
    gbs = alg / (ms * 1e-3) / 1e9
    kernels = _Progress({"rht_quant_bf16_65536x2048_g128": _entry(ms, **{"GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                                                                         "bytes": alg, "timing": how})})

    def hbm_entry(t, byts, **kw):
        return _entry(t, **{"GB/s": byts / t / 1e6, "frac_hbm": byts / t / 1e6 / HBM_PEAK_GBS,
                            "bytes": byts}, **kw)

    def gemm_entry(t, M, byts, **kw):
        ops = 2 * M * 4096 * 4096
        return _entry(t, **{"TOPS": ops / t / 1e9, "frac_int8_peak": ops / t / 1e9 / INT8_PEAK_TOPS,
                            "GB/s": byts / t / 1e6, "ops": ops, "bytes": byts}, **kw)

    if not args.only_main:
        s32 = [torch.empty((ROWS, N // 32), dtype=torch.float16, device=dev) for _ in range(nbuf)]
        ms32 = _timed(lambda i: hr.rotate_quant_int4(xs[i], 32, d, codes=codes[i], scales=s32[i]),
                      args.steps, args.warmup, nbuf)
        kernels["rht_quant_bf16_65536x2048_g32"] = hbm_entry(ms32, rht_alg_bytes(ROWS, N, 32))
        del s32
        # int8 activation codes for the W4A8 GEMM (one byte per code)
        c8 = [torch.empty((ROWS, N), dtype=torch.int8, device=dev) for _ in range(nbuf)]
        ms8 = _timed(lambda i: hr.rotate_quant_int8(xs[i], GROUP, d, codes=c8[i], scales=scales[i]),
                     args.steps, args.warmup, nbuf)
        kernels["rht_quant_int8_bf16_65536x2048_g128"] = hbm_entry(
            ms8, ROWS * N * 2 + ROWS * N + ROWS * (N // GROUP) * 2)
        del c8
        # the codes straight into the tiled fp6 operand format of the fp6 GEMM
        # (6 bits per code), scales transposed
        f6 = [torch.empty((ROWS, N * 3 // 4), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        sf6 = [torch.empty((N // GROUP, ROWS), dtype=torch.float16, device=dev) for _ in range(nbuf)]
        msf6 = _timed(lambda i: hr.rotate_quant_fp6(xs[i], GROUP, d, out=f6[i], out_scales=sf6[i]),
                      args.steps, args.warmup, nbuf)
        kernels["rht_quant_fp6_bf16_65536x2048_g128"] = hbm_entry(
            msf6, ROWS * N * 2 + ROWS * N * 3 // 4 + ROWS * (N // GROUP) * 2)
        del f6, sf6
        # the same quantization without the rotation (the probe's plain operands)
        msq = _timed(lambda i: hr.quant_int4(xs[i], GROUP, codes=codes[i], scales=scales[i]),
                     args.steps, args.warmup, nbuf)
        kernels["quant_int4_bf16_65536x2048_g128"] = hbm_entry(msq, alg)
        yf = torch.empty((ROWS, N), dtype=torch.float32, device=dev)
        msr = _timed(lambda i: hr.rotate(xs[i], d, out=yf), args.steps, args.warmup, nbuf)
        kernels["rotate_bf16_to_f32_65536x2048"] = hbm_entry(msr, ROWS * N * 2 + ROWS * N * 4)
        del yf
        dq = torch.empty((ROWS, N), dtype=torch.float32, device=dev)
        msd = _timed(lambda i: hr.dequant_int4(codes[i], scales[i], GROUP, out=dq),
                     args.steps, args.warmup, nbuf)
        kernels["dequant_int4_65536x2048_g128"] = hbm_entry(
            msd, ROWS * N // 2 + ROWS * (N // GROUP) * 2 + ROWS * N * 4)
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
                     max(5, args.steps // 2), min(args.warmup, 30))
        kernels["mixed_radix_quant_bf16_16384x14336_g128"] = hbm_entry(
            msm, rht_alg_bytes(mi.rows, mi.m * mi.p, 128))
        del xm, cm, sm

        # butterfly fp32 32768 x 4096 -> fp32, and fused G=64 quantization
        bi = hr_inputs.butterfly_inputs()
        xb = torch.from_numpy(bi.x).to(dev)
        co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(dev), False)
        pb = torch.from_numpy(bi.perm).to(dev)
        yb = torch.empty_like(xb)
        msb = _timed(lambda i: hr.butterfly_apply(xb, co, False, pb, out=yb),
                     max(5, args.steps // 2), min(args.warmup, 30))
        kernels["butterfly_f32_32768x4096"] = hbm_entry(msb, bi.rows * bi.n * 8)
        msbq = _timed(lambda i: hr.butterfly_apply(xb, co, False, pb, want_y=False, group=64),
                      max(5, args.steps // 2), min(args.warmup, 30))
        kernels["butterfly_quant_f32_32768x4096_g64"] = hbm_entry(
            msbq, bi.rows * bi.n * 4 + bi.rows * bi.n // 2 + bi.rows * (bi.n // 64) * 2)
        del xb, yb

        # HARP general processor: 4096 rows of d = 5120 = (8, 8, 8, 5, 2); two
        # buffer sets (336 MB with the fp32 output) alternate, so a call does
        # not find its rows in the 256 MB last-level cache
        hi = hr_inputs.harp_inputs()
        fb = torch.from_numpy(np.concatenate([f.ravel() for f in hi.fallbacks])).to(dev)
        hblk = hr.harp_blocks(hi.radices, torch.from_numpy(hi.theta).to(dev), fb)
        hx = [torch.from_numpy(hi.x).to(dev) for _ in range(2)]
        hy = [torch.empty_like(hx[0]) for _ in range(2)]
        tab = hblk.numel() * 4                 # the block table, read once
        msh = _timed(lambda i: hr.harp_apply(hx[i], hi.radices, hblk, out=hy[i]),
                     max(6, args.steps // 2), min(args.warmup, 30), 2)
        kernels["harp_f32_4096x5120_r88852"] = hbm_entry(msh, hi.rows * hi.d * 8 + tab,
                                                         buffers="2 sets alternating")
        mshq = _timed(lambda i: hr.harp_apply(hx[i], hi.radices, hblk, want_y=False, group=128),
                      max(6, args.steps // 2), min(args.warmup, 30), 2)
        kernels["harp_quant_f32_4096x5120_r88852_g128"] = hbm_entry(
            mshq, hi.rows * (hi.d * 4 + hi.d // 2 + (hi.d // 128) * 2) + tab, buffers="2 sets alternating")
        del hx, hy, hblk

        t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
        # W4A4 GEMM 4096^3 and M=16, G=128
        gi = hr_inputs.gemm_inputs(M=4096)
        ad, sad, wd, swd = t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales)
        cg = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        msg = _timed(lambda i: hr.w4a4_gemm(ad, sad, wd, swd, 128, out=cg), args.steps, args.warmup)
        kernels["w4a4_gemm_4096x4096x4096_g128"] = gemm_entry(
            msg, 4096, 4096 * 2048 * 2 + 8192 * 32 * 2 + 4096 * 4096 * 4, timing="eager launches")
        # the same product on fp6 matrix cores: weights converted once (as a
        # model would at load time); "gemm" times the GEMM on converted
        # operands, "with_a_convert" adds the per-call activation conversion
        a6, sta = hr.w4a4_to_fp6(ad, sad, 128)
        w6, stw = hr.w4a4_to_fp6(wd, swd, 128)
        b6 = 2 * 4096 * 3072 + 8192 * 32 * 2 + 4096 * 4096 * 4
        ms6 = _timed(lambda i: hr.w4a4_gemm_fp6(a6, sta, w6, stw, 128, 4096, out=cg), args.steps, args.warmup)
        kernels["w4a4_gemm_fp6_4096x4096x4096_g128"] = gemm_entry(
            ms6, 4096, b6, timing="eager launches", operands="tiled fp6 (hr_w4a4_to_fp6)")

        def conv_gemm(i):
            hr.w4a4_to_fp6(ad, sad, 128, out=a6, out_scales=sta)
            hr.w4a4_gemm_fp6(a6, sta, w6, stw, 128, 4096, out=cg)
        ms6c = _timed(conv_gemm, args.steps, args.warmup)
        kernels["w4a4_gemm_fp6_with_a_convert_4096x4096x4096_g128"] = gemm_entry(
            ms6c, 4096, b6 + 4096 * 2048 + 4096 * 32 * 2 + 4096 * 3072 + 4096 * 32 * 2, timing="eager launches",
            operands="packed int4 activations converted per call, weights converted once")
        # the whole activation path from bf16 (rotation + quantization, then
        # the GEMM): into fp6 tiles + fp6 GEMM, against packed int4 + int8 GEMM
        ri = hr_inputs.rht_inputs(rows=4096, n=4096)
        xa, da = ri.x.to(dev), t(ri.signs)

        def rq_fp6_gemm(i):
            hr.rotate_quant_fp6(xa, 128, da, out=a6, out_scales=sta)
            hr.w4a4_gemm_fp6(a6, sta, w6, stw, 128, 4096, out=cg)

        def rq_int4_gemm(i):
            hr.rotate_quant_int4(xa, 128, da, codes=ad, scales=sad)
            hr.w4a4_gemm(ad, sad, wd, swd, 128, out=cg)
        ms_rf = _timed(rq_fp6_gemm, args.steps, args.warmup)
        ms_ri = _timed(rq_int4_gemm, args.steps, args.warmup)
        xbytes = 4096 * 4096 * 2
        kernels["rotate_quant_fp6_then_gemm_fp6_4096x4096x4096_g128"] = gemm_entry(
            ms_rf, 4096, b6 + xbytes + 4096 * 3072 + 4096 * 32 * 2, timing="eager launches",
            operands="bf16 activations rotated into fp6 tiles per call, weights converted once")
        kernels["rotate_quant_int4_then_gemm_4096x4096x4096_g128"] = gemm_entry(
            ms_ri, 4096, 4096 * 2048 * 2 + 8192 * 32 * 2 + 4096 * 4096 * 4 + xbytes + 4096 * 2048 + 4096 * 32 * 2,
            timing="eager launches", operands="bf16 activations rotated into packed int4 per call")
        del ad, sad, cg, a6, sta, w6, stw, xa

        # decode shapes (M = 16): a call is shorter than the Python call that
        # issues it, so calls are captured in a HIP graph and replayed.  "hot":
        # one weight copy, which stays in the 256 MB last-level cache; "cold":
        # 40 weight copies (336 MB) in turn, so every call reads its weights
        # from HBM
        NW = 40
        gi = hr_inputs.gemm_inputs(M=16)
        a16, sa16 = t(gi.a_codes), t(gi.a_scales)
        wds = [wd] + [wd.clone() for _ in range(NW - 1)]
        swds = [swd] + [swd.clone() for _ in range(NW - 1)]
        c16 = torch.empty((16, 4096), dtype=torch.float32, device=dev)
        b16 = 16 * 2048 + 4096 * 2048 + (16 + 4096) * 32 * 2 + 16 * 4096 * 4
        for mode, nb in (("hot", 1), ("cold", NW)):
            tm = _timed_graph(lambda i: hr.w4a4_gemm(a16, sa16, wds[i], swds[i], 128, out=c16),
                              args.steps, args.warmup, per_graph=NW, nbuf=nb)
            kernels[f"w4a4_gemm_16x4096x4096_g128_{mode}"] = gemm_entry(
                tm, 16, b16, timing=f"HIP graph of {NW} launches over {nb} weight copies, replayed")

        # one decode step with online rotation: the 16 activation rows (bf16,
        # K = 4096) are rotated and quantized, then multiplied by the int4
        # weights.  Two launches (hr_rotate_quant_int4, then hr_w4a4_gemm) or
        # one (hr_rotate_quant_w4a4_gemm: rotation in the GEMM's prologue)
        ri = hr_inputs.rht_inputs(rows=16, n=4096, seed=7)
        xa, da = ri.x.to(dev), torch.from_numpy(ri.signs).to(dev)
        ac = torch.empty((16, 2048), dtype=torch.uint8, device=dev)
        asc = torch.empty((16, 32), dtype=torch.float16, device=dev)

        def decode_two(i):
            hr.rotate_quant_int4(xa, 128, da, codes=ac, scales=asc)
            hr.w4a4_gemm(ac, asc, wds[i], swds[i], 128, out=c16)

        def decode_fused(i):
            hr.rotate_quant_w4a4_gemm(xa, wds[i], swds[i], 128, da, out=c16)

        for mode, nb in (("hot", 1), ("cold", NW)):
            g_ms = kernels[f"w4a4_gemm_16x4096x4096_g128_{mode}"]["ms"]
            t2 = _timed_graph(decode_two, args.steps, args.warmup, per_graph=NW, nbuf=nb)
            kernels[f"decode_step_rotate_quant_w4a4_16x4096x4096_g128_{mode}"] = _entry(
                t2, gemm_alone_ms=g_ms, rotation_overhead=float(t2) / g_ms - 1.0,
                timing=f"HIP graph of {NW} steps (2 launches each) over {nb} weight copies, replayed")
            t1 = _timed_graph(decode_fused, args.steps, args.warmup, per_graph=NW, nbuf=nb)
            kernels[f"decode_step_fused_rotate_quant_w4a4_16x4096x4096_g128_{mode}"] = _entry(
                t1, gemm_alone_ms=g_ms, rotation_overhead=float(t1) / g_ms - 1.0,
                two_launch_ms=float(t2),
                timing=f"HIP graph of {NW} steps (1 launch each) over {nb} weight copies, replayed")
        del wds, swds

        # W4A8 GEMM: int8 activations, the same int4 weights
        gi = hr_inputs.gemm_w4a8_inputs(M=4096)
        ad, sad, wd, swd = t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales)
        cg = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        msg = _timed(lambda i: hr.w4a8_gemm(ad, sad, wd, swd, 128, out=cg), args.steps, args.warmup)
        kernels["w4a8_gemm_4096x4096x4096_g128"] = gemm_entry(
            msg, 4096, 4096 * 4096 + 4096 * 2048 + 8192 * 32 * 2 + 4096 * 4096 * 4, timing="eager launches")
        del ad, sad, cg
        gi = hr_inputs.gemm_w4a8_inputs(M=16)
        a16, sa16 = t(gi.a_codes), t(gi.a_scales)
        wds = [wd] + [wd.clone() for _ in range(NW - 1)]
        swds = [swd] + [swd.clone() for _ in range(NW - 1)]
        for mode, nb in (("hot", 1), ("cold", NW)):
            tm = _timed_graph(lambda i: hr.w4a8_gemm(a16, sa16, wds[i], swds[i], 128, out=c16),
                              args.steps, args.warmup, per_graph=NW, nbuf=nb)
            kernels[f"w4a8_gemm_16x4096x4096_g128_{mode}"] = gemm_entry(
                tm, 16, 16 * 4096 + 4096 * 2048 + (16 + 4096) * 32 * 2 + 16 * 4096 * 4,
                timing=f"HIP graph of {NW} launches over {nb} weight copies, replayed")
        del wds, swds

        # W8A8 GEMM: the W4A4 workload with its codes held one per byte
        g8 = hr_inputs.gemm_i8_inputs(M=4096)
        ad, sad, wd, swd = t(g8.a_codes), t(g8.a_scales), t(g8.w_codes), t(g8.w_scales)
        cg = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        msg = _timed(lambda i: hr.w8a8_gemm(ad, sad, wd, swd, 128, out=cg), args.steps, args.warmup)
        kernels["w8a8_gemm_4096x4096x4096_g128"] = gemm_entry(
            msg, 4096, 2 * 4096 * 4096 + 2 * 4096 * 32 * 2 + 4096 * 4096 * 4, timing="eager launches",
            codes="int4 values held in int8 (uniform -7..7)")

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
    g6 = kernels.get("w4a4_gemm_fp6_4096x4096x4096_g128")
    if g6:
        out["w4a4_gemm_fp6_tops"] = round(g6["TOPS"], 1)
        out["w4a4_gemm_fp6_frac_int8_peak"] = round(g6["frac_int8_peak"], 4)
        out["w4a4_gemm_fp6_frac_fp6_peak"] = round(g6["TOPS"] / FP6_PEAK_TOPS, 4)
    out["ms_per_step_median"] = round(ms.median, 5)
    out["ms_per_step_min"] = round(ms.min, 5)
    out["kernels"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in kernels.items()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
        try:
            out["cpu_fast_baseline"] = cpu_fast_baseline()
        except Exception as e:          # a host without gcc/OpenMP: report, do not fail the line
            out["cpu_fast_baseline"] = {"error": f"{type(e).__name__}: {e}"}
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
    "TA_TA_BUSY_sum TD_TD_BUSY_sum TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
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
             f"-- python3 bench.py {run_flag} --steps 10"]
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
        # GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles; TA_TA_BUSY_sum the 256 CUs' texture addressers
        ga, ta = vals.get("GRBM_GUI_ACTIVE"), vals.get("TA_TA_BUSY_sum")
        if ga and ta:
            lines.append(f"  TA busy cycles per CU / GPU busy cycles = {(ta / 256) / (ga / 8):.3f}")
        th, tm = vals.get("TCC_HIT_sum"), vals.get("TCC_MISS_sum")
        if th is not None and tm:
            lines.append(f"  L2 hit rate = {th / (th + tm):.3f}")
    with open(os.path.join(PROFILES, out_name), "w") as f:
        f.write("\n".join(lines) + "\n")


def _summarize_gemm_counters(d):
    _summarize_counters(d, "gemm_p", (("W4A4", "w4a4_gemm_tile_kernel<128, true, false, false>"),
                                      ("W4A8", "w4a4_gemm_tile_kernel<128, true, false, true>"),
                                      ("W4A4 on fp6 matrix cores", "w4a4_gemm_fp6_tile_kernel<128, true, false>")),
                        "w4a4_w4a8_gemm_4096_g128.counters.txt",
                        "the 4096^3 G=128 fp16-scale GEMM tile kernels", "--profile-gemm")


def _summarize_mixed_counters(d):
    _summarize_counters(d, "mixed_p", (("mixed radix m = 7", "mixed2048_mfma_kernel<7, 128, true, false, false>"),),
                        "mixed_radix_quant_bf16_16384x14336_g128.counters.txt",
                        "the bf16 16384x14336 (m = 7, O_7 dense) G=128 mixed-radix quantization kernel",
                        "--profile-mixed")


def _summarize_butterfly_counters(d):
    _summarize_counters(d, "bf_p", (("fp32 output", "butterfly4096_kernel<false, false, true, 0, false>"),
                                    ("codes only, G = 64", "butterfly4096_kernel<false, false, false, 64, true>")),
                        "butterfly4096_32768x4096.counters.txt",
                        "the fp32 32768x4096 butterfly (12 Givens stages + gather), fp32 output and G=64 codes only",
                        "--profile-butterfly")


def _summarize_harp_counters(d):
    _summarize_counters(d, "harp_p", (("HARP apply, fp32 output", "harp_apply_kernel"),),
                        "harp_apply_f32_4096x5120_r88852.counters.txt",
                        "the HARP processor on fp32 4096x5120, schedule (8, 8, 8, 5, 2), fp32 output",
                        "--profile-harp")


def summarize_profile(d):
    """Write the kernel-duration summary and the HBM-traffic summary of the
    headline kernel from rocprofv3 outputs under d/ktrace, d/fetch, d/write."""
    os.makedirs(PROFILES, exist_ok=True)
    # each summary is written only from runs present under d (the counter
    # passes of one kernel can be refreshed without the others)
    _summarize_gemm_counters(d)
    _summarize_mixed_counters(d)
    _summarize_butterfly_counters(d)
    _summarize_harp_counters(d)
    stats = _read_csv(os.path.join(d, "ktrace", "**", "*kernel_stats.csv"))
    if not stats:
        return 0
    lines = ["# rocprofv3 --kernel-trace --stats summary (times in microseconds)",
             "# command: rocprofv3 --kernel-trace --stats -d <dir>/ktrace -o run --output-format csv -- "
             "python3 bench.py --no-cpu-baseline",
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
           "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -d <dir>/fetch (<dir>/write) -o run "
                      "--output-format csv -- python3 bench.py --profile-run --steps 20",
           "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": nk,
           "copy_kernel_match": copy_kernel, "copy_bytes": COPY_BYTES, "copy_fetch_kib": cf,
           "copy_write_kib": cw, "copy_dispatches": nc}
    if nk == 0:
        return 0
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
