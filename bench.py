"""Benchmark of the rotated-basis ternary projection on one MI355X.

A step is one pass of the decode hot path over one batch of synthetic input
at the largest single-GPU workload: the signed Walsh-Hadamard transform of a
bf16 hidden row (K = 5120) and the PQ2_0_G128 decode GEMV against the
248320 x 5120 vocabulary head (337.7 MB of planes), issued as the library's
one-launch decode step (tq_rotated_gemv_rowsplit).  Inputs are resident in
HBM before the timed region.  Steps alternate between two distinct copies of
the planes (675 MB, more than twice the 256 MB Infinity Cache) so the weight
stream comes from HBM, and the steps are launched as one HIP graph.

Printed: one JSON line with the step throughput (algorithmic GB/s), the
roofline of the step's kernel (algorithmic bytes per launch over its mean
duration, from HIP events on its stream around the timed replay), the prefill
GEMM's TFLOP/s with its matrix-core roofline, the float64 oracle's CPU
throughput on a bounded sample of the same workload, and secondary figures for
the other workloads (the FFN gate/up decode step, the PTQ1_0 down projection
at batch 1/4/8, the one-launch head with the greedy token, embedding rows,
the plain-read bandwidth floor, the transcoder and the G64 expansion).
"""

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
INFINITY_CACHE = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    return ap.parse_args()


def copies_for(nbytes, minimum=2):
    return max(minimum, -(-2 * INFINITY_CACHE // nbytes))


def event_timed(torch, fn, launches):
    """Mean GPU duration (s) of fn(i) over `launches` calls.  The calls are
    captured once as a HIP graph on the current stream and the replay is
    bracketed by two HIP events on that stream: a host loop of launches
    cannot keep up with kernels of a few microseconds, so it would time the
    host, not the kernel."""
    stream = torch.cuda.current_stream()
    fn(0)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(launches):
            fn(i)
    g.replay()
    stream.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.replay()
    end.record(stream)
    end.synchronize()
    del g
    return start.elapsed_time(end) / 1e3 / launches


def load_counters(name, source):
    """Counter figures from a committed rocprofv3 summary, or None when the
    kernel source changed since they were taken."""
    path = os.path.join(HERE, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = open(os.path.join(HERE, "ternary_quantized_amd", "csrc", source), "rb").read()
    if rec.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the projection path here is single-device "
              "(multi-GPU sharding is a design note, not implemented); use --gpus 1",
              file=sys.stderr)
        return 2

    import torch
    import ternary_quantized_amd as tq
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bits_dev(a, dtype):
        return to_dev(np.asarray(a, np.uint16).view(np.int16)).view(dtype)

    # ------------------------------------- the step: config 4 vocabulary head
    c4 = synth.make_config(4)
    fmt, n, k = c4["fmt"], c4["n"], c4["k"]
    payload = tq.pack_rowsplit(fmt, c4["trits"], c4["scale_bits"])
    del c4["trits"]
    plane_bytes = payload.size
    ncopy = copies_for(plane_bytes)
    copies = [to_dev(payload)]
    copies += [copies[0].clone() for _ in range(ncopy - 1)]
    x = bits_dev(c4["x"], torch.bfloat16)
    signs = bits_dev(c4["sign_bits"], torch.bfloat16)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)

    def step(i):
        tq.rotated_gemv_rowsplit(copies[i % ncopy], fmt, n, k, x, signs, out=y)

    # algorithmic bytes of a step (one launch): planes + x (bf16) + signs
    # (bf16) + y (fp32)
    step_bytes = plane_bytes + 2 * k + 2 * k + 4 * n

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(ncopy):
            step(i)
    torch.cuda.synchronize()

    def capture(nsteps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(nsteps):
                step(i)
        return g

    g_warm = capture(max(1, args.warmup))
    g_timed = capture(args.steps)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if args.warmup > 0:
        with torch.cuda.stream(stream):
            g_warm.replay()
    torch.cuda.synchronize()
    # a graph replays on the current stream: make it the capture stream, so
    # that the events bracket the replay on the stream its kernels run on
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        ev0.record(stream)
        g_timed.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes * args.steps / elapsed / 1e9
    # every launch of the timed replay is the step's one kernel, so the HIP
    # events around the replay give its mean launch duration
    step_mean = ev0.elapsed_time(ev1) / 1e3 / args.steps

    # correctness spot check: the graph's last step equals an eager step on
    # the same copy, bit for bit
    y_graph = y.clone()
    step((args.steps - 1) % ncopy)
    torch.cuda.synchronize()
    if not torch.equal(y_graph, y):
        print("bench: graph replay result differs from eager result", file=sys.stderr)
        return 1
    del g_warm, g_timed

    achieved = step_bytes / step_mean / 1e9
    counters = load_counters("head_rotated_gemv_248320x5120_b1_counters.json", "tq_gemv_f4.h")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": counters["hbm_bytes_per_dispatch"] if counters else None,
                "kernel": "gemv_f4_kernel (fused signed transform + PQ2_0 GEMV on the fp8 x fp4 "
                          "matrix cores, 248320 x 5120, batch 1, bf16 x)",
                "bytes_per_launch": step_bytes, "mean_launch_us": round(step_mean * 1e6, 3),
                "launches": args.steps,
                "timing": "hip events on the launch stream around the timed graph replay"}

    # ------------------------------------------ prefill GEMM (config 5)
    with torch.cuda.stream(stream):
        prefill = bench_prefill(torch, tq, synth, to_dev, bits_dev)

    secondary = {}
    if not args.no_secondary:
        secondary.update(bench_secondary(torch, tq, synth, to_dev, bits_dev, stream, copies, c4))
    del copies
    torch.cuda.empty_cache()

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        secondary["copy_calibration_bytes"] = src.numel()

    # ------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(synth)
        if not args.no_secondary:
            cpu["other_rows"] = oracle_rows(synth)

    out = {
        "metric": "ternary GEMV achieved HBM GB/s (% of peak) + prefill GEMM TFLOP/s, 1xMI355X",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xternary->f32",
        "data": "synthetic (seeded; shapes and value recipes of the 27B model's vocabulary head, "
                "no real weights)",
        "config": {"workload": "vocabulary head decode step: signed WHT (K=5120, bf16 in) + "
                               "PQ2_0_G128 GEMV N=248320 K=5120 batch 1, one launch",
                   "n": n, "k": k, "batch": 1, "format": fmt,
                   "weight_copies_rotated": ncopy, "step_bytes": step_bytes,
                   "launch": "hip graph of all timed steps"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "prefill_gemm": prefill,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out))
    return 0


def bench_prefill(torch, tq, synth, to_dev, bits_dev):
    """Config 5: 2048 x 5120 bf16 rows -> signed transform (binary16 out) ->
    GEMM against the 17408 x 5120 PQ2_0 planes on the matrix cores."""
    c5 = synth.make_config(5)
    n5, k5 = c5["n"], c5["k"]
    p5 = to_dev(tq.pack_rowsplit(c5["fmt"], c5["trits"], c5["scale_bits"]))
    x5 = bits_dev(c5["x"], torch.bfloat16)
    s5 = bits_dev(c5["sign_bits"], torch.bfloat16)
    m5 = int(x5.shape[0])
    xr5 = torch.empty((m5, k5), dtype=torch.float16, device=x5.device)
    wmean = event_timed(torch, lambda i: tq.hadamard_signed(x5, s5, out=xr5), 10)
    y5 = torch.empty((m5, n5), dtype=torch.float32, device=x5.device)
    gmean = event_timed(torch, lambda i: tq.gemm_rowsplit(p5, c5["fmt"], n5, k5, xr5, out=y5), 20)
    flops = 2.0 * m5 * n5 * k5
    tflops = flops / gmean / 1e12
    # context only: the vendor BLAS on a plain fp16 GEMM of the same shape
    # (dense binary16 weights, no decode), on the same box
    wd = torch.randn((n5, k5), device=x5.device, dtype=torch.float16).t().contiguous()
    tmean = event_timed(torch, lambda i: torch.matmul(xr5, wd), 10)
    del wd
    # the same shape with the weights as PTQ1_0 planes
    p5t = to_dev(tq.pack_rowsplit("PTQ1_0_G128", c5["trits"], c5["scale_bits"]))
    pmean = event_timed(torch, lambda i: tq.gemm_rowsplit(p5t, "PTQ1_0_G128", n5, k5, xr5, out=y5), 10)
    del p5t, p5, y5
    torch.cuda.empty_cache()
    counters = load_counters("prefill_gemm_2048x17408x5120_counters.json", "tq_gemm.hip")
    return {
        "workload": "prefill GEMM: 2048 bf16 rows x K=5120 (signed WHT, binary16 out) against "
                    "PQ2_0_G128 N=17408, fp32 out",
        "m": m5, "n": n5, "k": k5, "flop_per_launch": flops,
        "tflops": round(tflops, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": counters["hbm_bytes_per_dispatch"] if counters else None,
                     "mfma_busy": counters["mfma_busy"] if counters else None,
                     "kernel": "gemm_planes_kernel<PQ2_0> (v_mfma_f32_32x32x16_f16)",
                     "mean_launch_us": round(gmean * 1e6, 2),
                     "timing": "hip events on the launch stream around a graph replay"},
        "ptq1_same_shape": {"mean_launch_us": round(pmean * 1e6, 2),
                            "tflops": round(flops / pmean / 1e12, 1)},
        "torch_matmul_fp16_same_shape_us": round(tmean * 1e6, 2),
        "wht_2048x5120_us": round(wmean * 1e6, 2),
        "wht_gbs": round(m5 * k5 * 4 / wmean / 1e9, 1),
    }


def bench_secondary(torch, tq, synth, to_dev, bits_dev, stream, head_copies, c4):
    res = {}
    with torch.cuda.stream(stream):
        # config 2: FFN gate/up decode step, PQ2_0 17408 x 5120 batch 1, one
        # launch and as two (transform, then GEMV on its binary16 output)
        c2 = synth.make_config(2)
        p2 = tq.pack_rowsplit(c2["fmt"], c2["trits"], c2["scale_bits"])
        n2, k2 = c2["n"], c2["k"]
        nc2 = copies_for(p2.size)
        cps2 = [to_dev(p2)]
        cps2 += [cps2[0].clone() for _ in range(nc2 - 1)]
        x2 = bits_dev(c2["x"], torch.bfloat16)
        s2 = bits_dev(c2["sign_bits"], torch.bfloat16)
        xr2 = torch.empty((1, k2), dtype=torch.float16, device=x2.device)
        y2 = torch.empty((1, n2), dtype=torch.float32, device=x2.device)
        launches = 8 * nc2
        mean = event_timed(torch, lambda i: tq.rotated_gemv_rowsplit(cps2[i % nc2], c2["fmt"], n2, k2,
                                                                      x2, s2, out=y2), launches)
        sbytes = p2.size + 2 * k2 + 2 * k2 + 4 * n2
        tq.hadamard_signed(x2, s2, out=xr2)
        gmean = event_timed(torch, lambda i: tq.gemv_rowsplit(cps2[i % nc2], c2["fmt"], n2, k2, xr2,
                                                               out=y2), launches)
        wmean = event_timed(torch, lambda i: tq.hadamard_signed(x2, s2, out=xr2), 64)
        gbytes2 = p2.size + 2 * k2 + 4 * n2
        res["cfg2_gate_up_step_b1"] = {"mean_launch_us": round(mean * 1e6, 3),
                                       "gbs": round(sbytes / mean / 1e9, 1),
                                       "frac_hbm": round(sbytes / mean / 1e9 / HBM_PEAK_GBS, 4),
                                       "gemv_alone_us": round(gmean * 1e6, 3),
                                       "gemv_alone_gbs": round(gbytes2 / gmean / 1e9, 1),
                                       "wht_k5120_b1_us": round(wmean * 1e6, 3)}
        # plain-read floor over the same number of bytes, same rotation
        sink = torch.zeros(1, dtype=torch.int32, device=x2.device)
        rmean = event_timed(torch, lambda i: tq.stream_read(cps2[i % nc2], sink), launches)
        res["read_floor_23_7MB"] = {"bytes": p2.size, "mean_launch_us": round(rmean * 1e6, 3),
                                    "gbs": round(p2.size / rmean / 1e9, 1),
                                    "frac_hbm": round(p2.size / rmean / 1e9 / HBM_PEAK_GBS, 4)}
        # config 2 shape at batch 4 and 8 (row-quad MFMA GEMV), then expanded
        # to G64 (+6% bytes over PQ2_0) at batch 1
        x2b = bits_dev(synth.activations_bf16_bits(np.random.default_rng(22), 8, k2), torch.bfloat16)
        for b in (4, 8):
            xr = tq.hadamard_signed(x2b[:b], s2, out_dtype=torch.float16)
            yb = torch.empty((b, n2), dtype=torch.float32, device=xr.device)
            mean = event_timed(torch, lambda i: tq.gemv_rowsplit(cps2[i % nc2], c2["fmt"], n2, k2, xr,
                                                                  out=yb), 4 * nc2)
            byts = p2.size + 2 * b * k2 + 4 * b * n2
            res["cfg2_shape_pq2_b%d" % b] = {"mean_launch_us": round(mean * 1e6, 3),
                                             "gbs": round(byts / mean / 1e9, 1),
                                             "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        gbytes = tq.g64_bytes(n2, k2)
        gcps = [tq.expand_g64(cps2[0], c2["fmt"], n2, k2) for _ in range(copies_for(gbytes))]
        del cps2
        ng = len(gcps)
        mean = event_timed(torch, lambda i: tq.gemv_g64(gcps[i % ng], n2, k2, xr2, out=y2), 4 * ng)
        byts = gbytes + 2 * k2 + 4 * n2
        res["cfg2_expanded_g64_b1"] = {"bytes": gbytes, "mean_launch_us": round(mean * 1e6, 3),
                                       "gbs": round(byts / mean / 1e9, 1),
                                       "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        del gcps
        torch.cuda.empty_cache()

        # config 3: PTQ1_0 down projection N=5120 K=17408, batch 1/4/8
        c3 = synth.make_config(3)
        p3 = tq.pack_rowsplit(c3["fmt"], c3["trits"], c3["scale_bits"])
        nc = copies_for(p3.size)
        cps = [to_dev(p3)]
        cps += [cps[0].clone() for _ in range(nc - 1)]
        n3, k3 = c3["n"], c3["k"]
        x3 = bits_dev(c3["x"], torch.bfloat16)
        s3 = bits_dev(c3["sign_bits"], torch.bfloat16)
        for b in (1, 4, 8):
            xr = tq.hadamard_signed(x3[:b], s3, out_dtype=torch.float16)
            yb = torch.empty((b, n3), dtype=torch.float32, device=xr.device)
            mean = event_timed(torch, lambda i: tq.gemv_rowsplit(cps[i % nc], c3["fmt"], n3, k3,
                                                                  xr, out=yb), 4 * nc)
            byts = p3.size + 2 * b * k3 + 4 * b * n3
            res["cfg3_ptq1_down_b%d" % b] = {"mean_launch_us": round(mean * 1e6, 3),
                                             "gbs": round(byts / mean / 1e9, 1),
                                             "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        # the same matrix expanded losslessly to 2-bit G64 blocks (+29% bytes,
        # codes without radix-3 digits), batch 1, and the expansion itself
        gbytes = tq.g64_bytes(n3, k3)
        gcps = [torch.empty(gbytes, dtype=torch.uint8, device=x3.device) for _ in range(copies_for(gbytes))]
        for g in gcps:
            tq.expand_g64(cps[0], c3["fmt"], n3, k3, out=g)
        emean = event_timed(torch, lambda i: tq.expand_g64(cps[i % nc], c3["fmt"], n3, k3,
                                                            out=gcps[i % len(gcps)]), 4 * nc)
        del cps
        xr = tq.hadamard_signed(x3[:1], s3, out_dtype=torch.float16)
        yb = torch.empty((1, n3), dtype=torch.float32, device=xr.device)
        ng = len(gcps)
        mean = event_timed(torch, lambda i: tq.gemv_g64(gcps[i % ng], n3, k3, xr, out=yb), 4 * ng)
        byts = gbytes + 2 * k3 + 4 * n3
        res["cfg3_expanded_g64_b1"] = {"bytes": gbytes, "mean_launch_us": round(mean * 1e6, 3),
                                       "gbs": round(byts / mean / 1e9, 1),
                                       "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4),
                                       "expand_us": round(emean * 1e6, 2),
                                       "expand_gbs": round((p3.size + gbytes) / emean / 1e9, 1)}
        del gcps
        # the same trits as PQ2_0 planes (the PQ2_0 model's down projection),
        # batch 1: the wave GEMV with each row split over a pair of waves
        pq = tq.pack_rowsplit("PQ2_0_G128", c3["trits"], c3["scale_bits"])
        ncq = copies_for(pq.size)
        cpq = [to_dev(pq)]
        cpq += [cpq[0].clone() for _ in range(ncq - 1)]
        mean = event_timed(torch, lambda i: tq.gemv_rowsplit(cpq[i % ncq], "PQ2_0_G128", n3, k3, xr,
                                                              out=yb), 4 * ncq)
        byts = pq.size + 2 * k3 + 4 * n3
        res["cfg3_shape_pq2_b1"] = {"bytes": int(pq.size), "mean_launch_us": round(mean * 1e6, 3),
                                    "gbs": round(byts / mean / 1e9, 1),
                                    "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        del cpq
        torch.cuda.empty_cache()

        # GatedDeltaNet output projection N=5120 K=6144 (48 value heads of 128,
        # gathered into the grouped head order before the transform), batch 1,
        # with config 2's value recipe
        rng = np.random.default_rng(46)
        n6, k6 = 5120, 6144
        t6 = synth.trits_sparse(rng, n6, k6)
        p6 = tq.pack_rowsplit("PQ2_0_G128", t6, synth.scale_bits_lognormal(rng, n6, k6 // 128))
        del t6
        s6 = bits_dev(synth.sign_bits(rng, k6), torch.bfloat16)
        x6 = bits_dev(synth.activations_bf16_bits(rng, 1, k6), torch.bfloat16)
        nc6 = copies_for(p6.size)
        cps6 = [to_dev(p6)]
        cps6 += [cps6[0].clone() for _ in range(nc6 - 1)]
        y6 = torch.empty((1, n6), dtype=torch.float32, device=x6.device)
        gmean = event_timed(torch, lambda i: tq.rotated_gemv_rowsplit_grouped(
            cps6[i % nc6], "PQ2_0_G128", n6, k6, x6, s6, out=y6), 4 * nc6)
        pmean = event_timed(torch, lambda i: tq.rotated_gemv_rowsplit(
            cps6[i % nc6], "PQ2_0_G128", n6, k6, x6, s6, out=y6), 4 * nc6)
        byts = p6.size + 2 * k6 + 2 * k6 + 4 * n6
        res["gdn_out_proj_grouped_step"] = {"n": n6, "k": k6, "mean_launch_us": round(gmean * 1e6, 3),
                                            "gbs": round(byts / gmean / 1e9, 1),
                                            "frac_hbm": round(byts / gmean / 1e9 / HBM_PEAK_GBS, 4),
                                            "same_step_without_gather_us": round(pmean * 1e6, 3)}
        del cps6
        torch.cuda.empty_cache()

        # config 4, beside the step: the head GEMV alone on a binary16 x', the
        # whole head step with RMSNorm and the greedy token in one launch, 64
        # embedding rows, and the plain-read floor over the head's bytes
        cps = head_copies
        n4, k4, fmt4 = c4["n"], c4["k"], c4["fmt"]
        pbytes = tq.geometry(fmt4, n4, k4)["payload_bytes"]
        x4 = bits_dev(c4["x"], torch.bfloat16)
        s4 = bits_dev(c4["sign_bits"], torch.bfloat16)
        xr = tq.hadamard_signed(x4, s4, out_dtype=torch.float16)
        y4 = torch.empty((1, n4), dtype=torch.float32, device=xr.device)
        mean = event_timed(torch, lambda i: tq.gemv_rowsplit(cps[i % 2], fmt4, n4, k4, xr, out=y4), 100)
        byts = pbytes + 2 * k4 + 4 * n4
        res["cfg4_head_gemv_alone_b1"] = {"mean_launch_us": round(mean * 1e6, 3),
                                          "gbs": round(byts / mean / 1e9, 1),
                                          "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        gnorm = bits_dev(synth.norm_weight_bits(np.random.default_rng(44), k4), torch.bfloat16)
        work = torch.zeros(2, dtype=torch.int64, device=xr.device)
        tok = torch.empty(1, dtype=torch.int32, device=xr.device)
        hmean = event_timed(torch, lambda i: tq.head_argmax(cps[i % 2], fmt4, n4, k4, x4, gnorm,
                                                             1e-6, s4, work, logits=y4[0], token=tok),
                            100)
        hbytes = pbytes + 3 * 2 * k4 + 4 * n4 + 4
        res["cfg4_head_greedy_one_launch"] = {"mean_launch_us": round(hmean * 1e6, 3),
                                              "gbs": round(hbytes / hmean / 1e9, 1),
                                              "frac_hbm": round(hbytes / hmean / 1e9 / HBM_PEAK_GBS, 4)}
        sink = torch.zeros(1, dtype=torch.int32, device=xr.device)
        rmean = event_timed(torch, lambda i: tq.stream_read(cps[i % 2], sink), 20)
        res["read_floor_337_7MB"] = {"bytes": pbytes, "mean_launch_us": round(rmean * 1e6, 3),
                                     "gbs": round(pbytes / rmean / 1e9, 1),
                                     "frac_hbm": round(pbytes / rmean / 1e9 / HBM_PEAK_GBS, 4)}
        ids = to_dev(c4["ids"])
        emb = torch.empty((64, k4), dtype=torch.float32, device=xr.device)
        mean = event_timed(torch, lambda i: tq.embed_rows_inverse(cps[i % 2], fmt4, n4, k4,
                                                                   ids, s4, out=emb), 20)
        res["cfg4_embed_64_rows_us"] = round(mean * 1e6, 3)
        # load-time step (a ranked next part): GGUF block stream -> planes of
        # the same head (337.7 MB in, 337.7 MB out), and back
        nblk = n4 * (k4 // 128) * 34
        blk = torch.empty(nblk, dtype=torch.uint8, device=xr.device)
        tq.planes_to_blocks(cps[0], fmt4, n4, k4, out=blk)
        tmean = event_timed(torch, lambda i: tq.blocks_to_planes(blk, fmt4, n4, k4, out=cps[1]), 4)
        bmean = event_timed(torch, lambda i: tq.planes_to_blocks(cps[1], fmt4, n4, k4, out=blk), 4)
        res["transcode_head_blocks_to_planes"] = {"us": round(tmean * 1e6, 1),
                                                  "gbs": round((nblk + pbytes) / tmean / 1e9, 1)}
        res["transcode_head_planes_to_blocks"] = {"us": round(bmean * 1e6, 1),
                                                  "gbs": round((nblk + pbytes) / bmean / 1e9, 1)}
        del blk
        gbytes = tq.g64_bytes(n4, k4)
        g4 = torch.empty(gbytes, dtype=torch.uint8, device=xr.device)
        emean = event_timed(torch, lambda i: tq.expand_g64(cps[i % 2], fmt4, n4, k4, out=g4), 4)
        res["expand_head_pq2_to_g64"] = {"us": round(emean * 1e6, 1),
                                         "gbs": round((pbytes + gbytes) / emean / 1e9, 1)}
        del g4
    torch.cuda.synchronize()
    return res


def _host():
    """What the CPU baseline ran on."""
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"os_cpu_count": os.cpu_count(), "usable_cpus": affinity, "cpu_model": model}


def cpu_baseline(synth, rows=16384, runs=3):
    """The float64 oracle (test infrastructure) on a bounded sample of the
    step's workload: the first `rows` rows of the vocabulary head recipe
    (K = 5120), transform + projection of the same hidden row, timed with
    all of the BLAS threads and with one, median of `runs` each."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import codec, projection as P, transform as T
    c = synth.make_config(4, n=rows)
    pay = codec.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
    x = T.bf16_bits_to_f64(c["x"])
    d = T.bf16_bits_to_f64(c["sign_bits"])
    sample_bytes = pay.size + 2 * c["k"] + 2 * c["k"] + 4 * rows

    def median_seconds():
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            P.projection(c["fmt"], rows, c["k"], pay, x, d)
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    blas = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    t_all = median_seconds()
    with threadpool_limits(1):
        t_one = median_seconds()
    return {"value": round(sample_bytes / t_all / 1e9, 5), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of the 248320 head rows (K=5120, head recipe): float64 signed transform "
                      "+ dequantised projection, median of %d" % (rows, runs),
            "seconds_per_sample": round(t_all, 3),
            "single_thread": {"value": round(sample_bytes / t_one / 1e9, 5), "unit": "GB/s",
                              "seconds_per_sample": round(t_one, 3)},
            "blas": [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in blas],
            "host": _host()}


def _timed(fn, min_seconds=1.0, max_reps=50):
    """(calls, seconds) of repeated fn() until min_seconds have passed."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            return reps, el


def oracle_rows(synth):
    """The oracle (test infrastructure) on bounded samples of the other
    workloads, one thread, in the unit of the matching secondary figure:
    payload-plus-activation GB/s for the projections, bytes moved for the
    expansion and the transcoder, TFLOP/s for the GEMM, microseconds for the
    64 embedding rows."""
    from threadpoolctl import threadpool_limits
    from oracle import codec, gdn, head as Hd, projection as P, q2g64, transform as T
    res = {}
    rows = 256
    with threadpool_limits(1):
        # FFN gate/up decode step (config 2 recipe): transform + projection
        c = synth.make_config(2, n=4 * rows)
        pay = codec.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
        xb, db = T.bf16_bits_to_f64(c["x"]), T.bf16_bits_to_f64(c["sign_bits"])
        reps, el = _timed(lambda: P.projection(c["fmt"], 4 * rows, c["k"], pay, xb, db))
        res["cfg2_gate_up_step_b1"] = {"gbs": round(pay.size * reps / el / 1e9, 5),
                                       "sample": "%d rows x %d" % (4 * rows, c["k"])}
        # PTQ1_0 down projection (config 3 recipe), batch 1
        c = synth.make_config(3, n=rows)
        pay = codec.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
        x = T.forward(T.bf16_bits_to_f64(c["x"][:1]), T.bf16_bits_to_f64(c["sign_bits"]))
        reps, el = _timed(lambda: P.project_payload(c["fmt"], rows, c["k"], pay, x))
        res["cfg3_ptq1_down_b1"] = {"gbs": round(pay.size * reps / el / 1e9, 5),
                                    "sample": "%d rows x %d" % (rows, c["k"])}
        # G64 expansion and the GEMV over the expanded stream
        reps, el = _timed(lambda: q2g64.expand(c["fmt"], rows, c["k"], pay))
        gb = q2g64.expanded_bytes(rows, c["k"])
        res["cfg3_expand_g64"] = {"gbs": round((pay.size + gb) * reps / el / 1e9, 5),
                                  "sample": "%d rows x %d" % (rows, c["k"])}
        st = q2g64.expand(c["fmt"], rows, c["k"], pay)
        reps, el = _timed(lambda: q2g64.project(st, rows, c["k"], x))
        res["cfg3_expanded_g64_b1"] = {"gbs": round(gb * reps / el / 1e9, 5),
                                       "sample": "%d rows x %d" % (rows, c["k"])}
        # the head step (config 4 recipe): norm, transform, projection, greedy
        c = synth.make_config(4, n=4 * rows)
        pay = codec.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
        g = T.bf16_bits_to_f64(synth.norm_weight_bits(np.random.default_rng(44), c["k"]))
        d = T.bf16_bits_to_f64(c["sign_bits"])
        xh = T.bf16_bits_to_f64(c["x"])
        reps, el = _timed(lambda: Hd.greedy(Hd.head(c["fmt"], 4 * rows, c["k"], pay, xh, g, 1e-6, d)[0]))
        res["cfg4_head_greedy"] = {"gbs": round(pay.size * reps / el / 1e9, 5),
                                   "sample": "%d rows x %d" % (4 * rows, c["k"])}
        # block stream -> planes (head recipe)
        blk = codec.planes_to_blocks(c["fmt"], 4 * rows, c["k"], pay)
        reps, el = _timed(lambda: codec.blocks_to_planes(c["fmt"], 4 * rows, c["k"], blk))
        res["transcode_blocks_to_planes"] = {"gbs": round((blk.size + pay.size) * reps / el / 1e9, 5),
                                             "sample": "%d rows x %d" % (4 * rows, c["k"])}
        # 64 embedding rows with the inverse transform
        cf = synth.make_config(4, n=4096)
        payf = codec.pack_rowsplit(cf["fmt"], cf["trits"], cf["scale_bits"])
        ids = cf["ids"] % 4096
        reps, el = _timed(lambda: P.embed_rows_inverse(cf["fmt"], 4096, cf["k"], payf, ids,
                                                       T.bf16_bits_to_f64(cf["sign_bits"])))
        res["cfg4_embed_64_rows"] = {"us": round(el / reps * 1e6, 1), "sample": "64 rows of a 4096-row table"}
        # GatedDeltaNet output projection with the grouped head order
        rng = np.random.default_rng(46)
        k6 = 6144
        t6 = synth.trits_sparse(rng, rows, k6)
        pay6 = codec.pack_rowsplit("PQ2_0_G128", t6, synth.scale_bits_lognormal(rng, rows, k6 // 128))
        d6 = T.bf16_bits_to_f64(synth.sign_bits(rng, k6))
        x6 = T.bf16_bits_to_f64(synth.activations_bf16_bits(rng, 1, k6))
        reps, el = _timed(lambda: P.project_payload("PQ2_0_G128", rows, k6, pay6,
                                                    gdn.forward_grouped(x6, d6)))
        res["gdn_out_proj_grouped_step"] = {"gbs": round(pay6.size * reps / el / 1e9, 5),
                                            "sample": "%d rows x %d" % (rows, k6)}
        # prefill GEMM (config 5 recipe): 16 token rows x 256 weight rows
        c = synth.make_config(5, n=rows, rows=16)
        pay = codec.pack_rowsplit(c["fmt"], c["trits"], c["scale_bits"])
        xr = T.forward(T.bf16_bits_to_f64(c["x"]), T.bf16_bits_to_f64(c["sign_bits"]))
        reps, el = _timed(lambda: P.project_payload(c["fmt"], rows, c["k"], pay, xr))
        res["cfg5_prefill_gemm"] = {"tflops": round(2.0 * 16 * rows * c["k"] * reps / el / 1e12, 6),
                                    "sample": "16 x %d x %d" % (rows, c["k"])}
    return res


if __name__ == "__main__":
    sys.exit(main())
