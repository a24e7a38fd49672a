"""Benchmark of the rotated-basis ternary projection on one MI355X.

A step is one pass of the decode hot path over one batch of synthetic input:
the signed Walsh-Hadamard transform of a bf16 activation row (K = 5120,
rounded to binary16) and the PQ2_0_G128 decode GEMV against the 17408 x 5120
FFN gate/up weight planes, issued as the library's one-launch decode step
(tq_rotated_gemv_rowsplit: the transform runs in every workgroup while its
first weight rows are in flight).  Inputs are resident in HBM before the
timed region.  Each step uses the next of 23 distinct weight copies
(23 x 23.7 MB, more than twice the 256 MB Infinity Cache) so the weight
stream comes from HBM, and the steps are launched as one HIP graph so the
host launch rate does not limit them.

Printed: one JSON line with the step throughput (algorithmic GB/s), the
roofline of the dominant kernel (the fused decode kernel: algorithmic bytes
per launch over its mean launch time from HIP events on its stream), the oracle's CPU
throughput on a bounded sample, and secondary figures for the other
workloads (PTQ1_0 down projection at batch 1/4/8, the vocabulary head and
embedding rows, and the prefill GEMM in TFLOP/s, beside the vendor BLAS on a
plain fp16 GEMM of the same shape for context).
"""

import argparse
import hashlib
import json
import os
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
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip configs 3-5")
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
    """HBM traffic from committed rocprofv3 counter runs, or None when the
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

    # ------------------------------------------------------ config 2 step
    c2 = synth.make_config(2)
    fmt, n, k = c2["fmt"], c2["n"], c2["k"]
    payload = tq.pack_rowsplit(fmt, c2["trits"], c2["scale_bits"])
    plane_bytes = payload.size
    ncopy = copies_for(plane_bytes)
    base = to_dev(payload)
    copies = [base.clone() for _ in range(ncopy)]
    x = bits_dev(c2["x"], torch.bfloat16)
    signs = bits_dev(c2["sign_bits"], torch.bfloat16)
    xrot = torch.empty((1, k), dtype=torch.float16, device=dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)

    def step(i):
        tq.rotated_gemv_rowsplit(copies[i % ncopy], fmt, n, k, x, signs, out=y)

    def step_two_launches(i):
        tq.hadamard_signed(x, signs, out=xrot)
        tq.gemv_rowsplit(copies[i % ncopy], fmt, n, k, xrot, out=y)

    # algorithmic bytes of a step (one launch): planes + x (bf16) + signs
    # (bf16) + y (fp32)
    step_bytes = plane_bytes + 2 * k + 2 * k + 4 * n
    # of the unfused GEMV launch: planes + x' (binary16) + y
    gemv_bytes = plane_bytes + 2 * k + 4 * n

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
    torch.cuda.synchronize()
    if args.warmup > 0:
        g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes * args.steps / elapsed / 1e9

    # correctness spot check of the last step against the library's own
    # first computation (same weights, same input): bitwise equal
    y_graph = y.clone()
    step((args.steps - 1) % ncopy)
    torch.cuda.synchronize()
    if not torch.equal(y_graph, y):
        print("bench: graph replay result differs from eager result", file=sys.stderr)
        return 1

    # ------------------------------ roofline of the fused decode kernel
    with torch.cuda.stream(stream):
        launches = 8 * ncopy
        step_mean = event_timed(torch, step, launches)
        # the same step as two launches (transform, then GEMV), for context
        tq.hadamard_signed(x, signs, out=xrot)
        gemv_mean = event_timed(
            torch, lambda i: tq.gemv_rowsplit(copies[i % ncopy], fmt, n, k, xrot, out=y), launches)
        wht_mean = event_timed(torch, lambda i: tq.hadamard_signed(x, signs, out=xrot), 64)
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=stream):
            for i in range(args.steps):
                step_two_launches(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g2.replay()
        torch.cuda.synchronize()
        two_launch_us = (time.perf_counter() - t0) * 1e6 / args.steps
        del g2
    achieved = step_bytes / step_mean / 1e9
    counters = load_counters("rotated_gemv_pq2_17408x5120_b1_counters.json", "tq_gemv_wave.h")
    traffic = None
    if counters:
        traffic = counters["hbm_bytes_per_dispatch"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gemv_wave_kernel<A=1, BQ=1, ring 6, x bf16, fused transform>",
                "bytes_per_launch": step_bytes, "mean_launch_us": round(step_mean * 1e6, 3),
                "launches": launches, "timing": "hip events around a graph replay of back-to-back launches"}
    del copies
    torch.cuda.empty_cache()

    # ------------------------------------------------ secondary workloads
    secondary = {"two_launch_step_us": round(two_launch_us, 3),
                 "wht_k5120_b1_mean_launch_us": round(wht_mean * 1e6, 3),
                 "gemv_unfused_mean_launch_us": round(gemv_mean * 1e6, 3),
                 "gemv_unfused_gbs": round(gemv_bytes / gemv_mean / 1e9, 1)}
    if not args.no_secondary:
        secondary.update(bench_secondary(torch, tq, synth, to_dev, bits_dev, stream))

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
        cpu = cpu_baseline(c2, step_bytes)
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
        "data": "synthetic (seeded; shapes and value recipes of the 27B model's FFN gate/up "
                "projection, no real weights)",
        "config": {"workload": "FFN gate/up decode: signed WHT (K=5120, bf16 in) + PQ2_0_G128 "
                               "GEMV N=17408 K=5120 batch 1, one launch",
                   "n": n, "k": k, "batch": 1, "format": fmt,
                   "weight_copies_rotated": ncopy, "step_bytes": step_bytes,
                   "launch": "hip graph of all timed steps"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out))
    return 0


def bench_secondary(torch, tq, synth, to_dev, bits_dev, stream):
    res = {}
    with torch.cuda.stream(stream):
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
        torch.cuda.empty_cache()

        # config 2 shape at batch 4 and 8 (row-quad MFMA GEMV), then expanded
        # to G64 (+6% bytes over PQ2_0) at batch 1
        c2 = synth.make_config(2)
        p2h = tq.pack_rowsplit(c2["fmt"], c2["trits"], c2["scale_bits"])
        n2, k2 = c2["n"], c2["k"]
        nc2 = copies_for(p2h.size)
        cps2 = [to_dev(p2h)]
        cps2 += [cps2[0].clone() for _ in range(nc2 - 1)]
        x2b = bits_dev(synth.activations_bf16_bits(np.random.default_rng(22), 8, k2), torch.bfloat16)
        s2b = bits_dev(c2["sign_bits"], torch.bfloat16)
        for b in (4, 8):
            xr = tq.hadamard_signed(x2b[:b], s2b, out_dtype=torch.float16)
            yb = torch.empty((b, n2), dtype=torch.float32, device=xr.device)
            mean = event_timed(torch, lambda i: tq.gemv_rowsplit(cps2[i % nc2], c2["fmt"], n2, k2, xr,
                                                                  out=yb), 4 * nc2)
            byts = p2h.size + 2 * b * k2 + 4 * b * n2
            res["cfg2_shape_pq2_b%d" % b] = {"mean_launch_us": round(mean * 1e6, 3),
                                             "gbs": round(byts / mean / 1e9, 1),
                                             "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        p2 = cps2[0]
        del cps2
        gbytes = tq.g64_bytes(n2, k2)
        gcps = [tq.expand_g64(p2, c2["fmt"], n2, k2) for _ in range(copies_for(gbytes))]
        x2 = bits_dev(c2["x"], torch.bfloat16)
        s2 = bits_dev(c2["sign_bits"], torch.bfloat16)
        xr = tq.hadamard_signed(x2, s2, out_dtype=torch.float16)
        yb = torch.empty((1, n2), dtype=torch.float32, device=xr.device)
        ng = len(gcps)
        mean = event_timed(torch, lambda i: tq.gemv_g64(gcps[i % ng], n2, k2, xr, out=yb), 4 * ng)
        byts = gbytes + 2 * k2 + 4 * n2
        res["cfg2_expanded_g64_b1"] = {"bytes": gbytes, "mean_launch_us": round(mean * 1e6, 3),
                                       "gbs": round(byts / mean / 1e9, 1),
                                       "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        del gcps, p2
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

        # config 4: vocabulary head N=248320 K=5120 batch 1 + 64 embedding rows
        c4 = synth.make_config(4)
        p4 = tq.pack_rowsplit(c4["fmt"], c4["trits"], c4["scale_bits"])
        n4, k4 = c4["n"], c4["k"]
        del c4["trits"]
        cps = [to_dev(p4), None]
        cps[1] = cps[0].clone()
        x4 = bits_dev(c4["x"], torch.bfloat16)
        s4 = bits_dev(c4["sign_bits"], torch.bfloat16)
        xr = tq.hadamard_signed(x4, s4, out_dtype=torch.float16)
        y4 = torch.empty((1, n4), dtype=torch.float32, device=xr.device)
        mean = event_timed(torch, lambda i: tq.gemv_rowsplit(cps[i % 2], c4["fmt"], n4, k4, xr,
                                                              out=y4), 20)
        byts = p4.size + 2 * k4 + 4 * n4
        res["cfg4_head_b1"] = {"mean_launch_us": round(mean * 1e6, 3),
                               "gbs": round(byts / mean / 1e9, 1),
                               "frac_hbm": round(byts / mean / 1e9 / HBM_PEAK_GBS, 4)}
        # the whole head step in one launch: RMSNorm, transform, head GEMV and
        # the greedy token (the logits are written too)
        gnorm = bits_dev(synth.norm_weight_bits(np.random.default_rng(44), k4), torch.bfloat16)
        work = torch.zeros(2, dtype=torch.int64, device=xr.device)
        tok = torch.empty(1, dtype=torch.int32, device=xr.device)
        hmean = event_timed(torch, lambda i: tq.head_argmax(cps[i % 2], c4["fmt"], n4, k4, x4, gnorm,
                                                             1e-6, s4, work, logits=y4[0], token=tok),
                            20)
        hbytes = p4.size + 3 * 2 * k4 + 4 * n4 + 4
        res["cfg4_head_greedy_one_launch"] = {"mean_launch_us": round(hmean * 1e6, 3),
                                              "gbs": round(hbytes / hmean / 1e9, 1),
                                              "frac_hbm": round(hbytes / hmean / 1e9 / HBM_PEAK_GBS, 4)}
        ids = to_dev(c4["ids"])
        emb = torch.empty((64, k4), dtype=torch.float32, device=xr.device)
        mean = event_timed(torch, lambda i: tq.embed_rows_inverse(cps[i % 2], c4["fmt"], n4, k4,
                                                                   ids, s4, out=emb), 20)
        res["cfg4_embed_64_rows_us"] = round(mean * 1e6, 3)
        # load-time step (a ranked next part): GGUF block stream -> planes of
        # the same head (337.7 MB in, 337.7 MB out), and back
        nblk = n4 * (k4 // 128) * 34
        blk = torch.empty(nblk, dtype=torch.uint8, device=xr.device)
        tq.planes_to_blocks(cps[0], c4["fmt"], n4, k4, out=blk)
        tmean = event_timed(torch, lambda i: tq.blocks_to_planes(blk, c4["fmt"], n4, k4, out=cps[1]), 4)
        bmean = event_timed(torch, lambda i: tq.planes_to_blocks(cps[1], c4["fmt"], n4, k4, out=blk), 4)
        res["transcode_head_blocks_to_planes"] = {"us": round(tmean * 1e6, 1),
                                                  "gbs": round((nblk + p4.size) / tmean / 1e9, 1)}
        res["transcode_head_planes_to_blocks"] = {"us": round(bmean * 1e6, 1),
                                                  "gbs": round((nblk + p4.size) / bmean / 1e9, 1)}
        del blk
        gbytes = tq.g64_bytes(n4, k4)
        g4 = torch.empty(gbytes, dtype=torch.uint8, device=xr.device)
        emean = event_timed(torch, lambda i: tq.expand_g64(cps[i % 2], c4["fmt"], n4, k4, out=g4), 4)
        res["expand_head_pq2_to_g64"] = {"us": round(emean * 1e6, 1),
                                         "gbs": round((p4.size + gbytes) / emean / 1e9, 1)}
        del cps, g4
        torch.cuda.empty_cache()

        # config 5: prefill 2048 x 5120 -> WHT (binary16 out) -> GEMM N=17408
        c5 = synth.make_config(5)
        p5 = to_dev(tq.pack_rowsplit(c5["fmt"], c5["trits"], c5["scale_bits"]))
        n5, k5 = c5["n"], c5["k"]
        x5 = bits_dev(c5["x"], torch.bfloat16)
        s5 = bits_dev(c5["sign_bits"], torch.bfloat16)
        xr5 = torch.empty((x5.shape[0], k5), dtype=torch.float16, device=x5.device)
        wmean = event_timed(torch, lambda i: tq.hadamard_signed(x5, s5, out=xr5), 10)
        y5 = torch.empty((x5.shape[0], n5), dtype=torch.float32, device=x5.device)
        gmean = event_timed(torch, lambda i: tq.gemm_rowsplit(p5, c5["fmt"], n5, k5, xr5,
                                                                  out=y5), 10)
        flops = 2.0 * x5.shape[0] * n5 * k5
        # context only: the vendor BLAS on a plain fp16 GEMM of the same shape
        # (dense binary16 weights, no decode), on the same box
        wd = torch.randn((n5, k5), device=x5.device, dtype=torch.float16).t().contiguous()
        tmean = event_timed(torch, lambda i: torch.matmul(xr5, wd), 10)
        del wd
        # the same shape with the weights as PTQ1_0 planes
        p5t = to_dev(tq.pack_rowsplit("PTQ1_0_G128", c5["trits"], c5["scale_bits"]))
        pmean = event_timed(torch, lambda i: tq.gemm_rowsplit(p5t, "PTQ1_0_G128", n5, k5, xr5,
                                                                  out=y5), 10)
        del p5t
        res["cfg5_shape_ptq1_gemm"] = {"mean_launch_us": round(pmean * 1e6, 2),
                                       "tflops": round(flops / pmean / 1e12, 1),
                                       "mfma_frac": round(flops / pmean / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
        res["cfg5_prefill_gemm"] = {"m": int(x5.shape[0]), "n": n5, "k": k5,
                                    "mean_launch_us": round(gmean * 1e6, 2),
                                    "tflops": round(flops / gmean / 1e12, 1),
                                    "mfma_frac": round(flops / gmean / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                                    "torch_matmul_fp16_same_shape_us": round(tmean * 1e6, 2),
                                    "wht_2048x5120_us": round(wmean * 1e6, 2),
                                    "wht_gbs": round(x5.numel() * 4 / wmean / 1e9, 1)}
    torch.cuda.synchronize()
    return res


def cpu_baseline(c2, step_bytes):
    """The float64 oracle (test infrastructure) timed on the host on whole
    config-2 steps: transform + projection of the same inputs, one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import codec, projection as P, transform as T
    payload = codec.pack_rowsplit(c2["fmt"], c2["trits"], c2["scale_bits"])
    x = T.bf16_bits_to_f64(c2["x"])
    d = T.bf16_bits_to_f64(c2["sign_bits"])
    reps, elapsed = 0, 0.0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while reps < 2 or (elapsed < 10.0 and reps < 8):
            P.projection(c2["fmt"], c2["n"], c2["k"], payload, x, d)
            reps += 1
            elapsed = time.perf_counter() - t0
    return {"value": round(step_bytes * reps / elapsed / 1e9, 5), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d full config-2 steps (float64 transform + projection of all 17408 rows)"
                      % reps,
            "seconds_per_step": round(elapsed / reps, 3)}


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
