#!/usr/bin/env python3
"""Benchmark of the VQ3R / VQ4P hot path on one MI355X.

One step = one pass of the whole path over one full routed-expert layer of
synthetic weights (256 experts x w1 [2048 x 7168] bf16, Student-t(5) x 0.02 x
per-row lognormal(0, 0.3)), inputs resident in HBM:
  1. Lloyd fit of the 3 x 256 VQ3R codebooks on 12 seeded-sampled experts (20 iters)
  2. VQ3R encode of all 256 experts (indices + fp16 row scales)
  3. VQ3R decode of all 256 experts to fp32
  4. relative Frobenius error per expert after 1, 2 and 3 stages
  5. repack of the indices into the GEMV runtime layout, then the fused
     dequant-GEMV at 1, 4 and 16 tokens, top-8 seeded routing, MALL flushed
  6. MXFP4 quantize-dequantize of the 12 sampled experts, VQ4P fit on them
     (4 x 64, 20 iters), VQ4P encode of all 256 experts, VQ4P dequant-GEMV
Prints one JSON line (value = layer weights per second of the whole step).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
ROWS, COLS = 2048, 7168
VEC_PER_EXPERT = ROWS * COLS // 8
FLOP_PER_VEC = {"vq3r": 3 * 256 * 8 * 2, "vq4p": 4 * 64 * 8 * 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--experts", type=int, default=256)
    ap.add_argument("--sample", type=int, default=12)
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--engine", default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=32768, help="oracle encode sample: first rows of the layer")
    ap.add_argument("--only", default="", help="comma list: fit,encode,decode,error,gemv,vq4p (default all)")
    ap.add_argument("--loop", default="", help="profiling helper: repeat one component (encode|encode4|fit|fit4|gemv1|gemv4|gemv16|decode) --steps times")
    ap.add_argument("--copy-calibration", action="store_true", help="also run a plain copy of known size")
    ap.add_argument("--layer", action="store_true", help="per-layer conversion measurement: w1 and w3 "
                    "[2048x7168] and w2 [7168x2048] of every expert, each family fit, encoded and measured, plus "
                    "the w2 dequant-GEMV (prints its own JSON line)")
    ap.add_argument("--gemm", default="", help="prompt-processing dequant-GEMM measurement on the layer: comma "
                    "list of token counts (top-8 each), e.g. 1024,4096,16384 (prints its own JSON line)")
    ap.add_argument("--ttp", action="store_true", help="Tied Trit-Planes codec on the layer: quantize, dequantize "
                    "and error of all experts (prints its own JSON line)")
    ap.add_argument("--container", default="", help="container measurement: write the layer's VQ3R records "
                    "into a container under this directory, then time streaming them into device memory and "
                    "verifying them (prints its own JSON line)")
    return ap.parse_args()


class Timer:
    """HIP events on the current stream around each component."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}

    def __call__(self, name):
        torch = self.torch
        timer = self

        class _Ctx:
            def __enter__(self_):
                self_.a = torch.cuda.Event(enable_timing=True)
                self_.b = torch.cuda.Event(enable_timing=True)
                self_.a.record()

            def __exit__(self_, *exc):
                self_.b.record()
                timer.ev.setdefault(name, []).append((self_.a, self_.b))

        return _Ctx()

    def mean_ms(self, name, skip=0):
        xs = [a.elapsed_time(b) for a, b in self.ev.get(name, [])[skip:]]
        return float(np.mean(xs)) if xs else float("nan")

    def reset(self):
        self.ev = {}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(one process drives one GPU). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic
    import residual_vector_quantization_amd as vq

    only = set(args.only.split(",")) if args.only else {"fit", "encode", "decode", "error", "gemv", "vq4p"}
    dev = "cuda"
    torch.cuda.set_device(0)
    E = args.experts
    t0 = time.time()
    W = torch.empty((E * ROWS, COLS), dtype=torch.bfloat16, device=dev)
    for e in range(E):
        synthetic.student_t_expert_torch(synthetic.expert_seed(3, e), ROWS, COLS, device=dev,
                                         out=W[e * ROWS:(e + 1) * ROWS])
    torch.cuda.synchronize()
    log("generated %d experts in %.1f s" % (E, time.time() - t0))
    sample = synthetic.sample_experts(E, min(args.sample, E), seed=3)
    mats = [W[e * ROWS:(e + 1) * ROWS] for e in sample]
    n_fit = len(mats) * VEC_PER_EXPERT
    init3 = synthetic.forgy_init(n_fit, 256, 3, seed=3)
    init4 = synthetic.forgy_init(n_fit, 64, 4, seed=4)
    nrows = E * ROWS
    # buffers and workspaces (allocated once, outside the timed region)
    cb3 = torch.empty((3, 256, 8), dtype=torch.float32, device=dev)
    cb4 = torch.empty((4, 64, 8), dtype=torch.float32, device=dev)
    fit_ws3 = vq.fit_workspace("vq3r", len(mats), ROWS, COLS)
    fit_ws4 = vq.fit_workspace("vq4p", len(mats), ROWS, COLS)
    idx3 = torch.empty((nrows, COLS // 8, 3), dtype=torch.uint8, device=dev)
    idx4 = torch.empty_like(idx3)
    sc3 = torch.empty(nrows, dtype=torch.float16, device=dev)
    sc4 = torch.empty_like(sc3)
    enc_ws = vq.encode_workspace("vq3r", nrows, COLS)
    need_dec = "decode" in only
    w_hat = torch.empty((nrows, COLS), dtype=torch.float32, device=dev) if need_dec else None
    err_ws = vq.error_workspace("vq3r", E, ROWS, COLS)
    sums = torch.empty((E, 4), dtype=torch.float64, device=dev)
    mx_out = torch.empty((len(mats) * ROWS, COLS), dtype=torch.float32, device=dev) if "vq4p" in only else None
    mx_ws = torch.empty(256, dtype=torch.uint8, device=dev)
    # cache eviction between GEMV reps: reading 1 GiB of other data evicts the packed experts from the
    # L2s and the MALL without leaving dirty lines whose write-back would land inside the timed kernel
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def evict():
        torch.sum(flush, dim=0, out=flush_out)
    gemv_cases = []
    for ntok in (1, 4, 16):
        x = torch.from_numpy(synthetic.activations_f16(ntok, COLS, seed=10 + ntok).view(np.float16)).to(dev)
        route = torch.from_numpy(synthetic.routing(ntok, E, 8, seed=20 + ntok)).to(dev)
        y = torch.empty((ntok, 8, ROWS), dtype=torch.float32, device=dev)
        ws = vq.gemv_workspace("vq3r", ROWS, COLS, ntok, 8)
        distinct = len(np.unique(route.cpu().numpy()))
        gemv_cases.append((ntok, x, route, y, ws, distinct))
    gemv_cases4 = [(ntok, x, route, y, vq.gemv_workspace("vq4p", ROWS, COLS, ntok, 8), d)
                   for ntok, x, route, y, ws, d in gemv_cases]
    idx3_e = idx3.view(E, ROWS, COLS // 8, 3)
    sc3_e = sc3.view(E, ROWS)
    idx4_e = idx4.view(E, ROWS, COLS // 8, 3)
    sc4_e = sc4.view(E, ROWS)
    pk3 = torch.empty((E, vq.lib().vq_gemv_packed_size(0, ROWS, COLS)), dtype=torch.uint8, device=dev)
    pk4 = torch.empty((E, vq.lib().vq_gemv_packed_size(1, ROWS, COLS)), dtype=torch.uint8, device=dev)
    T = Timer(torch)

    def step():
        if "fit" in only or not step.fitted:
            with T("fit3"):
                vq.fit_codebooks(mats, init3, fmt="vq3r", iters=args.iters, engine=args.engine, codebooks=cb3,
                                 workspace=fit_ws3, check=False)
            step.fitted = True
        if "encode" in only:
            with T("encode3"):
                vq.encode(W, cb3, fmt="vq3r", engine=args.engine, idx=idx3, scales=sc3, workspace=enc_ws,
                          check=False)
        if need_dec:
            with T("decode3"):
                vq.decode(idx3, sc3, cb3, fmt="vq3r", out=w_hat)
        if "error" in only:
            with T("error3"):
                vq.error_sums(W, idx3, sc3, cb3, fmt="vq3r", n_mats=E, sums=sums, workspace=err_ws, check=False)
        if "gemv" in only:
            with T("pack3"):
                vq.gemv_pack(idx3_e, fmt="vq3r", out=pk3)
            for ntok, x, route, y, ws, _ in gemv_cases:
                evict()
                with T("gemv3_%d" % ntok):
                    vq.dequant_gemv(pk3, sc3_e, cb3, x, route, ROWS, COLS, fmt="vq3r", y=y, workspace=ws)
        if "vq4p" in only:
            with T("mxfp4"):
                for i, m in enumerate(mats):
                    vq.mxfp4_qdq(m, out=mx_out[i * ROWS:(i + 1) * ROWS], workspace=mx_ws, check=False)
            with T("fit4"):
                vq.fit_codebooks([mx_out[i * ROWS:(i + 1) * ROWS] for i in range(len(mats))], init4, fmt="vq4p",
                                 iters=args.iters, engine=args.engine, codebooks=cb4, workspace=fit_ws4,
                                 check=False)
            with T("encode4"):
                vq.encode(W, cb4, fmt="vq4p", engine=args.engine, idx=idx4, scales=sc4, workspace=enc_ws,
                          check=False)
            with T("pack4"):
                vq.gemv_pack(idx4_e, fmt="vq4p", out=pk4)
            for ntok, x, route, y, ws4, _ in gemv_cases4:
                evict()
                with T("gemv4_%d" % ntok):
                    vq.dequant_gemv(pk4, sc4_e, cb4, x, route, ROWS, COLS, fmt="vq4p", y=y, workspace=ws4)
    step.fitted = False

    if args.ttp:
        ttp_bench(args, torch, vq, W, E)
        return

    if args.gemm:
        gemm_bench(args, torch, vq, synthetic, W, mats, init3, cb3, fit_ws3, idx3, sc3, enc_ws, E)
        return

    if args.layer:
        layer_bench(args, torch, vq, synthetic, W, E, evict)
        return

    if args.container:
        container_bench(args, torch, vq, W, mats, init3, cb3, fit_ws3, idx3, sc3, enc_ws, E)
        return

    if args.loop:
        # profiling helper: one component repeated, nothing else in the trace
        if args.loop not in ("fit", "fit4"):
            vq.fit_codebooks(mats, init3, fmt="vq3r", iters=args.iters, codebooks=cb3, workspace=fit_ws3)
            vq.encode(W, cb3, idx=idx3, scales=sc3, workspace=enc_ws)
            vq.gemv_pack(idx3_e, fmt="vq3r", out=pk3)
        if args.loop == "encode4":
            vq.fit_codebooks(mats, init4, fmt="vq4p", iters=args.iters, codebooks=cb4, workspace=fit_ws4)
        torch.cuda.synchronize()
        for i in range(args.steps):
            if args.loop == "encode":
                vq.encode(W, cb3, engine=args.engine, idx=idx3, scales=sc3, workspace=enc_ws, check=False)
            elif args.loop == "encode4":
                vq.encode(W, cb4, fmt="vq4p", engine=args.engine, idx=idx4, scales=sc4, workspace=enc_ws,
                          check=False)
            elif args.loop == "fit":
                vq.fit_codebooks(mats, init3, fmt="vq3r", iters=args.iters, codebooks=cb3, workspace=fit_ws3,
                                 check=False)
            elif args.loop == "fit4":
                vq.fit_codebooks(mats, init4, fmt="vq4p", iters=args.iters, codebooks=cb4, workspace=fit_ws4,
                                 check=False)
            elif args.loop.startswith("gemv"):
                ntok = int(args.loop[4:])
                c = [g for g in gemv_cases if g[0] == ntok][0]
                evict()
                vq.dequant_gemv(pk3, sc3_e, cb3, c[1], c[2], ROWS, COLS, y=c[3], workspace=c[4])
            elif args.loop == "decode":
                vq.decode(idx3, sc3, cb3, out=w_hat)
            torch.cuda.synchronize()
            log("loop %s %d done" % (args.loop, i))
        if args.copy_calibration:
            src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for i in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            log("copy calibration: 3 x 1 GiB copies done")
        return

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log("warmup step %d done" % i)
    T.reset()
    torch.cuda.synchronize()
    t_start = time.time()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.time() - t_start
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log("timed %d steps: %.2f ms/step (wall %.2f s)" % (args.steps, ms_step, wall))
    # correctness of the last step (status words + sanity of the error)
    comp = {}
    for k in sorted(T.ev):
        comp[k] = round(T.mean_ms(k), 4)
    weights = E * ROWS * COLS
    out = {}
    enc_ms = T.mean_ms("encode3")
    enc_tflops = E * VEC_PER_EXPERT * FLOP_PER_VEC["vq3r"] / (enc_ms * 1e-3) / 1e12
    out["encode_gweights_s"] = round(weights / (enc_ms * 1e-3) / 1e9, 3)
    out["encode_tflops_fp32_equiv"] = round(enc_tflops, 2)
    out["encode_frac_fp32_peak"] = round(enc_tflops / FP32_PEAK_TFLOPS, 4)
    gem = {}
    floors = {}
    for fmt in ("3", "4"):
        for ntok, x, route, y, ws, distinct in gemv_cases:
            key = "gemv%s_%d" % (fmt, ntok)
            if key not in T.ev:
                continue
            ms = T.mean_ms(key)
            alg = distinct * (VEC_PER_EXPERT * 3 + ROWS * 2) + ntok * COLS * 2 + ntok * 8 * ROWS * 4 + \
                (3 * 256 * 8 * 4 if fmt == "3" else 4 * 64 * 8 * 4)
            gbs = alg / (ms * 1e-3) / 1e9
            floor = floors.setdefault(alg // (1 << 20), read_floor_us(torch, alg, evict))
            gem[key] = {"us": round(ms * 1e3, 2), "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "distinct_experts": distinct, "alg_bytes": alg,
                        "plain_read_us": round(floor, 2), "frac_of_plain_read": round(floor / (ms * 1e3), 4)}
    # warm-cache GEMV (outside the timed region): the same call repeated back to back, so the packed
    # experts are still in the L2s and the MALL; reported next to the evicted figure above
    for fmt, pk, sce, cbk, cases, name in (("3", pk3, sc3_e, cb3, gemv_cases, "vq3r"),
                                          ("4", pk4, sc4_e, cb4, gemv_cases4, "vq4p")):
        for ntok, x, route, y, ws, distinct in cases:
            key = "gemv%s_%d" % (fmt, ntok)
            if key not in gem:
                continue
            ts = []
            for rep in range(8):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                vq.dequant_gemv(pk, sce, cbk, x, route, ROWS, COLS, fmt=name, y=y, workspace=ws)
                e0.record()
                vq.dequant_gemv(pk, sce, cbk, x, route, ROWS, COLS, fmt=name, y=y, workspace=ws)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            gem[key]["warm_us"] = round(sorted(ts)[len(ts) // 2], 2)
    if "error3" in T.ev:
        s = sums.double().cpu().numpy()
        out["rel_error_mean_after_stage"] = [round(float(np.mean(np.sqrt(s[:, t] / s[:, 3]))), 5) for t in range(3)]
    st = vq.read_status(enc_ws)
    out["encode_device_flags"] = st
    # roofline of the dominant kernel: the VQ3R encode
    roof = {"bound": "alu", "achieved": round(enc_tflops, 2), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(enc_tflops / FP32_PEAK_TFLOPS, 4), "traffic": encode_traffic() if E == 256 else None,
            "traffic_unit": "HBM bytes per encode call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "vq3r encode (k_encode + k_encode_exact)", "work": "12288 fp32 flop per 8-dim vector"}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, W, cb3, args.cpu_rows)
    line = {
        "metric": "VQ3R encode Gweights/s (%FP32 peak) + dequant-GEMV GB/s (%HBM peak), 1 GPU",
        "value": round(weights / (ms_step * 1e-3) / 1e9, 3),
        "unit": "Gweights/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "full routed-expert layer: %d experts x w1 [2048x7168] bf16, fit on %d sampled "
                               "experts x %d Lloyd iters, VQ3R+VQ4P encode, decode, error, dequant-GEMV at "
                               "1/4/16 tokens top-8" % (E, len(mats), args.iters),
                   "experts": E, "rows": ROWS, "cols": COLS, "parallelism": "single GPU"},
        "components_ms": comp,
        "encode": out,
        "gemv": gem,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def ttp_bench(args, torch, vq, W, E):
    """Tied Trit-Planes over the full layer (E x [2048 x 7168] bf16): quantize,
    dequantize and error, HIP-event timed; the rates are against HBM bytes."""
    dev = "cuda"
    n = E * ROWS * COLS
    codes = torch.empty((E * ROWS, COLS // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((E * ROWS, COLS // 256), dtype=torch.float16, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    out = torch.empty((E * ROWS, COLS), dtype=torch.float32, device=dev)
    sums = torch.empty((E, 2), dtype=torch.float64, device=dev)
    T = Timer(torch)
    for rep in range(args.warmup + max(3, args.steps)):
        if rep == args.warmup:
            T.reset()
        with T("quantize"):
            vq.ttp_quantize(W, codes=codes, scales=scales, workspace=ws, check=False)
        with T("dequantize"):
            vq.ttp_dequantize(codes, scales, out=out)
        with T("error"):
            vq.ttp_error_sums(W, codes, scales, n_mats=E, sums=sums, check=False)
    vq.read_status(ws)
    tot = sums.sum(dim=0)
    res = {}
    for k, nbytes in (("quantize", n * 2 + n // 2 + n // 128), ("dequantize", n // 2 + n // 128 + n * 4),
                      ("error", n * 2 + n // 2 + n // 128)):
        ms = T.mean_ms(k)
        res[k] = {"ms": round(ms, 3), "gweights_s": round(n / (ms * 1e-3) / 1e9, 1),
                  "hbm_GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "alg_bytes": nbytes}
    print(json.dumps({"ttp": res, "rel_err_layer": round(float((tot[0] / tot[1]).sqrt()), 5),
                      "bits_per_weight": 4.0625, "experts": E, "shape": [ROWS, COLS]}), flush=True)


FP16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak


def gemm_bench(args, torch, vq, synthetic, W, mats, init3, cb3, fit_ws3, idx3, sc3, enc_ws, E):
    """Dequant-GEMM on the full layer: T tokens, top-8 routing (uniform, seeded),
    y = W_hat_e x for all 8T pairs, timed with HIP events on the launch stream."""
    dev = "cuda"
    vq.fit_codebooks(mats, init3, fmt="vq3r", iters=args.iters, codebooks=cb3, workspace=fit_ws3)
    vq.encode(W, cb3, idx=idx3, scales=sc3, workspace=enc_ws)
    idx_e, sc_e = idx3.view(E, ROWS, COLS // 8, 3), sc3.view(E, ROWS)
    out = {}
    for T in [int(t) for t in args.gemm.split(",")]:
        x = torch.from_numpy(synthetic.activations_f16(T, COLS, seed=50 + T % 97).view(np.float16)).to(dev)
        route = torch.from_numpy(synthetic.routing(T, E, 8, seed=60 + T % 89)).to(dev)
        y = torch.empty((T, 8, ROWS), dtype=torch.float32, device=dev)
        ws = vq.gemm_workspace("vq3r", E, T, 8)
        ts = []
        for rep in range(args.warmup + max(3, args.steps)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            vq.dequant_gemm(idx_e, sc_e, cb3, x, route, y=y, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            if rep >= args.warmup:
                ts.append(e0.elapsed_time(e1))
        vq.read_status(ws)
        ms = float(np.median(ts))
        flop = 2.0 * T * 8 * ROWS * COLS
        tf = flop / (ms * 1e-3) / 1e12
        out["tokens_%d" % T] = {"pairs_per_expert": T * 8 / E, "ms": round(ms, 4), "tflops": round(tf, 1),
                                "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4),
                                "records_GB_s": round(E * VEC_PER_EXPERT * 3 / (ms * 1e-3) / 1e9, 1)}
        log("gemm T=%d: %.3f ms, %.1f TFLOP/s" % (T, ms, tf))
    print(json.dumps({"gemm": out, "experts": E, "shape": [ROWS, COLS], "topk": 8}), flush=True)


def layer_bench(args, torch, vq, synthetic, W1, E, evict):
    """Per-layer conversion: three matrix families per expert, each with its own
    codebooks fit on the 12 sampled experts (w1 is the main workload's matrix;
    w3 and w2 are drawn with the same recipe and seed families 6 and 7; w2 is
    [7168 x 2048]). Times fit, encode and error per family, then the fused
    dequant-GEMV on w2 at 1 / 4 / 16 tokens, top-8."""
    dev = "cuda"
    fams = {"w1": W1.view(E, ROWS, COLS)}
    for name, cfgid, (r, c) in (("w3", 6, (ROWS, COLS)), ("w2", 7, (COLS, ROWS))):
        t = torch.empty((E, r, c), dtype=torch.bfloat16, device=dev)
        for e in range(E):
            synthetic.student_t_expert_torch(synthetic.expert_seed(cfgid, e), r, c, device=dev, out=t[e])
        fams[name] = t
    torch.cuda.synchronize()
    sample = synthetic.sample_experts(E, min(args.sample, E), seed=3)
    T = Timer(torch)
    out = {}
    for name, Wn in fams.items():
        _, r, c = Wn.shape
        n_fit = len(sample) * r * c // 8
        init = synthetic.forgy_init(n_fit, 256, 3, seed=3)
        mats = [Wn[e] for e in sample]
        flat = Wn.view(E * r, c)
        fit_ws = vq.fit_workspace("vq3r", len(mats), r, c)
        enc_ws = vq.encode_workspace("vq3r", E * r, c)
        cb = torch.empty((3, 256, 8), dtype=torch.float32, device=dev)
        idx = torch.empty((E * r, c // 8, 3), dtype=torch.uint8, device=dev)
        sc = torch.empty(E * r, dtype=torch.float16, device=dev)
        err_ws = vq.error_workspace("vq3r", E, r, c)
        sums = torch.empty((E, 4), dtype=torch.float64, device=dev)
        for rep in range(args.warmup + args.steps):
            if rep == args.warmup:
                T.reset()
            with T(name + "_fit"):
                vq.fit_codebooks(mats, init, fmt="vq3r", iters=args.iters, engine=args.engine, codebooks=cb,
                                 workspace=fit_ws, check=False)
            with T(name + "_encode"):
                vq.encode(flat, cb, fmt="vq3r", engine=args.engine, idx=idx, scales=sc, workspace=enc_ws,
                          check=False)
            with T(name + "_error"):
                vq.error_sums(flat, idx, sc, cb, fmt="vq3r", n_mats=E, sums=sums, workspace=err_ws, check=False)
        vq.read_status(enc_ws)
        tot = sums.sum(dim=0)
        enc_ms = T.mean_ms(name + "_encode")
        wts = E * r * c
        out[name] = {"shape": [r, c], "fit_ms": round(T.mean_ms(name + "_fit"), 3), "encode_ms": round(enc_ms, 3),
                     "error_ms": round(T.mean_ms(name + "_error"), 3),
                     "encode_gweights_s": round(wts / (enc_ms * 1e-3) / 1e9, 2),
                     "encode_frac_fp32_peak": round(wts / 8 * 12288 / (enc_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4),
                     "rel_err_all": [round(float(v), 5) for v in (tot[:3] / tot[3]).sqrt()]}
        log("%s: fit %.1f ms, encode %.1f ms, error %.2f ms" % (name, out[name]["fit_ms"], enc_ms,
                                                               out[name]["error_ms"]))
        if name == "w2":
            pk = vq.gemv_pack(idx.view(E, r, c // 8, 3), fmt="vq3r")
            gem = {}
            for ntok in (1, 4, 16):
                x = torch.from_numpy(synthetic.activations_f16(ntok, c, seed=30 + ntok).view(np.float16)).to(dev)
                route = torch.from_numpy(synthetic.routing(ntok, E, 8, seed=40 + ntok)).to(dev)
                y = torch.empty((ntok, 8, r), dtype=torch.float32, device=dev)
                ws = vq.gemv_workspace("vq3r", r, c, ntok, 8)
                ts = []
                for rep in range(10):
                    evict()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    vq.dequant_gemv(pk, sc.view(E, r), cb, x, route, r, c, fmt="vq3r", y=y, workspace=ws)
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3)
                us = float(np.median(ts[2:]))
                distinct = len(np.unique(route.cpu().numpy()))
                alg = distinct * (r * (c // 8) * 3 + r * 2) + ntok * c * 2 + ntok * 8 * r * 4 + 3 * 256 * 8 * 4
                floor = read_floor_us(torch, alg, evict)
                gbs = alg / (us * 1e-6) / 1e9
                gem["gemv_%d" % ntok] = {"us": round(us, 2), "GB_s": round(gbs, 1),
                                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "distinct_experts": distinct,
                                         "alg_bytes": alg, "plain_read_us": round(floor, 2),
                                         "frac_of_plain_read": round(floor / us, 4)}
            out["w2"]["gemv"] = gem
    print(json.dumps({"layer": out, "experts": E, "fit_sample": len(sample), "iters": args.iters}), flush=True)


def container_bench(args, torch, vq, W, mats, init3, cb3, fit_ws3, idx3, sc3, enc_ws, E):
    """Expert-record container over the whole layer: write (host), load into
    device memory through the pinned staging buffer, verify on the GPU. The
    load is timed against a plain pinned host-to-device copy of the same bytes."""
    vq.fit_codebooks(mats, init3, fmt="vq3r", iters=args.iters, codebooks=cb3, workspace=fit_ws3)
    vq.encode(W, cb3, idx=idx3, scales=sc3, workspace=enc_ws)
    sums = vq.error_sums(W, idx3, sc3, cb3, fmt="vq3r", n_mats=E)
    rel = vq.rel_errors(sums)
    os.makedirs(args.container, exist_ok=True)
    path = os.path.join(args.container, "w1_vq3r.vqc")
    idx_e, sc_e = idx3.view(E, ROWS, COLS // 8, 3), sc3.view(E, ROWS)
    torch.cuda.synchronize()
    t0 = time.time()
    vq.write_container(path, "vq3r", cb3, idx_e, sc_e, rel_err=rel)
    t_write = time.time() - t0
    log("container written: %.1f s" % t_write)
    payload = E * (ROWS * (COLS // 8) * 3 + ROWS * 2)
    loads = []
    for i in range(max(1, args.steps)):
        torch.cuda.synchronize()
        t0 = time.time()
        _, ix, sc, _ = vq.load_container(path)
        torch.cuda.synchronize()
        loads.append(time.time() - t0)
        log("load %d: %.3f s" % (i, loads[-1]))
    same = bool(torch.equal(ix, idx_e) and torch.equal(sc.view(torch.int16), sc_e.view(torch.int16)))
    del ix, sc
    pin = torch.empty(payload, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(payload, dtype=torch.uint8, device="cuda")
    h2d = []
    for i in range(3):
        torch.cuda.synchronize()
        t0 = time.time()
        dst.copy_(pin, non_blocking=True)
        torch.cuda.synchronize()
        h2d.append(time.time() - t0)
    del pin, dst
    sample = np.random.default_rng(0).integers(0, 256, 256 << 20, dtype=np.uint8).tobytes()
    t0 = time.time()
    vq.crc32(sample)
    crc_gbs = len(sample) / (time.time() - t0) / 1e9
    torch.cuda.synchronize()
    t0 = time.time()
    v = vq.verify_container(path, [W[e * ROWS:(e + 1) * ROWS] for e in range(E)])
    torch.cuda.synchronize()
    t_verify = time.time() - t0
    ncpu = len(os.sched_getaffinity(0))
    print(json.dumps({"container": {
        "records": E, "record_shape": [ROWS, COLS], "payload_bytes": payload, "file_bytes": os.path.getsize(path),
        "write_s": round(t_write, 3), "load_s_best": round(min(loads), 4),
        "load_GB_s": round(payload / min(loads) / 1e9, 2),
        "pinned_h2d_copy_GB_s": round(payload / min(h2d) / 1e9, 2),
        "crc32_single_thread_GB_s": round(crc_gbs, 2), "host_threads": ncpu,
        "verify_s": round(t_verify, 3), "verify_match": v["match"], "load_bit_exact": same}}), flush=True)
    os.remove(path)


def encode_traffic():
    """HBM bytes per VQ3R encode call from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None once the encode sources differ from the ones it measured."""
    path = os.path.join(ROOT, "profiles", "k_encode_vq3r_layer_256x2048x7168_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and line.startswith("    "):
            k, v = line.strip().split(":", 1)
            kv[k.strip()] = v.strip()
    files = kv.get("source_files", "").split()
    if not files or "traffic_bytes_per_launch" not in kv:
        return None
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(ROOT, "residual_vector_quantization_amd", "csrc", f), "rb").read())
    if h.hexdigest() != kv.get("source_sha256"):
        return None
    return int(kv["traffic_bytes_per_launch"])


def read_floor_us(torch, nbytes, evict, reps=5):
    """Time of a plain device read of nbytes after the same cache eviction as the
    GEMV: torch row sums over [n/1024, 1024] fp32, the fastest plain torch read
    here (one pass; its output is 1/1024 of the input). The reference point for
    the GEMV's HBM rate."""
    rows = max(1, -(-nbytes // 4096))
    buf = torch.ones((rows, 1024), dtype=torch.float32, device="cuda")
    out = torch.empty(rows, dtype=torch.float32, device="cuda")
    best = None
    for _ in range(reps):
        evict()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.sum(buf, dim=1, out=out)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e3
        best = t if best is None else min(best, t)
    del buf
    return best


def cpu_baseline(torch, W, cb3, nrows):
    """The oracle (plain C, all host threads) encoding a bounded sample of the
    same workload: the first `nrows` weight rows of the layer (experts 0, 1, ...)
    with the fitted codebooks."""
    import oracle
    w = W[:nrows].float().cpu().numpy()
    cb = cb3.cpu().numpy()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.time()
    oracle.encode(w, cb)
    dt = time.time() - t0
    return {"value": round(w.size / dt / 1e9, 6), "unit": "Gweights/s", "cores": threads, "kind": "oracle",
            "sample": "VQ3R encode of the first %d rows x 7168 of the layer (%d experts, %.1f s)"
                      % (nrows, -(-nrows // ROWS), dt)}


if __name__ == "__main__":
    main()
