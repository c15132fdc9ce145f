#!/usr/bin/env python3
"""Benchmark of the VQ3R / VQ4P hot path on one MI355X.

One step = one pass of the whole path over one full routed-expert layer of
synthetic weights (256 experts x w1 [2048 x 7168] bf16, Student-t(5) x 0.02 x
per-row lognormal(0, 0.3)), inputs resident in HBM:
  1. Lloyd fit of the 3 x 256 VQ3R codebooks on 12 seeded-sampled experts (20 iters)
  2. VQ3R encode of all 256 experts (indices + fp16 row scales)
  3. VQ3R decode of all 256 experts to fp32
  4. relative Frobenius error per expert after 1, 2 and 3 stages
  5. the fused dequant-GEMV at 1, 4 and 16 tokens, top-8 seeded routing, caches
     evicted before each call: on the GEMV layout (repacked once per step) and on
     the stored records
  6. the MXFP4 source path: MXFP4 quantize-dequantize of all 256 experts; VQ3R
     and VQ4P (4 x 64) each fit on the 12 sampled MXFP4 experts (20 iters) and
     encode all 256 of them; errors against the MXFP4 source and against the
     original weights; VQ4P decode and dequant-GEMV
Prints one JSON line (value = layer weights per second of the whole step, with
the metric's own figures -- encode Gweights/s and GEMV GB/s -- beside it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_PEAK_TFLOPS = 157.3
FP16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak
HBM_PEAK_GBS = 8000.0
ROWS, COLS = 2048, 7168
VEC_PER_EXPERT = ROWS * COLS // 8
FLOP_PER_VEC = {"vq3r": 3 * 256 * 8 * 2, "vq4p": 4 * 64 * 8 * 2}
CB_BYTES = {"vq3r": 3 * 256 * 8 * 4, "vq4p": 4 * 64 * 8 * 4}
GEMV_ROUTINGS = 8  # seeded top-8 routings per batch size, one per timed step in turn
# VALU issue: 1024 SIMDs (256 CUs x 4), one wave64 instruction per 4 cycles, 2.4 GHz
VALU_ISSUE_PER_S = 1024 * 2.4e9 / 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--experts", type=int, default=256)
    ap.add_argument("--sample", type=int, default=12)
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--engine", default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=32768, help="oracle encode sample: first rows of the layer")
    ap.add_argument("--only", default="", help="comma list: fit,encode,decode,error,gemv,mx (default all)")
    ap.add_argument("--loop", default="", help="profiling helper: repeat one component (encode|encode4|encodef32|"
                    "fit|fit4|gemv1|gemv4|gemv16|gemvs1|gemvs4|gemvs16|decode|error|read) --steps times")
    ap.add_argument("--copy-calibration", action="store_true", help="also run a plain copy of known size")
    ap.add_argument("--report", action="store_true", help="error tables: configs 1, 2 and 5 against the RTN "
                    "baselines and the oracle (prints its own JSON line)")
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

    def median_ms(self, name):
        xs = [a.elapsed_time(b) for a, b in self.ev.get(name, [])]
        return float(np.median(xs)) if xs else float("nan")

    def reset(self):
        self.ev = {}


def gemv_alg_bytes(distinct, ntok, fmt, rows=ROWS, cols=COLS):
    """Algorithmic bytes of one dequant-GEMV call: the records and fp16 row scales
    of each distinct routed expert, the fp16 activations, the fp32 outputs (top-8)
    and the codebooks."""
    return distinct * (rows * (cols // 8) * 3 + rows * 2) + ntok * cols * 2 + ntok * 8 * rows * 4 + CB_BYTES[fmt]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(one process drives one GPU). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic
    import residual_vector_quantization_amd as vq

    if args.report:
        report(args, torch, vq, synthetic)
        return
    only = set(args.only.split(",")) if args.only else {"fit", "encode", "decode", "error", "gemv", "mx"}
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
    cb3m = torch.empty_like(cb3)
    cb4 = torch.empty((4, 64, 8), dtype=torch.float32, device=dev)
    fit_ws3 = vq.fit_workspace("vq3r", len(mats), ROWS, COLS)
    fit_ws4 = vq.fit_workspace("vq4p", len(mats), ROWS, COLS)
    idx3 = torch.empty((nrows, COLS // 8, 3), dtype=torch.uint8, device=dev)
    idx3m = torch.empty_like(idx3)
    idx4 = torch.empty_like(idx3)
    sc3 = torch.empty(nrows, dtype=torch.float16, device=dev)
    sc3m = torch.empty_like(sc3)
    sc4 = torch.empty_like(sc3)
    enc_ws = vq.encode_workspace("vq3r", nrows, COLS)
    need_dec = "decode" in only
    w_hat = torch.empty((nrows, COLS), dtype=torch.float32, device=dev) if need_dec else None
    err_ws = vq.error_workspace("vq4p", E, ROWS, COLS)  # the larger of the two formats
    sums3 = torch.empty((E, 4), dtype=torch.float64, device=dev)
    sums_mx = {k: torch.empty((E, 4 if k[0] == "3" else 5), dtype=torch.float64, device=dev)
               for k in ("3s", "3o", "4s", "4o")}
    rel3 = torch.empty((E, 3), dtype=torch.float64, device=dev)
    rel3_all = torch.empty(3, dtype=torch.float64, device=dev)
    rel_mx = {k: (torch.empty((E, 3 if k[0] == "3" else 4), dtype=torch.float64, device=dev),
                  torch.empty(3 if k[0] == "3" else 4, dtype=torch.float64, device=dev)) for k in sums_mx}
    do_mx = "mx" in only
    # the MXFP4 source as bf16 (exact: vq_mxfp4_qdq_bf16)
    mx = torch.empty((nrows, COLS), dtype=torch.bfloat16, device=dev) if do_mx else None
    mx_mats = [mx[e * ROWS:(e + 1) * ROWS] for e in sample] if do_mx else None
    mx_ws = torch.empty(256, dtype=torch.uint8, device=dev)
    # cache eviction between GEMV reps: reading 1 GiB of other data evicts the experts from the L2s and the
    # MALL without leaving dirty lines whose write-back would land inside the timed kernel
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def evict():
        torch.sum(flush, dim=0, out=flush_out)
    gemv_cases = []
    for ntok in (1, 4, 16):
        x = torch.from_numpy(synthetic.activations_f16(ntok, COLS, seed=10 + ntok).view(np.float16)).to(dev)
        # GEMV_ROUTINGS seeded routings per batch size; timed step i uses routing i mod GEMV_ROUTINGS
        routes_np = [synthetic.routing(ntok, E, 8, seed=20 + ntok + 1000 * r) for r in range(GEMV_ROUTINGS)]
        routes = [torch.from_numpy(rt).to(dev) for rt in routes_np]
        y = torch.empty((ntok, 8, ROWS), dtype=torch.float32, device=dev)
        distincts = [len(np.unique(rt)) for rt in routes_np]
        gemv_cases.append({"ntok": ntok, "x": x, "route": routes[0], "y": y, "distinct": distincts[0],
                           "routes": routes, "distincts": distincts, "calls": {},
                           "ws3": vq.gemv_packed_workspace("vq3r", ROWS, COLS, ntok, 8),
                           "ws4": vq.gemv_packed_workspace("vq4p", ROWS, COLS, ntok, 8),
                           "wss": vq.gemv_workspace("vq3r", ROWS, COLS, ntok, 8, E)})
    idx3_e, sc3_e = idx3.view(E, ROWS, COLS // 8, 3), sc3.view(E, ROWS)
    idx4_e, sc4_e = idx4.view(E, ROWS, COLS // 8, 3), sc4.view(E, ROWS)
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
                vq.error_sums(W, idx3, sc3, cb3, fmt="vq3r", n_mats=E, sums=sums3, workspace=err_ws, check=False,
                              rel=rel3, rel_all=rel3_all)
        rsel = step.n % GEMV_ROUTINGS
        step.n += 1

        def routed(c, key):
            c["calls"].setdefault(key, []).append(c["distincts"][rsel])
            return c["routes"][rsel]
        if "gemv" in only:
            with T("pack3"):
                vq.gemv_pack(idx3_e, fmt="vq3r", out=pk3)
            for c in gemv_cases:
                evict()
                rt = routed(c, "gemv3_%d" % c["ntok"])
                with T("gemv3_%d" % c["ntok"]):
                    vq.dequant_gemv_packed(pk3, sc3_e, cb3, c["x"], rt, ROWS, COLS, fmt="vq3r", y=c["y"],
                                           workspace=c["ws3"])
            for c in gemv_cases:
                evict()
                rt = routed(c, "gemvs3_%d" % c["ntok"])
                with T("gemvs3_%d" % c["ntok"]):
                    vq.dequant_gemv(idx3_e, sc3_e, cb3, c["x"], rt, fmt="vq3r", y=c["y"], workspace=c["wss"])
        if do_mx:
            with T("mxfp4"):
                vq.mxfp4_qdq(W, out=mx, workspace=mx_ws, check=False)
            with T("fit3_mx"):
                vq.fit_codebooks(mx_mats, init3, fmt="vq3r", iters=args.iters, engine=args.engine, codebooks=cb3m,
                                 workspace=fit_ws3, check=False)
            with T("encode3_mx"):
                vq.encode(mx, cb3m, fmt="vq3r", engine=args.engine, idx=idx3m, scales=sc3m, workspace=enc_ws,
                          check=False)
            with T("fit4_mx"):
                vq.fit_codebooks(mx_mats, init4, fmt="vq4p", iters=args.iters, engine=args.engine, codebooks=cb4,
                                 workspace=fit_ws4, check=False)
            with T("encode4_mx"):
                vq.encode(mx, cb4, fmt="vq4p", engine=args.engine, idx=idx4, scales=sc4, workspace=enc_ws,
                          check=False)
            with T("error_mx"):
                for key, (ref, ix, sc, cb, fmt) in {"3s": (mx, idx3m, sc3m, cb3m, "vq3r"),
                                                    "3o": (W, idx3m, sc3m, cb3m, "vq3r"),
                                                    "4s": (mx, idx4, sc4, cb4, "vq4p"),
                                                    "4o": (W, idx4, sc4, cb4, "vq4p")}.items():
                    vq.error_sums(ref, ix, sc, cb, fmt=fmt, n_mats=E, sums=sums_mx[key],
                                  workspace=err_ws, check=False, rel=rel_mx[key][0], rel_all=rel_mx[key][1])
            if need_dec:
                with T("decode4"):
                    vq.decode(idx4, sc4, cb4, fmt="vq4p", out=w_hat)
            if "gemv" in only:
                with T("pack4"):
                    vq.gemv_pack(idx4_e, fmt="vq4p", out=pk4)
                for c in gemv_cases:
                    evict()
                    rt = routed(c, "gemv4_%d" % c["ntok"])
                    with T("gemv4_%d" % c["ntok"]):
                        vq.dequant_gemv_packed(pk4, sc4_e, cb4, c["x"], rt, ROWS, COLS, fmt="vq4p",
                                               y=c["y"], workspace=c["ws4"])
    step.fitted = False
    step.n = 0

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
        loop_bench(args, torch, vq, W, mats, init3, init4, cb3, cb4, fit_ws3, fit_ws4, idx3, sc3, idx4, sc4,
                   enc_ws, pk3, sc3_e, idx3_e, gemv_cases, evict, w_hat, flush, (err_ws, sums3, rel3, rel3_all))
        return

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log("warmup step %d done" % i)
    T.reset()
    for c in gemv_cases:
        c["calls"] = {}
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
    comp = {k: round(T.mean_ms(k), 4) for k in sorted(T.ev)}
    weights = E * ROWS * COLS
    # the exact pass of the last encode in the step that used the workspace (VQ3R of the bf16 layer unless the
    # MXFP4 path ran after it): re-encode once, read its counter
    vq.encode(W, cb3, fmt="vq3r", engine=args.engine, idx=idx3, scales=sc3, workspace=enc_ws, check=False)
    enc_flags = vq.read_status(enc_ws)
    n_exact = int(enc_ws[4:8].cpu().view(torch.int32)[0])
    enc_ms = T.mean_ms("encode3")
    enc = {}
    if "encode3" in T.ev:
        alg_flop = E * VEC_PER_EXPERT * FLOP_PER_VEC["vq3r"]
        enc = {"ms": round(enc_ms, 3), "gweights_s": round(weights / (enc_ms * 1e-3) / 1e9, 3),
               "tflops_fp32_equiv": round(alg_flop / (enc_ms * 1e-3) / 1e12, 2),
               "frac_fp32_equiv": round(alg_flop / (enc_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4),
               "frac_fp16_mfma_peak": round(alg_flop / (enc_ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
               "exact_pass_vectors": n_exact, "exact_pass_fraction": round(n_exact / (E * VEC_PER_EXPERT), 7),
               "tie_band_mismatches": 0, "device_flags": enc_flags}
        prof = "k_encode_vq3r_layer_256x2048x7168_counters.md"
        valu = profile_value(prof, "valu_instructions_per_call")
        if valu is not None:
            # from the committed counters: VALU issue at the clock measured during them, and at 2.4 GHz over
            # this run's time
            enc["valu_issue_frac"] = profile_value(prof, "valu_issue_frac")
            enc["matrix_pipe_busy_frac"] = profile_value(prof, "matrix_pipe_busy_frac")
            enc["valu_issue_frac_at_2p4ghz"] = round(valu / VALU_ISSUE_PER_S / (enc_ms * 1e-3), 4)
    if "encode3" in T.ev:
        enc["engines"] = engine_legs(torch, vq, W, cb3, idx3, sc3, enc_ws, E, enc_ms)
    gem = gemv_report(torch, vq, T, gemv_cases, evict, pk3, pk4, sc3_e, sc4_e, cb3, cb4, idx3_e)
    # the HBM-bound steps of the layer, over their algorithmic bytes: records (3 B per vector), fp16 row
    # scales and fp32 output for the decodes; bf16 weights, records and scales for the relative errors
    rec_b, sc_b = weights // 8 * 3, E * ROWS * 2
    hbm = {}
    for key, what, nbytes in (("decode3", "VQ3R decode of the layer, fp32 output", rec_b + sc_b + 4 * weights),
                              ("decode4", "VQ4P decode of the layer (MXFP4 source), fp32 output",
                               rec_b + sc_b + 4 * weights),
                              ("error3", "relative errors after each stage, VQ3R, bf16 weights",
                               2 * weights + rec_b + sc_b)):
        if key in comp:
            gbs = nbytes / (comp[key] * 1e-3) / 1e9
            hbm[key] = {"ms": comp[key], "alg_bytes": nbytes, "GB_s": round(gbs, 1),
                        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "what": what}
    errors = {}
    if "error3" in T.ev:
        errors["vq3r_bf16_layer"] = {"rel_err_all_after_stage": [round(float(v), 6) for v in rel3_all.cpu()],
                                     "rel_err_expert_mean": [round(float(v), 6) for v in rel3.mean(dim=0).cpu()]}
    if do_mx:
        for key, name in (("3s", "vq3r_mxfp4_vs_source"), ("3o", "vq3r_mxfp4_vs_original"),
                          ("4s", "vq4p_mxfp4_vs_source"), ("4o", "vq4p_mxfp4_vs_original")):
            errors[name] = [round(float(v), 6) for v in rel_mx[key][1].cpu()]
    # roofline of the dominant kernel: the VQ3R encode call
    roof = None
    if "encode3" in T.ev:
        alg_tf = E * VEC_PER_EXPERT * FLOP_PER_VEC["vq3r"] / (enc_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(alg_tf, 2), "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(alg_tf / FP16_PEAK_TFLOPS, 4),
                "traffic": profile_value("k_encode_vq3r_layer_256x2048x7168_counters.md",
                                         "traffic_bytes_per_launch") if E == 256 else None,
                "traffic_unit": "HBM bytes per encode call (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": "vq3r encode call (k_encode + k_encode_exact)",
                "work": "12288 flop per 8-dim vector (3 stages x 256 codewords x 8 dims x 2)",
                "pipe": "fp16 matrix cores (hi/lo split: 4 issued matrix flops per algorithmic flop)",
                "binding_resource": "VALU issue (top-2 selection of the scores)",
                "valu_issue_frac": enc.get("valu_issue_frac"),
                "fp32_equiv_frac": enc.get("frac_fp32_equiv")}
    cpu, legs = None, None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, W, cb3, args.cpu_rows)
        legs = cpu_baseline_legs(torch, vq, synthetic, W, mats, cb3, idx3_e, sc3_e, gemv_cases[0])
    line = {
        "metric": "VQ3R encode Gweights/s (%FP32 peak) + dequant-GEMV GB/s (%HBM peak), 1 GPU",
        "value": round(weights / (ms_step * 1e-3) / 1e9, 3),
        "unit": "Gweights/s",
        "encode_gweights_s": enc.get("gweights_s"),
        "gemv_GB_s": {str(c["ntok"]): gem.get("gemv3_%d" % c["ntok"], {}).get("GB_s") for c in gemv_cases},
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "full routed-expert layer: %d experts x w1 [2048x7168] bf16; VQ3R fit on %d sampled "
                               "experts x %d Lloyd iters, encode, decode, error, dequant-GEMV at 1/4/16 tokens "
                               "top-8; MXFP4 source path: VQ3R and VQ4P fit/encode/error, VQ4P decode and GEMV"
                               % (E, len(mats), args.iters),
                   "experts": E, "rows": ROWS, "cols": COLS, "parallelism": "single GPU"},
        "components_ms": comp,
        "encode": enc,
        "gemv": gem,
        "hbm_steps": hbm,
        "errors": errors,
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baseline_legs": legs,
    }
    print(json.dumps(line), flush=True)


def engine_legs(torch, vq, W, cb3, idx3, sc3, enc_ws, E, auto_ms):
    """The VQ3R encode of the same layer with the fp32 engines (outside the timed
    step): fp32 matrix cores and fp32 VALU, each timed with HIP events and
    checked bit for bit against the default engine's indices and scales."""
    ref_idx, ref_sc = idx3.clone(), sc3.clone()
    flop = E * VEC_PER_EXPERT * FLOP_PER_VEC["vq3r"]
    out = {"mfma_f16x": {"ms": round(auto_ms, 3), "pipe": "fp16 matrix cores (hi/lo split)",
                         "tflops_fp32_equiv": round(flop / (auto_ms * 1e-3) / 1e12, 2),
                         "frac_fp32_peak": round(flop / (auto_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4)}}
    for eng, pipe, reps in (("mfma_f32", "fp32 matrix cores", 3), ("valu_f32", "fp32 VALU", 1)):
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            vq.encode(W, cb3, fmt="vq3r", engine=eng, idx=idx3, scales=sc3, workspace=enc_ws, check=False)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        tf = flop / (ms * 1e-3) / 1e12
        out[eng] = {"ms": round(ms, 3), "pipe": pipe, "tflops_fp32": round(tf, 2),
                    "frac_fp32_peak": round(tf / FP32_PEAK_TFLOPS, 4),
                    "bit_exact_vs_default": bool(torch.equal(idx3, ref_idx) and torch.equal(sc3, ref_sc))}
        log("encode engine %s: %.2f ms" % (eng, ms))
    idx3.copy_(ref_idx)
    sc3.copy_(ref_sc)
    return out


def gemv_report(torch, vq, T, cases, evict, pk3, pk4, sc3_e, sc4_e, cb3, cb4, idx3_e):
    """Per GEMV call: event time, algorithmic GB/s and fraction of the 8 TB/s
    peak, the time of a plain streaming read of the same number of bytes after
    the same eviction (vq_stream_read), and the warm-cache time."""
    gem = {}
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    floors = {}
    for c in cases:
        for fmt, key in (("vq3r", "gemv3_%d"), ("vq3r", "gemvs3_%d"), ("vq4p", "gemv4_%d")):
            k = key % c["ntok"]
            if k not in T.ev:
                continue
            # per call: its routing's distinct experts -> algorithmic bytes -> GB/s; medians over the calls
            ts = np.array([a.elapsed_time(b) for a, b in T.ev[k]])
            dist = np.array(c["calls"].get(k, [c["distinct"]] * len(ts))[:len(ts)])
            algs = np.array([gemv_alg_bytes(int(d), c["ntok"], fmt) for d in dist])
            ms = float(np.median(ts))
            gbs = float(np.median(algs / (ts * 1e-3) / 1e9))
            alg = int(np.median(algs))
            if alg // (1 << 20) not in floors:
                floors[alg // (1 << 20)] = read_floor_us(torch, vq, alg, evict, out)
            floor = floors[alg // (1 << 20)]
            gem[k] = {"us": round(ms * 1e3, 2), "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "calls": len(ts), "routings": min(len(ts), GEMV_ROUTINGS),
                      "distinct_experts": round(float(dist.mean()), 2), "alg_bytes": alg,
                      "plain_read_us": round(floor, 2), "frac_of_plain_read": round(floor / (ms * 1e3), 4)}
            if k.startswith("gemvs"):
                gem[k]["layout"] = "stored records (lists the routed experts and repacks them each call)"
            tr = profile_value("k_gemv_vq3r_256x2048x7168_counters.md", "traffic_bytes_per_call_%s" % k)
            if tr is not None:  # counted on the first routing (the profiling loop's)
                alg0 = gemv_alg_bytes(c["distinct"], c["ntok"], fmt)
                gem[k]["traffic_bytes"] = tr
                gem[k]["traffic_over_alg"] = round(tr / alg0, 3)
    # warm caches: the same call back to back, outside the timed region
    for c in cases:
        for fmt, key, pk, sce, cbk, ws in (("vq3r", "gemv3_%d", pk3, sc3_e, cb3, c["ws3"]),
                                           ("vq4p", "gemv4_%d", pk4, sc4_e, cb4, c["ws4"])):
            k = key % c["ntok"]
            if k not in gem:
                continue
            ts = []
            for rep in range(8):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                vq.dequant_gemv_packed(pk, sce, cbk, c["x"], c["route"], ROWS, COLS, fmt=fmt, y=c["y"], workspace=ws)
                e0.record()
                vq.dequant_gemv_packed(pk, sce, cbk, c["x"], c["route"], ROWS, COLS, fmt=fmt, y=c["y"], workspace=ws)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            gem[k]["warm_us"] = round(sorted(ts)[len(ts) // 2], 2)
    for c in cases:
        k = "gemv3_%d" % c["ntok"]
        if k in gem and "gemv4_%d" % c["ntok"] in gem:
            gem["vq4p_over_vq3r_speed_%d" % c["ntok"]] = round(gem[k]["us"] / gem["gemv4_%d" % c["ntok"]]["us"], 3)
    return gem


def read_floor_us(torch, vq, nbytes, evict, out, reps=5):
    """Time of a plain streaming read (vq_stream_read) of nbytes after the same
    cache eviction as the GEMV: the read floor the GEMV's rate is compared with."""
    n = max(16, -(-nbytes // 16) * 16)
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    best = None
    for _ in range(reps):
        evict()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        vq.stream_read(buf, out)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e3
        best = t if best is None else min(best, t)
    del buf
    return best


def loop_bench(args, torch, vq, W, mats, init3, init4, cb3, cb4, fit_ws3, fit_ws4, idx3, sc3, idx4, sc4, enc_ws,
               pk3, sc3_e, idx3_e, gemv_cases, evict, w_hat, flush, err_bufs):
    """Profiling helper: one component repeated, nothing else in the trace."""
    if args.loop not in ("fit", "fit4"):
        vq.fit_codebooks(mats, init3, fmt="vq3r", iters=args.iters, codebooks=cb3, workspace=fit_ws3)
        vq.encode(W, cb3, idx=idx3, scales=sc3, workspace=enc_ws)
        vq.gemv_pack(idx3_e, fmt="vq3r", out=pk3)
    if args.loop == "encode4":
        vq.fit_codebooks(mats, init4, fmt="vq4p", iters=args.iters, codebooks=cb4, workspace=fit_ws4)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for i in range(args.steps):
        if args.loop == "encode":
            vq.encode(W, cb3, engine=args.engine, idx=idx3, scales=sc3, workspace=enc_ws, check=False)
        elif args.loop == "encodef32":
            vq.encode(W, cb3, engine="mfma_f32", idx=idx3, scales=sc3, workspace=enc_ws, check=False)
        elif args.loop == "encode4":
            vq.encode(W, cb4, fmt="vq4p", engine=args.engine, idx=idx4, scales=sc4, workspace=enc_ws, check=False)
        elif args.loop == "fit":
            vq.fit_codebooks(mats, init3, fmt="vq3r", iters=args.iters, codebooks=cb3, workspace=fit_ws3,
                             check=False)
        elif args.loop == "fit4":
            vq.fit_codebooks(mats, init4, fmt="vq4p", iters=args.iters, codebooks=cb4, workspace=fit_ws4,
                             check=False)
        elif args.loop.startswith("gemvs"):
            c = [g for g in gemv_cases if g["ntok"] == int(args.loop[5:])][0]
            evict()
            vq.dequant_gemv(idx3_e, sc3_e, cb3, c["x"], c["route"], y=c["y"], workspace=c["wss"])
        elif args.loop.startswith("gemv"):
            c = [g for g in gemv_cases if g["ntok"] == int(args.loop[4:])][0]
            evict()
            vq.dequant_gemv_packed(pk3, sc3_e, cb3, c["x"], c["route"], ROWS, COLS, y=c["y"], workspace=c["ws3"])
        elif args.loop == "decode":
            vq.decode(idx3, sc3, cb3, out=w_hat)
        elif args.loop == "error":
            err_ws, sums3, rel3, rel3_all = err_bufs
            vq.error_sums(W, idx3, sc3, cb3, fmt="vq3r", n_mats=W.shape[0] // ROWS, sums=sums3, workspace=err_ws,
                          check=False, rel=rel3, rel_all=rel3_all)
        elif args.loop == "read":
            evict()
            vq.stream_read(flush, out)
        torch.cuda.synchronize()
        log("loop %s %d done" % (args.loop, i))
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for i in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB copies done")


# ------------------------------------------------------------------ error tables
def report(args, torch, vq, synthetic):
    """Gate-3 style error tables ([VQ3R page] §3.1 table: rtn2-g64 / vq2 / vq3 /
    rtn3-g64 / rtn4-row; §3.2: requantizing an MXFP4 source; §5: VQ4P) on the
    synthetic configurations:
      config 1: W [256 x 1024] fp32 N(0,1) x lognormal(0, 0.5) rows, seed 0; codebooks
                from 10 Lloyd iterations on W (Forgy seed 0);
      config 2: the 12 sampled experts of the layer (w1 [2048 x 7168] bf16), 20 iterations;
      config 5: the same 12 experts MXFP4 quantize-dequantized, VQ3R and VQ4P.
    VQ errors come from the library (vq_error's relative errors); each table's
    oracle check re-encodes with the CPU oracle and compares within 1e-5 (config 1:
    all of W, bit-exact codebooks; configs 2 and 5: two experts). The RTN
    baselines are the oracle's (CPU)."""
    import oracle
    dev = "cuda"
    t_all = time.time()
    out = {}

    def rtn_rows(ws):
        num = {k: 0.0 for k in ("rtn4-row", "rtn3-g64", "rtn2-g64")}
        den = 0.0
        for w in ws:
            for name, b, g in (("rtn4-row", 4, None), ("rtn3-g64", 3, 64), ("rtn2-g64", 2, 64)):
                d, ww = oracle.error_sums(w, oracle.rtn(w, b, g)[0])
                num[name] += d
            den += float(np.sum(np.asarray(w, np.float64) ** 2))
        return {k: round(float(np.sqrt(v / den)), 6) for k, v in num.items()}

    # config 1
    W1 = synthetic.gaussian_rows(256, 1024, seed=0)
    t1 = {"shape": [256, 1024], "iters": 10}
    for fmt in ("vq3r", "vq4p"):
        S, K = vq.stages_entries(fmt)
        init = synthetic.forgy_init(256 * 128, K, S, seed=0)
        cb = vq.fit_codebooks([torch.from_numpy(W1).to(dev)], init, fmt=fmt, iters=10)
        idx, sc = vq.encode(torch.from_numpy(W1).to(dev), cb, fmt=fmt)
        rel = vq.rel_errors(torch.from_numpy(W1).to(dev), idx, sc, cb, fmt=fmt)[0].cpu().numpy()[0]
        cb_o, _ = oracle.fit([W1], S, K, 10, init)
        i_o, s_o = oracle.encode(W1, cb_o)
        ref = [oracle.rel_error(W1, oracle.decode(i_o, s_o, cb_o, stages_used=su)) for su in range(1, S + 1)]
        t1[fmt] = {"rel_err_after_stage": [round(float(v), 6) for v in rel],
                   "oracle_rel_err_after_stage": [round(float(v), 6) for v in ref],
                   "codebooks_bit_exact": bool(np.array_equal(cb.cpu().numpy().view(np.uint32), cb_o.view(np.uint32))),
                   "max_abs_diff_vs_oracle": float(np.max(np.abs(rel - np.array(ref))))}
    t1.update(rtn_rows([W1]))
    out["config1"] = t1
    log("config 1 done (%.1f s)" % (time.time() - t_all))
    # configs 2 and 5: the 12 sampled experts
    E = args.experts
    sample = synthetic.sample_experts(E, min(args.sample, E), seed=3)
    mats = [synthetic.student_t_expert_torch(synthetic.expert_seed(3, int(e)), ROWS, COLS, device=dev)
            for e in sample]
    Wst = torch.cat(mats, dim=0)
    mx = vq.mxfp4_qdq(Wst)
    mx_mats = [mx[i * ROWS:(i + 1) * ROWS] for i in range(len(mats))]
    n_fit = len(mats) * VEC_PER_EXPERT
    check = [0, len(mats) - 1]
    host = {i: mats[i].float().cpu().numpy() for i in range(len(mats))}
    host_mx = {i: mx_mats[i].cpu().numpy() for i in range(len(mats))}
    for name, src, srcs_host, fmts in (("config2", mats, host, ("vq3r",)),
                                       ("config5", mx_mats, host_mx, ("vq3r", "vq4p"))):
        tab = {"experts": [int(e) for e in sample], "shape": [ROWS, COLS], "iters": args.iters}
        flat = torch.cat(src, dim=0)
        for fmt in fmts:
            S, K = vq.stages_entries(fmt)
            init = synthetic.forgy_init(n_fit, K, S, seed=3 if fmt == "vq3r" else 4)
            t0 = time.time()
            cb = vq.fit_codebooks(src, init, fmt=fmt, iters=args.iters)
            idx, sc = vq.encode(flat, cb, fmt=fmt)
            rel, rel_all, _ = vq.rel_errors(flat, idx, sc, cb, fmt=fmt, n_mats=len(src))
            ent = {"rel_err_all_after_stage": [round(float(v), 6) for v in rel_all.cpu()],
                   "rel_err_per_expert_final": [round(float(v), 6) for v in rel[:, S - 1].cpu()],
                   "gpu_fit_encode_s": round(time.time() - t0, 2)}
            if name == "config5":
                # the same records against the original (pre-MXFP4) weights
                _, rel_o, _ = vq.rel_errors(Wst, idx, sc, cb, fmt=fmt, n_mats=len(src))
                ent["rel_err_vs_original_after_stage"] = [round(float(v), 6) for v in rel_o.cpu()]
            cbh = cb.cpu().numpy()
            diffs = []
            for i in check:
                i_o, s_o = oracle.encode(srcs_host[i], cbh)
                rec_ok = bool(np.array_equal(oracle.unpack(fmt, idx[i * ROWS:(i + 1) * ROWS].cpu().numpy()), i_o))
                for su in range(1, S + 1):
                    r_o = oracle.rel_error(srcs_host[i], oracle.decode(i_o, s_o, cbh, stages_used=su))
                    diffs.append(abs(float(rel[i, su - 1]) - r_o))
                ent.setdefault("oracle_checked_experts", []).append({"expert": int(sample[i]),
                                                                     "indices_bit_exact": rec_ok})
            ent["max_abs_diff_vs_oracle"] = max(diffs)
            tab[fmt] = ent
            log("%s %s done (%.1f s)" % (name, fmt, time.time() - t_all))
        tab.update(rtn_rows([srcs_host[i] for i in range(len(mats))]))
        if name == "config5":
            tab["rtn_vs_original"] = rtn_rows([host[i] for i in range(len(mats))])
            tab["mxfp4_vs_original"] = round(float(np.sqrt(
                sum(oracle.error_sums(host[i], host_mx[i])[0] for i in host) /
                sum(float(np.sum(host[i].astype(np.float64) ** 2)) for i in host))), 6)
        out[name] = tab
    out["bits_per_weight"] = {"vq3r": 3.0, "vq3r_with_row_scales": round(3 + 16 / COLS, 4), "vq4p": 3.0,
                              "rtn4-row": round(4 + 16 / COLS, 4), "rtn3-g64": 3.25, "rtn2-g64": 2.25, "mxfp4": 4.25}
    out["seconds"] = round(time.time() - t_all, 1)
    print(json.dumps({"report": out}), flush=True)


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
        rel = torch.empty((E, 3), dtype=torch.float64, device=dev)
        rel_all = torch.empty(3, dtype=torch.float64, device=dev)
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
                vq.error_sums(flat, idx, sc, cb, fmt="vq3r", n_mats=E, sums=sums, workspace=err_ws, check=False,
                              rel=rel, rel_all=rel_all)
        vq.read_status(enc_ws)
        tot = sums.sum(dim=0)
        enc_ms = T.mean_ms(name + "_encode")
        wts = E * r * c
        out[name] = {"shape": [r, c], "fit_ms": round(T.mean_ms(name + "_fit"), 3), "encode_ms": round(enc_ms, 3),
                     "error_ms": round(T.mean_ms(name + "_error"), 3),
                     "encode_gweights_s": round(wts / (enc_ms * 1e-3) / 1e9, 2),
                     "encode_frac_fp32_peak": round(wts / 8 * 12288 / (enc_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4),
                     "rel_err_all": [round(float(v), 5) for v in rel_all.cpu()]}
        log("%s: fit %.1f ms, encode %.1f ms, error %.2f ms" % (name, out[name]["fit_ms"], enc_ms,
                                                               out[name]["error_ms"]))
        if name == "w2":
            pk = vq.gemv_pack(idx.view(E, r, c // 8, 3), fmt="vq3r")
            gem = {}
            for ntok in (1, 4, 16):
                x = torch.from_numpy(synthetic.activations_f16(ntok, c, seed=30 + ntok).view(np.float16)).to(dev)
                route = torch.from_numpy(synthetic.routing(ntok, E, 8, seed=40 + ntok)).to(dev)
                y = torch.empty((ntok, 8, r), dtype=torch.float32, device=dev)
                ws = vq.gemv_packed_workspace("vq3r", r, c, ntok, 8)
                ts = []
                for rep in range(10):
                    evict()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    vq.dequant_gemv_packed(pk, sc.view(E, r), cb, x, route, r, c, fmt="vq3r", y=y, workspace=ws)
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3)
                us = float(np.median(ts[2:]))
                distinct = len(np.unique(route.cpu().numpy()))
                alg = distinct * (r * (c // 8) * 3 + r * 2) + ntok * c * 2 + ntok * 8 * r * 4 + 3 * 256 * 8 * 4
                floor = read_floor_us(torch, vq, alg, evict, torch.zeros(1, dtype=torch.int32, device=dev))
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
    rel = vq.rel_errors(W, idx3, sc3, cb3, fmt="vq3r", n_mats=E)[0]
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




def profile_value(fname, key):
    """A number from the machine-readable block of a committed profile summary,
    or None once the kernel sources differ from the ones it measured."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and line.startswith("    "):
            k, v = line.strip().split(":", 1)
            kv[k.strip()] = v.strip()
    files = kv.get("source_files", "").split()
    if not files or key not in kv:
        return None
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(ROOT, "residual_vector_quantization_amd", "csrc", f), "rb").read())
    if h.hexdigest() != kv.get("source_sha256"):
        return None
    return float(kv[key])


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, W, cb3, nrows):
    """The oracle (plain C, all host threads) encoding a bounded sample of the
    same workload: the first `nrows` weight rows of the layer (experts 0, 1, ...)
    with the fitted codebooks."""
    import oracle
    w = W[:nrows].float().cpu().numpy()
    cb = cb3.cpu().numpy()
    threads = oracle.max_threads()
    t0 = time.time()
    oracle.encode(w, cb)
    dt = time.time() - t0
    return {"value": round(w.size / dt / 1e9, 6), "unit": "Gweights/s", "cores": threads, "kind": "oracle",
            "sample": "VQ3R encode of the first %d rows x 7168 of the layer (%d experts, %.1f s)"
                      % (nrows, -(-nrows // ROWS), dt), "cpu_model": cpu_model()}


def cpu_baseline_legs(torch, vq, synthetic, W, mats, cb3, idx3_e, sc3_e, case1):
    """The other oracle legs: config 1 fit + encode (VQ3R, 10 iterations on
    [256 x 1024]), the encode of 2 of the 12 sampled experts (config 2, scaled
    per weight), and the fp64 GEMV reference at 1 token (decode of the 8 routed
    experts + fp64 products)."""
    import oracle
    threads = oracle.max_threads()
    legs = {}
    W1 = synthetic.gaussian_rows(256, 1024, seed=0)
    init = synthetic.forgy_init(256 * 128, 256, 3, seed=0)
    t0 = time.time()
    cb, _ = oracle.fit([W1], 3, 256, 10, init)
    oracle.encode(W1, cb)
    legs["config1_fit_encode_s"] = round(time.time() - t0, 3)
    w2 = torch.cat(mats[:2]).float().cpu().numpy()
    t0 = time.time()
    oracle.encode(w2, cb3.cpu().numpy())
    dt = time.time() - t0
    legs["config2_encode_gweights_s"] = round(w2.size / dt / 1e9, 6)
    legs["config2_encode_sample"] = "2 of the 12 sampled experts (%.1f s)" % dt
    route = case1["route"].cpu().numpy()[0]
    xf = synthetic.f16_bits_to_f32(case1["x"].cpu().view(torch.int16).numpy().view(np.uint16)).reshape(-1)
    cbh = cb3.cpu().numpy()
    t0 = time.time()
    for e in route:
        idx = oracle.unpack("vq3r", idx3_e[int(e)].cpu().numpy())
        s = sc3_e[int(e)].cpu().view(torch.int16).numpy().view(np.uint16)
        oracle.gemv_ref(oracle.decode(idx, s, cbh), xf)
    legs["gemv_ref_1_token_s"] = round(time.time() - t0, 3)
    legs["gemv_ref_1_token_GB_s"] = round(gemv_alg_bytes(len(set(route.tolist())), 1, "vq3r") /
                                          (time.time() - t0) / 1e9, 4)
    legs["cores"] = threads
    legs["kind"] = "oracle"
    return legs


if __name__ == "__main__":
    main()
