"""Benchmark of the TTT-layer forward on one MI355X.

A step is one ttt_forward over one batch of synthetic input: key statistics,
fused forward/backward of the inner model, weight update and readout (every
kernel of the layer).  Default workload: B=8, H=12, N=6084 (1248^2 image at
patch 16), d=64, inner GELU MLP of width 256 (r=4), MSE loss, eta=1, one
full-batch step, key instance norm, bf16 tensors with fp32 accumulation.
Other workloads (--workload): the ViT-S, DiT and LaCT shapes, the ViT3 block,
the LaCT update rules, the update variants and the outer-loop backward.

Prints one JSON line with the whole-job throughput (tokens/s, tokens = B*N),
the spread of the step time (median, p10, p90 over bursts of steps), the
roofline position of the dominant kernel (timed with HIP events inside the
timed region, on the stream it runs on), the shader clock observed under the
workload, a micro-benchmarked bf16 MFMA peak next to the published one, and
the float64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (published)
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32, vector and dense matrix (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
METRIC = "TTT-layer tokens/sec on 1 MI355X (N=6084, r=4) + % of bf16 MFMA peak"

# name -> (workload, ttt_options keywords or None, mode, roofline bound)
#   mode "forward": ttt_forward_ex; "backward": ttt_backward (the outer-loop gradients)
#   bound: what bounds the dominant kernel ("mfma": bf16 matrix cores on its
#   algorithmic flops; "hbm": its algorithmic bytes; "alu": fp32 vector units)
VARIANTS = {
    "c3_hires_r4": ("c3_hires_r4", None, "forward", "mfma"),
    "c2_vits_r1": ("c2_vits_r1", None, "forward", "mfma"),
    "c2_vits_r4": ("c2_vits_r4", None, "forward", "mfma"),
    "c4_dit_h64": ("c4_dit_h64", None, "forward", "hbm"),
    "c5_lact_swiglu": ("c5_lact_swiglu", None, "forward", "mfma"),
    "c5_lact_momentum": ("c5_lact_swiglu", dict(rule="momentum", beta=0.9), "forward", "mfma"),
    "c5_lact_muon": ("c5_lact_swiglu", dict(rule="muon", beta=0.9, muon_scale=0.02), "forward", "mfma"),
    "c5_lact_video_mask": ("c5_lact_swiglu", dict(chunk_update=[1, 0] * 8), "forward", "mfma"),
    "c3_first_layer_only": ("c3_hires_r4", dict(update_mask=1), "forward", "mfma"),
    "c3_epochs3": ("c3_hires_r4", dict(epochs=3), "forward", "mfma"),
    "vit3_hires": ("vit3_hires", None, "forward", "mfma"),
    "c3_outer_backward": ("c3_hires_r4", None, "backward", "mfma"),
}


def bench_workloads():
    from synth_inputs import WORKLOADS, Workload

    w = dict(WORKLOADS)
    # the ViT3 block at 1248^2: one depthwise-convolution head and 11 GLU
    # heads, dot loss, one full-batch epoch; eta = 1/N, i.e. eta = 1 on the
    # token-mean of the summed dot loss
    w["vit3_hires"] = Workload("vit3_hires", B=8, H=12, N=6084, d=64, hidden=64, inner="vit3", loss="dot",
                               key_norm=True, eta=1.0 / 6084, grid=(78, 78), conv_k=3, seed=1006)
    return w


def gemm_flops(w, tokens_per_pair, mode="forward"):
    """Algorithmic flops (2*m*n*k per product) of one pass over the tokens, per
    pair: (update-side products, readout products)."""
    g = 2.0 * tokens_per_pair * w.d * w.hidden
    if w.inner == "mlp_gelu":
        if mode == "backward":
            # step (5 with V_hat), readout backward (Z_q, A_q_bar, dQ, dW1*, dW2*),
            # tangent and reverse of phi (Z_dot, F, F_dot x2, A_dot_bar, A_bar x2,
            # dX x2, dW1, dW2 x2)
            return g * (5 + 5 + 12 + (1 if w.loss == "mse" else 0)), 0.0
        n_fb = 5 if w.loss == "mse" else 4          # Z, [V_hat], dW2, dA, dW1
        n_q = 2
    elif w.inner == "swiglu":
        n_fb = 7 if w.loss == "mse" else 6          # Z1, Z3, [V_hat], dW2, dH, dW1, dW3
        n_q = 3
    elif w.inner in ("glu", "vit3"):
        g = 2.0 * tokens_per_pair * w.d * w.d      # two d x d maps (the convolution head is not a GEMM)
        n_fb = 4 if w.loss == "dot" else 5          # U, Z, dW1, dW2 [+ F for MSE]
        n_q = 2
    else:
        g = 2.0 * tokens_per_pair * w.d * w.d
        n_fb = 2 if w.loss == "mse" else 1
        n_q = 1
    return g * n_fb, g * n_q


def kernel_source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "linear_complexity_attention_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), only if
    they were taken on the kernel sources as they are now."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
        e = d.get(f"{kernel}@{workload}")
        if e and e.get("source_hash") == kernel_source_hash():
            return e.get("bytes_per_launch")
    except (OSError, ValueError):
        return None
    return None


def cpu_baseline(w, budget_s, inputs, okw, mode):
    """The float64 oracle on whole (b, h) pairs of the same workload and inputs,
    pair after pair (wrapping round) until `budget_s` seconds have passed;
    scaled to tokens/s of the whole layer."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import ttt_oracle as orc

    q, k, v, W0, et = inputs
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    done, t_total = 0, 0.0
    rng = np.random.default_rng(0)
    while t_total < budget_s:
        p = done % (w.B * w.H)
        b, h = divmod(p, w.H)
        # the ViT3 split needs a head's own model: keep every head index
        hs = slice(0, w.H) if w.inner == "vit3" else slice(h, h + 1)
        sl = (slice(b, b + 1), hs)
        args = [a[sl].astype(np.float64) for a in (q, k, v)]
        W = [m[hs].astype(np.float64) for m in W0]
        eta_tok = None if et is None else et[sl].astype(np.float64)
        kw = dict(eta_scale=w.eta, eta_tok=eta_tok, loss=w.loss, inner=w.inner, key_norm=w.key_norm)
        t = time.perf_counter()
        if mode == "backward":
            dO = rng.standard_normal(args[0].shape)
            orc.oracle_backward(*args, W, dO, **kw)
        else:
            if w.conv_k:
                kw["grid"] = w.grid
            orc.oracle_forward(*args, W, chunk=w.chunk, renorm=w.renorm, **kw, **okw)
        t_total += time.perf_counter() - t
        done += 1
    pairs = done * (w.H if w.inner == "vit3" else 1)
    pair_tokens_per_s = pairs * w.N / t_total
    return {"value": pair_tokens_per_s / w.H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} (b,h) {'blocks' if w.inner == 'vit3' else 'pairs'} of the same workload's inputs "
                      f"({pairs * w.N} pair-tokens), {t_total:.1f} s of float64 NumPy "
                      f"({'outer-loop backward' if mode == 'backward' else 'forward'}); tokens/s = pair-tokens/s / H"}


def oracle_kwargs(opts, nm):
    """ttt_options keywords -> the oracle's keywords."""
    if not opts:
        return {}
    kw = dict(opts)
    if "update_mask" in kw:
        kw["update_mask"] = [bool(kw["update_mask"] >> i & 1) for i in range(nm)]
    return kw


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    i = (len(xs) - 1) * q
    lo, hi = int(i), min(int(i) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)


def measure_mfma_peak(torch, blib):
    """bf16 MFMA throughput of a chip-filling micro-benchmark (TFLOP/s) and the
    shader clock (MHz) one of its blocks saw."""
    blocks, iters = 8 * 256, 5000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    args = lambda it: (blocks, it, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clk.data_ptr()),
                       ctypes.c_void_p(stream))
    for _ in range(2):
        blib.bench_mfma_peak_launch(*args(500))
    torch.cuda.synchronize()
    best, mhz = None, None
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        blib.bench_mfma_peak_launch(*args(iters))
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        if best is None or ms < best:
            best = ms
            c, r = clk.cpu().tolist()
            mhz = c * 100.0 / r if r else None
    return blib.bench_mfma_peak_flops(blocks, iters) / (best * 1e-3) / 1e12, mhz


def measure_overlap(torch):
    """Times of the overlap probe: 16 MFMAs (16x16x32 bf16) and/or NV packed
    f16 FMAs per wave and iteration, one or two waves per SIMD, no memory."""
    blib = ctypes.CDLL(os.path.join(ROOT, "linear_complexity_attention_amd", "libttt_bench.so"))
    blib.bench_overlap_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    sink = torch.empty(cu * 512, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    names = ["1 wave/SIMD: 16 MFMA", "1 wave/SIMD: 64 VALU", "1 wave/SIMD: 16 MFMA + 32 VALU in one wave",
             "1 wave/SIMD: 16 MFMA + 64 VALU in one wave", "2 waves/SIMD: 16 MFMA each",
             "2 waves/SIMD: one 16 MFMA, the other 64 VALU", "2 waves/SIMD: 16 MFMA + 64 VALU in each"]
    out = {"iterations": iters, "cus": cu, "ms": {}}
    for i, name in enumerate(names):
        blib.bench_overlap_launch(i, cu, 200, ctypes.c_void_p(sink.data_ptr()), stream)
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            blib.bench_overlap_launch(i, cu, iters, ctypes.c_void_p(sink.data_ptr()), stream)
            b.record()
            torch.cuda.synchronize()
            best = a.elapsed_time(b) if best is None else min(best, a.elapsed_time(b))
        out["ms"][name] = round(best, 3)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3_hires_r4", choices=sorted(VARIANTS))
    ap.add_argument("--burst", type=int, default=10, help="steps between the spread events")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the clock probe and the MFMA micro-benchmark")
    ap.add_argument("--mfma-valu-overlap", action="store_true",
                    help="only run the MFMA / packed-f16 VALU overlap micro-benchmark and print its times")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (fp32 read + write) five times; its "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "runs on one GPU only; --gpus must be 1 (sharding over (batch, head) "
                                   "pairs across GPUs is not built)"}))
        sys.exit(2)

    import torch

    if args.mfma_valu_overlap:
        print(json.dumps(measure_overlap(torch)))
        return

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))
        return

    from linear_complexity_attention_amd import ttt
    from synth_inputs import make_inputs

    wname, opts, mode, bound = VARIANTS[args.workload]
    w = bench_workloads()[wname]
    dev = torch.device("cuda:0")
    q, k, v, W0, et = make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    tq, tk, tv = (torch.from_numpy(a).to(dev).to(tdt).contiguous() for a in (q, k, v))
    tW = [torch.from_numpy(m).to(dev).contiguous() for m in W0]
    tet = torch.from_numpy(et).to(dev).contiguous() if et is not None else None
    layer = ttt.TTTLayer(w.B, w.H, w.N, w.d, w.hidden, dtype=w.dtype, key_norm=w.key_norm, eps=1e-5,
                         renorm=w.renorm, grid=w.grid, conv_k=w.conv_k)
    options = ttt.make_options(**opts) if opts else None
    out = torch.empty_like(tq)
    stream = torch.cuda.current_stream(dev)
    if mode == "backward":
        dO = torch.from_numpy(make_inputs(w, seed=w.seed + 7)[0]).to(dev).to(tdt).contiguous()

        def step():
            layer.backward(tq, tk, tv, tW, dO, eta=w.eta, eta_tok=tet, loss=w.loss, inner=w.inner)
    else:
        def step():
            layer.forward(tq, tk, tv, tW, eta=w.eta, eta_tok=tet, loss=w.loss, inner=w.inner, chunk=w.chunk,
                          out=out, options=options)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps.  Inside it the library records two HIP events per
    # step on its own stream around the dominant kernel family (the gradient of
    # the first update batch), for the roofline, and one event marks every
    # burst of steps, for the spread of the step time.  (Every recorded event
    # adds a little time between kernels, so no others are recorded here.)
    timed_events = mode == "forward"
    ev_grad = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] if timed_events else []
    burst = max(1, min(args.burst, args.steps))
    nburst = args.steps // burst
    ev_burst = [torch.cuda.Event(enable_timing=True) for _ in range(nburst + 1)]
    for a, b in ev_grad:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_burst[0].record(stream)
    for i in range(args.steps):
        if timed_events:
            a, b = ev_grad[i]
            ttt.ttt_set_timing_events(layer.handle, [None, None, a.cuda_event, b.cuda_event, None, None, None, None])
        step()
        if (i + 1) % burst == 0 and (i + 1) // burst <= nburst:
            ev_burst[(i + 1) // burst].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ttt.ttt_set_timing_events(layer.handle, None)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_step = [ev_burst[j].elapsed_time(ev_burst[j + 1]) / burst for j in range(nburst)]
    grad_ms = sum(a.elapsed_time(b) for a, b in ev_grad) / len(ev_grad) if ev_grad else None

    # Per-family breakdown, outside the timed region: all four families timed
    # with events on a few more steps.
    kern_ms = None
    if mode == "forward":
        nb = min(args.steps, 20)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(nb)]
        for row in evs:
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        for i in range(nb):
            ttt.ttt_set_timing_events(layer.handle, [e.cuda_event for e in evs[i]])
            step()
        torch.cuda.synchronize()
        ttt.ttt_set_timing_events(layer.handle, None)
        fam = {"key_stats": 0, "grad": 1, "update": 2, "readout": 3}
        kern_ms = {n: sum(evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for i in range(nb)) / nb
                   for n, j in fam.items()}

    # shader clock under the workload (a probe after each of 30 more steps) and
    # the MFMA micro-benchmark
    extras = {}
    if not args.no_extras:
        from linear_complexity_attention_amd import build_lib

        if os.path.exists(build_lib.BENCH_LIB):
            blib = ctypes.CDLL(build_lib.BENCH_LIB)
            blib.bench_mfma_peak_flops.restype = ctypes.c_double
            blib.bench_mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int]
            slots = torch.zeros((30, 3), dtype=torch.int64, device=dev)
            for i in range(30):
                step()
                blib.bench_clock_probe_launch(2000, ctypes.c_void_p(slots[i].data_ptr()),
                                              ctypes.c_void_p(stream.cuda_stream))
            torch.cuda.synchronize()
            s = slots.cpu().tolist()
            mhz = sorted(c * 100.0 / r for c, r, _ in s if r > 0)
            extras["shader_clock_mhz"] = {"median": percentile(mhz, 0.5), "min": mhz[0], "max": mhz[-1],
                                          "how": "s_memtime / s_memrealtime (100 MHz) of a probe wave "
                                                 "enqueued after each of 30 steps"}
            peak, peak_mhz = measure_mfma_peak(torch, blib)
            extras["mfma_bf16_microbench_tflops"] = peak
            extras["mfma_microbench_clock_mhz"] = peak_mhz
        else:
            extras["note"] = "libttt_bench.so not built: no clock probe or MFMA micro-benchmark"

    tokens = w.B * w.N
    value = tokens / (ms_per_step * 1e-3)
    P = w.B * w.H
    chunks = 1 if w.chunk == 0 else (w.N + w.chunk - 1) // w.chunk
    f_fb, f_q = gemm_flops(w, w.N, mode)
    epochs = (opts or {}).get("epochs", 1)
    layer_flops = P * (f_fb * epochs + f_q)
    path = layer.path_name(w.loss, w.inner, w.chunk, options) if mode == "forward" else "backward_generic"
    first_tokens = w.N if w.chunk == 0 else min(w.chunk, w.N)
    roof = {"bound": bound}
    if mode == "backward":
        # the whole step: batched products on the fp32 matrix cores plus elementwise passes
        achieved = layer_flops / (ms_per_step * 1e-3) / 1e12
        roof.update(kernel="outer-loop backward step (fp32 MFMA products + elementwise passes)", achieved=achieved,
                    peak=PEAK_FP32_TFLOPS, unit="TFLOP/s", frac=achieved / PEAK_FP32_TFLOPS, traffic=None,
                    algorithmic_flops_per_launch=layer_flops)
    else:
        kname = {"mfma": "fused forward/backward (k_mfma_grad)",
                 "mfma_fused": "fused forward/backward, gradient step and readout (k_mfma_grad, whole pairs)",
                 "mfma_swiglu": "SwiGLU forward/backward (k_lact_grad), first chunk"}.get(
                     path, "gradient kernels of the first update batch")
        fp32_mfma = path.startswith("mfma_f32")
        if fp32_mfma:
            kname = "fp32 matrix-core step (k_gemm_f32 products + passes), first update batch"
        grad_flops = P * gemm_flops(w, first_tokens)[0]
        if path == "mfma_fused":          # the same kernel also computes the readout
            grad_flops += P * f_q
        if w.inner == "vit3":
            grad_flops = w.B * (w.H - 1) * gemm_flops(w, first_tokens)[0]
            kname = f"GLU gradient (k_glu_grad, MFMA bf16), heads 1..{w.H - 1} of the block"
        if bound == "hbm":
            nbytes = P * first_tokens * w.d * 2 * (2 if w.dtype == "bf16" else 4)   # K and V once
            achieved = nbytes / (grad_ms * 1e-3) / 1e9
            roof.update(kernel=kname, achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s", frac=achieved / PEAK_HBM_GBS,
                        traffic=stored_traffic("grad", args.workload), algorithmic_bytes_per_launch=nbytes)
        else:
            peak = PEAK_BF16_TFLOPS if bound == "mfma" and not fp32_mfma else PEAK_FP32_TFLOPS
            achieved = grad_flops / (grad_ms * 1e-3) / 1e12
            roof.update(kernel=kname, achieved=achieved, peak=peak, unit="TFLOP/s", frac=achieved / peak,
                        traffic=stored_traffic("grad", args.workload), algorithmic_flops_per_launch=grad_flops)
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} hidden={w.hidden} "
                               f"inner={w.inner} loss={w.loss} eta={w.eta:.6g} chunk={w.chunk} "
                               f"key_norm={w.key_norm} renorm={w.renorm} options={opts} mode={mode} "
                               f"({w.dtype} tensors, fp32 accumulation)",
                   "global_batch": w.B, "seq_len": w.N, "heads": w.H, "head_dim": w.d, "hidden": w.hidden,
                   "path": path},
        "step_ms": {"median": percentile(per_step, 0.5), "p10": percentile(per_step, 0.1),
                    "p90": percentile(per_step, 0.9), "bursts": nburst, "steps_per_burst": burst},
        "layer_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "frac_of_bf16_peak": layer_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "kernel_ms": kern_ms,
        "kernel_ms_note": "per-family times from a separate pass with events around every kernel "
                          "(outside the timed region); roofline uses the timed region's own events",
        "roofline": roof,
    }
    res.update(extras)
    if "mfma_bf16_microbench_tflops" in res:
        res["frac_of_microbench_peak"] = res["layer_tflops"] / res["mfma_bf16_microbench_tflops"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, (q, k, v, W0, et),
                                           oracle_kwargs(opts, len(W0)), mode)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
