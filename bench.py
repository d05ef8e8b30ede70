"""Benchmark of the TTT-layer forward on one MI355X.

A step is one ttt_forward over one batch of synthetic input: key statistics,
fused forward/backward of the inner model, weight update and readout (every
kernel of the layer).  Default workload: B=8, H=12, N=6084 (1248^2 image at
patch 16), d=64, inner GELU MLP of width 256 (r=4), MSE loss, eta=1, one
full-batch step, key instance norm, bf16 tensors with fp32 accumulation.

Prints one JSON line with the whole-job throughput (tokens/s, tokens = B*N),
the roofline position of the dominant kernel (timed with HIP events inside the
timed region, on the stream it runs on) and the float64 CPU oracle timed on a
bounded sample of the same workload.
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

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)


def gemm_flops(w, tokens_per_pair):
    """Algorithmic flops (2*m*n*k per product) of one pass over the tokens."""
    g = 2.0 * tokens_per_pair * w.d * w.hidden
    if w.inner == "mlp_gelu":
        n_fb = 5 if w.loss == "mse" else 4          # Z, [V_hat], dW2, dA, dW1
        n_q = 2
    elif w.inner == "swiglu":
        n_fb = 7 if w.loss == "mse" else 6          # Z1, Z3, [V_hat], dW2, dH, dW1, dW3
        n_q = 3
    else:
        g = 2.0 * tokens_per_pair * w.d * w.d
        n_fb = 2 if w.loss == "mse" else 1
        n_q = 1
    return g * n_fb, g * n_q


def kernel_source_hash():
    h = hashlib.sha256()
    for name in sorted(os.listdir(os.path.join(ROOT, "linear_complexity_attention_amd", "csrc"))):
        with open(os.path.join(ROOT, "linear_complexity_attention_amd", "csrc", name), "rb") as f:
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


def cpu_baseline(w, budget_s, inputs):
    """The float64 oracle on whole (b, h) pairs of the same workload and inputs,
    pair after pair (wrapping round) until `budget_s` seconds have passed;
    scaled to tokens/s of the whole layer."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import ttt_oracle as orc

    q, k, v, W0, et = inputs
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    done, t_total = 0, 0.0
    while t_total < budget_s:
        p = done % (w.B * w.H)
        b, h = divmod(p, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = [a[sl].astype(np.float64) for a in (q, k, v)]
        W = [m[h:h + 1].astype(np.float64) for m in W0]
        eta_tok = None if et is None else et[sl].astype(np.float64)
        t = time.perf_counter()
        orc.oracle_forward(*args, W, eta_scale=w.eta, eta_tok=eta_tok, loss=w.loss, inner=w.inner,
                           chunk=w.chunk, key_norm=w.key_norm, renorm=w.renorm)
        t_total += time.perf_counter() - t
        done += 1
    pair_tokens_per_s = done * w.N / t_total
    return {"value": pair_tokens_per_s / w.H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} (b,h) pair runs of the same workload's inputs ({done * w.N} pair-tokens, "
                      f"{w.B * w.H} distinct pairs cycled), {t_total:.1f} s of float64 NumPy; "
                      f"tokens/s = pair-tokens/s / H"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3_hires_r4")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (fp32 read + write) five times; its "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is described in DESIGN.md, not built)"}))
        sys.exit(2)

    import torch

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
    from synth_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v, W0, et = make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    tq, tk, tv = (torch.from_numpy(a).to(dev).to(tdt).contiguous() for a in (q, k, v))
    tW = [torch.from_numpy(m).to(dev).contiguous() for m in W0]
    tet = torch.from_numpy(et).to(dev).contiguous() if et is not None else None
    layer = ttt.TTTLayer(w.B, w.H, w.N, w.d, w.hidden, dtype=w.dtype, key_norm=w.key_norm, eps=1e-5,
                         renorm=w.renorm)
    out = torch.empty_like(tq)
    stream = torch.cuda.current_stream(dev)

    def step():
        layer.forward(tq, tk, tv, tW, eta=w.eta, eta_tok=tet, loss=w.loss, inner=w.inner, chunk=w.chunk,
                      out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps; inside it the library records two HIP events per
    # step on its own stream, around the dominant kernel (the forward/backward
    # of the first update batch), for the roofline figure.  (Every recorded
    # event adds a little time between kernels, so no others are recorded here.)
    ev_grad = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a, b in ev_grad:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        a, b = ev_grad[i]
        ttt.ttt_set_timing_events(layer.handle, [None, None, a.cuda_event, b.cuda_event, None, None, None, None])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    grad_ms = sum(a.elapsed_time(b) for a, b in ev_grad) / args.steps

    # Per-kernel breakdown, outside the timed region: all four families timed
    # with events on a few more steps.
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

    tokens = w.B * w.N
    value = tokens / (ms_per_step * 1e-3)
    P = w.B * w.H
    chunks = 1 if w.chunk == 0 else (w.N + w.chunk - 1) // w.chunk
    f_fb, f_q = gemm_flops(w, w.N)
    layer_flops = P * (f_fb + f_q)
    # dominant kernel: the fused forward/backward of the first (here: only) update batch
    first_tokens = w.N if w.chunk == 0 else min(w.chunk, w.N)
    grad_flops = P * gemm_flops(w, first_tokens)[0]
    achieved = grad_flops / (grad_ms * 1e-3) / 1e12
    path = layer.path_name(w.loss, w.inner, w.chunk)
    traffic = stored_traffic("grad", args.workload)
    res = {
        "metric": "TTT-layer tokens/sec on 1 MI355X (N=6084, r=4) + % of bf16 MFMA peak",
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
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} hidden={w.hidden} inner={w.inner} "
                               f"loss={w.loss} eta={w.eta} chunk={w.chunk} key_norm={w.key_norm} "
                               f"renorm={w.renorm} ({w.dtype} tensors, fp32 accumulation)",
                   "global_batch": w.B, "seq_len": w.N, "heads": w.H, "head_dim": w.d, "hidden": w.hidden,
                   "path": path},
        "layer_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "frac_of_bf16_peak": layer_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "kernel_ms": kern_ms,
        "kernel_ms_note": "per-family times from a separate pass with events around every kernel "
                          "(outside the timed region); roofline uses the timed region's own events",
        "roofline": {"kernel": {"mfma": "fused forward/backward (k_mfma_grad)",
                                "mfma_swiglu": "SwiGLU forward/backward (k_lact_grad), first chunk"}.get(path, "grad"),
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "algorithmic_flops_per_launch": grad_flops},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, (q, k, v, W0, et))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
