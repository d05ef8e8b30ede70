"""Shared helpers of the GPU parity tests: run the HIP library through its
binding and the float64 oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

from oracle import ttt_oracle as orc
from synth_inputs import WORKLOADS, Workload, make_inputs


def device_inputs(w: Workload, *, B=None, H=None, N=None, seed=None, shared_w0=True):
    """Seeded inputs on cuda:0 in the workload's dtype, plus the exact float64
    values the GPU receives (bf16-rounded inputs upcast) for the oracle."""
    q, k, v, W0, et = make_inputs(w, B=B, H=H, N=N, seed=seed, shared_w0=shared_w0)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(a).to(dev).to(tdt).contiguous() for a in (q, k, v))
    tW = [torch.from_numpy(m).to(dev).contiguous() for m in W0]
    tet = torch.from_numpy(et).to(dev).contiguous() if et is not None else None
    exact = dict(q=tq.double().cpu().numpy(), k=tk.double().cpu().numpy(), v=tv.double().cpu().numpy(),
                 W0=[m.astype(np.float64) for m in W0], eta_tok=None if et is None else et.astype(np.float64))
    return (tq, tk, tv, tW, tet), exact


def run_gpu(w: Workload, dev_in, *, flags=0, eta=None, return_weights=True, chunk=None, eps=1e-5, options=None):
    from linear_complexity_attention_amd import ttt

    tq, tk, tv, tW, tet = dev_in
    B, H, N, d = tq.shape
    layer = ttt.TTTLayer(B, H, N, d, w.hidden, dtype=w.dtype, key_norm=w.key_norm, eps=eps,
                         renorm=w.renorm, flags=flags, grid=w.grid, conv_k=w.conv_k)
    W_out = None
    if return_weights:
        W_out = [torch.empty((B, H) + tuple(m.shape[-2:]), dtype=torch.float32, device=tq.device) for m in tW]
    O = layer.forward(tq, tk, tv, tW, eta=w.eta if eta is None else eta, eta_tok=tet, loss=w.loss,
                      inner=w.inner, chunk=w.chunk if chunk is None else chunk, W_out=W_out, options=options)
    torch.cuda.synchronize()
    path = layer.path_name(w.loss, w.inner, w.chunk if chunk is None else chunk, options)
    return O, W_out, path


def run_oracle(w: Workload, exact, *, pairs=None, eta=None, chunk=None, eps=1e-5, okw=None):
    """Oracle on all pairs, or on the listed (b, h) pairs only (each pair is
    independent, so a slice of the inputs gives that pair's exact result);
    okw: extra oracle keywords (update variants)."""
    kw = dict(eta_scale=w.eta if eta is None else eta, loss=w.loss, inner=w.inner,
              chunk=w.chunk if chunk is None else chunk, key_norm=w.key_norm, eps=eps, renorm=w.renorm)
    if w.conv_k:
        kw["grid"] = w.grid
    kw.update(okw or {})
    if pairs is None:
        return orc.oracle_forward(exact["q"], exact["k"], exact["v"], exact["W0"], eta_tok=exact["eta_tok"], **kw)
    Os, Ws = [], []
    for (b, h) in pairs:
        sl = (slice(b, b + 1), slice(h, h + 1))
        W0 = [m[h:h + 1] if m.ndim == 3 else m[b:b + 1, h:h + 1] for m in exact["W0"]]
        et = None if exact["eta_tok"] is None else exact["eta_tok"][sl]
        O, Wf = orc.oracle_forward(exact["q"][sl], exact["k"][sl], exact["v"][sl], W0, eta_tok=et, **kw)
        Os.append(O[0, 0])
        Ws.append([m[0, 0] for m in Wf])
    return Os, Ws


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / denom) if denom > 0 else float(np.max(np.abs(got)))


TOL = {"bf16": 1e-2, "f32": 1e-4}
