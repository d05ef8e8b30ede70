"""Seeded synthetic inputs for the TTT-layer workloads.

This module only draws random numbers: it holds none of the layer's arithmetic,
so both the HIP path's tests/benchmark and the float64 CPU oracle can take their
inputs from it without sharing any of the method.  Every array is drawn with
NumPy's PCG64 generator (``numpy.random.default_rng(seed)``) in float32, in the
fixed order Q, K, V, W1, W2[, W3], eta.  Casting to bfloat16 (round to nearest
even) is left to the caller.

The shapes stand in for the pages' workloads (ImageNet ViT-S with 14x14 patches,
1248^2 images at patch 16 = 6084 tokens, a 128x128 DiT latent, 32K-token LaCT
language training); none of those datasets is available, so seeded Gaussians
take their place.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    hidden: int
    dtype: str = "bf16"           # dtype of q, k, v, o ("f32" or "bf16")
    inner: str = "mlp_gelu"       # "linear" | "mlp_gelu" | "swiglu"
    loss: str = "mse"             # "mse" | "dot"
    chunk: int = 0                # 0: full batch; C > 0: causal chunks of C tokens
    key_norm: bool = True
    renorm: bool = False
    eta: float = 1.0
    per_token_eta: bool = False
    key_shift: float = 0.5        # constant added to every key channel
    unit_columns: bool = False    # W0 columns scaled to unit L2 norm
    seed: int = 0
    grid: tuple = (0, 0)          # token raster (convolution inner models)
    conv_k: int = 0               # convolution kernel size
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.B * self.N


WORKLOADS = {
    "c1_tiny_fp32": Workload("c1_tiny_fp32", B=1, H=1, N=256, d=32, hidden=32,
                             dtype="f32", seed=1001),
    "c2_vits_r1": Workload("c2_vits_r1", B=64, H=6, N=196, d=64, hidden=64, seed=1002),
    "c2_vits_r4": Workload("c2_vits_r4", B=64, H=6, N=196, d=64, hidden=256, seed=1012),
    "c3_hires_r4": Workload("c3_hires_r4", B=8, H=12, N=6084, d=64, hidden=256, seed=1003),
    "c4_dit_h64": Workload("c4_dit_h64", B=2, H=24, N=16384, d=64, hidden=64, seed=1004),
    "c5_lact_swiglu": Workload("c5_lact_swiglu", B=1, H=4, N=32768, d=128, hidden=256,
                               inner="swiglu", loss="dot", chunk=2048, key_norm=False,
                               renorm=True, per_token_eta=True, key_shift=0.0,
                               unit_columns=True, seed=1005),
}


def matrix_shapes(inner: str, d: int, hidden: int, conv_k: int = 3):
    if inner == "linear":
        return [(d, d)]
    if inner == "mlp_gelu":
        return [(d, hidden), (hidden, d)]
    if inner == "swiglu":
        return [(d, hidden), (hidden, d), (d, hidden)]
    if inner == "glu":
        return [(d, d), (d, d)]
    if inner == "dwconv":
        return [(d, conv_k * conv_k)]
    if inner == "vit3":
        return [(d, d), (d, d), (d, conv_k * conv_k)]
    raise ValueError(inner)


def make_inputs(w: Workload, *, B=None, H=None, N=None, seed=None, shared_w0=True):
    """Draw q, k, v [B,H,N,d], W0 (list of [H,in,out] float32) and eta_tok.

    Q, K, V ~ N(0, 1), then ``key_shift`` is added to every key channel (the
    constant key shift the key normalisation must cancel).  W0 ~ N(0, 1/d) for
    every matrix, or Gaussian columns scaled to unit L2 norm when
    ``unit_columns``; a convolution kernel [d, k*k] ~ N(0, 1/k^2) (each output
    is a sum of k^2 taps).  eta_tok = 0.1 * softplus(z), z ~ N(0, 1) per (b, h, n),
    when ``per_token_eta`` (else None).  With ``shared_w0=False`` W0 gets a
    leading batch axis ([B, H, in, out]).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (B, H, N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.key_shift:
        k += np.float32(w.key_shift)
    lead = (H,) if shared_w0 else (B, H)
    W0 = []
    shapes = matrix_shapes(w.inner, w.d, w.hidden, w.conv_k)
    for i, (fi, fo) in enumerate(shapes):
        m = rng.standard_normal(lead + (fi, fo), dtype=np.float32)
        conv = (w.inner == "dwconv") or (w.inner == "vit3" and i == 2)
        if conv:
            m *= np.float32(1.0 / w.conv_k)
        elif w.unit_columns:
            m /= np.sqrt((m.astype(np.float64) ** 2).sum(axis=-2, keepdims=True)).astype(np.float32)
        else:
            m *= np.float32(1.0 / np.sqrt(w.d))
        W0.append(np.ascontiguousarray(m))
    eta_tok = None
    if w.per_token_eta:
        z = rng.standard_normal((B, H, N), dtype=np.float32)
        eta_tok = (0.1 * np.logaddexp(0.0, z.astype(np.float64))).astype(np.float32)
    return q, k, v, W0, eta_tok
