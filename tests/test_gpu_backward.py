"""GPU parity of the outer-loop backward (gradients through the inner update)
against the float64 oracle's hand backward (itself pinned by finite
differences and torch autograd), through the C ABI, on every pair: dQ, dK,
dV, dW0 and d eta, for the linear and GELU-MLP inner models, both losses, key
norm on and off, shared and per-batch W0, bf16 and fp32 tensors; the GELU-MLP
shapes with d and h multiples of 16 take the fp32 matrix-core path, the
others the generic kernels.  The
backward computes in fp32, so the bar is the fp32 one on every output:
max|err| / max|ref| <= 1e-4."""
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as orc
from synth_inputs import Workload
from tests.gpu_common import device_inputs, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("inner,loss,key_norm,dtype,shared,N,d,hidden", [
    ("mlp_gelu", "mse", True, "bf16", True, 333, 64, 256),
    ("mlp_gelu", "dot", False, "bf16", False, 200, 64, 128),
    ("mlp_gelu", "mse", False, "f32", True, 150, 32, 64),
    ("mlp_gelu", "dot", True, "f32", False, 77, 48, 96),
    ("mlp_gelu", "mse", True, "bf16", True, 100, 40, 72),    # d, h not multiples of 16: generic kernels
    ("linear", "mse", True, "bf16", True, 300, 64, 64),
    ("linear", "dot", False, "f32", False, 120, 128, 128),
])
def test_outer_backward(inner, loss, key_norm, dtype, shared, N, d, hidden):
    from linear_complexity_attention_amd import ttt

    w = Workload("bwd", B=2, H=3, N=N, d=d, hidden=hidden, dtype=dtype, inner=inner, loss=loss, key_norm=key_norm,
                 per_token_eta=True, eta=2.0 if loss == "mse" else 0.05, seed=900 + N)
    dev_in, exact = device_inputs(w, shared_w0=shared)
    tq, tk, tv, tW, tet = dev_in
    tdt = tq.dtype
    dO = torch.from_numpy(np.random.default_rng(w.seed + 1).standard_normal((2, 3, N, d), dtype=np.float32)).to(
        tq.device).to(tdt).contiguous()
    layer = ttt.TTTLayer(2, 3, N, d, hidden, dtype=dtype, key_norm=key_norm)
    g = layer.backward(tq, tk, tv, tW, dO, eta=w.eta, eta_tok=tet, loss=loss, inner=inner)
    torch.cuda.synchronize()
    ref = orc.oracle_backward(exact["q"], exact["k"], exact["v"], exact["W0"], dO.double().cpu().numpy(),
                              eta_scale=w.eta, eta_tok=exact["eta_tok"], loss=loss, inner=inner, key_norm=key_norm,
                              eps=1e-5)
    tag = f"{inner} {loss} kn={key_norm} {dtype} shared={shared}"
    for name in ("dq", "dk", "dv", "deta"):
        e = rel_err(g[name].cpu().numpy(), ref[name])
        assert e <= 1e-4, f"{tag}: {name} rel err {e:.3e}"
    for i, (a, b) in enumerate(zip(g["dW0"], ref["dW0"])):
        e = rel_err(a.cpu().numpy(), b)
        assert e <= 1e-4, f"{tag}: dW0[{i}] rel err {e:.3e}"
