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


def test_outer_backward_c3_full_size():
    """The outer-loop backward at c3 size (B=8, H=12, N=6084, d=64, h=256,
    MSE, key norm, shared W0), as the benchmark runs it: dq, dk, dv and deta
    of sampled pairs and dW0 of sampled heads (a shared W0 sums its pairs, so
    a head's dW0 is checked against the sum of the oracle's per-pair
    gradients over the batch)."""
    from linear_complexity_attention_amd import ttt
    from synth_inputs import WORKLOADS

    w = WORKLOADS["c3_hires_r4"]
    B, H, N, d = w.B, w.H, w.N, w.d
    dev_in, exact = device_inputs(w)
    tq, tk, tv, tW, tet = dev_in
    dO = torch.from_numpy(np.random.default_rng(w.seed + 7).standard_normal((B, H, N, d), dtype=np.float32)).to(
        tq.device).to(tq.dtype).contiguous()
    layer = ttt.TTTLayer(B, H, N, d, w.hidden, dtype=w.dtype, key_norm=w.key_norm)
    g = layer.backward(tq, tk, tv, tW, dO, eta=w.eta, eta_tok=tet, loss=w.loss, inner=w.inner)
    torch.cuda.synchronize()
    dO64 = dO.double().cpu().numpy()
    heads = (0, 7, 11)
    dW0_ref = [np.zeros((len(heads),) + m.shape[1:]) for m in exact["W0"]]
    for b in range(B):
        sl = np.s_[b:b + 1]
        for hi, h in enumerate(heads):
            hs = np.s_[h:h + 1]
            ref = orc.oracle_backward(exact["q"][sl][:, hs], exact["k"][sl][:, hs], exact["v"][sl][:, hs],
                                      [m[hs] for m in exact["W0"]], dO64[sl][:, hs], eta_scale=w.eta,
                                      eta_tok=None, loss=w.loss, inner=w.inner, key_norm=w.key_norm, eps=1e-5)
            for i in range(2):
                dW0_ref[i][hi] += ref["dW0"][i][0]
            if b in (0, 5):
                for name in ("dq", "dk", "dv", "deta"):
                    e = rel_err(g[name][b, h].cpu().numpy(), ref[name][0, 0])
                    assert e <= 1e-4, f"c3 backward pair ({b}, {h}): {name} rel err {e:.3e}"
    for i in range(2):
        got = g["dW0"][i][list(heads)].cpu().numpy()
        e = rel_err(got, dW0_ref[i])
        assert e <= 1e-4, f"c3 backward: dW0[{i}] rel err {e:.3e}"
