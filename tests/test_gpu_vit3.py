"""GPU parity of ViT3's inner models against the float64 oracle, through the C
ABI, on every pair: the simplified GLU FC(x)*SiLU(FC(x)), the depthwise
convolution over the token raster (kernel sizes 1..7, square and ragged
rasters, both channel blocks of a lane), and the ViT3 block that gives head 0
the convolution and the other heads the GLU.  Bar: max|err| / max|ref| <= 1e-2
(bf16) or 1e-4 (fp32) on O and on dW of every matrix a head uses."""
import numpy as np
import pytest

from synth_inputs import Workload
from tests.gpu_common import TOL, device_inputs, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _check(w, *, opts=None, okw=None, path=None, flags=0):
    from linear_complexity_attention_amd import ttt
    from oracle import ttt_oracle as orc

    options = ttt.make_options(**opts) if opts else None
    dev_in, exact = device_inputs(w)
    O, W_out, got = run_gpu(w, dev_in, options=options, flags=flags)
    O_ref, W_ref = run_oracle(w, exact, okw=okw)
    tol = TOL[w.dtype]
    tag = f"{w.name} {w.inner} {w.dtype} {w.loss} kn={w.key_norm} grid={w.grid} k={w.conv_k} path={got}"
    e = rel_err(O.float().cpu().numpy(), O_ref)
    assert e <= tol, f"{tag}: O rel err {e:.3e}"
    Wg = [m.cpu().numpy() for m in W_out]
    for h in range(w.H):
        _, used = orc.head_model(w.inner, h)
        for i in used:
            w0 = exact["W0"][i][h]
            e = rel_err(Wg[i][:, h] - w0, W_ref[i][:, h] - w0)
            assert e <= tol, f"{tag}: head {h} dW{i} rel err {e:.3e}"
    if path is not None:
        assert got == path, tag


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("loss,key_norm,d", [("dot", True, 64), ("mse", False, 64), ("dot", False, 32),
                                             ("mse", True, 128)])
def test_glu(dtype, loss, key_norm, d):
    w = Workload("glu", B=2, H=3, N=333, d=d, hidden=d, dtype=dtype, inner="glu", loss=loss, key_norm=key_norm,
                 per_token_eta=loss == "dot", eta=1.0 if loss == "mse" else 0.01, seed=601 + d)
    # bf16 at d = 64 takes the MFMA GLU kernels, everything else the generic ones
    _check(w, path="mfma_glu" if dtype == "bf16" and d == 64 else "generic")


@pytest.mark.parametrize("loss", ["dot", "mse"])
def test_glu_generic_forced_and_mfma_ragged(loss):
    """The generic GLU kernels on bf16 tensors (forced), and the MFMA ones on a
    ragged token count that leaves a partial last tile in several splits."""
    w = Workload("glu2", B=3, H=2, N=1001, d=64, hidden=64, inner="glu", loss=loss, key_norm=True,
                 per_token_eta=True, eta=1.0 if loss == "mse" else 0.003, seed=650)
    _check(w, path="generic", flags=0x2)
    _check(w, path="mfma_glu")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("k,grid,d,loss,key_norm", [
    (3, (14, 14), 64, "dot", True),
    (3, (13, 17), 64, "mse", False),
    (1, (9, 11), 64, "mse", True),
    (5, (12, 10), 128, "dot", False),
    (7, (11, 9), 48, "mse", True),
    (3, (10, 21), 128, "mse", True),
    (7, (20, 19), 64, "dot", True),
    (3, (17, 9), 32, "dot", False),
    (5, (1, 37), 16, "mse", True),
    (3, (190, 190), 64, "dot", True),
])
def test_dwconv(dtype, k, grid, d, loss, key_norm):
    """The LDS-tiled kernels take d in {8, ..., 128} whose window fits 64 KiB
    (8 x 8 tiles, ragged edges, one tile row, more tiles than workgroups at
    190 x 190); d = 48 and k = 5 at d = 128 take the direct kernels."""
    N = grid[0] * grid[1]
    w = Workload("dw", B=2, H=2, N=N, d=d, hidden=d, dtype=dtype, inner="dwconv", loss=loss, key_norm=key_norm,
                 per_token_eta=loss == "dot", eta=1.0 if loss == "mse" else 0.01, grid=grid, conv_k=k,
                 seed=700 + k + d)
    _check(w, path="dwconv")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,loss", [(4, "dot"), (3, "mse"), (1, "dot")])
def test_vit3_block(dtype, H, loss):
    w = Workload("vit3", B=2, H=H, N=196, d=64, hidden=64, dtype=dtype, inner="vit3", loss=loss, key_norm=True,
                 eta=1.0 / 196 if loss == "dot" else 1.0, grid=(14, 14), conv_k=3, seed=800 + H)
    _check(w, path="dwconv+mfma_glu" if dtype == "bf16" and H > 1 else "dwconv+generic")


def test_dwconv_with_epochs_and_momentum():
    w = Workload("dwe", B=1, H=2, N=150, d=64, hidden=64, inner="dwconv", loss="mse", key_norm=True,
                 grid=(10, 15), conv_k=3, seed=810)
    _check(w, opts=dict(epochs=3, rule="momentum", beta=0.5), okw=dict(epochs=3, rule="momentum", beta=0.5))


def test_vit3_block_full_size():
    """The ViT3 block at 1248^2 in the benchmark's configuration (B=8, H=12,
    N=6084 on a 78 x 78 raster, d=64, 3 x 3 convolution head, dot loss,
    eta = 1/N), every pair: the LDS-tiled convolution with a hundred tiles
    per pair, the GLU kernels' full token splits and the statistics merge."""
    w = Workload("vit3_hires", B=8, H=12, N=6084, d=64, hidden=64, inner="vit3", loss="dot", key_norm=True,
                 eta=1.0 / 6084, grid=(78, 78), conv_k=3, seed=1006)
    _check(w, path="dwconv+mfma_glu")
