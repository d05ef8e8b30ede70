"""GPU parity: the HIP library (through the C ABI) against the float64 oracle
on the same seeded inputs.  Pass bar: max|O_gpu - O_ref| / max|O_ref| <= 1e-2
on the bf16 path and <= 1e-4 on the fp32 path, and the same bound on the
update itself (dW = W_out - W0, dO = O - F_W0(Q)) so that a wrong backward
cannot hide behind a small step."""
import numpy as np
import pytest
import torch

from oracle import ttt_oracle as orc
from synth_inputs import WORKLOADS, Workload
from tests.gpu_common import TOL, device_inputs, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

GENERIC = 0x2   # TTT_FLAG_FORCE_GENERIC
LOG = 0x4       # TTT_FLAG_LOG


def _w0_pair(exact, b, h):
    return [m[h] if m.ndim == 3 else m[b, h] for m in exact["W0"]]


def _all_pairs(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def _check_pairs(w, dev_in, exact, pairs, *, flags=0, tol=None, eta=None, chunk=None, tag="", eps=1e-5):
    """O and dW = W_out - W0 of every listed pair, element by element, against
    the oracle (pairs=None: all pairs)."""
    tol = TOL[w.dtype] if tol is None else tol
    pairs = _all_pairs(w) if pairs is None else pairs
    O, W_out, path = run_gpu(w, dev_in, flags=flags, eta=eta, chunk=chunk, eps=eps)
    O_ref, W_ref = run_oracle(w, exact, pairs=pairs, eta=eta, chunk=chunk, eps=eps)
    Og = O.float().cpu().numpy()
    Wg = [m.cpu().numpy() for m in W_out]
    for i, (b, h) in enumerate(pairs):
        e = rel_err(Og[b, h], O_ref[i])
        assert e <= tol, f"{tag} O pair {(b, h)} rel err {e:.3e} > {tol} (path {path})"
        w0 = _w0_pair(exact, b, h)
        for m in range(len(w0)):
            dW_ref = W_ref[i][m] - w0[m]
            if np.max(np.abs(dW_ref)) == 0.0:
                np.testing.assert_allclose(Wg[m][b, h], W_ref[i][m], atol=1e-6)
                continue
            e = rel_err(Wg[m][b, h] - w0[m], dW_ref)
            assert e <= tol, f"{tag} dW{m} pair {(b, h)} rel err {e:.3e} > {tol} (path {path})"
    return O, W_out, path


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------
def test_c1_tiny_fp32_full():
    w = WORKLOADS["c1_tiny_fp32"]
    dev_in, exact = device_inputs(w)
    O, W_out, path = _check_pairs(w, dev_in, exact, [(0, 0)], tag="c1")
    # the output change caused by the update, against the oracle's
    O0 = orc.oracle_readout(exact["q"], [m[None] for m in exact["W0"]], w.inner)
    O_ref, _ = run_oracle(w, exact)
    assert rel_err(O.double().cpu().numpy() - O0, O_ref - O0) <= 1e-4


@pytest.mark.parametrize("name", ["c2_vits_r1", "c2_vits_r4"])
def test_c2_vit_small_all_pairs(name):
    w = WORKLOADS[name]
    dev_in, exact = device_inputs(w)
    O, W_out, path = run_gpu(w, dev_in)
    O_ref, W_ref = run_oracle(w, exact)
    assert rel_err(O.float().cpu().numpy(), O_ref) <= 1e-2, path
    for m in range(2):
        dW = W_out[m].cpu().numpy() - exact["W0"][m][None]
        assert rel_err(dW, W_ref[m] - exact["W0"][m][None]) <= 1e-2, (path, m)
    _check_output_change(w, dev_in, exact, O, [(0, 0), (17, 2), (63, 5)], name)


def _check_output_change(w, dev_in, exact, O, pairs, tag):
    """dO = O - F_W0(Q), the output change the update causes, against the
    oracle's.  The GPU's F_W0(Q) comes from the same kernels at eta = 0, so the
    readout's smooth approximation errors largely cancel; what cannot cancel
    is rounding that differs between the two runs: the bf16 outputs (half an
    ulp each, 2^-9 of |O|) and the bf16 copies of W1* and W0 the readout
    stages (of the same order), hence tolerance
    1e-2 * max|dO_ref| + 2^-7 * max|O_ref|.  (A 5 % error in dW, with dO about
    a third of O, exceeds it.)"""
    O0g, _, _ = run_gpu(w, dev_in, eta=0.0, return_weights=False)
    O_ref, _ = run_oracle(w, exact, pairs=pairs)
    O0_ref, _ = run_oracle(w, exact, pairs=pairs, eta=0.0)
    Og, O0 = O.float().cpu().numpy(), O0g.float().cpu().numpy()
    for i, (b, h) in enumerate(pairs):
        d_ref = O_ref[i] - O0_ref[i]
        err = np.max(np.abs((Og[b, h] - O0[b, h]) - d_ref))
        tol = 1e-2 * np.max(np.abs(d_ref)) + 2.0 ** -7 * np.max(np.abs(O_ref[i]))
        assert err <= tol, f"{tag} dO pair {(b, h)}: max err {err:.3e} > {tol:.3e}"


# c3, c4, c5 at full size, in the launch configuration the benchmark times:
# O and dW of every (b, h) pair against the oracle (which computes each pair
# alone; pairs are independent), plus the output change on a sample of pairs
def test_c3_hires_all_pairs():
    w = WORKLOADS["c3_hires_r4"]
    dev_in, exact = device_inputs(w)
    O, _, path = _check_pairs(w, dev_in, exact, None, tag="c3")
    assert path == "mfma"
    _check_output_change(w, dev_in, exact, O, [(0, 0), (3, 7), (7, 11)], "c3")


def test_c4_dit_all_pairs():
    w = WORKLOADS["c4_dit_h64"]
    dev_in, exact = device_inputs(w)
    O, _, path = _check_pairs(w, dev_in, exact, None, tag="c4")
    assert path == "mfma"
    _check_output_change(w, dev_in, exact, O, [(0, 0), (1, 23)], "c4")


def test_c5_lact_all_pairs():
    w = WORKLOADS["c5_lact_swiglu"]
    dev_in, exact = device_inputs(w)
    _, _, path = _check_pairs(w, dev_in, exact, None, tag="c5")
    assert path == "mfma_swiglu"


# ---------------------------------------------------------------------------
# Every inner model x loss x mode, several tiles with a ragged tail
# ---------------------------------------------------------------------------
COMBOS = [
    ("mlp_gelu", "mse", 0, True, False),
    ("mlp_gelu", "dot", 0, True, False),
    ("swiglu", "dot", 0, True, True),
    ("swiglu", "mse", 0, False, False),
    ("linear", "mse", 0, True, False),
    ("linear", "dot", 0, False, True),
    ("swiglu", "dot", 96, False, True),
    ("mlp_gelu", "mse", 100, False, False),
    ("mlp_gelu", "dot", 64, False, True),
    # raw (not normalised) keys on the GELU-MLP MFMA kernel, and its stream-K
    # update followed by the column re-norm
    ("mlp_gelu", "mse", 0, False, False),
    ("mlp_gelu", "dot", 0, False, True),
    ("mlp_gelu", "mse", 0, True, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("inner,loss,chunk,key_norm,renorm", COMBOS)
@pytest.mark.parametrize("generic", [False, True])
def test_combos_ragged(inner, loss, chunk, key_norm, renorm, dtype, generic):
    w = Workload("combo", B=2, H=3, N=333, d=64, hidden=128, dtype=dtype, inner=inner, loss=loss, chunk=chunk,
                 key_norm=key_norm, renorm=renorm, per_token_eta=(loss == "dot"), seed=77,
                 unit_columns=renorm, eta=1.0 if loss == "mse" else 0.5)
    dev_in, exact = device_inputs(w)
    _check_pairs(w, dev_in, exact, [(0, 0), (1, 2)], flags=GENERIC if generic else 0,
                 tag=f"{inner}/{loss}/{chunk}/{dtype}/{'gen' if generic else 'auto'}")


# every instance of the GELU-MLP MFMA gradient kernel: hidden 64/128/256 x
# MSE/dot x key norm on/off, full batch, ragged N that spans several stream-K
# ranges (pairs x tiles > workgroups), with and without the column re-norm
@pytest.mark.parametrize("hidden", [64, 128, 256])
@pytest.mark.parametrize("loss", ["mse", "dot"])
@pytest.mark.parametrize("key_norm", [False, True])
def test_mfma_mlp_instances(hidden, loss, key_norm):
    renorm = loss == "dot"
    w = Workload("inst", B=3, H=5, N=1111, d=64, hidden=hidden, loss=loss, key_norm=key_norm, renorm=renorm,
                 per_token_eta=(loss == "dot"), unit_columns=renorm, seed=900 + hidden + 2 * key_norm,
                 eta=1.0 if loss == "mse" else 0.05)
    dev_in, exact = device_inputs(w)
    _, _, path = _check_pairs(w, dev_in, exact, None, tag=f"h={hidden} {loss} kn={key_norm}")
    assert path == "mfma"


# the direct mode of the same kernel (one workgroup per pair, which applies the
# gradient step itself): as many pairs as CUs, ragged N, every instance;
# sampled pairs (first, last and scattered), O and dW
@pytest.mark.parametrize("hidden", [64, 128, 256])
@pytest.mark.parametrize("loss", ["mse", "dot"])
@pytest.mark.parametrize("key_norm", [False, True])
def test_mfma_direct_instances(hidden, loss, key_norm, capfd):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = Workload("direct", B=cus // 8, H=8, N=77, d=64, hidden=hidden, loss=loss, key_norm=key_norm,
                 per_token_eta=(loss == "dot"), seed=700 + hidden + 2 * key_norm,
                 eta=1.0 if loss == "mse" else 0.05)
    dev_in, exact = device_inputs(w)
    pairs = [(0, 0), (1, 3), (w.B // 2, 5), (w.B - 1, 7)]
    _, _, path = _check_pairs(w, dev_in, exact, pairs, flags=LOG, tag=f"direct h={hidden} {loss} kn={key_norm}")
    assert path == "mfma_fused"
    assert "grad=mfma_direct" in capfd.readouterr().err


def test_mfma_direct_without_w_out():
    """The direct step with no W_out requested (as the benchmark calls it):
    O of sampled pairs against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = Workload("direct_o", B=cus // 8, H=8, N=77, d=64, hidden=256, seed=760)
    dev_in, exact = device_inputs(w)
    O, _, path = run_gpu(w, dev_in, return_weights=False)
    assert path == "mfma_fused"
    pairs = [(0, 0), (w.B // 2, 3), (w.B - 1, 7)]
    O_ref, _ = run_oracle(w, exact, pairs=pairs)
    for i, (b, h) in enumerate(pairs):
        assert rel_err(O[b, h].float().cpu().numpy(), O_ref[i]) <= 1e-2, (b, h, path)


def test_mfma_direct_batch_specific_w0():
    """The direct step with a W0 per (batch, head) (the step's W is read
    through the batch stride): O and dW of sampled pairs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = Workload("direct_bw0", B=cus // 8, H=8, N=100, d=64, hidden=64, seed=770)
    dev_in, exact = device_inputs(w, shared_w0=False)
    pairs = [(0, 1), (w.B // 3, 6), (w.B - 1, 0)]
    _, _, path = _check_pairs(w, dev_in, exact, pairs, flags=LOG, tag="direct per-batch W0")
    assert path == "mfma_fused"


# the direct step inside the stream-K split: more pairs than slots, short
# pairs, so some workgroups hold whole pairs (stepped by the gradient kernel)
# and others split pairs (finished by the update kernel); every 7th pair
@pytest.mark.parametrize("hidden,loss,key_norm", [(64, "mse", True), (256, "mse", True), (128, "dot", False)])
def test_mfma_direct_mixed(hidden, loss, key_norm, capfd):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pairs_per_slot = 2.5 if hidden == 64 else 1.25
    w = Workload("direct_mixed", B=int(cus * pairs_per_slot) // 8, H=8, N=100, d=64, hidden=hidden, loss=loss,
                 key_norm=key_norm, per_token_eta=(loss == "dot"), seed=730 + hidden,
                 eta=1.0 if loss == "mse" else 0.05)
    dev_in, exact = device_inputs(w)
    pairs = [divmod(i, w.H) for i in range(0, w.B * w.H, 7)]
    _, _, path = _check_pairs(w, dev_in, exact, pairs, flags=LOG, tag=f"direct mixed h={hidden} {loss}")
    assert path == "mfma"
    assert "grad=mfma_direct" in capfd.readouterr().err


@pytest.mark.parametrize("d,hidden,N", [(32, 32, 256), (64, 64, 130), (64, 256, 517), (128, 256, 300),
                                        (16, 48, 77), (64, 192, 250)])
def test_shapes_mlp_mse(d, hidden, N):
    w = Workload("shape", B=1, H=2, N=N, d=d, hidden=hidden, seed=5 + d + hidden + N)
    dev_in, exact = device_inputs(w)
    _check_pairs(w, dev_in, exact, [(0, 0), (0, 1)], tag=f"shape d={d} h={hidden} N={N}")


# the remaining kernel instances and the largest widths: SwiGLU at (d, h) =
# (64, 256) and (128, 128) (the LaCT kernels' other two shapes), the GELU MLP
# at h = 512 (the widest supported: the fp32 matrix-core step, and the generic
# kernels when forced) and the linear model at d = 128
@pytest.mark.parametrize("inner,loss,d,hidden,chunk,renorm,path", [
    ("swiglu", "dot", 64, 256, 100, True, "mfma_swiglu"),
    ("swiglu", "dot", 128, 128, 128, True, "mfma_swiglu"),
    ("mlp_gelu", "mse", 64, 512, 0, False, "mfma_f32_grad"),
    ("mlp_gelu", "mse", 64, 512, 0, False, "generic"),
    ("linear", "mse", 128, 128, 0, False, "generic"),
])
def test_shapes_other_kernels(inner, loss, d, hidden, chunk, renorm, path):
    w = Workload("shape2", B=1, H=2, N=300, d=d, hidden=hidden, inner=inner, loss=loss, chunk=chunk,
                 key_norm=(chunk == 0), renorm=renorm, per_token_eta=(loss == "dot"), unit_columns=renorm,
                 seed=11 + d + hidden, eta=0.3 if loss == "dot" else 1.0)
    dev_in, exact = device_inputs(w)
    flags = GENERIC if (inner == "mlp_gelu" and path == "generic") else 0
    _, _, got = _check_pairs(w, dev_in, exact, [(0, 0), (0, 1)], flags=flags,
                             tag=f"{inner} d={d} h={hidden} chunk={chunk} {path}")
    assert got == path


def test_large_eta_exposes_backward():
    """100x the step: the update dominates O, so an error in dW shows in O."""
    w = Workload("eta100", B=2, H=2, N=1000, d=64, hidden=256, seed=31, eta=100.0)
    dev_in, exact = device_inputs(w)
    _check_pairs(w, dev_in, exact, [(0, 0), (1, 1)], tag="eta100")


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
def test_single_token_with_key_norm_keeps_w0():
    w = Workload("n1", B=2, H=2, N=1, d=64, hidden=64, seed=41)
    dev_in, exact = device_inputs(w)
    O, W_out, _ = run_gpu(w, dev_in)
    for m, w0 in zip(W_out, dev_in[3]):
        torch.testing.assert_close(m, w0[None].expand_as(m), rtol=0, atol=1e-7)
    O_ref, _ = run_oracle(w, exact)
    assert rel_err(O.float().cpu().numpy(), O_ref) <= 1e-2


def test_single_token_tiny_eps_padding_rows():
    """N = 1 with a tiny eps: rstd is 1e5, so -mean * rstd of the 31 padding
    rows of the only tile is beyond the f16 range; those rows must not poison
    dW (W stays exactly W0, O is finite and equals the oracle)."""
    w = Workload("n1eps", B=1, H=3, N=1, d=64, hidden=256, seed=48)
    dev_in, exact = device_inputs(w)
    O, W_out, path = run_gpu(w, dev_in, eps=1e-10)
    assert path == "mfma_fused"      # three one-tile pairs: each workgroup holds one whole
    for m, w0 in zip(W_out, dev_in[3]):
        torch.testing.assert_close(m, w0[None].expand_as(m), rtol=0, atol=1e-7)
    assert torch.isfinite(O.float()).all()
    O_ref, _ = run_oracle(w, exact, eps=1e-10)
    assert rel_err(O.float().cpu().numpy(), O_ref) <= 1e-2


def test_binding_rejects_bad_tensors():
    """The binding checks every tensor's device, dtype, layout and shape before
    the C call, so a mismatch cannot reach the kernels."""
    from linear_complexity_attention_amd import ttt

    w = Workload("val", B=2, H=2, N=64, d=64, hidden=128, seed=49)
    (tq, tk, tv, tW, _), _ = device_inputs(w)
    layer = ttt.TTTLayer(2, 2, 64, 64, 128)
    bad_w0 = [
        [tW[0][:, :32].contiguous(), tW[1]],                     # wrong inner shape
        [tW[0], tW[1].transpose(-1, -2).contiguous()],             # W2 stored [d, h]
        [tW[0].double(), tW[1]],                                   # dtype
        [tW[0][None].expand(2, -1, -1, -1).contiguous(), tW[1]],   # mixed layouts
        [tW[0]],                                                   # too few matrices
    ]
    for W0 in bad_w0:
        with pytest.raises(ValueError):
            layer.forward(tq, tk, tv, W0)
    with pytest.raises(ValueError):
        layer.forward(tq, tk, tv, tW, eta_tok=torch.ones(2, 2, 63, device=tq.device))
    with pytest.raises(ValueError):
        layer.forward(tq, tk, tv, tW, out=torch.empty(2, 2, 64, 32, dtype=torch.bfloat16, device=tq.device))
    with pytest.raises(ValueError):
        layer.forward(tq, tk, tv, tW, W_out=[torch.empty(2, 2, 64, 128, device=tq.device),
                                             torch.empty(2, 2, 64, 128, device=tq.device)])
    with pytest.raises(ValueError):
        layer.forward(tq[:, :, :, :32], tk, tv, tW)
    O = layer.forward(tq, tk, tv, tW)          # the valid call still works
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all()


def test_eta_zero_reads_w0():
    w = Workload("eta0", B=1, H=3, N=200, d=64, hidden=256, seed=42, eta=0.0)
    dev_in, exact = device_inputs(w)
    O, W_out, _ = run_gpu(w, dev_in)
    O0 = orc.oracle_readout(exact["q"], [m[None] for m in exact["W0"]], w.inner)
    assert rel_err(O.float().cpu().numpy(), O0) <= 1e-2


# (chunk, N, eta): many sequential updates make the recurrence sensitive to
# rounding (a relative perturbation of W0 grows with every chunk), so the step
# sizes are chosen where the oracle's own amplification of a 1e-6 perturbation
# stays below ~10x; the stress workload c5 is covered above.
@pytest.mark.parametrize("chunk,N,eta", [(1, 40, 0.2), (7, 333, 0.1), (333, 333, 0.5), (5000, 333, 0.5)])
def test_chunk_edges(chunk, N, eta):
    w = Workload("chunks", B=1, H=2, N=N, d=64, hidden=128, inner="swiglu", loss="dot", chunk=chunk,
                 key_norm=False, renorm=True, per_token_eta=True, unit_columns=True, seed=43, eta=eta)
    dev_in, exact = device_inputs(w)
    _check_pairs(w, dev_in, exact, [(0, 0), (0, 1)], tag=f"chunk={chunk}")


def test_batch_specific_w0_and_continuation():
    """W0 with a batch axis, and a sequence split at a chunk boundary into two
    calls (the second seeded with W_out of the first) equals one call."""
    w = Workload("cont", B=2, H=2, N=256, d=64, hidden=128, inner="swiglu", loss="dot", chunk=64,
                 key_norm=False, renorm=True, per_token_eta=True, unit_columns=True, seed=44)
    dev_in, exact = device_inputs(w, shared_w0=False)
    _check_pairs(w, dev_in, exact, [(0, 1), (1, 0)], tag="bstride")
    tq, tk, tv, tW, tet = dev_in
    O_full, W_full, _ = run_gpu(w, dev_in)
    half = lambda t: t[:, :, :128].contiguous()
    rest = lambda t: t[:, :, 128:].contiguous()
    w_half = Workload(**{**w.__dict__, "N": 128})
    O1, W1, _ = run_gpu(w_half, (half(tq), half(tk), half(tv), tW, half(tet)))
    O2, W2, _ = run_gpu(w_half, (rest(tq), rest(tk), rest(tv), W1, rest(tet)))
    got = torch.cat([O1, O2], dim=2).float()
    assert (got - O_full.float()).abs().max().item() <= 1e-2 * O_full.float().abs().max().item()
    for a, b in zip(W2, W_full):
        assert (a - b).abs().max().item() <= 1e-4 * b.abs().max().item()


def test_deterministic_bitwise():
    w = Workload("det", B=2, H=3, N=1500, d=64, hidden=256, seed=45)
    dev_in, _ = device_inputs(w)
    O1, W1, _ = run_gpu(w, dev_in)
    O2, W2, _ = run_gpu(w, dev_in)
    assert torch.equal(O1, O2)
    for a, b in zip(W1, W2):
        assert torch.equal(a, b)


def test_check_finite_flag():
    from linear_complexity_attention_amd import ttt

    w = Workload("nan", B=1, H=2, N=100, d=64, hidden=64, seed=46)
    dev_in, _ = device_inputs(w)
    tq, tk, tv, tW, tet = dev_in
    layer = ttt.TTTLayer(1, 2, 100, 64, 64, dtype="bf16", flags=ttt.TTT_FLAG_CHECK_FINITE)
    layer.forward(tq, tk, tv, tW)            # clean inputs pass
    tv2 = tv.clone()
    tv2[0, 1, 17, 3] = float("nan")
    with pytest.raises(ttt.TTTError) as ei:
        layer.forward(tq, tk, tv2, tW)
    assert ei.value.status == ttt.TTT_ERR_NONFINITE


def test_generic_and_fast_paths_agree():
    w = WORKLOADS["c2_vits_r4"]
    dev_in, _ = device_inputs(w, B=4)
    Oa, Wa, pa = run_gpu(w, dev_in)
    Ob, Wb, pb = run_gpu(w, dev_in, flags=GENERIC)
    assert pb == "generic"
    assert rel_err(Oa.float().cpu().numpy(), Ob.float().cpu().numpy()) <= 1e-2


def test_f16_range_of_the_mlp_fast_path():
    """The GELU-MLP MFMA kernels carry the loss gradient in f16: values past its
    range are reported as non-finite (TTT_FLAG_CHECK_FINITE), and the generic
    fp32 kernels (TTT_FLAG_FORCE_GENERIC) still compute the layer."""
    from linear_complexity_attention_amd import ttt

    w = Workload("range", B=1, H=2, N=100, d=64, hidden=64, seed=47)
    dev_in, exact = device_inputs(w)
    tq, tk, tv, tW, tet = dev_in
    big = (tv.float() * 1.0e5).to(torch.bfloat16)
    fast = ttt.TTTLayer(1, 2, 100, 64, 64, dtype="bf16", flags=ttt.TTT_FLAG_CHECK_FINITE)
    assert fast.path_name("mse", "mlp_gelu", 0) == "mfma"
    with pytest.raises(ttt.TTTError) as ei:
        fast.forward(tq, tk, big, tW)
    assert ei.value.status == ttt.TTT_ERR_NONFINITE
    slow = ttt.TTTLayer(1, 2, 100, 64, 64, dtype="bf16",
                        flags=ttt.TTT_FLAG_CHECK_FINITE | ttt.TTT_FLAG_FORCE_GENERIC)
    O = slow.forward(tq, tk, big, tW)
    torch.cuda.synchronize()
    O_ref, _ = orc.oracle_forward(exact["q"], exact["k"], big.double().cpu().numpy(), exact["W0"],
                                  eta_scale=1.0, loss="mse", inner="mlp_gelu", chunk=0, key_norm=True, eps=1e-5)
    assert rel_err(O.float().cpu().numpy(), O_ref) <= TOL["bf16"]
