"""GPU parity of the update variants (ttt_forward_ex options) against the
float64 oracle, through the C ABI, on every pair: several epochs per batch,
only some matrices updated (first layer only), sequential mini-batches read at
the end (write-then-query), read-only chunks, heavy-ball momentum and Muon.
Same bar as the plain layer: max|err| / max|ref| <= 1e-2 (bf16 tensors) or
1e-4 (fp32) on O and on dW = W_out - W0 of every matrix."""
import numpy as np
import pytest

from synth_inputs import Workload
from tests.gpu_common import TOL, device_inputs, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _check(w, opts, okw, *, path=None, flags=0):
    from linear_complexity_attention_amd import ttt

    options = ttt.make_options(**opts)
    dev_in, exact = device_inputs(w)
    O, W_out, got_path = run_gpu(w, dev_in, options=options, flags=flags)
    O_ref, W_ref = run_oracle(w, exact, okw=okw)
    tol = TOL[w.dtype]
    tag = f"{w.name} {opts} path={got_path}"
    e = rel_err(O.float().cpu().numpy(), O_ref)
    assert e <= tol, f"{tag}: O rel err {e:.3e}"
    W0 = [m[None] if m.ndim == 3 else m for m in exact["W0"]]
    mask = okw.get("update_mask")
    for i, (g, r, w0) in enumerate(zip(W_out, W_ref, W0)):
        g = g.cpu().numpy()
        if mask is not None and not mask[i]:
            np.testing.assert_array_equal(g, np.broadcast_to(w0, g.shape).astype(np.float32),
                                          err_msg=f"{tag}: matrix {i} outside the mask changed")
            continue
        e = rel_err(g - w0, r - w0)
        assert e <= tol, f"{tag}: dW{i} rel err {e:.3e}"
    if path is not None:
        assert got_path == path, tag
    return got_path


def _mlp(dtype="bf16", **kw):
    base = dict(B=2, H=3, N=333, d=64, hidden=128, dtype=dtype, seed=501)
    base.update(kw)
    return Workload("mlp", **base)


def _swiglu(dtype="bf16", **kw):
    base = dict(B=1, H=3, N=600, d=64, hidden=128, dtype=dtype, inner="swiglu", loss="dot", chunk=128,
                key_norm=False, renorm=True, per_token_eta=True, key_shift=0.0, unit_columns=True, seed=502,
                eta=0.5)
    base.update(kw)
    return Workload("swiglu", **base)


# several epochs [ViT3 guideline 2]
def test_epochs_c3_full_size():
    """c3 (B=8, H=12, N=6084, d=64, h=256) with three epochs, in the
    benchmark's configuration: the fp32 matrix-core step at full size, every
    pair."""
    from synth_inputs import WORKLOADS

    _check(WORKLOADS["c3_hires_r4"], dict(epochs=3), dict(epochs=3), path="mfma_f32_grad+mfma_query")



@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_epochs_full_batch(dtype):
    _check(_mlp(dtype), dict(epochs=3), dict(epochs=3))


def test_epochs_chunked_swiglu():
    _check(_swiglu(), dict(epochs=2), dict(epochs=2), path="mfma_swiglu")


# only the first layer adjusted [TvS]: on the MFMA path (stream-K update) and
# with the re-norm, the second matrix stays W0 bit for bit
@pytest.mark.parametrize("key_norm,renorm,loss", [(True, False, "mse"), (False, True, "dot")])
def test_first_layer_only_mfma(key_norm, renorm, loss):
    w = _mlp(key_norm=key_norm, renorm=renorm, loss=loss, unit_columns=renorm, per_token_eta=loss == "dot",
             eta=1.0 if loss == "mse" else 0.2)
    _check(w, dict(update_mask=1), dict(update_mask=[True, False]), path="mfma")


def test_mask_chunked_swiglu():
    _check(_swiglu(), dict(update_mask=0b101), dict(update_mask=[True, False, True]), path="mfma_swiglu")


# sequential mini-batches that all write before the queries read [ViT3
# guideline 2, LaCT sets]: with key norm (generic gradient) and without (LaCT
# kernels)
@pytest.mark.parametrize("key_norm", [False, True])
def test_write_then_query_swiglu(key_norm):
    w = _swiglu(key_norm=key_norm)
    _check(w, dict(order="write_then_query"), dict(order="write_then_query"))


def test_write_then_query_mlp_f32():
    w = _mlp("f32", chunk=100, key_norm=True)
    _check(w, dict(order="write_then_query", epochs=2), dict(order="write_then_query", epochs=2))


# read-only chunks [LaCT video: clean chunks write, noisy chunks read]
def test_read_only_chunks():
    mask = [1, 0, 1, 1, 0]
    _check(_swiglu(), dict(chunk_update=mask), dict(chunk_update=mask), path="mfma_swiglu")


def test_read_only_last_chunk_and_all_read_only():
    _check(_swiglu(), dict(chunk_update=[1, 1, 0, 1, 0]), dict(chunk_update=[1, 1, 0, 1, 0]))
    _check(_swiglu(N=256), dict(chunk_update=[0, 0]), dict(chunk_update=[0, 0]))


# momentum [LaCT]: chunked (LaCT kernels), full batch on the MFMA path, the
# generic path, and with a mask
@pytest.mark.parametrize("case", ["swiglu", "mlp_mfma", "mlp_generic_f32", "mlp_masked_epochs"])
def test_momentum(case):
    if case == "swiglu":
        _check(_swiglu(), dict(rule="momentum", beta=0.9), dict(rule="momentum", beta=0.9), path="mfma_swiglu")
    elif case == "mlp_mfma":
        _check(_mlp(), dict(rule="momentum", beta=0.9), dict(rule="momentum", beta=0.9), path="mfma")
    elif case == "mlp_generic_f32":
        w = _mlp("f32", chunk=111, key_norm=False)
        _check(w, dict(rule="momentum", beta=0.5), dict(rule="momentum", beta=0.5))
    else:
        _check(_mlp(), dict(rule="momentum", beta=0.5, epochs=3, update_mask=2),
               dict(rule="momentum", beta=0.5, epochs=3, update_mask=[False, True]))


# Muon [LaCT]: Newton-Schulz on the momentum, then the re-norm
@pytest.mark.parametrize("case", ["swiglu", "swiglu_d128", "mlp_mfma", "linear_f32", "mlp_masked"])
def test_muon(case):
    if case == "swiglu":
        w, opts = _swiglu(), dict(rule="muon", beta=0.5, muon_scale=0.1)
    elif case == "swiglu_d128":
        w, opts = _swiglu(d=128, hidden=256, N=512, chunk=256), dict(rule="muon", beta=0.0, muon_scale=0.1,
                                                                      ns_steps=5)
    elif case == "mlp_mfma":
        w, opts = _mlp(renorm=True, unit_columns=True), dict(rule="muon", beta=0.0, muon_scale=0.05)
    elif case == "linear_f32":
        w = Workload("lin", B=2, H=2, N=300, d=32, hidden=32, dtype="f32", inner="linear", loss="dot", chunk=100,
                     key_norm=False, per_token_eta=True, seed=503)
        opts = dict(rule="muon", beta=0.9, muon_scale=0.2, ns_steps=3)
    else:
        w, opts = _mlp(), dict(rule="muon", beta=0.0, muon_scale=0.05, update_mask=2)
    okw = dict(opts)
    if "update_mask" in okw:
        okw["update_mask"] = [bool(okw["update_mask"] >> i & 1) for i in range(2)]
    _check(w, opts, okw)
