"""ttt_forward_noalloc (the entry point for callers that cannot allocate)
against ttt_forward on the same inputs: two calls in a row on one GPU, the
second with a smaller input, each through the C ABI, outputs and final weights
bit-identical to those of ttt_forward (the same kernels in the same order; only
the scratch memory differs).  An over-size request is rejected before anything
is enqueued."""
import pytest
import torch

from synth_inputs import Workload
from tests.gpu_common import device_inputs

pytestmark = pytest.mark.gpu


def _raw_call(layer, w, dev_in, noalloc):
    from linear_complexity_attention_amd import ttt

    tq, tk, tv, tW, tet = dev_in
    li, ii = ttt.LOSSES[w.loss], ttt.INNERS[w.inner]
    out = torch.empty_like(tq)
    # zero-filled: a ViT3 request writes each matrix only for the heads of its range
    W_out = [torch.zeros((w.B, w.H) + tuple(m.shape[-2:]), dtype=torch.float32, device=tq.device) for m in tW]
    wts = ttt.ttt_weights()
    for i, m in enumerate(tW):
        wts.w[i] = m.data_ptr()
    wts.batch_stride = 0
    e = ttt.ttt_eta(float(w.eta), tet.data_ptr() if tet is not None else None)
    wo = ttt.ttt_weights_out()
    for i, m in enumerate(W_out):
        wo.w[i] = m.data_ptr()
    stream = torch.cuda.current_stream(tq.device).cuda_stream
    if noalloc:
        rc = ttt.ttt_forward_noalloc(layer.handle, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), wts, e, li, ii,
                                     w.chunk, out.data_ptr(), wo, stream)
    else:
        nbytes = layer.workspace_bytes(w.loss, w.inner, w.chunk)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=tq.device)
        rc = ttt.ttt_forward(layer.handle, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), wts, e, li, ii, w.chunk,
                             out.data_ptr(), wo, ws.data_ptr(), nbytes, stream)
    assert rc == ttt.TTT_OK, ttt.ttt_last_error(layer.handle)
    torch.cuda.synchronize()
    return out, W_out


def test_noalloc_matches_forward_twice_second_smaller():
    from linear_complexity_attention_amd import ttt

    cases = [
        Workload("na_mlp", B=4, H=6, N=3000, d=64, hidden=256, seed=61),
        Workload("na_lact", B=1, H=4, N=1000, d=128, hidden=256, inner="swiglu", loss="dot", chunk=256,
                 key_norm=False, renorm=True, per_token_eta=True, key_shift=0.0, unit_columns=True, seed=62),
    ]
    sizes = []
    for w in cases:
        print(f"no-alloc case {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} h={w.hidden} chunk={w.chunk}", flush=True)
        dev_in, _ = device_inputs(w)
        layer = ttt.TTTLayer(w.B, w.H, w.N, w.d, w.hidden, dtype=w.dtype, key_norm=w.key_norm, renorm=w.renorm)
        need = layer.workspace_bytes(w.loss, w.inner, w.chunk)
        assert need <= ttt.TTT_NOALLOC_SCRATCH_BYTES
        sizes.append(w.B * w.H * w.N * w.d)
        O_ref, W_ref = _raw_call(layer, w, dev_in, noalloc=False)
        O, W = _raw_call(layer, w, dev_in, noalloc=True)
        assert torch.equal(O, O_ref), f"{w.name}: O differs from ttt_forward"
        for a, b in zip(W, W_ref):
            assert torch.equal(a, b), f"{w.name}: final weights differ from ttt_forward"
        assert torch.isfinite(O.float()).all()
    assert sizes[1] < sizes[0]


def test_vit3_block_serial_and_concurrent_ranges_agree():
    """The ViT3 block's two head ranges run one after another through the
    no-alloc entry point on a fresh handle (it creates no stream), then on
    the handle's second stream through ttt_forward (which creates it), then
    on that stream through the no-alloc entry point again: O and the final
    weights are bit-identical every time."""
    from linear_complexity_attention_amd import ttt

    w = Workload("na_vit3", B=4, H=6, N=400, d=64, hidden=64, inner="vit3", loss="dot", key_norm=True,
                 eta=1.0 / 400, grid=(20, 20), conv_k=3, seed=63)
    print(f"no-alloc case {w.name}: B={w.B} H={w.H} N={w.N} grid={w.grid}", flush=True)
    dev_in, _ = device_inputs(w)
    layer = ttt.TTTLayer(w.B, w.H, w.N, w.d, w.hidden, dtype=w.dtype, key_norm=w.key_norm, renorm=w.renorm,
                         grid=w.grid, conv_k=w.conv_k)
    runs = [_raw_call(layer, w, dev_in, noalloc=True), _raw_call(layer, w, dev_in, noalloc=False),
            _raw_call(layer, w, dev_in, noalloc=True)]
    O_ref, W_ref = runs[0]
    assert torch.isfinite(O_ref.float()).all()
    for O, W in runs[1:]:
        assert torch.equal(O, O_ref)
        for a, b in zip(W, W_ref):
            assert torch.equal(a, b)


def test_noalloc_fused_gradient_and_readout():
    """A request on the fused path (every pair held whole by one gradient
    workgroup, which also reads it out) through both entry points: O and the
    final weights bit-identical."""
    from linear_complexity_attention_amd import ttt

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = Workload("na_fused", B=cus // 8, H=8, N=196, d=64, hidden=256, seed=64)
    print(f"no-alloc case {w.name}: B={w.B} H={w.H} N={w.N} h={w.hidden}", flush=True)
    dev_in, _ = device_inputs(w)
    layer = ttt.TTTLayer(w.B, w.H, w.N, w.d, w.hidden, dtype=w.dtype, key_norm=w.key_norm, renorm=w.renorm)
    assert layer.path_name(w.loss, w.inner, w.chunk) == "mfma_fused"
    O_ref, W_ref = _raw_call(layer, w, dev_in, noalloc=False)
    O, W = _raw_call(layer, w, dev_in, noalloc=True)
    assert torch.isfinite(O_ref.float()).all()
    assert torch.equal(O, O_ref)
    for a, b in zip(W, W_ref):
        assert torch.equal(a, b)


def test_noalloc_rejects_oversize_request():
    from linear_complexity_attention_amd import ttt

    layer = ttt.TTTLayer(64, 16, 8192, 64, 512, key_norm=True)
    need = layer.workspace_bytes("mse", "mlp_gelu", 0)
    assert need > ttt.TTT_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20   # never dereferenced: the size check comes first
    W = ttt.ttt_weights()
    W.w[0] = W.w[1] = fake
    rc = ttt.ttt_forward_noalloc(layer.handle, fake, fake, fake, W, ttt.ttt_eta(1.0, None), ttt.TTT_LOSS_MSE,
                                 ttt.TTT_INNER_MLP_GELU, 0, fake, None, None)
    assert rc == ttt.TTT_ERR_WORKSPACE
    assert "ttt_forward_noalloc" in ttt.ttt_last_error(layer.handle)
