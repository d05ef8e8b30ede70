"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names what it pins and why a plausible mistake in the oracle (a
dropped term, a wrong sign, index or constant, a transposed operand) fails it:
hand-worked cases (tests/golden), finite differences, an independent
torch.autograd derivation built on library routines (instance_norm, gelu,
silu, mse_loss), closed forms stated by the pages, and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle import ttt_oracle as orc
from synth_inputs import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_cases.json")


def _arr4(x):
    return np.asarray(x, dtype=np.float64)[None, None]


def _rand_case(rng, B=1, H=1, N=12, d=4, h=6, inner=orc.INNER_MLP, shift=0.5, wscale=None):
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) + shift
    v = rng.standard_normal((B, H, N, d))
    wscale = (1.0 / math.sqrt(d)) if wscale is None else wscale
    shapes = {orc.INNER_LINEAR: [(d, d)], orc.INNER_MLP: [(d, h), (h, d)],
              orc.INNER_SWIGLU: [(d, h), (h, d), (d, h)]}[inner]
    W0 = [rng.standard_normal((H,) + s) * wscale for s in shapes]
    return q, k, v, W0


# --------------------------------------------------------------------------
# Hand-worked golden cases
# --------------------------------------------------------------------------
def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_worked(case):
    W0 = [np.asarray(w, dtype=np.float64)[None] for w in case["W0"]]
    O, Wf = orc.oracle_forward(_arr4(case["q"]), _arr4(case["k"]), _arr4(case["v"]), W0,
                               eta_scale=case["eta"], loss=case["loss"], inner=case["inner"],
                               chunk=case["chunk"], key_norm=case["key_norm"],
                               renorm=case["renorm"])
    np.testing.assert_allclose(O[0, 0], np.asarray(case["O"]), rtol=1e-12, atol=1e-12)
    for got, want in zip(Wf, case["W_final"]):
        np.testing.assert_allclose(got[0, 0], np.asarray(want), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Activations against independent library routines
# --------------------------------------------------------------------------
def test_gelu_is_z_times_normal_cdf():
    z = np.linspace(-8, 8, 2001)
    np.testing.assert_allclose(orc.gelu(z), z * norm.cdf(z), rtol=1e-13, atol=1e-15)
    t = torch.tensor(z, dtype=torch.float64)
    np.testing.assert_allclose(orc.gelu(z), torch.nn.functional.gelu(t).numpy(), rtol=1e-13, atol=1e-15)


def test_activation_derivatives_by_finite_difference():
    z = np.linspace(-7, 7, 1401)
    e = 1e-6
    np.testing.assert_allclose(orc.gelu_prime(z), (orc.gelu(z + e) - orc.gelu(z - e)) / (2 * e),
                               rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(orc.silu_prime(z), (orc.silu(z + e) - orc.silu(z - e)) / (2 * e),
                               rtol=1e-7, atol=1e-9)
    t = torch.tensor(z, dtype=torch.float64)
    np.testing.assert_allclose(orc.silu(z), torch.nn.functional.silu(t).numpy(), rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# P1: hand backward == central finite differences of the loss
# --------------------------------------------------------------------------
@pytest.mark.parametrize("inner", [orc.INNER_LINEAR, orc.INNER_MLP, orc.INNER_SWIGLU])
@pytest.mark.parametrize("loss", [orc.LOSS_MSE, orc.LOSS_DOT])
def test_backward_matches_finite_differences(inner, loss):
    rng = np.random.default_rng(7)
    N, d, h = 9, 4, 6
    X = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    eta = 0.3 + rng.random(N)
    _, _, _, W0 = _rand_case(rng, N=N, d=d, h=h, inner=inner)
    W = [w[0] for w in W0]

    def L(Ws):
        Vh, _ = orc.inner_forward(inner, Ws, X)
        # loss definitions written from their names: mean squared error over
        # all N*d entries, negative dot product, each token weighted by eta_n
        if loss == orc.LOSS_MSE:
            return float(np.sum(eta[:, None] * (Vh - V) ** 2) / V.size)
        return float(-np.sum(eta[:, None] * Vh * V))

    Vh, cache = orc.inner_forward(inner, W, X)
    G = orc.loss_grad(loss, Vh, V, eta)
    dW = orc.inner_backward(inner, W, X, G, cache)
    step = 1e-6
    for i, w in enumerate(W):
        fd = np.zeros_like(w)
        for idx in np.ndindex(w.shape):
            wp = [x.copy() for x in W]
            wm = [x.copy() for x in W]
            wp[i][idx] += step
            wm[i][idx] -= step
            fd[idx] = (L(wp) - L(wm)) / (2 * step)
        np.testing.assert_allclose(dW[i], fd, rtol=1e-6, atol=1e-9)


# --------------------------------------------------------------------------
# P2: an independent derivation with torch.autograd in float64
# --------------------------------------------------------------------------
def _torch_layer(q, k, v, W0, eta_scale, eta_tok, loss, inner, chunk, key_norm, eps, renorm):
    """The layer written with library pieces: F.instance_norm for the key
    statistics, F.gelu / F.silu, F.mse_loss, and autograd for dL/dW."""
    F = torch.nn.functional
    q, k, v = (torch.tensor(a, dtype=torch.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    if key_norm:
        kk = k.reshape(B * H, N, d).transpose(1, 2)            # [BH, d, N]
        k = F.instance_norm(kk, eps=eps).transpose(1, 2).reshape(B, H, N, d)
    eta = torch.full((B, H, N), float(eta_scale), dtype=torch.float64)
    if eta_tok is not None:
        eta = eta * torch.tensor(eta_tok, dtype=torch.float64)

    def fwd(Ws, x):
        if inner == orc.INNER_LINEAR:
            return x @ Ws[0]
        if inner == orc.INNER_MLP:
            return F.gelu(x @ Ws[0]) @ Ws[1]
        return (F.silu(x @ Ws[0]) * (x @ Ws[2])) @ Ws[1]

    O = torch.zeros_like(q)
    for b in range(B):
        for h in range(H):
            ref = [torch.tensor(np.asarray(w)[h], dtype=torch.float64) for w in W0]
            Ws = [w.clone() for w in ref]
            bounds = [(0, N)] if chunk == 0 else [(s, min(s + chunk, N)) for s in range(0, N, chunk)]
            for (s, e) in bounds:
                if chunk:
                    O[b, h, s:e] = fwd(Ws, q[b, h, s:e])
                Wg = [w.clone().requires_grad_(True) for w in Ws]
                Vh = fwd(Wg, k[b, h, s:e])
                et = eta[b, h, s:e]
                if loss == orc.LOSS_MSE:
                    if eta_tok is None:
                        Lv = float(eta_scale) * F.mse_loss(Vh, v[b, h, s:e], reduction="mean")
                    else:
                        Lv = (et[:, None] * (Vh - v[b, h, s:e]) ** 2).mean()
                else:
                    Lv = -(et[:, None] * Vh * v[b, h, s:e]).sum()
                grads = torch.autograd.grad(Lv, Wg)
                Ws = [w - g for w, g in zip(Ws, grads)]
                if renorm:
                    Ws = [w * (r.norm(dim=0, keepdim=True) / w.norm(dim=0, keepdim=True).clamp_min(1e-12))
                          for w, r in zip(Ws, ref)]
            if not chunk:
                O[b, h] = fwd(Ws, q[b, h])
    return O.detach().numpy()


@pytest.mark.parametrize("inner,loss,chunk,key_norm,renorm,pertok", [
    (orc.INNER_MLP, orc.LOSS_MSE, 0, True, False, False),
    (orc.INNER_MLP, orc.LOSS_DOT, 0, True, False, False),
    (orc.INNER_SWIGLU, orc.LOSS_DOT, 0, True, True, True),
    (orc.INNER_SWIGLU, orc.LOSS_MSE, 0, False, False, True),
    (orc.INNER_LINEAR, orc.LOSS_MSE, 0, True, False, False),
    (orc.INNER_SWIGLU, orc.LOSS_DOT, 5, False, True, True),
    (orc.INNER_MLP, orc.LOSS_MSE, 4, False, False, False),
    (orc.INNER_MLP, orc.LOSS_DOT, 7, False, True, True),
])
def test_oracle_matches_autograd_layer(inner, loss, chunk, key_norm, renorm, pertok):
    rng = np.random.default_rng(11)
    q, k, v, W0 = _rand_case(rng, B=2, H=2, N=17, d=5, h=7, inner=inner)
    eta_tok = (0.1 + rng.random((2, 2, 17))) if pertok else None
    args = dict(eta_scale=0.8, eta_tok=eta_tok, loss=loss, inner=inner, chunk=chunk,
                key_norm=key_norm, renorm=renorm)
    O, _ = orc.oracle_forward(q, k, v, W0, eps=1e-5, **args)
    O_ref = _torch_layer(q, k, v, W0, args["eta_scale"], eta_tok, loss, inner, chunk, key_norm, 1e-5, renorm)
    np.testing.assert_allclose(O, O_ref, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# Closed forms and special cases stated by the pages
# --------------------------------------------------------------------------
@pytest.mark.parametrize("inner", [orc.INNER_MLP, orc.INNER_SWIGLU, orc.INNER_LINEAR])
def test_eta_zero_reads_initial_weights(inner):
    """P3: eta = 0 leaves W0 untouched, so O = F_W0(Q)."""
    rng = np.random.default_rng(3)
    q, k, v, W0 = _rand_case(rng, B=2, H=3, N=10, d=4, h=6, inner=inner)
    O, Wf = orc.oracle_forward(q, k, v, W0, eta_scale=0.0, inner=inner)
    Wb = [np.broadcast_to(w[None], (2,) + w.shape) for w in W0]
    np.testing.assert_allclose(O, orc.oracle_readout(q, Wb, inner), rtol=0, atol=0)
    for a, b in zip(Wf, Wb):
        np.testing.assert_array_equal(a, b)


def test_linear_mse_closed_form():
    """P4: linear inner model, MSE: W* = W0 - eta*2/(N d) * K^T (K W0 - V), O = Q W*."""
    rng = np.random.default_rng(4)
    N, d, eta = 13, 5, 0.7
    q, k, v, W0 = _rand_case(rng, N=N, d=d, inner=orc.INNER_LINEAR)
    O, Wf = orc.oracle_forward(q, k, v, W0, eta_scale=eta, loss=orc.LOSS_MSE,
                               inner=orc.INNER_LINEAR, key_norm=False)
    K, V, Q, W = k[0, 0], v[0, 0], q[0, 0], W0[0][0]
    Ws = W - eta * 2.0 / (N * d) * K.T @ (K @ W - V)
    np.testing.assert_allclose(Wf[0][0, 0], Ws, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O[0, 0], Q @ Ws, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("key_norm", [False, True])
def test_linear_dot_zero_init_is_linear_attention(key_norm):
    """P5: linear inner, W0 = 0, dot loss: O = eta * Q (K_hat^T V) -- the
    linear-attention special case (ViT3 page, section 01 / glossary)."""
    rng = np.random.default_rng(5)
    q, k, v, W0 = _rand_case(rng, B=2, H=2, N=11, d=3, inner=orc.INNER_LINEAR)
    W0 = [np.zeros_like(W0[0])]
    eta = 1.3
    O, _ = orc.oracle_forward(q, k, v, W0, eta_scale=eta, loss=orc.LOSS_DOT,
                              inner=orc.INNER_LINEAR, key_norm=key_norm)
    for b in range(2):
        for h in range(2):
            K = k[b, h]
            if key_norm:
                t = torch.tensor(K.T[None], dtype=torch.float64)
                K = torch.nn.functional.instance_norm(t, eps=1e-5)[0].numpy().T
            np.testing.assert_allclose(O[b, h], eta * q[b, h] @ (K.T @ v[b, h]), rtol=1e-12, atol=1e-12)


def test_chunked_linear_dot_is_block_causal_linear_attention():
    """P6: chunked, linear, dot, W0 = 0, no re-norm:
    O_c = Q_c * sum_{c' < c} K_c'^T diag(eta_c') V_c' (read-then-update)."""
    rng = np.random.default_rng(6)
    N, d, C = 23, 4, 5
    q, k, v, W0 = _rand_case(rng, N=N, d=d, inner=orc.INNER_LINEAR)
    W0 = [np.zeros_like(W0[0])]
    et = 0.05 + rng.random((1, 1, N))
    O, Wf = orc.oracle_forward(q, k, v, W0, eta_tok=et, loss=orc.LOSS_DOT, inner=orc.INNER_LINEAR,
                               chunk=C, key_norm=False)
    Q, K, V, e = q[0, 0], k[0, 0], v[0, 0], et[0, 0]
    for s in range(0, N, C):
        S = (K[:s] * e[:s, None]).T @ V[:s]
        np.testing.assert_allclose(O[0, 0, s:s + C], Q[s:s + C] @ S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Wf[0][0, 0], (K * e[:, None]).T @ V, rtol=1e-12, atol=1e-12)


def test_one_chunk_longer_than_sequence_reads_w0():
    """P7: causal mode with chunk >= N: every query reads W0."""
    rng = np.random.default_rng(8)
    q, k, v, W0 = _rand_case(rng, B=1, H=2, N=9, d=4, h=5, inner=orc.INNER_SWIGLU)
    O, _ = orc.oracle_forward(q, k, v, W0, loss=orc.LOSS_DOT, inner=orc.INNER_SWIGLU, chunk=64,
                              key_norm=False, renorm=True)
    Wb = [np.broadcast_to(w[None], (1,) + w.shape) for w in W0]
    np.testing.assert_allclose(O, orc.oracle_readout(q, Wb, orc.INNER_SWIGLU), rtol=0, atol=0)


def test_constant_per_token_eta_equals_scalar_eta():
    """P8: eta_tok == c everywhere is the same as eta_scale = c."""
    rng = np.random.default_rng(9)
    q, k, v, W0 = _rand_case(rng, B=1, H=2, N=12, d=4, h=6, inner=orc.INNER_SWIGLU)
    a, _ = orc.oracle_forward(q, k, v, W0, eta_tok=np.full((1, 2, 12), 0.37), loss=orc.LOSS_DOT,
                              inner=orc.INNER_SWIGLU, chunk=5, key_norm=False, renorm=True)
    b, _ = orc.oracle_forward(q, k, v, W0, eta_scale=0.37, loss=orc.LOSS_DOT,
                              inner=orc.INNER_SWIGLU, chunk=5, key_norm=False, renorm=True)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_key_norm_cancels_constant_shift_and_scale():
    """P9: the key statistics are per channel over tokens, so adding any
    constant vector to every key leaves O unchanged, and scaling keys by
    alpha > 0 changes O only through eps.  A norm over the wrong axis fails."""
    rng = np.random.default_rng(10)
    q, k, v, W0 = _rand_case(rng, B=1, H=2, N=30, d=6, h=8)
    base, _ = orc.oracle_forward(q, k, v, W0)
    shift = rng.standard_normal((1, 1, 1, 6)) * 3.0
    shifted, _ = orc.oracle_forward(q, k + shift, v, W0)
    np.testing.assert_allclose(shifted, base, rtol=1e-10, atol=1e-11)
    scaled, _ = orc.oracle_forward(q, 7.0 * k, v, W0, eps=0.0)
    plain, _ = orc.oracle_forward(q, k, v, W0, eps=0.0)
    np.testing.assert_allclose(scaled, plain, rtol=1e-10, atol=1e-11)
    # without the norm the shift does change the output
    a, _ = orc.oracle_forward(q, k, v, W0, key_norm=False)
    c, _ = orc.oracle_forward(q, k + shift, v, W0, key_norm=False)
    assert np.max(np.abs(a - c)) > 1e-3


def test_key_norm_matches_library_instance_norm():
    rng = np.random.default_rng(12)
    K = rng.standard_normal((40, 7)) * 2.0 + 0.5
    t = torch.tensor(K.T[None], dtype=torch.float64)
    np.testing.assert_allclose(orc.key_instnorm(K, 1e-5),
                               torch.nn.functional.instance_norm(t, eps=1e-5)[0].numpy().T,
                               rtol=1e-12, atol=1e-12)


def test_renorm_restores_w0_column_norms():
    """P10: after every update each output column has W0's column norm."""
    w = WORKLOADS["c5_lact_swiglu"]
    q, k, v, W0, et = make_inputs(w, H=1, N=96)
    W0 = [x.astype(np.float64) for x in W0]
    shrunk = [x[:, :16, :24] if i != 1 else x[:, :24, :16] for i, x in enumerate(W0)]
    shrunk = [x / np.sqrt((x ** 2).sum(axis=-2, keepdims=True)) for x in shrunk]
    _, Wf = orc.oracle_forward(q[..., :16], k[..., :16], v[..., :16], shrunk, eta_tok=et,
                               loss=orc.LOSS_DOT, inner=orc.INNER_SWIGLU, chunk=32,
                               key_norm=False, renorm=True)
    for m in Wf:
        np.testing.assert_allclose(np.sqrt((m ** 2).sum(axis=-2)), 1.0, rtol=1e-12)


def test_chunk_boundary_continuation():
    """P11: splitting at a chunk boundary into two calls (the second seeded
    with the first call's final weights) equals one call."""
    rng = np.random.default_rng(13)
    q, k, v, W0 = _rand_case(rng, B=2, H=1, N=20, d=4, h=6, inner=orc.INNER_SWIGLU)
    et = 0.1 + rng.random((2, 1, 20))
    kw = dict(loss=orc.LOSS_DOT, inner=orc.INNER_SWIGLU, chunk=5, key_norm=False, renorm=True)
    # continuing needs the re-norm targets of the original W0: unit-norm W0 makes them 1
    W0u = [w / np.sqrt((w ** 2).sum(axis=-2, keepdims=True)) for w in W0]
    O, Wf = orc.oracle_forward(q, k, v, W0u, eta_tok=et, **kw)
    O1, W1 = orc.oracle_forward(q[:, :, :10], k[:, :, :10], v[:, :, :10], W0u, eta_tok=et[:, :, :10], **kw)
    O2, W2 = orc.oracle_forward(q[:, :, 10:], k[:, :, 10:], v[:, :, 10:], W1, eta_tok=et[:, :, 10:], **kw)
    np.testing.assert_allclose(np.concatenate([O1, O2], axis=2), O, rtol=1e-12, atol=1e-13)
    for a, b in zip(W2, Wf):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_full_batch_is_permutation_equivariant_and_pairs_independent():
    """P12: full batch treats tokens as a set; each (b, h) is independent."""
    rng = np.random.default_rng(14)
    q, k, v, W0 = _rand_case(rng, B=2, H=3, N=15, d=4, h=6)
    O, _ = orc.oracle_forward(q, k, v, W0)
    p = rng.permutation(15)
    Op, _ = orc.oracle_forward(q[:, :, p], k[:, :, p], v[:, :, p], W0)
    np.testing.assert_allclose(Op, O[:, :, p], rtol=1e-12, atol=1e-13)
    O11, _ = orc.oracle_forward(q[1:2, 2:3], k[1:2, 2:3], v[1:2, 2:3], [w[2:3] for w in W0])
    np.testing.assert_allclose(O11[0, 0], O[1, 2], rtol=1e-13, atol=1e-14)


def test_eta_equivalent_to_scaling_k_and_v():
    """P13: linear inner + MSE (no key norm): eta*s^2 with (K, V) equals eta
    with (sK, sV) -- the equivalence stated in the ViT3 page, guideline 3."""
    rng = np.random.default_rng(15)
    q, k, v, W0 = _rand_case(rng, B=1, H=2, N=14, d=5, inner=orc.INNER_LINEAR)
    s, eta = 1.7, 0.45
    a, _ = orc.oracle_forward(q, k, v, W0, eta_scale=eta * s * s, inner=orc.INNER_LINEAR, key_norm=False)
    b, _ = orc.oracle_forward(q, s * k, s * v, W0, eta_scale=eta, inner=orc.INNER_LINEAR, key_norm=False)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_causal_mode_never_reads_future_tokens():
    """Read-then-update: perturbing keys/values/queries at or after a chunk
    boundary leaves every earlier output unchanged (LaCT page, order of
    operations)."""
    rng = np.random.default_rng(16)
    q, k, v, W0 = _rand_case(rng, B=1, H=1, N=24, d=4, h=6, inner=orc.INNER_SWIGLU)
    kw = dict(loss=orc.LOSS_DOT, inner=orc.INNER_SWIGLU, chunk=6, key_norm=False)
    O, _ = orc.oracle_forward(q, k, v, W0, **kw)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[:, :, 12:] += 5.0
    v2[:, :, 12:] -= 3.0
    q2[:, :, 12:] *= 2.0
    O2, _ = orc.oracle_forward(q2, k2, v2, W0, **kw)
    np.testing.assert_array_equal(O2[:, :, :12], O[:, :, :12])
    assert np.max(np.abs(O2[:, :, 12:] - O[:, :, 12:])) > 1e-3


def test_causal_mode_rejects_key_norm():
    rng = np.random.default_rng(17)
    q, k, v, W0 = _rand_case(rng)
    with pytest.raises(ValueError):
        orc.oracle_forward(q, k, v, W0, chunk=4, key_norm=True)


def test_synthetic_inputs_follow_recipe():
    w = WORKLOADS["c1_tiny_fp32"]
    q, k, v, W0, et = make_inputs(w)
    assert q.shape == (1, 1, 256, 32) and q.dtype == np.float32
    assert abs(float(k.mean()) - 0.5) < 0.05 and abs(float(q.mean())) < 0.05
    assert abs(float(W0[0].std()) * math.sqrt(32) - 1.0) < 0.1
    assert et is None
    q2, *_ = make_inputs(w)
    np.testing.assert_array_equal(q, q2)
    w5 = WORKLOADS["c5_lact_swiglu"]
    q, k, v, W0, et = make_inputs(w5, N=64)
    for m in W0:
        np.testing.assert_allclose(np.sqrt((m.astype(np.float64) ** 2).sum(axis=-2)), 1.0, rtol=1e-5)
    assert et.shape == (1, 4, 64) and float(et.min()) > 0.0
