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
def _torch_layer(q, k, v, W0, eta_scale, eta_tok, loss, inner, chunk, key_norm, eps, renorm, *, epochs=1,
                 update_mask=None, write_then_query=False, chunk_update=None, beta=None):
    """The layer written with library pieces: F.instance_norm for the key
    statistics, F.gelu / F.silu, F.mse_loss, and autograd for dL/dW.  Options:
    several epochs per batch, a per-matrix update mask, chunks that all write
    before the queries read, read-only chunks, heavy-ball momentum (beta)."""
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
            mom = [torch.zeros_like(w) for w in ref]
            upd = [True] * len(ref) if update_mask is None else list(update_mask)
            bounds = [(0, N)] if chunk == 0 else [(s, min(s + chunk, N)) for s in range(0, N, chunk)]
            causal = chunk > 0 and not write_then_query
            for ci, (s, e) in enumerate(bounds):
                if causal:
                    O[b, h, s:e] = fwd(Ws, q[b, h, s:e])
                if chunk_update is not None and not chunk_update[ci]:
                    continue
                for _ in range(epochs):
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
                    new = []
                    for i, (w, g) in enumerate(zip(Ws, grads)):
                        if not upd[i]:
                            new.append(w)
                            continue
                        if beta is not None:
                            mom[i] = beta * mom[i] + g
                            g = mom[i]
                        w = w - g
                        if renorm:
                            w = w * (ref[i].norm(dim=0, keepdim=True) / w.norm(dim=0, keepdim=True).clamp_min(1e-12))
                        new.append(w)
                    Ws = new
            if not causal:
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


# the update variants against the same independent derivation: epochs,
# first-layer-only, sequential mini-batches read at the end, read-only chunks,
# heavy-ball momentum (with re-norm where the pages pair it with the rule)
@pytest.mark.parametrize("inner,loss,chunk,opts", [
    (orc.INNER_MLP, orc.LOSS_MSE, 0, dict(epochs=3)),
    (orc.INNER_SWIGLU, orc.LOSS_DOT, 0, dict(epochs=2, renorm=True)),
    (orc.INNER_MLP, orc.LOSS_MSE, 0, dict(update_mask=[True, False])),
    (orc.INNER_SWIGLU, orc.LOSS_DOT, 5, dict(update_mask=[True, False, True], renorm=True)),
    (orc.INNER_MLP, orc.LOSS_MSE, 4, dict(write_then_query=True)),
    (orc.INNER_SWIGLU, orc.LOSS_DOT, 5, dict(write_then_query=True, key_norm=True, epochs=2)),
    (orc.INNER_SWIGLU, orc.LOSS_DOT, 4, dict(chunk_update=[1, 0, 0, 1, 1], renorm=True)),
    (orc.INNER_MLP, orc.LOSS_DOT, 6, dict(chunk_update=[0, 1, 0], write_then_query=True)),
    (orc.INNER_SWIGLU, orc.LOSS_DOT, 5, dict(beta=0.9, renorm=True)),
    (orc.INNER_MLP, orc.LOSS_MSE, 0, dict(beta=0.5, epochs=3, update_mask=[False, True])),
])
def test_update_variants_match_autograd_layer(inner, loss, chunk, opts):
    rng = np.random.default_rng(12)
    q, k, v, W0 = _rand_case(rng, B=2, H=2, N=17, d=5, h=7, inner=inner)
    eta_tok = 0.1 + rng.random((2, 2, 17))
    opts = dict(opts)
    key_norm = opts.pop("key_norm", False)
    renorm = opts.pop("renorm", False)
    beta = opts.pop("beta", None)
    O, _ = orc.oracle_forward(q, k, v, W0, eta_scale=0.8, eta_tok=eta_tok, loss=loss, inner=inner, chunk=chunk,
                              key_norm=key_norm, renorm=renorm,
                              rule=orc.RULE_GD if beta is None else orc.RULE_MOMENTUM, beta=beta or 0.0,
                              order=orc.ORDER_WRITE_THEN_QUERY if opts.get("write_then_query") else orc.ORDER_CAUSAL,
                              epochs=opts.get("epochs", 1), update_mask=opts.get("update_mask"),
                              chunk_update=opts.get("chunk_update"))
    O_ref = _torch_layer(q, k, v, W0, 0.8, eta_tok, loss, inner, chunk, key_norm, 1e-5, renorm, beta=beta, **opts)
    np.testing.assert_allclose(O, O_ref, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# Newton-Schulz orthogonalisation (Muon) and the update rules in closed form
# --------------------------------------------------------------------------
def _ns_by_svd(M, steps):
    """What the published iteration does, through the SVD: every singular value
    s of M / ||M||_F goes through p(s) = a s + b s^3 + c s^5 `steps` times; the
    singular vectors stay."""
    a, b, c = 3.4445, -4.7750, 2.0315
    U, S, Vt = np.linalg.svd(M, full_matrices=False)
    s = S / (np.linalg.norm(M) + 1e-7)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


@pytest.mark.parametrize("shape", [(5, 8), (8, 5), (6, 6), (16, 48)])
@pytest.mark.parametrize("steps", [1, 5])
def test_newton_schulz_acts_on_singular_values(shape, steps):
    M = np.random.default_rng(21).standard_normal(shape)
    np.testing.assert_allclose(orc.newton_schulz(M, steps), _ns_by_svd(M, steps), rtol=1e-9, atol=1e-11)


def test_newton_schulz_five_steps_nearly_orthogonal():
    """Muon's five steps bring every singular value of a well-conditioned
    matrix into roughly [0.7, 1.2] (the quintic is tuned for fast, not exact,
    convergence)."""
    M = np.random.default_rng(22).standard_normal((32, 64))
    s = np.linalg.svd(orc.newton_schulz(M, 5), compute_uv=False)
    assert s.min() > 0.6 and s.max() < 1.25, s


def _lin_dot_case(rng, N=24, d=4):
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    eta_tok = 0.2 + rng.random((1, 1, N))
    return q, k, v, [np.zeros((1, d, d))], eta_tok


def test_momentum_linear_dot_closed_form():
    """Linear inner model, dot loss, W0 = 0: the chunk gradient g_j =
    -K_j^T diag(eta_j) V_j does not depend on W, so heavy-ball momentum gives
    W_c = sum_{j<c} (1 - beta^(c-j)) / (1 - beta) K_j^T diag(eta_j) V_j and
    O_c = Q_c W_c (block-causal linear attention with geometric weights)."""
    rng = np.random.default_rng(23)
    q, k, v, W0, et = _lin_dot_case(rng)
    C, beta = 6, 0.7
    O, _ = orc.oracle_forward(q, k, v, W0, eta_tok=et, loss=orc.LOSS_DOT, inner=orc.INNER_LINEAR, chunk=C,
                              key_norm=False, rule=orc.RULE_MOMENTUM, beta=beta)
    Q, K, V, E = q[0, 0], k[0, 0], v[0, 0], et[0, 0]
    for c in range(4):
        W = np.zeros((4, 4))
        for j in range(c):
            sl = slice(j * C, (j + 1) * C)
            W += (1 - beta ** (c - j)) / (1 - beta) * K[sl].T @ (E[sl, None] * V[sl])
        np.testing.assert_allclose(O[0, 0, c * C:(c + 1) * C], Q[c * C:(c + 1) * C] @ W, rtol=1e-11, atol=1e-12)


def test_muon_linear_dot_closed_form():
    """Linear inner model, dot loss, W0 = 0, Muon without momentum: each chunk
    adds s NS(K_j^T diag(eta_j) V_j) (NS is odd), with NS through the SVD."""
    rng = np.random.default_rng(24)
    q, k, v, W0, et = _lin_dot_case(rng, N=30, d=5)
    C, scale = 10, 0.3
    O, Wf = orc.oracle_forward(q, k, v, W0, eta_tok=et, loss=orc.LOSS_DOT, inner=orc.INNER_LINEAR, chunk=C,
                               key_norm=False, rule=orc.RULE_MUON, beta=0.0, muon_scale=scale, ns_steps=5)
    Q, K, V, E = q[0, 0], k[0, 0], v[0, 0], et[0, 0]
    W = np.zeros((5, 5))
    for c in range(3):
        sl = slice(c * C, (c + 1) * C)
        np.testing.assert_allclose(O[0, 0, sl], Q[sl] @ W, rtol=1e-9, atol=1e-11)
        W = W + scale * _ns_by_svd(K[sl].T @ (E[sl, None] * V[sl]), 5)
    np.testing.assert_allclose(Wf[0][0, 0], W, rtol=1e-9, atol=1e-11)


def test_epochs_linear_mse_closed_form():
    """E epochs of full-batch GD on the linear model with MSE:
    W_E = (I - a S)^E W0 + sum_{j<E} (I - a S)^j a K^T V, S = K^T K,
    a = eta 2 / (N d) (key norm off)."""
    rng = np.random.default_rng(25)
    N, d, E, eta = 20, 4, 4, 3.0
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    W0 = [rng.standard_normal((1, d, d)) * 0.5]
    _, Wf = orc.oracle_forward(q, k, v, W0, eta_scale=eta, loss=orc.LOSS_MSE, inner=orc.INNER_LINEAR, chunk=0,
                               key_norm=False, epochs=E)
    K, V = k[0, 0], v[0, 0]
    a = eta * 2.0 / (N * d)
    T = np.eye(d) - a * K.T @ K
    want = np.linalg.matrix_power(T, E) @ W0[0][0]
    want += sum(np.linalg.matrix_power(T, j) @ (a * K.T @ V) for j in range(E))
    np.testing.assert_allclose(Wf[0][0, 0], want, rtol=1e-11, atol=1e-12)


def test_first_layer_only_keeps_second_layer():
    """Only the first layer adjusted [TvS]: W2 stays W0's, W1 takes the same
    step as in the full update (both gradients are taken at W0)."""
    rng = np.random.default_rng(26)
    q, k, v, W0 = _rand_case(rng, B=2, H=2, N=15, d=4, h=6)
    O, Wf = orc.oracle_forward(q, k, v, W0, update_mask=[True, False])
    _, Wfull = orc.oracle_forward(q, k, v, W0)
    np.testing.assert_array_equal(Wf[1], np.broadcast_to(W0[1][None], Wf[1].shape))
    np.testing.assert_allclose(Wf[0], Wfull[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(O, orc.oracle_readout(q, Wf, orc.INNER_MLP), rtol=1e-13, atol=1e-14)


def test_write_then_query_dot_linear_equals_full_batch():
    """With the dot loss the linear model's gradient does not depend on W, so
    sequential mini-batches that all write before the queries read give the
    full-batch result: linear attention eta Q (K^T V) at W0 = 0."""
    rng = np.random.default_rng(27)
    q, k, v, W0, et = _lin_dot_case(rng, N=23)
    args = dict(eta_tok=et, loss=orc.LOSS_DOT, inner=orc.INNER_LINEAR, key_norm=False)
    O_seq, W_seq = orc.oracle_forward(q, k, v, W0, chunk=5, order=orc.ORDER_WRITE_THEN_QUERY, **args)
    O_full, W_full = orc.oracle_forward(q, k, v, W0, chunk=0, **args)
    np.testing.assert_allclose(O_seq, O_full, rtol=1e-12, atol=1e-13)
    Q, K, V, E = q[0, 0], k[0, 0], v[0, 0], et[0, 0]
    np.testing.assert_allclose(O_full[0, 0], Q @ (K.T @ (E[:, None] * V)), rtol=1e-12, atol=1e-13)


def test_read_only_chunks_block_causal():
    """Read-only chunks [LaCT, video]: O_c = Q_c sum_{j<c, j writes}
    K_j^T diag(eta_j) V_j for the linear model with dot loss at W0 = 0; with
    no writing chunk every query reads W0 and W0 is returned."""
    rng = np.random.default_rng(28)
    q, k, v, W0, et = _lin_dot_case(rng, N=25)
    C, mask = 5, [1, 0, 1, 0, 1]
    args = dict(eta_tok=et, loss=orc.LOSS_DOT, inner=orc.INNER_LINEAR, key_norm=False, chunk=C)
    O, _ = orc.oracle_forward(q, k, v, W0, chunk_update=mask, **args)
    Q, K, V, E = q[0, 0], k[0, 0], v[0, 0], et[0, 0]
    for c in range(5):
        W = sum((K[j * C:(j + 1) * C].T @ (E[j * C:(j + 1) * C, None] * V[j * C:(j + 1) * C])
                 for j in range(c) if mask[j]), np.zeros((4, 4)))
        np.testing.assert_allclose(O[0, 0, c * C:(c + 1) * C], Q[c * C:(c + 1) * C] @ W, rtol=1e-11, atol=1e-12)
    rng2 = np.random.default_rng(29)
    q2, k2, v2, W02 = _rand_case(rng2, N=12, d=4, h=6, inner=orc.INNER_SWIGLU)
    O2, Wf2 = orc.oracle_forward(q2, k2, v2, W02, inner=orc.INNER_SWIGLU, loss=orc.LOSS_DOT, chunk=4,
                                 key_norm=False, chunk_update=[0, 0, 0], renorm=True)
    np.testing.assert_array_equal(O2, orc.oracle_readout(q2, [w[None] for w in W02], orc.INNER_SWIGLU))
    for a, b in zip(Wf2, W02):
        np.testing.assert_array_equal(a[0, 0], b[0])


def test_renorm_applies_to_updated_matrices_only():
    rng = np.random.default_rng(30)
    q, k, v, W0 = _rand_case(rng, N=12, d=4, h=6, inner=orc.INNER_SWIGLU, wscale=1.0)
    _, Wf = orc.oracle_forward(q, k, v, W0, inner=orc.INNER_SWIGLU, loss=orc.LOSS_DOT, chunk=4, key_norm=False,
                               renorm=True, update_mask=[False, True, True], rule=orc.RULE_MOMENTUM, beta=0.5)
    np.testing.assert_array_equal(Wf[0][0, 0], W0[0][0])
    for i in (1, 2):
        np.testing.assert_allclose(np.linalg.norm(Wf[i][0, 0], axis=0), np.linalg.norm(W0[i][0], axis=0),
                                   rtol=1e-12)
        assert np.max(np.abs(Wf[i][0, 0] - W0[i][0])) > 1e-3


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


# --------------------------------------------------------------------------
# ViT3's inner models: simplified GLU and the depthwise convolution, and the
# ViT3 head split (one convolution head, the others GLU heads)
# --------------------------------------------------------------------------
def _grid_case(rng, B=1, H=1, gh=5, gw=6, d=4, k=3, shift=0.5):
    N = gh * gw
    q = rng.standard_normal((B, H, N, d))
    kk = rng.standard_normal((B, H, N, d)) + shift
    v = rng.standard_normal((B, H, N, d))
    return q, kk, v, (gh, gw), N


@pytest.mark.parametrize("loss", [orc.LOSS_MSE, orc.LOSS_DOT])
def test_glu_and_dwconv_backward_by_finite_differences(loss):
    rng = np.random.default_rng(40)
    gh, gw, d, k = 4, 5, 3, 3
    N = gh * gw
    X = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    eta = 0.3 + rng.random(N)
    for inner, W in ((orc.INNER_GLU, [rng.standard_normal((d, d)) * 0.7, rng.standard_normal((d, d)) * 0.7]),
                     (orc.INNER_DWCONV, [rng.standard_normal((d, k * k)) * 0.5])):
        def L(Ws):
            Vh, _ = orc.inner_forward(inner, Ws, X, (gh, gw))
            if loss == orc.LOSS_MSE:
                return float(np.sum(eta[:, None] * (Vh - V) ** 2) / V.size)
            return float(-np.sum(eta[:, None] * Vh * V))

        Vh, cache = orc.inner_forward(inner, W, X, (gh, gw))
        dW = orc.inner_backward(inner, W, X, orc.loss_grad(loss, Vh, V, eta), cache, (gh, gw))
        for i, w in enumerate(W):
            fd = np.zeros_like(w)
            for idx in np.ndindex(w.shape):
                wp = [x.copy() for x in W]
                wm = [x.copy() for x in W]
                wp[i][idx] += 1e-6
                wm[i][idx] -= 1e-6
                fd[idx] = (L(wp) - L(wm)) / 2e-6
            np.testing.assert_allclose(dW[i], fd, rtol=1e-6, atol=1e-9, err_msg=f"{inner} dW{i}")


def _torch_vit3(q, k, v, W0, grid, eta_scale, eta_tok, loss, inner, key_norm, epochs, beta=None):
    """GLU with F.silu, the depthwise convolution with F.conv2d(groups=d),
    gradients by autograd; inner "vit3" = head 0 convolution, other heads GLU."""
    F = torch.nn.functional
    q, k, v = (torch.tensor(a, dtype=torch.float64) for a in (q, k, v))
    B, H, N, d = q.shape
    gh, gw = grid
    if key_norm:
        k = F.instance_norm(k.reshape(B * H, N, d).transpose(1, 2), eps=1e-5).transpose(1, 2).reshape(B, H, N, d)
    eta = torch.full((B, H, N), float(eta_scale), dtype=torch.float64)
    if eta_tok is not None:
        eta = eta * torch.tensor(eta_tok, dtype=torch.float64)

    def conv(x, w):                       # x [N, d], w [d, k*k]
        kk = int(round(math.sqrt(w.shape[1])))
        img = x.T.reshape(1, d, gh, gw)
        out = F.conv2d(img, w.reshape(d, 1, kk, kk), padding=(kk - 1) // 2, groups=d)
        return out.reshape(d, N).T

    def fwd(model, Ws, x):
        if model == orc.INNER_GLU:
            return (x @ Ws[0]) * F.silu(x @ Ws[1])
        return conv(x, Ws[0])

    O = torch.zeros_like(q)
    for b in range(B):
        for h in range(H):
            model, used = orc.head_model(inner, h)
            Ws = [torch.tensor(np.asarray(W0[i])[h], dtype=torch.float64) for i in used]
            mom = [torch.zeros_like(w) for w in Ws]
            for _ in range(epochs):
                Wg = [w.clone().requires_grad_(True) for w in Ws]
                Vh = fwd(model, Wg, k[b, h])
                et = eta[b, h]
                if loss == orc.LOSS_MSE:
                    Lv = (et[:, None] * (Vh - v[b, h]) ** 2).mean()
                else:
                    Lv = -(et[:, None] * Vh * v[b, h]).sum()
                grads = torch.autograd.grad(Lv, Wg)
                if beta is not None:
                    mom = [beta * m + g for m, g in zip(mom, grads)]
                    grads = mom
                Ws = [w - g for w, g in zip(Ws, grads)]
            O[b, h] = fwd(model, Ws, q[b, h])
    return O.numpy()


@pytest.mark.parametrize("inner,loss,key_norm,epochs,beta", [
    (orc.INNER_GLU, orc.LOSS_DOT, True, 1, None),
    (orc.INNER_GLU, orc.LOSS_MSE, False, 2, None),
    (orc.INNER_DWCONV, orc.LOSS_DOT, True, 1, None),
    (orc.INNER_DWCONV, orc.LOSS_MSE, False, 3, 0.5),
    (orc.INNER_VIT3, orc.LOSS_DOT, True, 1, None),
    (orc.INNER_VIT3, orc.LOSS_MSE, True, 2, None),
])
def test_vit3_models_match_autograd_layer(inner, loss, key_norm, epochs, beta):
    rng = np.random.default_rng(41)
    B, H, d, k = 2, 3, 5, 3
    q, kk, v, grid, N = _grid_case(rng, B=B, H=H, d=d, k=k)
    W0 = {orc.INNER_GLU: [rng.standard_normal((H, d, d)) * 0.4, rng.standard_normal((H, d, d)) * 0.4],
          orc.INNER_DWCONV: [rng.standard_normal((H, d, k * k)) * 0.3]}
    W0[orc.INNER_VIT3] = W0[orc.INNER_GLU] + W0[orc.INNER_DWCONV]
    eta_tok = 0.2 + rng.random((B, H, N))
    O, _ = orc.oracle_forward(q, kk, v, W0[inner], eta_scale=0.9, eta_tok=eta_tok, loss=loss, inner=inner, chunk=0,
                              key_norm=key_norm, epochs=epochs, grid=grid,
                              rule=orc.RULE_GD if beta is None else orc.RULE_MOMENTUM, beta=beta or 0.0)
    O_ref = _torch_vit3(q, kk, v, W0[inner], grid, 0.9, eta_tok, loss, inner, key_norm, epochs, beta)
    np.testing.assert_allclose(O, O_ref, rtol=1e-10, atol=1e-12)


def test_dwconv_dot_zero_init_closed_form():
    """Depthwise convolution, dot loss, W0 = 0 (key norm off): the updated
    kernel of channel c is eta times the cross-correlation of the padded key
    channel with the value channel, and O is Q cross-correlated with it
    ('same' mode) -- both through scipy.signal.correlate2d."""
    from scipy.signal import correlate2d

    rng = np.random.default_rng(42)
    gh, gw, d, k, eta = 6, 7, 3, 3, 0.7
    q, kk, v, grid, N = _grid_case(rng, gh=gh, gw=gw, d=d, k=k)
    O, Wf = orc.oracle_forward(q, kk, v, [np.zeros((1, d, k * k))], eta_scale=eta, loss=orc.LOSS_DOT,
                               inner=orc.INNER_DWCONV, chunk=0, key_norm=False, grid=grid)
    Q, K, V = (a[0, 0].reshape(gh, gw, d) for a in (q, kk, v))
    for c in range(d):
        w = eta * correlate2d(np.pad(K[:, :, c], 1), V[:, :, c], mode="valid")     # [k, k]
        np.testing.assert_allclose(Wf[0][0, 0, c].reshape(k, k), w, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(O[0, 0, :, c].reshape(gh, gw), correlate2d(Q[:, :, c], w, mode="same"),
                                   rtol=1e-11, atol=1e-12)


def test_dwconv_1x1_is_channel_scaling_closed_form():
    """A 1 x 1 depthwise kernel scales every channel: with MSE,
    w_c* = w_c - eta 2/(N d) sum_t (w_c x_tc - v_tc) x_tc and O = Q w*."""
    rng = np.random.default_rng(43)
    q, kk, v, grid, N = _grid_case(rng, gh=4, gw=5, d=3)
    w0 = rng.standard_normal((1, 3, 1))
    eta = 1.3
    O, Wf = orc.oracle_forward(q, kk, v, [w0], eta_scale=eta, loss=orc.LOSS_MSE, inner=orc.INNER_DWCONV, chunk=0,
                               key_norm=False, grid=grid)
    X, V = kk[0, 0], v[0, 0]
    w = w0[0, :, 0] - eta * 2.0 / (N * 3) * np.sum((X * w0[0, :, 0] - V) * X, axis=0)
    np.testing.assert_allclose(Wf[0][0, 0, :, 0], w, rtol=1e-12)
    np.testing.assert_allclose(O[0, 0], q[0, 0] * w, rtol=1e-12)


def test_vit3_heads_are_the_two_models():
    """The ViT3 block: head 0 is exactly the convolution layer on that head,
    the other heads exactly the GLU layer on theirs."""
    rng = np.random.default_rng(44)
    B, H, d, k = 2, 3, 4, 3
    q, kk, v, grid, N = _grid_case(rng, B=B, H=H, d=d)
    W1, W2 = rng.standard_normal((H, d, d)) * 0.5, rng.standard_normal((H, d, d)) * 0.5
    Wc = rng.standard_normal((H, d, k * k)) * 0.3
    args = dict(loss=orc.LOSS_DOT, chunk=0, key_norm=True, grid=grid)
    O, Wf = orc.oracle_forward(q, kk, v, [W1, W2, Wc], inner=orc.INNER_VIT3, **args)
    Oc, Wfc = orc.oracle_forward(q[:, :1], kk[:, :1], v[:, :1], [Wc[:1]], inner=orc.INNER_DWCONV, **args)
    Og, Wfg = orc.oracle_forward(q[:, 1:], kk[:, 1:], v[:, 1:], [W1[1:], W2[1:]], inner=orc.INNER_GLU, **args)
    np.testing.assert_array_equal(O[:, :1], Oc)
    np.testing.assert_array_equal(O[:, 1:], Og)
    np.testing.assert_array_equal(Wf[2][:, :1], Wfc[0])
    np.testing.assert_array_equal(Wf[0][:, 1:], Wfg[0])
    np.testing.assert_array_equal(Wf[1][:, 1:], Wfg[1])


# --------------------------------------------------------------------------
# Outer-loop backward (gradient through the inner update)
# --------------------------------------------------------------------------
def _outer_case(rng, inner, B=1, H=2, N=7, d=3, h=4, shared=True):
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) + 0.5
    v = rng.standard_normal((B, H, N, d))
    dO = rng.standard_normal((B, H, N, d))
    shapes = [(d, d)] if inner == orc.INNER_LINEAR else [(d, h), (h, d)]
    lead = (H,) if shared else (B, H)
    W0 = [rng.standard_normal(lead + s) * 0.6 for s in shapes]
    eta_tok = 0.5 + rng.random((B, H, N))
    return q, k, v, dO, W0, eta_tok


@pytest.mark.parametrize("inner", [orc.INNER_LINEAR, orc.INNER_MLP])
@pytest.mark.parametrize("loss", [orc.LOSS_MSE, orc.LOSS_DOT])
@pytest.mark.parametrize("key_norm", [False, True])
def test_outer_backward_matches_finite_differences(inner, loss, key_norm):
    """Brute force: central differences of S = sum(dO * O) with respect to
    every element of q, k, v, W0 and the per-token rates."""
    rng = np.random.default_rng(50)
    q, k, v, dO, W0, et = _outer_case(rng, inner, B=2, H=1, shared=True)
    scale = 0.7

    def S(q_, k_, v_, W_, et_):
        O, _ = orc.oracle_forward(q_, k_, v_, W_, eta_scale=scale, eta_tok=et_, loss=loss, inner=inner, chunk=0,
                                  key_norm=key_norm, eps=1e-5)
        return float(np.sum(dO * O))

    g = orc.oracle_backward(q, k, v, W0, dO, eta_scale=scale, eta_tok=et, loss=loss, inner=inner,
                            key_norm=key_norm, eps=1e-5)
    e = 1e-6
    for name, pos in (("dq", 0), ("dk", 1), ("dv", 2)):
        base = [q, k, v]
        num = np.zeros_like(q)
        for ix in np.ndindex(q.shape):
            p_, m_ = [a.copy() for a in base], [a.copy() for a in base]
            p_[pos][ix] += e
            m_[pos][ix] -= e
            num[ix] = (S(*p_, W0, et) - S(*m_, W0, et)) / (2 * e)
        np.testing.assert_allclose(g[name], num, rtol=1e-5, atol=1e-7, err_msg=name)
    for i in range(len(W0)):
        num = np.zeros_like(W0[i])
        for ix in np.ndindex(W0[i].shape):
            wp, wm = [w.copy() for w in W0], [w.copy() for w in W0]
            wp[i][ix] += e
            wm[i][ix] -= e
            num[ix] = (S(q, k, v, wp, et) - S(q, k, v, wm, et)) / (2 * e)
        np.testing.assert_allclose(g["dW0"][i], num, rtol=1e-5, atol=1e-7, err_msg=f"dW0[{i}]")
    num = np.zeros_like(et)
    for ix in np.ndindex(et.shape):
        ep, em = et.copy(), et.copy()
        ep[ix] += e
        em[ix] -= e
        num[ix] = (S(q, k, v, W0, ep) - S(q, k, v, W0, em)) / (2 * e)
    # deta is the gradient with respect to eta_n = scale * eta_tok[n]
    np.testing.assert_allclose(g["deta"] * scale, num, rtol=1e-5, atol=1e-7, err_msg="deta")


@pytest.mark.parametrize("inner,loss,key_norm,shared", [
    (orc.INNER_MLP, orc.LOSS_MSE, True, True),
    (orc.INNER_MLP, orc.LOSS_DOT, False, False),
    (orc.INNER_LINEAR, orc.LOSS_MSE, True, False),
    (orc.INNER_LINEAR, orc.LOSS_DOT, True, True),
])
def test_outer_backward_matches_autograd(inner, loss, key_norm, shared):
    """Independent derivation: the layer in torch with F.instance_norm and
    F.gelu, the inner gradient by autograd with create_graph=True, and the
    outer gradients by autograd through it."""
    F = torch.nn.functional
    rng = np.random.default_rng(51)
    q, k, v, dO, W0, et = _outer_case(rng, inner, B=2, H=2, N=9, d=4, h=5, shared=shared)
    scale = 0.8
    g = orc.oracle_backward(q, k, v, W0, dO, eta_scale=scale, eta_tok=et, loss=loss, inner=inner,
                            key_norm=key_norm, eps=1e-5)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    tW = [torch.tensor(w, requires_grad=True) for w in W0]
    teta = torch.tensor(et * scale, requires_grad=True)          # effective per-token rate
    B, H, N, d = q.shape
    kk = tk
    if key_norm:
        kk = F.instance_norm(tk.reshape(B * H, N, d).transpose(1, 2), eps=1e-5).transpose(1, 2).reshape(B, H, N, d)

    def fwd(Ws, x):
        return x @ Ws[0] if inner == orc.INNER_LINEAR else F.gelu(x @ Ws[0]) @ Ws[1]

    S = 0.0
    for b in range(B):
        for h in range(H):
            Ws = [w[h] if shared else w[b, h] for w in tW]
            Vh = fwd(Ws, kk[b, h])
            en = teta[b, h][:, None]
            if loss == orc.LOSS_MSE:
                Lv = (en * (Vh - tv[b, h]) ** 2).sum() / (N * d)
            else:
                Lv = -(en * Vh * tv[b, h]).sum()
            grads = torch.autograd.grad(Lv, Ws, create_graph=True)
            Wst = [w - gg for w, gg in zip(Ws, grads)]
            S = S + (torch.tensor(dO[b, h]) * fwd(Wst, tq[b, h])).sum()
    S.backward()
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(g["dk"], tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(g["dv"], tv.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(g["deta"], teta.grad.numpy(), rtol=1e-9, atol=1e-11)
    for a, t in zip(g["dW0"], tW):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_gelu_second_derivative_by_finite_difference():
    z = np.linspace(-6, 6, 1201)
    e = 1e-6
    np.testing.assert_allclose(orc.gelu_second(z), (orc.gelu_prime(z + e) - orc.gelu_prime(z - e)) / (2 * e),
                               rtol=1e-6, atol=1e-8)
