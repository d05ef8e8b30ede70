"""Float64 CPU oracle for the Test-Time-Training (TTT) layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
this file: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

It is a plain, slow, direct transcription of what the pages define, in NumPy
float64 (matmul is the only library primitive used for the algebra; ``erf`` comes
from SciPy).  Pages cited:

* [ViT3]  ViT³ paper summary (app.podcasttoinsight.top, papers/vit3-test-time-
  training-vision), §02 "method essence" -- the
  inner-loop update equation (forward on keys, one gradient step with rate eta,
  readout on queries); §03 guideline 1 (losses MSE / dot product), guideline 2
  (single epoch, full batch B = N), guideline 3 (eta = 1.0), guideline 4 (two-layer
  MLP widened to r*d), glossary entry "linear attention" (W = K^T V).
* [LaCT]  "Test-Time Training Done Right" analysis (www.iplexlaw.co.kr, blog/lact-
  large-chunk-test-time-training), sections
  "Fast weights as memory of the current context" (large chunks), "Nonlinear
  memory complements local attention" (SwiGLU fast weights with three matrices,
  negative dot-product loss, chunk gradients summed with per-token learning
  rates, L2 normalisation after the update), "Order of operations excludes
  leaking the future" (read-then-update per chunk; write-then-query for sets).
* [TvS]   "Test-Time Training vs Sleep" compare page (researchpapers.dev, en/
  compare/test-time-training-vs-sleep), section "Side one"
  (key instance normalisation removes the constant key shift; NaN without it).

The update variants follow the same pages:
* update rules [LaCT "Nonlinear memory..."]: plain gradient step, momentum,
  and Muon (the momentum matrix orthogonalised by Newton-Schulz iterations);
  L2 normalisation after every update;
* several epochs over one update batch, and sequential mini-batches that all
  write before any query reads [ViT3 §03 guideline 2];
* only the first layer adjusted [TvS "Side one"];
* chunks that only read while others write (video: clean chunks write, noisy
  chunks read) [LaCT "Order of operations..."].

Every pinned property of this file is exercised by ``tests/test_oracle.py``.
Points the pages leave open (MSE reduction constant, norm axis, epsilon,
activation, re-norm axis, ...) are readings, not page facts; each function
states the reading it implements.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf, expit

INNER_LINEAR = "linear"
INNER_MLP = "mlp_gelu"
INNER_SWIGLU = "swiglu"
INNER_GLU = "glu"
INNER_DWCONV = "dwconv"
INNER_VIT3 = "vit3"
LOSS_MSE = "mse"
LOSS_DOT = "dot"

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ---------------------------------------------------------------------------
# Activations.  Exact erf-GELU (reading: the configs name GELU, no page fixes
# the variant; the exact form is the definition).  SiLU is the gate of SwiGLU
# [LaCT "Nonlinear memory..."].
# ---------------------------------------------------------------------------
def gelu(z):
    return 0.5 * z * (1.0 + erf(z / _SQRT2))


def gelu_prime(z):
    return 0.5 * (1.0 + erf(z / _SQRT2)) + z * np.exp(-0.5 * z * z) * _INV_SQRT_2PI


def sigmoid(z):
    return expit(z)


def silu(z):
    return z * sigmoid(z)


def silu_prime(z):
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


# ---------------------------------------------------------------------------
# Key instance normalisation [TvS "Side one"]: pretrained keys carry a constant
# shift that softmax cancels and the inner optimisation does not.  Reading: the
# statistics are per channel over the tokens of one (batch, head), biased
# variance, eps inside the square root, no affine parameters, keys only.
# ---------------------------------------------------------------------------
def key_instnorm(K, eps):
    """K: [N, d] -> (K - mean_n K) / sqrt(var_n K + eps), per channel."""
    mu = K.mean(axis=0, keepdims=True)
    var = ((K - mu) ** 2).mean(axis=0, keepdims=True)
    return (K - mu) / np.sqrt(var + eps)


# ---------------------------------------------------------------------------
# Inner model F_W  [ViT3 §02; §03 guideline 4; LaCT "Nonlinear memory..."].
# Row-vector convention: x is [n, d]; every matrix is stored [in, out].
#   linear : F(x) = x W
#   mlp    : F(x) = gelu(x W1) W2,            W1 [d, h], W2 [h, d]
#   swiglu : F(x) = (silu(x W1) * (x W3)) W2, W1, W3 [d, h], W2 [h, d]
# W is a list: [W] / [W1, W2] / [W1, W2, W3].
# ---------------------------------------------------------------------------
# ViT3 §03 guideline 6 / §04 and its glossary: the simplified gated linear
# unit FC(x) * SiLU(FC(x)) (two d x d maps, no output projection; reading: no
# biases, W[0] is the plain branch, W[1] the gated one) and the depthwise
# convolution, whose kernel is the fast weight: the tokens form a gh x gw
# raster (token t = i gw + j) and channel c of the output is the k x k
# cross-correlation of channel c of the input with w[c] (reading: zero padding
# of (k - 1) / 2 on every side, stride 1, no bias; w stored [d, k*k], tap
# (a, b) at a k + b).
def _pad_raster(X, grid, r):
    gh, gw = grid
    return np.pad(X.reshape(gh, gw, -1), ((r, r), (r, r), (0, 0)))


def dwconv(X, w, grid):
    """Depthwise k x k cross-correlation of the [N, d] raster X with w [d, k*k]."""
    gh, gw = grid
    k = int(round(math.sqrt(w.shape[1])))
    r = (k - 1) // 2
    Xp = _pad_raster(X, grid, r)
    out = np.zeros((gh, gw, X.shape[1]))
    for a in range(k):
        for b in range(k):
            out += Xp[a:a + gh, b:b + gw, :] * w[:, a * k + b]
    return out.reshape(gh * gw, -1)


def dwconv_weight_grad(X, G, grid, k):
    """dL/dw [d, k*k] of the depthwise convolution given G = dL/dout [N, d]."""
    gh, gw = grid
    r = (k - 1) // 2
    Xp = _pad_raster(X, grid, r)
    Gr = G.reshape(gh, gw, -1)
    dw = np.zeros((G.shape[1], k * k))
    for a in range(k):
        for b in range(k):
            dw[:, a * k + b] = np.sum(Gr * Xp[a:a + gh, b:b + gw, :], axis=(0, 1))
    return dw


def inner_forward(inner, W, X, grid=None):
    """Returns (F_W(X), cache) -- cache holds what the hand backward needs."""
    if inner == INNER_LINEAR:
        return X @ W[0], None
    if inner == INNER_GLU:
        U = X @ W[0]
        Z = X @ W[1]
        return U * silu(Z), (U, Z)
    if inner == INNER_DWCONV:
        return dwconv(X, W[0], grid), None
    if inner == INNER_MLP:
        Z = X @ W[0]
        A = gelu(Z)
        return A @ W[1], (Z, A)
    if inner == INNER_SWIGLU:
        Z1 = X @ W[0]
        Z3 = X @ W[2]
        Hh = silu(Z1) * Z3
        return Hh @ W[1], (Z1, Z3, Hh)
    raise ValueError(f"unknown inner model {inner!r}")


def inner_backward(inner, W, X, G, cache, grid=None):
    """Hand-derived dL/dW given G = dL/dF_W(X) ([ViT3 §02], step (ii)).

    MLP   : dW2 = A^T G ; dZ = (G W2^T) * gelu'(Z) ; dW1 = X^T dZ
    SwiGLU: dW2 = Hh^T G ; dH = G W2^T ; dZ1 = dH * Z3 * silu'(Z1) ;
            dZ3 = dH * silu(Z1) ; dW1 = X^T dZ1 ; dW3 = X^T dZ3
    linear: dW = X^T G
    GLU   : dU = G * silu(Z) ; dZ = G * U * silu'(Z) ; dW1 = X^T dU ; dW2 = X^T dZ
    DWConv: dw[c, tap] = sum over tokens of G[., c] times the tap's shifted X[., c]
    """
    if inner == INNER_LINEAR:
        return [X.T @ G]
    if inner == INNER_GLU:
        U, Z = cache
        return [X.T @ (G * silu(Z)), X.T @ (G * U * silu_prime(Z))]
    if inner == INNER_DWCONV:
        k = int(round(math.sqrt(W[0].shape[1])))
        return [dwconv_weight_grad(X, G, grid, k)]
    if inner == INNER_MLP:
        Z, A = cache
        dW2 = A.T @ G
        dZ = (G @ W[1].T) * gelu_prime(Z)
        dW1 = X.T @ dZ
        return [dW1, dW2]
    if inner == INNER_SWIGLU:
        Z1, Z3, Hh = cache
        dW2 = Hh.T @ G
        dH = G @ W[1].T
        dZ1 = dH * Z3 * silu_prime(Z1)
        dZ3 = dH * silu(Z1)
        return [X.T @ dZ1, dW2, X.T @ dZ3]
    raise ValueError(f"unknown inner model {inner!r}")


# ---------------------------------------------------------------------------
# Reconstruction losses [ViT3 §03 guideline 1 / loss table; LaCT "Nonlinear
# memory..."].  Per-token learning rates eta_n weight each token's gradient in
# the sum over the batch [LaCT]; a scalar eta is the constant case [ViT3 §02].
#   MSE (reading: mean over all n*d entries of the batch):
#       L = sum_n eta_n * (1/(n_b d)) * ||F(k_n) - v_n||^2
#       G_n = eta_n * 2/(n_b d) * (F(k_n) - v_n)
#   dot (reading: sum, negative):
#       L = - sum_n eta_n * <F(k_n), v_n>,    G_n = - eta_n v_n
# eta is folded into G, so the update below is W <- W - dW.
# ---------------------------------------------------------------------------
def loss_value(loss, Vhat, V, eta_n):
    nb, d = V.shape
    if loss == LOSS_MSE:
        return float(np.sum(eta_n[:, None] * (Vhat - V) ** 2) / (nb * d))
    if loss == LOSS_DOT:
        return float(-np.sum(eta_n[:, None] * Vhat * V))
    raise ValueError(f"unknown loss {loss!r}")


def loss_grad(loss, Vhat, V, eta_n):
    nb, d = V.shape
    if loss == LOSS_MSE:
        return eta_n[:, None] * (2.0 / (nb * d)) * (Vhat - V)
    if loss == LOSS_DOT:
        return -eta_n[:, None] * V
    raise ValueError(f"unknown loss {loss!r}")


def column_renorm(W, Wref):
    """L2 re-normalisation after an update [LaCT "Nonlinear memory..."].

    Reading: every output column of an [in, out] matrix is rescaled to the norm
    that column had in the initial weights W0 (unit norm for unit-norm W0).
    """
    n_new = np.sqrt((W * W).sum(axis=0, keepdims=True))
    n_ref = np.sqrt((Wref * Wref).sum(axis=0, keepdims=True))
    return W * (n_ref / np.maximum(n_new, 1e-12))


# ---------------------------------------------------------------------------
# Update rules [LaCT "Nonlinear memory complements local attention": plain
# gradient descent, momentum, and Muon, which turns the matrix gradient into
# an orthogonalised matrix by Newton-Schulz iterations; L2 normalisation after
# the update].  The page names the rules only.  Readings:
#   momentum: M <- beta M + G,   W <- W - M        (heavy ball, M starts at 0)
#   Muon    : M <- beta M + G,   W <- W - s NS(M)   (beta = 0: no momentum)
# where G is the eta-weighted chunk gradient and NS is the Newton-Schulz
# orthogonalisation of the published Muon optimiser (Jordan et al., 2024):
# X = M / (||M||_F + 1e-7); k times X <- a X + (b A + c A A) X with A = X X^T,
# (a, b, c) = (3.4445, -4.7750, 2.0315), computed on the wide orientation
# (rows <= cols; a tall matrix is transposed first and back after).  Each step
# maps every singular value sigma of X to a sigma + b sigma^3 + c sigma^5 and
# keeps the singular vectors.
# ---------------------------------------------------------------------------
RULE_GD = "gd"
RULE_MOMENTUM = "momentum"
RULE_MUON = "muon"
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def newton_schulz(M, steps):
    a, b, c = NS_COEFFS
    tall = M.shape[0] > M.shape[1]
    X = M.T if tall else M
    X = X / (np.sqrt(np.sum(X * X)) + 1e-7)
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    return X.T if tall else X


def apply_rule(W, dW, M, rule, beta, muon_scale, ns_steps, update):
    """One update of the matrices flagged in ``update`` (the others keep their
    values and their momentum).  dW already carries eta.  Returns (W, M)."""
    W, M = list(W), list(M)
    for i, (w, g) in enumerate(zip(W, dW)):
        if not update[i]:
            continue
        if rule == RULE_GD:
            W[i] = w - g
        elif rule == RULE_MOMENTUM:
            M[i] = beta * M[i] + g
            W[i] = w - M[i]
        elif rule == RULE_MUON:
            M[i] = beta * M[i] + g
            W[i] = w - muon_scale * newton_schulz(M[i], ns_steps)
        else:
            raise ValueError(f"unknown update rule {rule!r}")
    return W, M


def inner_step(inner, loss, W, X, V, eta_n, grid=None):
    """One gradient step of the inner model on the mini-dataset (X, V).

    [ViT3 §02]: V̂ = F_W(X); W <- W - eta * dL(V̂, V)/dW.  Returns (W_new, dW).
    """
    Vhat, cache = inner_forward(inner, W, X, grid)
    G = loss_grad(loss, Vhat, V, eta_n)
    dW = inner_backward(inner, W, X, G, cache, grid)
    return [w - g for w, g in zip(W, dW)], dW


def n_matrices(inner):
    return {INNER_LINEAR: 1, INNER_MLP: 2, INNER_SWIGLU: 3, INNER_GLU: 2, INNER_DWCONV: 1, INNER_VIT3: 3}[inner]


def head_model(inner, h):
    """ViT3 block [ViT3 §04]: one head uses the depthwise convolution, the other
    heads the simplified GLU (reading: head 0 is the convolution head).  W0 of
    "vit3" is [W1, W2, w_conv]; returns (inner model of head h, indices of the
    matrices it uses)."""
    if inner != INNER_VIT3:
        return inner, list(range(n_matrices(inner)))
    return (INNER_DWCONV, [2]) if h == 0 else (INNER_GLU, [0, 1])


def _pair_weights(W0, b, h):
    """W0 matrices are [H, in, out] (shared over the batch) or [B, H, in, out]."""
    out = []
    for w in W0:
        w = np.asarray(w, dtype=np.float64)
        out.append(w[h].copy() if w.ndim == 3 else w[b, h].copy())
    return out


ORDER_CAUSAL = "causal"
ORDER_WRITE_THEN_QUERY = "write_then_query"


def oracle_forward(q, k, v, W0, *, eta_scale=1.0, eta_tok=None, loss=LOSS_MSE,
                   inner=INNER_MLP, chunk=0, key_norm=True, eps=1e-5,
                   renorm=False, epochs=1, update_mask=None, order=ORDER_CAUSAL,
                   chunk_update=None, rule=RULE_GD, beta=0.0, muon_scale=1.0,
                   ns_steps=5, grid=None):
    """TTT-layer forward.  q, k, v: [B, H, N, d]; W0: list of matrices
    ([H, in, out] or [B, H, in, out]); eta_tok: None or [B, H, N].

    chunk == 0 : full batch, one update batch of all N tokens, then every
                 query reads the updated weights (write-then-query) [ViT3 §03
                 guideline 2; LaCT "Order of operations"].
    chunk == C : update batches of C tokens (the last may be shorter).
                 order "causal": each chunk first reads the weights left by
                 the earlier chunks, then takes its own step [LaCT "Order of
                 operations"]; order "write_then_query": every chunk writes in
                 turn (sequential mini-batches), then every query reads the
                 final weights [ViT3 §03 guideline 2; LaCT, sets of images].
    epochs     : gradient steps on each update batch [ViT3 §03 guideline 2].
    update_mask: which matrices the steps change (None: all); e.g. [True,
                 False] adjusts only the first layer [TvS "Side one"].
    chunk_update: None or one flag per chunk; a chunk with a false flag only
                 reads (video: clean chunks write, noisy chunks read) [LaCT].
    rule, beta, muon_scale, ns_steps: the update rule (see apply_rule).
    renorm     : after every update, each updated matrix's columns get their
                 W0 norms back [LaCT].
    grid       : (gh, gw) token raster of the depthwise convolution (inner
                 "dwconv", and "vit3", whose head 0 is a convolution head and
                 whose other heads are GLU heads).
    Returns (O [B, H, N, d], W_final list of [B, H, in, out]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if chunk < 0:
        raise ValueError("chunk must be >= 0")
    if order not in (ORDER_CAUSAL, ORDER_WRITE_THEN_QUERY):
        raise ValueError(f"unknown order {order!r}")
    causal = chunk > 0 and order == ORDER_CAUSAL
    if causal and key_norm:
        raise ValueError("key instance norm over the whole sequence would read "
                         "future keys in causal chunked mode")
    if epochs < 1:
        raise ValueError("epochs must be >= 1")
    nm = n_matrices(inner)
    if len(W0) != nm:
        raise ValueError(f"{inner} needs {nm} matrices, got {len(W0)}")
    update_all = [True] * nm if update_mask is None else [bool(x) for x in update_mask]
    if len(update_all) != nm:
        raise ValueError("update_mask needs one flag per matrix")
    if inner in (INNER_DWCONV, INNER_VIT3):
        if grid is None or grid[0] * grid[1] != N:
            raise ValueError("the convolution needs a token grid with gh * gw == N")
        if chunk > 0:
            raise ValueError("the convolution inner model is full batch only")
        if rule == RULE_MUON or renorm:
            raise ValueError("Muon and the column re-norm are defined for matrices, not convolution kernels")
    span = chunk if chunk > 0 else N
    nb = (N + span - 1) // span
    if chunk_update is not None and len(chunk_update) != nb:
        raise ValueError(f"chunk_update needs {nb} flags")
    O = np.zeros_like(q)
    W_final = [np.zeros((B, H) + np.asarray(w).shape[-2:]) for w in W0]
    for b in range(B):
        for h in range(H):
            model, used = head_model(inner, h)
            allw = _pair_weights(W0, b, h)
            Wref = [allw[i] for i in used]
            update = [update_all[i] for i in used]
            W = [w.copy() for w in Wref]
            M = [np.zeros_like(w) for w in Wref]
            Q, K, V = q[b, h], k[b, h], v[b, h]
            eta = np.full(N, float(eta_scale))
            if eta_tok is not None:
                eta = eta * np.asarray(eta_tok, dtype=np.float64)[b, h]
            Kh = key_instnorm(K, eps) if key_norm else K
            for c in range(nb):
                s, e = c * span, min((c + 1) * span, N)
                if causal:
                    O[b, h, s:e] = inner_forward(model, W, Q[s:e])[0]   # read
                if chunk_update is not None and not chunk_update[c]:
                    continue                                              # read-only chunk
                for _ in range(epochs):
                    Vhat, cache = inner_forward(model, W, Kh[s:e], grid)
                    G = loss_grad(loss, Vhat, V[s:e], eta[s:e])
                    dW = inner_backward(model, W, Kh[s:e], G, cache, grid)
                    W, M = apply_rule(W, dW, M, rule, beta, muon_scale, ns_steps, update)
                    if renorm:
                        W = [column_renorm(w, r) if u else w for w, r, u in zip(W, Wref, update)]
            if not causal:
                O[b, h] = inner_forward(model, W, Q, grid)[0]             # write, then query
            for i in range(nm):                 # matrices a head does not use stay W0
                W_final[i][b, h] = W[used.index(i)] if i in used else allw[i]
    return O, W_final


def oracle_readout(q, W, inner, grid=None):
    """O = F_W(Q) for per-pair weights W ([B, H, in, out] each) -- step (iii)."""
    q = np.asarray(q, dtype=np.float64)
    B, H = q.shape[:2]
    O = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            model, used = head_model(inner, h)
            O[b, h] = inner_forward(model, [np.asarray(W[i], np.float64)[b, h] for i in used], q[b, h], grid)[0]
    return O


# ---------------------------------------------------------------------------
# Outer-loop backward [ViT3 §02: the whole inner update is differentiable and
# trained end to end with the outer network (a gradient of a gradient);
# §03 guideline 1: the value projection learns through the mixed second
# derivative of the loss].  Given dO = dS/dO of an outer loss S, the gradients
# of S with respect to Q, K, V, W0 and the per-token rates eta_n, for the full-
# batch single gradient step (chunk 0, one epoch, plain gradient descent, no
# re-norm), for the linear and the GELU-MLP inner models.
#
# Steps, per (b, h):
#   1. forward: K_hat, W* = W0 - g(W0), g = dL/dW at W0 (as oracle_forward)
#   2. readout backward at W*: U = dS/dW* and dQ (the inner backward with X = Q
#      and G = dO, plus the input gradient)
#   3. W* = W0 - g(W0, K_hat, V, eta): with phi = <g, U> = the derivative of L
#      along U (forward-mode tangent F_dot of the inner model along U, phi =
#      sum <G, F_dot>), dW0 = U - dphi/dW0, dK_hat = -dphi/dK_hat,
#      dV = -dphi/dV, deta = -dphi/deta (reverse mode through phi)
#   4. key-norm backward: dK = rstd (dK_hat - mean_n dK_hat - K_hat mean_n(dK_hat K_hat))
# Reading: W0 shared over the batch ([H, in, out]) gets the sum over b of its
# pairs' gradients; deta is the gradient with respect to the effective rate
# eta_n = eta_scale * eta_tok[n] of each token.
# ---------------------------------------------------------------------------
def gelu_second(z):
    """gelu''(z) = phi(z) (2 - z^2), phi the standard normal density."""
    return np.exp(-0.5 * z * z) * _INV_SQRT_2PI * (2.0 - z * z)


def _readout_backward(inner, W, Q, dO):
    """dS/dW and dS/dQ of O = F_W(Q) given dO."""
    if inner == INNER_LINEAR:
        return [Q.T @ dO], dO @ W[0].T
    Z = Q @ W[0]
    A = gelu(Z)
    dZ = (dO @ W[1].T) * gelu_prime(Z)
    return [Q.T @ dZ, A.T @ dO], dZ @ W[0].T


def _phi_backward(inner, loss, W, U, X, V, eta):
    """Reverse mode of phi = <dL/dW, U> = sum_n <G_n, F_dot_n> with respect to
    (W, X, V, eta).  Returns (dW list, dX, dV, deta)."""
    nb, d = V.shape
    c = 1.0 / (nb * d)
    # forward and tangent along U
    if inner == INNER_LINEAR:
        F = X @ W[0]
        Fd = X @ U[0]
    else:
        Z = X @ W[0]
        A = gelu(Z)
        F = A @ W[1]
        Zd = X @ U[0]
        Ad = gelu_prime(Z) * Zd
        Fd = Ad @ W[1] + A @ U[1]
    G = loss_grad(loss, F, V, eta)
    # reverse: phi = <G, Fd>
    Gb = Fd                                   # d phi / d G
    if loss == LOSS_MSE:
        Fb = 2.0 * c * eta[:, None] * Gb      # through G = 2 c eta (F - V)
        Vb = -Fb
        etab = 2.0 * c * np.sum(Gb * (F - V), axis=1)
    else:
        Fb = np.zeros_like(F)                 # G = -eta V does not depend on F
        Vb = -eta[:, None] * Gb
        etab = -np.sum(Gb * V, axis=1)
    Fdb = G                                   # d phi / d Fd
    if inner == INNER_LINEAR:
        Wb = [X.T @ Fb]                       # F = X W
        Xb = Fdb @ U[0].T + Fb @ W[0].T       # Fd = X U, F = X W
        return Wb, Xb, Vb, etab
    Adb = Fdb @ W[1].T                        # Fd = Ad W2 + A U2
    W2b = Ad.T @ Fdb + A.T @ Fb               # ... and F = A W2
    Ab = Fdb @ U[1].T + Fb @ W[1].T
    Zdb = gelu_prime(Z) * Adb                 # Ad = gelu'(Z) Zd
    Zb = gelu_second(Z) * Zd * Adb + gelu_prime(Z) * Ab
    Xb = Zdb @ U[0].T + Zb @ W[0].T           # Zd = X U1, Z = X W1
    W1b = X.T @ Zb
    return [W1b, W2b], Xb, Vb, etab


def key_instnorm_backward(K, dKh, eps):
    mu = K.mean(axis=0, keepdims=True)
    rstd = 1.0 / np.sqrt(((K - mu) ** 2).mean(axis=0, keepdims=True) + eps)
    Kh = (K - mu) * rstd
    return rstd * (dKh - dKh.mean(axis=0, keepdims=True) - Kh * (dKh * Kh).mean(axis=0, keepdims=True))


def oracle_backward(q, k, v, W0, dO, *, eta_scale=1.0, eta_tok=None, loss=LOSS_MSE, inner=INNER_MLP,
                    key_norm=True, eps=1e-5):
    """Gradients of S = sum(dO * O) for the full-batch single-step layer.
    Returns dict(dq, dk, dv [B, H, N, d], dW0 (list, W0's layout), deta [B, H, N])."""
    if inner not in (INNER_LINEAR, INNER_MLP):
        raise ValueError("the outer-loop backward covers the linear and GELU-MLP inner models")
    q, k, v, dO = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dO))
    B, H, N, d = q.shape
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(q), dv=np.zeros_like(q), deta=np.zeros((B, H, N)),
               dW0=[np.zeros(np.asarray(w).shape) for w in W0])
    for b in range(B):
        for h in range(H):
            W = _pair_weights(W0, b, h)
            Q, K, V = q[b, h], k[b, h], v[b, h]
            eta = np.full(N, float(eta_scale))
            if eta_tok is not None:
                eta = eta * np.asarray(eta_tok, dtype=np.float64)[b, h]
            Kh = key_instnorm(K, eps) if key_norm else K
            Ws, _ = inner_step(inner, loss, W, Kh, V, eta)                 # 1
            U, dQ = _readout_backward(inner, Ws, Q, dO[b, h])              # 2
            Wb, Xb, Vb, etab = _phi_backward(inner, loss, W, U, Kh, V, eta)  # 3
            dKh = -Xb
            out["dq"][b, h] = dQ
            out["dv"][b, h] = -Vb
            out["deta"][b, h] = -etab
            out["dk"][b, h] = key_instnorm_backward(K, dKh, eps) if key_norm else dKh   # 4
            for i, (u, wb) in enumerate(zip(U, Wb)):
                if np.asarray(W0[i]).ndim == 3:
                    out["dW0"][i][h] += u - wb
                else:
                    out["dW0"][i][b, h] = u - wb
    return out
