"""Float64 CPU oracle for the Test-Time-Training (TTT) layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
this file: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

It is a plain, slow, direct transcription of what the pages define, in NumPy
float64 (matmul is the only library primitive used for the algebra; ``erf`` comes
from SciPy).  Pages cited (full addresses in the design doc):

* [ViT3]  ViT³ paper summary (podcasttoinsight), §02 "method essence" -- the
  inner-loop update equation (forward on keys, one gradient step with rate eta,
  readout on queries); §03 guideline 1 (losses MSE / dot product), guideline 2
  (single epoch, full batch B = N), guideline 3 (eta = 1.0), guideline 4 (two-layer
  MLP widened to r*d), glossary entry "linear attention" (W = K^T V).
* [LaCT]  "Test-Time Training Done Right" analysis (iplexlaw blog), sections
  "Fast weights as memory of the current context" (large chunks), "Nonlinear
  memory complements local attention" (SwiGLU fast weights with three matrices,
  negative dot-product loss, chunk gradients summed with per-token learning
  rates, L2 normalisation after the update), "Order of operations excludes
  leaking the future" (read-then-update per chunk; write-then-query for sets).
* [TvS]   "Test-Time Training vs Sleep" compare page, section "Side one"
  (key instance normalisation removes the constant key shift; NaN without it).

Every pinned property of this file is exercised by ``tests/test_oracle.py``.
Readings of points the pages leave open (MSE reduction constant, norm axis,
epsilon, activation, re-norm axis, ...) are listed in the design doc; each function
names the reading it implements.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf, expit

INNER_LINEAR = "linear"
INNER_MLP = "mlp_gelu"
INNER_SWIGLU = "swiglu"
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
def inner_forward(inner, W, X):
    """Returns (F_W(X), cache) -- cache holds what the hand backward needs."""
    if inner == INNER_LINEAR:
        return X @ W[0], None
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


def inner_backward(inner, W, X, G, cache):
    """Hand-derived dL/dW given G = dL/dF_W(X) ([ViT3 §02], step (ii)).

    MLP   : dW2 = A^T G ; dZ = (G W2^T) * gelu'(Z) ; dW1 = X^T dZ
    SwiGLU: dW2 = Hh^T G ; dH = G W2^T ; dZ1 = dH * Z3 * silu'(Z1) ;
            dZ3 = dH * silu(Z1) ; dW1 = X^T dZ1 ; dW3 = X^T dZ3
    linear: dW = X^T G
    """
    if inner == INNER_LINEAR:
        return [X.T @ G]
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


def inner_step(inner, loss, W, X, V, eta_n):
    """One gradient step of the inner model on the mini-dataset (X, V).

    [ViT3 §02]: V̂ = F_W(X); W <- W - eta * dL(V̂, V)/dW.  Returns (W_new, dW).
    """
    Vhat, cache = inner_forward(inner, W, X)
    G = loss_grad(loss, Vhat, V, eta_n)
    dW = inner_backward(inner, W, X, G, cache)
    return [w - g for w, g in zip(W, dW)], dW


def n_matrices(inner):
    return {INNER_LINEAR: 1, INNER_MLP: 2, INNER_SWIGLU: 3}[inner]


def _pair_weights(W0, b, h):
    """W0 matrices are [H, in, out] (shared over the batch) or [B, H, in, out]."""
    out = []
    for w in W0:
        w = np.asarray(w, dtype=np.float64)
        out.append(w[h].copy() if w.ndim == 3 else w[b, h].copy())
    return out


def oracle_forward(q, k, v, W0, *, eta_scale=1.0, eta_tok=None, loss=LOSS_MSE,
                   inner=INNER_MLP, chunk=0, key_norm=True, eps=1e-5,
                   renorm=False):
    """TTT-layer forward.  q, k, v: [B, H, N, d]; W0: list of matrices
    ([H, in, out] or [B, H, in, out]); eta_tok: None or [B, H, N].

    chunk == 0 : full batch, one step over all N tokens, then every query reads
                 the updated weights (write-then-query) [ViT3 §03 guideline 2;
                 LaCT "Order of operations"].
    chunk == C : causal large chunks of C tokens (the last may be shorter); each
                 chunk first reads the weights left by the earlier chunks, then
                 takes its own step [LaCT "Order of operations"].
    Returns (O [B, H, N, d], W_final list of [B, H, in, out]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if chunk < 0:
        raise ValueError("chunk must be >= 0")
    if chunk > 0 and key_norm:
        raise ValueError("key instance norm over the whole sequence would read "
                         "future keys in causal chunked mode")
    nm = n_matrices(inner)
    if len(W0) != nm:
        raise ValueError(f"{inner} needs {nm} matrices, got {len(W0)}")
    O = np.zeros_like(q)
    W_final = [np.zeros((B, H) + np.asarray(w).shape[-2:]) for w in W0]
    for b in range(B):
        for h in range(H):
            Wref = _pair_weights(W0, b, h)
            W = [w.copy() for w in Wref]
            Q, K, V = q[b, h], k[b, h], v[b, h]
            eta = np.full(N, float(eta_scale))
            if eta_tok is not None:
                eta = eta * np.asarray(eta_tok, dtype=np.float64)[b, h]
            Kh = key_instnorm(K, eps) if key_norm else K
            if chunk == 0:
                W, _ = inner_step(inner, loss, W, Kh, V, eta)
                if renorm:
                    W = [column_renorm(w, r) for w, r in zip(W, Wref)]
                O[b, h] = inner_forward(inner, W, Q)[0]
            else:
                for s in range(0, N, chunk):
                    e = min(s + chunk, N)
                    O[b, h, s:e] = inner_forward(inner, W, Q[s:e])[0]   # read
                    W, _ = inner_step(inner, loss, W, Kh[s:e], V[s:e], eta[s:e])
                    if renorm:
                        W = [column_renorm(w, r) for w, r in zip(W, Wref)]
            for i in range(nm):
                W_final[i][b, h] = W[i]
    return O, W_final


def oracle_readout(q, W, inner):
    """O = F_W(Q) for per-pair weights W ([B, H, in, out] each) -- step (iii)."""
    q = np.asarray(q, dtype=np.float64)
    B, H = q.shape[:2]
    O = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            O[b, h] = inner_forward(inner, [np.asarray(w, np.float64)[b, h] for w in W], q[b, h])[0]
    return O
