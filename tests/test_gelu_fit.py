"""Accuracy of the packed-f16 GELU polynomials compiled into the MFMA kernels.

The coefficients are read from the kernel source and evaluated here in
emulated f16 arithmetic (each FMA rounded once, as the hardware does), in the
two forms the kernels use, against the exact GELU z * Phi(z) (scipy's erf).
This pins the error bounds the kernels' comments and the design notes state;
the GPU parity tests then check the kernels end to end.
"""
import os
import re

import numpy as np
import pytest
from scipy.special import erf

SRC = os.path.join(os.path.dirname(__file__), "..", "linear_complexity_attention_amd", "csrc", "k_mfma_full.hip")
H = np.float16


def _fit(name):
    src = open(SRC).read()
    body = re.search(r"struct %s \{(.*?)\n\};" % name, src, re.S).group(1)
    c = float(re.search(r"float c = ([0-9.]+)f;", body).group(1))
    coef = lambda k: [float(x.rstrip("f")) for x in re.search(r"float %s\[\d+\] = \{([^}]*)\};" % k, body).group(1).split(",")]
    return c, coef("P"), coef("Q")


def _fma(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(H)


def _horner(co, v, scale):
    acc = np.full_like(v, H(co[-1] * scale))
    for k in range(len(co) - 2, -1, -1):
        acc = _fma(acc, v, H(co[k] * scale))
    return acc


def _cdf(z):
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def _pdf(z):
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def _all_f16():
    x = np.arange(65536, dtype=np.uint16).view(H)
    return x[np.isfinite(x)]


def test_gradient_fit_input_clamped():
    """c Phi = c/2 + w P(v)/sqrt2 and gelu' = 1/2 + w Q(v)/sqrt2 with w = clamp(zh, +-sqrt2)."""
    c, P, Q = _fit("GeluFitG")
    r2 = np.sqrt(0.5)
    zh = _all_f16()
    z = zh.astype(np.float64) * c / np.sqrt(2.0)
    w = np.clip(zh, H(-np.sqrt(2.0)), H(np.sqrt(2.0)))
    v = _fma(w, w, H(-1.0))
    cphi = _fma(w, _horner(P, v, r2), H(c / 2.0))
    with np.errstate(over="ignore"):                  # A' overflows f16 for the largest zh
        a = (zh.astype(np.float64) * cphi.astype(np.float64)).astype(H).astype(np.float64) * r2   # = gelu
    gelu = z * _cdf(z)
    inner = np.abs(z) <= 4.0
    assert np.abs(a - gelu)[inner].max() < 6.0e-3
    # beyond |Z| = 4 the clamped Phi is within 1e-3 of 0 or 1: error relative to |Z|
    # (up to |Z| = 1e4; A' = sqrt(2) gelu(Z) leaves the f16 range near 4.6e4)
    outer = ~inner & (np.abs(z) <= 1.0e4)
    assert (np.abs(a - gelu)[outer] / np.abs(z[outer])).max() < 1.5e-3
    gp = _fma(w, _horner(Q, v, r2), H(0.5)).astype(np.float64)
    assert np.abs(gp - (_cdf(z) + z * _pdf(z))).max() < 2.6e-3


def test_readout_fit_output_clamped():
    """Phi = clamp01(1/2 + zh P(zh^2 - 1)/(sqrt2 c)) on the unclamped zh, every finite f16 zh."""
    c, P, _ = _fit("GeluFit4")
    zh = _all_f16()
    z = zh.astype(np.float64) * c / np.sqrt(2.0)
    with np.errstate(over="ignore", invalid="ignore"):
        v = _fma(zh, zh, H(-1.0))
        phi = _fma(zh, _horner(P, v, np.sqrt(0.5) / c), H(0.5)).astype(np.float64)
    assert not np.isnan(phi).any()
    phi = np.clip(phi, 0.0, 1.0)
    # outside a small interval Phi is exactly 0 or 1, with the sign of Z
    far = np.abs(z) > 3.5
    assert np.array_equal(phi[far], (z[far] > 0).astype(np.float64))
    a = (zh.astype(np.float64) * phi).astype(H).astype(np.float64) * c / np.sqrt(2.0)
    gelu = z * _cdf(z)
    assert (np.abs(a - gelu) - np.abs(gelu) * 2.0 ** -11).max() < 3.0e-3


@pytest.mark.parametrize("name", ["GeluFitG", "GeluFit4"])
def test_fit_constants_match_the_fitting_script(name):
    """The compiled coefficients are the ones fit_gelu.py derives (to the printed digits)."""
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", "linear_complexity_attention_amd"))
    import fit_gelu
    c, P, Q = _fit(name)
    Pf, Qf = fit_gelu.fits(c, len(P) - 1, len(Q) - 1 if name == "GeluFitG" else None)
    assert np.allclose(P, Pf, rtol=0, atol=2e-6)
    if name == "GeluFitG":
        assert np.allclose(Q, Qf, rtol=0, atol=2e-6)
