"""Derive the packed-f16 GELU polynomials of the MLP MFMA kernels.

With a clamp point c, zh = sqrt(2) Z / c, w = clamp(zh, -sqrt(2), sqrt(2)) and
v = w^2 - 1, the kernels evaluate
    c Phi(Z) = c/2 + w P(v) / sqrt(2)      gelu'(Z) = 1/2 + w Q(v) / sqrt(2)
in f16 Horner form.  P and Q are Lawson (iteratively reweighted least squares,
converging to minimax) fits on v in [-1, 1]; the errors printed here are those
of the f16 evaluation the kernels perform (fma in one rounding, RNE
conversions), over Z in [-4, 4].
The readout evaluates the same P on the unclamped zh and clamps the output:
    Phi(Z) = clamp01(1/2 + zh P(zh^2 - 1) / (sqrt(2) c)),   A = zh Phi(Z).
For that form the error is taken over every finite f16 value of zh (the part
beyond the f16 rounding of the result, relative 2^-11), and the values that
do not clamp and the NaN results are counted.  Run: python fit_gelu.py
"""
import numpy as np
from scipy.special import erf


def cdf(z):
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def pdf(z):
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def lawson(fun, deg, weight):
    u = (np.cos(np.linspace(0.0, np.pi, 6000)) + 1.0) / 2.0     # w0^2 on Chebyshev nodes
    w0 = np.sqrt(u)
    w0[w0 == 0.0] = 1e-9
    f, v = fun(w0), 2.0 * u - 1.0
    V = np.vander(v, deg + 1, increasing=True)
    wt = np.ones_like(u)
    for _ in range(100):
        co = np.linalg.lstsq(V * np.sqrt(wt)[:, None], f * np.sqrt(wt), rcond=None)[0]
        wt = wt * (np.abs(V @ co - f) * w0 * weight + 1e-30)
        wt /= wt.sum()
    return co


def f16_errors(c, P, Q=None):
    h = np.float16
    fma = lambda a, b, cc: (a.astype(np.float64) * b.astype(np.float64) + np.float64(cc)).astype(h)
    r2 = np.sqrt(0.5)
    z = np.linspace(-4.0, 4.0, 400001)
    zh = (np.sqrt(2.0) / c * z).astype(np.float32).astype(h)
    w = np.clip(zh, h(-np.sqrt(2.0)), h(np.sqrt(2.0)))
    v = fma(w, w, h(-1.0))

    def horner(co):
        acc = np.full_like(v, h(co[-1] * r2))
        for k in range(len(co) - 2, -1, -1):
            acc = fma(acc, v, h(co[k] * r2))
        return acc
    cphi = fma(w, horner(P), h(c / 2.0))
    a = (zh.astype(np.float64) * cphi.astype(np.float64)).astype(h).astype(np.float64) * r2
    err_a = np.abs(a - z * cdf(z)).max()
    err_g = None
    if Q is not None:
        gp = fma(w, horner(Q), h(0.5)).astype(np.float64)
        err_g = np.abs(gp - (cdf(z) + z * pdf(z))).max()
    return err_a, err_g


def f16_errors_out_clamp(c, P):
    h = np.float16
    fma = lambda a, b, cc: (a.astype(np.float64) * b.astype(np.float64) + np.float64(cc)).astype(h)
    zh = np.arange(65536, dtype=np.uint16).view(h)
    zh = zh[np.isfinite(zh)]                           # every finite f16 zh
    z = zh.astype(np.float64) * c / np.sqrt(2.0)
    s = np.sqrt(0.5) / c
    with np.errstate(over="ignore", invalid="ignore"):
        v = fma(zh, zh, h(-1.0))                       # +inf for |zh| > 256
        acc = np.full_like(v, h(P[-1] * s))
        for k in range(len(P) - 2, -1, -1):
            acc = fma(acc, v, h(P[k] * s))
        phi = fma(zh, acc, h(0.5)).astype(np.float64)
    n_nan = int(np.isnan(phi).sum())
    z_open = np.abs(z[(phi > 0.0) & (phi < 1.0)]).max()  # beyond it Phi is exactly 0 or 1
    phi = np.clip(phi, 0.0, 1.0)
    a = (zh.astype(np.float64) * phi).astype(h).astype(np.float64) * c / np.sqrt(2.0)
    g = z * cdf(z)
    return (np.abs(a - g) - np.abs(g) * 2.0 ** -11).max(), z_open, n_nan


def fits(c, deg_p, deg_q=None):
    P = lawson(lambda w0: (c * cdf(c * w0) - c / 2.0) / w0, deg_p, c)
    Q = None if deg_q is None else lawson(lambda w0: (cdf(c * w0) + c * w0 * pdf(c * w0) - 0.5) / w0, deg_q, 1.0)
    return P, Q


if __name__ == "__main__":
    for name, c, dp, dq in (("GeluFitG (gradient)", 3.5, 4, 5), ("GeluFit4 (readout)", 3.125, 4, None)):
        P, Q = fits(c, dp, dq)
        ea, eg = f16_errors(c, P, Q)
        print(f"{name}: c = {c}")
        print("  P =", np.array2string(P, precision=9, separator=", "))
        if Q is not None:
            print("  Q =", np.array2string(Q, precision=9, separator=", "))
        print(f"  max |error| gelu {ea:.2e}" + ("" if eg is None else f", gelu' {eg:.2e}"))
        if Q is None:
            eo, zo, nn = f16_errors_out_clamp(c, P)
            print(f"  output-clamped form: max |error| gelu {eo:.2e} beyond the result's rounding,"
                  f" Phi exactly 0 or 1 for |Z| > {zo:.3f}, NaN results: {nn}")
