"""Fit the coefficients of the FMA-polynomial exp2 used by the forward kernel.

The explainer pages on FlashAttention-4 (gist.science technical summary,
methodology item 2) replace part of the hardware exponentials by a degree 3
or 5 polynomial evaluated with FMAs, accurate to bf16 precision.  They give
no coefficients, so this script derives them:

  2^x = 2^n * 2^f,  n = floor(x),  f = x - n in [0, 1)
  2^f ~ p(f) = 1 + c1 f + ... + cD f^D

with p(0) = 1 pinned (integer x is then exact) and c1..cD chosen to minimise
the maximum relative error  max_f |p(f) / 2^f - 1|  over a dense grid of
[0, 1].  That minimax problem is a linear program in (c1..cD, t):

  minimise t  subject to  -t <= (1 + sum_k c_k f^k) 2^-f - 1 <= t.

Run it to print the coefficients pasted into exp2_poly.h and the error each
set reaches in exact arithmetic.
"""
import numpy as np
from scipy.optimize import linprog


def fit(degree: int, npts: int = 4001):
    f = np.linspace(0.0, 1.0, npts)
    w = 2.0 ** -f
    # variables: c1..cD, t
    cols = [w * f ** k for k in range(1, degree + 1)]
    A = np.stack(cols, axis=1)
    ones = np.ones((npts, 1))
    # (1 + A c) w - 1 <= t   ->  A c - t <= 1 - w
    # -(1 + A c) w + 1 <= t  -> -A c - t <= w - 1
    A_ub = np.vstack([np.hstack([A, -ones]), np.hstack([-A, -ones])])
    b_ub = np.concatenate([1.0 - w, w - 1.0])
    c = np.zeros(degree + 1)
    c[-1] = 1.0
    res = linprog(c, A_ub=A_ub, b_ub=b_ub, bounds=[(None, None)] * (degree + 1), method="highs")
    assert res.success, res.message
    coef = res.x[:degree]
    ff = np.linspace(0.0, 1.0, 200001)
    p = 1.0 + sum(coef[k] * ff ** (k + 1) for k in range(degree))
    err = np.max(np.abs(p * 2.0 ** -ff - 1.0))
    return coef, err


if __name__ == "__main__":
    for deg in (3, 5):
        coef, err = fit(deg)
        print(f"degree {deg}: max relative error {err:.3e}")
        for k, cval in enumerate(coef, start=1):
            print(f"  c{k} = {np.float32(cval)!r}  ({cval:.17g})")
