"""Coefficients of exp2_poly.h: the minimax polynomial (relative error) of
2^f on [-1/2, 1/2], by the Remez exchange algorithm.

python gen_exp2_poly.py [degree]   prints the coefficients c0..cn (rounded to
fp32) and the maximum relative error of the fp32-rounded polynomial in exact
arithmetic on a dense grid.
"""

import sys

import numpy as np


def remez(n, a=-0.5, b=0.5, iters=40, grid=200001):
    """Degree-n polynomial p minimising max |p(f) - 2^f| / 2^f on [a, b]."""
    x = (a + b) / 2 + (b - a) / 2 * np.cos(np.pi * np.arange(n + 2) / (n + 1))[::-1]  # Chebyshev extrema
    g = np.linspace(a, b, grid)
    c = None
    for _ in range(iters):
        # p(x_i) - 2^x_i = (-1)^i E 2^x_i on the reference points
        A = np.zeros((n + 2, n + 2))
        for i, xi in enumerate(x):
            A[i, :n + 1] = xi ** np.arange(n + 1)
            A[i, n + 1] = -((-1) ** i) * 2.0 ** xi
        sol = np.linalg.solve(A, 2.0 ** x)
        c = sol[:n + 1]
        err = (np.polyval(c[::-1], g) - 2.0 ** g) / 2.0 ** g
        # new reference: the largest |err| between consecutive sign changes
        ext, start = [], 0
        sign = np.sign(err)
        for j in range(1, len(g)):
            if sign[j] != sign[j - 1]:
                ext.append(start + int(np.argmax(np.abs(err[start:j]))))
                start = j
        ext.append(start + int(np.argmax(np.abs(err[start:]))))
        if len(ext) != n + 2:
            break
        x = g[ext]
    return c


def main():
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 3
    c = np.float32(remez(n)).astype(np.float64)
    g = np.linspace(-0.5, 0.5, 400001)
    err = np.abs(np.polyval(c[::-1], g) - 2.0 ** g) / 2.0 ** g
    for i, ci in enumerate(c):
        print("c%d = %.17gf" % (i, ci))
    print("max relative error (fp32 coefficients, exact arithmetic): %.3g" % err.max())


if __name__ == "__main__":
    main()
