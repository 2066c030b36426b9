"""Coefficients of the polynomial SiLU used by the bf16 attention kernel.

With x' = log2(e) * x, the kernel needs g(x') = log2(e) * SiLU(x) =
x' / (1 + 2^-x'). Its odd part is x'/2 and its even part is a smooth function
of y = x'^2, so on |x| <= R

    g(x') ~= 0.5 x' + y * (c0 + c1 y + c2 y^2).

The coefficients are a y-weighted least-squares fit on Chebyshev nodes of
y in [0, (R log2 e)^2] (R = 2). Running this script prints them, the
maximum absolute error of g on a dense grid (about 3.3e-4) and the largest
relative error where |g| > 0.05 (about 1.1e-3, below the bf16 half-ulp of
2^-9 that the kernel rounds the result to). A cubic (deg=3) reaches 2.8e-5
for one more FMA per score.
"""
import numpy as np

R = 2.0
L = 1.0 / np.log(2.0)


def g_exact(xp):
    return xp / (1.0 + np.exp2(-xp))


def fit(deg=2, R=R):
    Rp = R * L
    yc = (np.cos(np.linspace(0.0, np.pi, 400)) + 1.0) / 2.0 * Rp * Rp
    xc = np.sqrt(yc)
    with np.errstate(invalid="ignore", divide="ignore"):
        tc = (g_exact(xc) - 0.5 * xc) / yc
    tc[yc < 1e-12] = 0.25 / L  # limit of (g - x'/2) / x'^2 at 0
    return np.polynomial.polynomial.polyfit(yc, tc, deg, w=yc)


if __name__ == "__main__":
    c = fit()
    xs = np.linspace(-R * L, R * L, 200001)
    y = xs * xs
    g = 0.5 * xs + y * np.polynomial.polynomial.polyval(y, c)
    print("coefficients c0..c%d:" % (len(c) - 1), ", ".join(f"{v:.9e}f" for v in c))
    err = np.abs(g - g_exact(xs))
    big = np.abs(g_exact(xs)) > 0.05
    print("max |g - g_exact| on |x| <= R:", err.max())
    print("max relative error where |g| > 0.05:", (err[big] / np.abs(g_exact(xs))[big]).max())
