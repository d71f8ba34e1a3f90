"""Coefficients of gelu16 (device_common.hpp): a degree-5 polynomial Q(s) with

    erfc(z) ~= 2 s 2^(Q(s) - log2(e) z^2),   s = 1 / (2 + z),   z >= 0,

fitted (Lawson-reweighted least squares, which converges to the minimax fit) to
ln(erfc(z) / t) + z^2 in t = 2 s over Chebyshev nodes of t in (0, 1], then moved to
base 2 and to s. Run with numpy and scipy: prints the coefficients (highest
degree first, as the kernel evaluates them) and the fit's erfc relative error.
Not used at run time; the kernel carries the printed constants."""
import numpy as np
from scipy.special import erfcx

LOG2E = 1.0 / np.log(2.0)


def g(t):
    z = 2.0 * (1.0 / t - 1.0)
    return np.log(erfcx(z)) - np.log(t)  # ln(erfc(z) / t) + z^2


def fit(deg=5, nodes=6000, rounds=300):
    x = np.clip(0.5 * (1 - np.cos(np.pi * (np.arange(nodes) + 0.5) / nodes)), 1e-7, 1.0)
    y = g(x)
    V = np.vander(x, deg + 1, increasing=True)
    w = np.ones_like(x)
    for _ in range(rounds):
        c, *_ = np.linalg.lstsq(V * np.sqrt(w)[:, None], y * np.sqrt(w), rcond=None)
        w = w * (np.abs(V @ c - y) + 1e-30)
        w /= w.sum()
    return (LOG2E * c * 2.0 ** np.arange(deg + 1)).astype(np.float32)


if __name__ == "__main__":
    cs = fit()
    t = np.linspace(1e-7, 1.0, 400001)
    err = np.max(np.abs(np.polyval(cs.astype(np.float64)[::-1], t / 2) - LOG2E * g(t))) / LOG2E
    print("Q, highest degree first:", ", ".join(f"{v:.9g}" for v in cs[::-1]))
    print(f"erfc relative error {err:.2e}")
