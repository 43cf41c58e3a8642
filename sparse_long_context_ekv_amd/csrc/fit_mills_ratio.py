"""Coefficients of the Mills-ratio polynomial used by the Gaussian threshold
kernel (select.hip, `upper_tail`).

The standard normal upper tail is written Q(x) = phi(x) R(x) for x >= 0,
with R the Mills ratio.  With t = 1/(1 + K x), t in (0, 1], the function
h(t) = R(x)/t is smooth on [0, 1] (h(0) = K, from R(x) ~ 1/x), so a
polynomial of degree DEG in t, fitted here by weighted least squares on the
relative error at Chebyshev nodes, gives R(x) ~ t * h(t) over all x >= 0.
R is evaluated in float64 through the scaled complementary error function,
R(x) = sqrt(pi/2) erfcx(x / sqrt(2)).

    python fit_mills_ratio.py      # prints the C table and its error bounds
"""

import numpy as np
from scipy.special import erfcx

K = 0.4
DEG = 11


def mills(x):
    return np.sqrt(np.pi / 2.0) * erfcx(x / np.sqrt(2.0))


def fit(k=K, deg=DEG, nodes=4000):
    t = 0.5 * (1.0 - np.cos(np.pi * (np.arange(nodes) + 0.5) / nodes))
    t = t[t > 1e-6]
    h = mills((1.0 / t - 1.0) / k) / t
    a = np.vander(t, deg + 1, increasing=True) / h[:, None]
    c, *_ = np.linalg.lstsq(a, np.ones_like(t), rcond=None)
    return c


def max_rel_error(c, k=K, dtype=np.float64):
    x = np.concatenate([np.linspace(0.0, 12.0, 200001), np.linspace(12.0, 40.0, 2001)]).astype(dtype)
    t = (dtype(1) / (dtype(1) + dtype(k) * x)).astype(dtype)
    p = np.zeros_like(t)
    for ci in np.asarray(c, dtype=dtype)[::-1]:
        p = (p * t + ci).astype(dtype)
    return float(np.max(np.abs((p * t).astype(np.float64) / mills(x.astype(np.float64)) - 1.0)))


if __name__ == "__main__":
    c = fit()
    print(f"// t = 1/(1 + {K}f x); R(x) ~ t * sum_i c[i] t^i  (degree {DEG})")
    print(f"// max relative error of R: {max_rel_error(c):.2e} (float64 Horner), "
          f"{max_rel_error(c, dtype=np.float32):.2e} (float32 Horner)")
    print("constexpr float kMillsC[%d] = {" % (DEG + 1))
    print(",\n".join("    %.9ef" % v for v in np.float32(c)) + "};")
