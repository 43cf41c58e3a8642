"""alpha-entmax and softmax in float64 (oracle; test infrastructure only).

[EKV] = "EntmaxKV: Support-Aware Decoding for Entmax Attention".

Definition followed ([EKV] section 2.2, whose display survives only as its
left-hand side, completed from the "(alpha-1) s_i" argument of Appendix B.2
and the beta = 1/(alpha-1) case labels of Appendix C.2; reading R2):

    x_i = (alpha - 1) * s_i,    beta = 1 / (alpha - 1)
    p_i = [x_i - tau]_+ ** beta,  with tau the unique value making sum(p) = 1.

The support is S = {i : x_i > tau}; every other p_i is exactly 0.  For
alpha = 1 the transformation is softmax ([EKV] section 2.1) and the value
reported in place of tau is the log-partition log(sum(exp(s))).

Two independent ways of finding tau are kept so that they can pin each other:

* ``threshold_sort``: for beta in {1, 2}.  The logits are sorted in
  decreasing order; for every candidate support size k the equation restricted
  to the top k is solved in closed form, and the k whose solution is
  consistent with the ordering is the support size.
* ``threshold_bisect``: any beta.  Bisection on the bracket
  [max(x) - 1, max(x) - n**(1-alpha)] (the first end keeps the largest term
  at most 1, the second makes every term at most 1/n), followed for
  beta in {1, 2} by the closed form on the support it found.
"""

from __future__ import annotations

import numpy as np


def beta_of(alpha: float) -> float:
    """Exponent 1/(alpha-1) of the entmax mapping ([EKV] Appendix C.2 case labels)."""
    if not alpha > 1.0:
        raise ValueError("entmax exponent needs alpha > 1")
    return 1.0 / (alpha - 1.0)


def _is_int_beta(beta: float, value: int) -> bool:
    return abs(beta - value) < 1e-12


def closed_form_tau(xs_top: np.ndarray, beta: float) -> float:
    """tau solving sum_{i in S} (x_i - tau)**beta = 1 for a given support S.

    beta = 1:  tau = (sum x - 1) / k.
    beta = 2:  sum (x - tau)^2 = V + k (m - tau)^2 = 1 with m the mean and
               V the centred sum of squares, so tau = m - sqrt((1 - V)/k);
               returns nan when V > 1 (no real root: S cannot be the support).
    """
    xs_top = np.asarray(xs_top, dtype=np.float64)
    k = xs_top.size
    if _is_int_beta(beta, 1):
        return float((xs_top.sum() - 1.0) / k)
    if _is_int_beta(beta, 2):
        m = xs_top.mean()
        v = float(np.sum((xs_top - m) ** 2))
        if v > 1.0:
            return float("nan")
        return float(m - np.sqrt((1.0 - v) / k))
    raise ValueError("closed form only for beta in {1, 2}")


def threshold_sort(x: np.ndarray, alpha: float) -> tuple[float, int]:
    """Exact tau and support size by scanning support sizes (beta in {1, 2}).

    The support size k* is the one k for which the closed-form tau_k of the
    top-k logits satisfies x_(k) > tau_k >= x_(k+1) (x_(n+1) = -inf).
    """
    beta = beta_of(alpha)
    xs = np.sort(np.asarray(x, dtype=np.float64))[::-1]
    xs = xs[np.isfinite(xs)]
    n = xs.size
    if n == 0:
        raise ValueError("entmax of an empty set is undefined")
    found = None
    for k in range(1, n + 1):
        tau = closed_form_tau(xs[:k], beta)
        if not np.isfinite(tau):
            continue
        nxt = xs[k] if k < n else -np.inf
        if xs[k - 1] > tau >= nxt:
            found = (tau, k)
            break
    if found is None:
        raise RuntimeError("no consistent support size found")
    return found


def _objective(x: np.ndarray, tau: float, beta: float) -> float:
    return float(np.sum(np.maximum(x - tau, 0.0) ** beta) - 1.0)


def threshold_bisect(x: np.ndarray, alpha: float, iters: int = 100) -> tuple[float, int]:
    """tau by bisection on sum [x - tau]_+^beta = 1, then the closed form on
    the support found when beta is 1 or 2.  Returns (tau, support size)."""
    beta = beta_of(alpha)
    x = np.asarray(x, dtype=np.float64)
    x = x[np.isfinite(x)]
    n = x.size
    if n == 0:
        raise ValueError("entmax of an empty set is undefined")
    xmax = float(x.max())
    lo = xmax - 1.0
    hi = xmax - float(n) ** (1.0 - alpha)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if _objective(x, mid, beta) >= 0.0:
            lo = mid
        else:
            hi = mid
    tau = 0.5 * (lo + hi)
    if _is_int_beta(beta, 1) or _is_int_beta(beta, 2):
        sup = x[x > lo]
        tau_cf = closed_form_tau(sup, beta)
        if np.isfinite(tau_cf) and sup.min() > tau_cf:
            rest = x[x <= lo]
            if rest.size == 0 or tau_cf >= rest.max():
                tau = tau_cf
    return tau, int(np.count_nonzero(x > tau))


def entmax(s: np.ndarray, alpha: float, method: str = "auto"):
    """alpha-entmax of one score vector.

    Returns (p, tau, support_size).  tau is in the units of x = (alpha-1) s;
    for alpha = 1 the result is softmax and tau is log(sum(exp(s))).
    Non-finite scores (-inf marks an invalid slot) get probability 0.
    """
    s = np.asarray(s, dtype=np.float64)
    if alpha == 1.0:
        p, lse = softmax(s)
        return p, lse, int(np.count_nonzero(p > 0))
    beta = beta_of(alpha)
    x = (alpha - 1.0) * s
    if method == "auto":
        method = "sort" if (_is_int_beta(beta, 1) or _is_int_beta(beta, 2)) else "bisect"
    if method == "sort":
        tau, k = threshold_sort(x, alpha)
    elif method == "bisect":
        tau, k = threshold_bisect(x, alpha)
    else:
        raise ValueError(method)
    p = np.zeros_like(x)
    fin = np.isfinite(x)
    p[fin] = np.maximum(x[fin] - tau, 0.0) ** beta
    return p, tau, k


def softmax(s: np.ndarray):
    """Max-shifted softmax ([EKV] section 2.1 with pi = softmax).
    Returns (p, log-partition)."""
    s = np.asarray(s, dtype=np.float64)
    fin = np.isfinite(s)
    m = s[fin].max()
    e = np.zeros_like(s)
    e[fin] = np.exp(s[fin] - m)
    z = e.sum()
    return e / z, float(m + np.log(z))
