"""Candidate page selection in float64 (oracle; test infrastructure only).

[EKV] = "EntmaxKV: Support-Aware Decoding for Entmax Attention".

Two policies ([EKV] section 4.3):

* top-k: the k pages with the largest pooled box score (reading R7 for ties:
  larger score first, then lower logical page index; reading R8: no forced
  sink or recent pages).
* Gaussian-aware: each page's token scores for head h are modelled as
  N(mu_{h,p}, sigma_{h,p}^2); the threshold estimate tau_hat_h solves the
  distributional entmax equation (Appendix C.2, "Solving for the
  distributional threshold", Eq. (18))

      F_h(tau) = sum_p n_p E[ g_alpha(S^(p); tau) ] = 1,
      g_alpha(s; tau) = [(alpha-1) s - tau]_+^beta,

  with the closed-form expectations of the cases alpha = 2, 3/2, 4/3
  (beta = 1, 2, 3).  The page rule of Eq. (21) did not survive extraction;
  reading R10 selects every page whose pooled margin
  t_{g,p} = max_{h in g} (mu_{h,p} - tau_hat_h/(alpha-1)) / sigma_{h,p}
  reaches -z (default z = 3), ranked by margin, capped, at least one page
  (reading R11).  The pages print no worked example of Eq. (21), so the
  choice of this reading cannot be checked against them; its arithmetic is
  pinned by hand-worked cases (tests/test_oracle_pins_by_hand.py) that a
  sigma^2 divisor, a mean or minimum over heads, an undivided or dropped
  threshold, a flipped sign or a strict comparison at -z would fail.
"""

from __future__ import annotations

import numpy as np
from scipy.special import ndtr

_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


def topk_pages(U: np.ndarray, k: int) -> np.ndarray:
    """Indices (ascending) of the k largest entries of U; ties go to the
    lower index (R7).  All pages when M <= k."""
    U = np.asarray(U, dtype=np.float64)
    M = U.size
    if M <= k:
        return np.arange(M)
    order = np.lexsort((np.arange(M), -U))   # primary: U descending; then index
    return np.sort(order[:k])


def gauss_expect(m, v, beta: int):
    """E[(Y)_+^beta] for Y ~ N(m, v^2), v >= 0, beta in {1, 2, 3}.

    Integrating the truncated normal with z = m/v, Phi/phi the standard
    normal CDF/PDF:
        beta = 1:  m Phi + v phi
        beta = 2:  (m^2 + v^2) Phi + m v phi
        beta = 3:  (m^3 + 3 m v^2) Phi + v (m^2 + 2 v^2) phi
    v = 0 gives [m]_+^beta (reading R9).
    """
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(np.broadcast(m, v).shape)
    m, v = np.broadcast_arrays(m, v)
    zero = v <= 0.0
    out[zero] = np.maximum(m[zero], 0.0) ** beta
    mm, vv = m[~zero], v[~zero]
    z = mm / vv
    Phi = ndtr(z)
    phi = np.exp(-0.5 * z * z) * _INV_SQRT_2PI
    if beta == 1:
        e = mm * Phi + vv * phi
    elif beta == 2:
        e = (mm * mm + vv * vv) * Phi + mm * vv * phi
    elif beta == 3:
        e = (mm ** 3 + 3.0 * mm * vv * vv) * Phi + vv * (mm * mm + 2.0 * vv * vv) * phi
    else:
        raise ValueError("closed forms exist for beta in {1, 2, 3} only")
    out[~zero] = e
    return out


def _beta_int(alpha: float) -> int:
    beta = 1.0 / (alpha - 1.0)
    b = int(round(beta))
    if abs(beta - b) > 1e-9 or b not in (1, 2, 3):
        raise ValueError("Gaussian selector needs alpha in {2, 3/2, 4/3}")
    return b


def gauss_F(tau: float, mu: np.ndarray, sigma: np.ndarray, n_p: np.ndarray, alpha: float) -> float:
    """F(tau) - 1 of Eq. (18) for one head."""
    a = alpha - 1.0
    e = gauss_expect(a * mu - tau, a * sigma, _beta_int(alpha))
    return float(np.sum(n_p * e) - 1.0)


def gauss_tau_hat(mu: np.ndarray, sigma: np.ndarray, n_p: np.ndarray, alpha: float,
                  iters: int = 100) -> float:
    """tau_hat of Eq. (18) for one head by fp64 bisection.

    F is decreasing in tau.  At lo = max_p (alpha-1) mu_p - 1 the page with
    the largest mean already gives n_p E[Y_+^beta] >= n_p ([E Y]_+)^beta >= 1
    (Jensen), so F(lo) >= 1; hi starts at max_p (alpha-1)(mu_p + 10 sigma_p)
    and is widened until F(hi) <= 1.
    """
    a = alpha - 1.0
    mu = np.asarray(mu, dtype=np.float64)
    sigma = np.asarray(sigma, dtype=np.float64)
    lo = float(np.max(a * mu)) - 1.0
    hi = float(np.max(a * (mu + 10.0 * sigma)))
    if hi <= lo:
        hi = lo + 1.0
    while gauss_F(hi, mu, sigma, n_p, alpha) > 0.0:
        hi += (hi - lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if gauss_F(mid, mu, sigma, n_p, alpha) >= 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def gauss_margins(mu: np.ndarray, sigma: np.ndarray, tau_hat: np.ndarray, alpha: float) -> np.ndarray:
    """Pooled margins t_{g,p} = max_h (mu_{h,p} - theta_h) / sigma_{h,p},
    theta_h = tau_hat_h/(alpha-1), over the r heads of one group (R5, R10).
    sigma = 0: +inf when mu > theta, -inf otherwise (a token exactly at the
    threshold gets probability 0).  mu, sigma: [r][M]; tau_hat: [r]."""
    mu = np.asarray(mu, dtype=np.float64)
    sigma = np.asarray(sigma, dtype=np.float64)
    theta = np.asarray(tau_hat, dtype=np.float64)[:, None] / (alpha - 1.0)
    diff = mu - theta
    t = np.empty_like(diff)
    pos = sigma > 0.0
    t[pos] = diff[pos] / sigma[pos]
    t[~pos] = np.where(diff[~pos] > 0.0, np.inf, -np.inf)
    return t.max(axis=0)


def gauss_select(mu: np.ndarray, sigma: np.ndarray, tau_hat: np.ndarray, alpha: float,
                 z: float, cap: int) -> np.ndarray:
    """Reading R10/R11 of Eq. (21): pages with pooled margin >= -z, ranked by
    margin (ties to the lower index), at most cap of them, at least one;
    returned in ascending order."""
    t = gauss_margins(mu, sigma, tau_hat, alpha)
    M = t.size
    order = np.lexsort((np.arange(M), -t))
    count = int(np.count_nonzero(t >= -z))
    take = max(1, min(count, cap))
    return np.sort(order[:take])


def superset_pages(U: np.ndarray, tau_lo: np.ndarray, alpha: float, cap: int) -> np.ndarray:
    """Support-superset selection for one KV group ([EKV] Appendix B.2): with
    U_p an upper bound on every token score of page p (the box score) and
    tau_lo_h no larger than head h's threshold, any token j with
    (alpha-1) s_j > tau_h lies in a page with (alpha-1) U_p > tau_lo_h.  One
    page set serves the group (reading R5), so the group's threshold is the
    smallest of its heads': select every page with
    U_p > min_h tau_lo_h / (alpha-1), ranked by U (ties to the lower index),
    at most cap pages, at least one; ascending order.

    U: [M] pooled box scores; tau_lo: [r] per-head thresholds in x units."""
    U = np.asarray(U, dtype=np.float64)
    theta = float(np.min(np.asarray(tau_lo, dtype=np.float64))) / (alpha - 1.0)
    M = U.size
    order = np.lexsort((np.arange(M), -U))
    count = int(np.count_nonzero(U > theta))
    take = max(1, min(count, cap))
    return np.sort(order[:take])
