"""Paged KV view, page statistics and page scores in float64 (oracle; test
infrastructure only).

[EKV] = "EntmaxKV: Support-Aware Decoding for Entmax Attention".

Notation: P tokens per page, G key/value groups, H query heads, r = H/G,
head h reads group g(h) = floor(h / r) (reading R1, the usual GQA repeat of
"EntroPrefill" section 2.1 Eq. (1)).  A sequence of n tokens has
M = ceil(n / P) logical pages; page p holds the valid tokens
J_p = [p P, min((p+1) P, n)), n_p = |J_p|.
"""

from __future__ import annotations

import numpy as np


def num_pages(n: int, page_size: int) -> int:
    return (int(n) + page_size - 1) // page_size


def gather_logical(cache: np.ndarray, page_table_row: np.ndarray, n: int) -> np.ndarray:
    """Logical-order view [n][G][d] of one sequence of a paged cache
    [num_phys][G][P][d] (the paged layout of [EKV] section 4, after
    PagedAttention: logical page p lives in physical page page_table_row[p])."""
    num_phys, G, P, d = cache.shape
    M = num_pages(n, P)
    phys = np.asarray(page_table_row[:M], dtype=np.int64)
    tiles = np.asarray(cache[phys], dtype=np.float64)       # [M][G][P][d]
    tok = tiles.transpose(0, 2, 1, 3).reshape(M * P, G, d)  # [M*P][G][d]
    return tok[:n]


def head_group(h: int, num_q_heads: int, num_groups: int) -> int:
    """g(h) = floor(h / r), r = H/G (reading R1)."""
    r = num_q_heads // num_groups
    return h // r


def page_stats(K: np.ndarray, page_size: int):
    """Per page, group and channel: min, max, mean and population variance of
    the keys over the page's valid tokens ([EKV] section 4.2 and Appendix
    B.1 for min/max; mean/variance are the per-page statistics the Gaussian
    selector of section 4.3 reads; divisor n_p, reading R3).

    K: [n][G][d].  Returns four arrays [M][G][d].
    """
    K = np.asarray(K, dtype=np.float64)
    n, G, d = K.shape
    M = num_pages(n, page_size)
    kmin = np.empty((M, G, d))
    kmax = np.empty((M, G, d))
    mean = np.empty((M, G, d))
    var = np.empty((M, G, d))
    for p in range(M):
        tile = K[p * page_size:min((p + 1) * page_size, n)]  # [n_p][G][d]
        kmin[p] = tile.min(axis=0)
        kmax[p] = tile.max(axis=0)
        mu = tile.mean(axis=0)
        mean[p] = mu
        var[p] = ((tile - mu) ** 2).mean(axis=0)
    return kmin, kmax, mean, var


def round_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest value of the 8-bit float format E4M3 of the OCP 8-bit floating
    point specification (1 sign bit; 4 exponent bits, bias 7; 3 mantissa bits;
    subnormal step 2^-9 below 2^-6; no infinities; largest finite 448), ties
    to the even mantissa.  Finite magnitudes beyond 448 become 448 (the
    storage reading for page mean/variance kept in this format, an option in
    the spirit of R4); NaN stays NaN.

    Written from the format definition: within the binade [2^e, 2^(e+1)),
    e >= -6, the representable values are multiples of 2^(e-3); below 2^-6
    they are multiples of 2^-9.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3)
    with np.errstate(invalid="ignore"):
        v = np.minimum(np.round(a / step) * step, 448.0)   # np.round: half to even
    return np.where(np.isnan(x), np.nan, np.copysign(v, x))


def page_valid_counts(n: int, page_size: int) -> np.ndarray:
    """n_p for every logical page of a sequence of n tokens."""
    M = num_pages(n, page_size)
    counts = np.full(M, page_size, dtype=np.int64)
    if M and n % page_size:
        counts[-1] = n % page_size
    return counts


def box_scores(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray):
    """Quest-style box bound ([EKV] section 4.2 and Appendix B.1):

        u_{h,p} = (1/sqrt(d)) sum_i max(q_{h,i} kmax_{p,i}, q_{h,i} kmin_{p,i}),

    the largest q.k/sqrt(d) over the axis-aligned box spanned by the page's
    keys, hence an upper bound on every token score in the page.  Pooled per
    group by the maximum over its r heads (reading R5).

    q: [H][d]; kmin, kmax: [M][G][d].  Returns (u [H][M], U [G][M]).
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    M, G, _ = kmin.shape
    r = H // G
    u = np.empty((H, M))
    for h in range(H):
        g = h // r
        a = q[h][None, :] * kmax[:, g, :]
        b = q[h][None, :] * kmin[:, g, :]
        u[h] = np.maximum(a, b).sum(axis=1) / np.sqrt(d)
    U = u.reshape(G, r, M).max(axis=1)
    return u, U


def gauss_moments(q: np.ndarray, mean: np.ndarray, var: np.ndarray):
    """Per-head score moments of each page for the Gaussian selector ([EKV]
    section 4.3, "score moments per head" of section 4.4), diagonal model
    (reading R6):

        mu_{h,p}    = (1/sqrt(d)) sum_i q_{h,i} mean_{p,i}
        sigma2_{h,p} = (1/d)      sum_i q_{h,i}^2 var_{p,i}

    mu is exactly the mean of the page's token scores; sigma^2 is their
    variance when the channels of the page's keys are uncorrelated.
    Returns (mu [H][M], sigma [H][M]).
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    M, G, _ = mean.shape
    r = H // G
    mu = np.empty((H, M))
    sig = np.empty((H, M))
    for h in range(H):
        g = h // r
        mu[h] = mean[:, g, :] @ q[h] / np.sqrt(d)
        sig[h] = np.sqrt(var[:, g, :] @ (q[h] ** 2) / d)
    return mu, sig


def token_scores(q: np.ndarray, K: np.ndarray, tokens: np.ndarray | None = None):
    """s_{h,j} = q_h . k_{g(h), j} / sqrt(d) ([EKV] section 2.1).
    q: [H][d]; K: [n][G][d]; tokens: optional index array.  Returns [H][len]."""
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    Kt = np.asarray(K if tokens is None else K[tokens], dtype=np.float64)
    G = Kt.shape[1]
    r = H // G
    s = np.empty((H, Kt.shape[0]))
    for h in range(H):
        s[h] = Kt[:, h // r, :] @ q[h] / np.sqrt(d)
    return s
