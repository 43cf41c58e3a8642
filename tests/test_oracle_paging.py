"""Pins of the oracle's paged view, page statistics and page scores.

Source: "EntmaxKV: Support-Aware Decoding for Entmax Attention", section 4.2
(per-channel page min/max; box score) and Appendix B.1 (the box score bounds
every score in its page), section 4.3 (Gaussian page moments).
"""

import numpy as np
import pytest

from oracle import paged as pg
from oracle import select as sel


def _random_paged(rng, n, G, P, d, num_phys_extra=3):
    M = pg.num_pages(n, P)
    num_phys = M + num_phys_extra
    cache = rng.normal(size=(num_phys, G, P, d))
    table = rng.permutation(num_phys)[:M]
    return cache, table


def test_gather_follows_page_table():
    rng = np.random.default_rng(1)
    n, G, P, d = 37, 2, 4, 3
    cache, table = _random_paged(rng, n, G, P, d)
    K = pg.gather_logical(cache, table, n)
    for j in range(n):
        np.testing.assert_array_equal(K[j], cache[table[j // P], :, j % P, :])


def test_stats_arithmetic_progression():
    """Keys k_j = a + b j on a full page: mean a + b (P-1)/2, population
    variance b^2 (P^2 - 1)/12, min/max at the ends."""
    P, G, d = 16, 1, 3
    a = np.array([0.5, -2.0, 3.0])
    b = np.array([1.0, 0.25, -0.5])
    K = (a[None, :] + np.arange(P)[:, None] * b[None, :])[:, None, :]
    kmin, kmax, mean, var = pg.page_stats(K, P)
    np.testing.assert_allclose(mean[0, 0], a + b * (P - 1) / 2, atol=1e-14)
    np.testing.assert_allclose(var[0, 0], b ** 2 * (P * P - 1) / 12, atol=1e-13)
    np.testing.assert_array_equal(kmin[0, 0], np.minimum(a, a + (P - 1) * b))
    np.testing.assert_array_equal(kmax[0, 0], np.maximum(a, a + (P - 1) * b))


def test_stats_partial_last_page_uses_valid_tokens_only():
    P = 16
    K = np.zeros((21, 1, 1))
    K[16:, 0, 0] = [1, 2, 3, 4, 5]         # 5 valid tokens in page 1
    kmin, kmax, mean, var = pg.page_stats(K, P)
    assert kmin[1, 0, 0] == 1 and kmax[1, 0, 0] == 5
    assert mean[1, 0, 0] == 3 and abs(var[1, 0, 0] - 2.0) < 1e-15   # (4+1+0+1+4)/5
    np.testing.assert_array_equal(pg.page_valid_counts(21, P), [16, 5])


def test_identical_keys_zero_variance():
    """Stored keys are fp32/bf16 values, so k * c sums exactly in fp64 and the
    page mean of identical keys is the key itself: variance exactly 0."""
    c = np.array([0.3, -1.2], dtype=np.float32).astype(np.float64)
    K = np.tile(c[None, None, :], (21, 1, 1))
    _, _, _, var = pg.page_stats(K, 16)
    assert np.all(var == 0.0)


@pytest.mark.parametrize("P", [1, 4, 16])
def test_box_score_bounds_every_token(P):
    rng = np.random.default_rng(3)
    n, G, d, H = 203, 2, 16, 6
    K = rng.normal(size=(n, G, d))
    q = rng.normal(size=(H, d)) * 2
    kmin, kmax, _, _ = pg.page_stats(K, P)
    u, U = pg.box_scores(q, kmin, kmax)
    s = pg.token_scores(q, K)
    M = pg.num_pages(n, P)
    for h in range(H):
        for p in range(M):
            page_max = s[h, p * P:min((p + 1) * P, n)].max()
            assert u[h, p] >= page_max - 1e-12
            if min((p + 1) * P, n) - p * P == 1:
                assert abs(u[h, p] - page_max) < 1e-12     # single-token page: exact
    r = H // G
    np.testing.assert_array_equal(U, u.reshape(G, r, M).max(axis=1))


def test_single_token_pages_reduce_topk_to_token_topk():
    rng = np.random.default_rng(4)
    n, d = 300, 8
    K = rng.normal(size=(n, 1, d))
    q = rng.normal(size=(1, d))
    kmin, kmax, _, _ = pg.page_stats(K, 1)
    _, U = pg.box_scores(q, kmin, kmax)
    s = pg.token_scores(q, K)[0]
    np.testing.assert_allclose(U[0], s, atol=1e-12)
    want = np.sort(np.argsort(-s, kind="stable")[:25])
    np.testing.assert_array_equal(sel.topk_pages(U[0], 25), want)


def test_gauss_mu_is_mean_page_score():
    """mu_{h,p} is exactly the mean of the page's token scores (linearity)."""
    rng = np.random.default_rng(5)
    n, G, d, H, P = 100, 2, 8, 4, 16
    K = rng.normal(size=(n, G, d))
    q = rng.normal(size=(H, d))
    _, _, mean, var = pg.page_stats(K, P)
    mu, sig = pg.gauss_moments(q, mean, var)
    s = pg.token_scores(q, K)
    for p in range(pg.num_pages(n, P)):
        np.testing.assert_allclose(mu[:, p], s[:, p * P:min((p + 1) * P, n)].mean(axis=1), atol=1e-12)


def test_gauss_sigma_is_score_std_for_uncorrelated_channels():
    """With Hadamard-orthogonal channel patterns the page's channels are
    exactly uncorrelated, so sigma^2 equals the population variance of the
    page's token scores."""
    P, d, H = 16, 15, 3
    Hd = np.array([[1.0]])
    while Hd.shape[0] < P:
        Hd = np.block([[Hd, Hd], [Hd, -Hd]])          # Sylvester Hadamard 16x16
    rng = np.random.default_rng(6)
    scale = rng.uniform(0.5, 2.0, size=d)
    offs = rng.normal(size=d)
    K = (offs[None, :] + Hd[:, 1:d + 1] * scale[None, :])[:, None, :]   # [16][1][15]
    q = rng.normal(size=(H, d))
    _, _, mean, var = pg.page_stats(K, P)
    mu, sig = pg.gauss_moments(q, mean, var)
    s = pg.token_scores(q, K)
    np.testing.assert_allclose(sig[:, 0], s.std(axis=1), atol=1e-12)
    np.testing.assert_allclose(mu[:, 0], s.mean(axis=1), atol=1e-12)


def test_head_group_map_consecutive():
    assert [pg.head_group(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


def test_results_independent_of_physical_placement():
    rng = np.random.default_rng(7)
    n, G, P, d = 70, 2, 16, 4
    cache, table = _random_paged(rng, n, G, P, d)
    K1 = pg.gather_logical(cache, table, n)
    perm = rng.permutation(cache.shape[0])
    cache2 = np.empty_like(cache)
    cache2[perm] = cache
    K2 = pg.gather_logical(cache2, perm[table], n)
    np.testing.assert_array_equal(K1, K2)
