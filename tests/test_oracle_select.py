"""Pins of the oracle's page selection: top-k and the Gaussian-aware selector.

Source: "EntmaxKV: Support-Aware Decoding for Entmax Attention", section 4.3
(top-k and Gaussian-aware policies) and Appendix C.2 (closed-form
expectations for alpha = 2, 3/2, 4/3 and the distributional threshold
equation, Eq. (18)).
"""

import os

import numpy as np
import pytest
from scipy.integrate import quad

from oracle import entmax as em
from oracle import paged as pg
from oracle import select as sel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split(";")]


def test_topk_ties_prefer_lower_index():
    U = np.array([3, 1, 3, 2, 3, 2, 0], dtype=float)
    np.testing.assert_array_equal(sel.topk_pages(U, 2), [0, 2])
    np.testing.assert_array_equal(sel.topk_pages(U, 4), [0, 2, 3, 4])
    np.testing.assert_array_equal(sel.topk_pages(U, 10), np.arange(7))


def test_topk_brute_force():
    rng = np.random.default_rng(2)
    for _ in range(200):
        M = int(rng.integers(1, 40))
        k = int(rng.integers(1, 45))
        U = rng.integers(0, 6, size=M).astype(float)     # many ties
        got = sel.topk_pages(U, k)
        assert list(got) == sorted(got)
        assert len(got) == min(k, M)
        chosen = set(got.tolist())
        for i in range(M):
            for j in range(M):
                if i in chosen and j not in chosen:
                    # every kept page beats every dropped one, ties to the lower index
                    assert U[i] > U[j] or (U[i] == U[j] and i < j)


@pytest.mark.parametrize("row", list(_rows("gauss_moments.txt")))
def test_gauss_moments_golden(row):
    beta, m, v = int(row[0]), float(row[1]), float(row[2])
    want = eval(row[3])
    got = float(sel.gauss_expect(m, v, beta))
    assert abs(got - want) < 1e-14 * max(1.0, abs(want))


@pytest.mark.parametrize("beta", [1, 2, 3])
def test_gauss_closed_forms_equal_quadrature(beta):
    for m, v in [(0.3, 1.0), (-1.7, 0.4), (2.5, 0.1), (-0.2, 3.0), (1.0, 2.0), (-4.0, 1.0)]:
        f = lambda y: max(y, 0.0) ** beta * np.exp(-0.5 * ((y - m) / v) ** 2) / (v * np.sqrt(2 * np.pi))  # noqa: E731
        ref, _ = quad(f, 0.0, m + 40 * v, epsabs=1e-15, epsrel=1e-13, limit=400)
        got = float(sel.gauss_expect(m, v, beta))
        assert abs(got - ref) <= 1e-11 * max(1.0, abs(ref))


def _paged_scores(K, q, P):
    _, _, mean, var = pg.page_stats(K, P)
    return pg.gauss_moments(q, mean, var)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 4.0 / 3.0])
def test_eq18_single_token_pages_is_exact_entmax(alpha):
    """With P = 1 every page is one token (sigma = 0, n_p = 1): Eq. (18) is
    the entmax threshold equation itself."""
    rng = np.random.default_rng(8)
    n, d = 500, 16
    K = rng.normal(size=(n, 1, d))
    q = rng.normal(size=(1, d)) * 2
    mu, sig = _paged_scores(K, q, 1)
    assert np.all(sig == 0.0)
    tau_hat = sel.gauss_tau_hat(mu[0], sig[0], np.ones(n), alpha)
    _, tau, _ = em.entmax(pg.token_scores(q, K)[0], alpha)
    assert abs(tau_hat - tau) < 1e-12


def test_eq18_identical_keys_in_each_page_is_exact_entmax():
    """All keys of a page identical: sigma = 0 and E = n_p [m]_+^beta, so
    tau_hat equals the exact threshold over all tokens (including a partial
    last page)."""
    rng = np.random.default_rng(9)
    P, M, d = 16, 40, 8
    base = rng.normal(size=(M, 1, d)).astype(np.float32).astype(np.float64)
    K = np.repeat(base, P, axis=0)[: M * P - 7]            # last page has 9 tokens
    q = (rng.normal(size=(1, d)) * 3).astype(np.float32).astype(np.float64)
    mu, sig = _paged_scores(K, q, P)
    assert np.all(sig == 0.0)
    n_p = pg.page_valid_counts(K.shape[0], P)
    tau_hat = sel.gauss_tau_hat(mu[0], sig[0], n_p, 1.5)
    _, tau, _ = em.entmax(pg.token_scores(q, K)[0], 1.5)
    assert abs(tau_hat - tau) < 1e-11


@pytest.mark.parametrize("alpha", [1.5, 2.0, 4.0 / 3.0])
def test_eq18_residual(alpha):
    rng = np.random.default_rng(10)
    mu = rng.normal(size=800) * 0.5
    sig = rng.uniform(0.0, 1.5, size=800)
    sig[::7] = 0.0
    n_p = np.full(800, 16)
    n_p[-1] = 5
    tau_hat = sel.gauss_tau_hat(mu, sig, n_p, alpha)
    assert abs(sel.gauss_F(tau_hat, mu, sig, n_p, alpha)) < 1e-10


def test_gauss_tau_hat_moves_with_variance():
    """More spread per page puts more expected mass above any threshold, so
    the estimate rises (F increasing in sigma for fixed tau)."""
    mu = np.zeros(100)
    n_p = np.full(100, 16)
    t_small = sel.gauss_tau_hat(mu, np.full(100, 0.2), n_p, 1.5)
    t_large = sel.gauss_tau_hat(mu, np.full(100, 1.0), n_p, 1.5)
    assert t_large > t_small


def test_gauss_select_invariants():
    rng = np.random.default_rng(12)
    r, M = 4, 300
    mu = rng.normal(size=(r, M))
    sig = rng.uniform(0.05, 1.0, size=(r, M))
    n_p = np.full(M, 16)
    tau_hat = np.array([sel.gauss_tau_hat(mu[h], sig[h], n_p, 1.5) for h in range(r)])
    t = sel.gauss_margins(mu, sig, tau_hat, 1.5)
    prev = None
    for z in (0.5, 1.0, 2.0, 3.0, 5.0):
        s = sel.gauss_select(mu, sig, tau_hat, 1.5, z, cap=M)
        assert list(s) == sorted(s) and len(s) >= 1
        np.testing.assert_array_equal(s, np.flatnonzero(t >= -z) if np.any(t >= -z) else s)
        if prev is not None:
            assert set(prev) <= set(s)                   # larger z: superset
        prev = s
    capped = sel.gauss_select(mu, sig, tau_hat, 1.5, 5.0, cap=17)
    assert len(capped) == 17
    kept_min = t[capped].min()
    dropped = np.setdiff1d(np.arange(M), capped)
    assert np.all(t[dropped] <= kept_min)               # the cap keeps the largest margins
    everything = sel.gauss_select(mu, sig, tau_hat, 1.5, 1e9, cap=M)
    np.testing.assert_array_equal(everything, np.arange(M))


def test_gauss_select_keeps_at_least_one_page():
    mu = np.array([[-5.0, -4.0, -6.0]])
    sig = np.array([[0.01, 0.01, 0.01]])
    s = sel.gauss_select(mu, sig, np.array([10.0]), 1.5, z=0.0, cap=3)
    np.testing.assert_array_equal(s, [1])


def test_gauss_margin_zero_sigma():
    mu = np.array([[1.0, 0.0, 2.0]])
    sig = np.zeros((1, 3))
    t = sel.gauss_margins(mu, sig, np.array([0.5]), 1.5)     # theta = 1.0
    assert t[0] == -np.inf and t[1] == -np.inf and t[2] == np.inf


def test_chunked_selection_equals_one_level():
    """The decomposition behind the GPU's two-level selection of long rows:
    under the order "larger key first, then lower page index", keeping the
    top min(k, chunk) pages of every chunk and then the top k of their union
    (kept in page order) gives exactly the one-level top k, with exact ties,
    chunks of any size and a partial last chunk.  Also with a cutoff: the
    count of keys at or above it, summed over chunks, decides how many pages
    the one-level rule keeps (max(1, min(k, count)))."""
    rng = np.random.default_rng(31)
    for _ in range(300):
        M = int(rng.integers(1, 400))
        k = int(rng.integers(1, 60))
        C = int(rng.integers(1, 70))
        U = rng.integers(-6, 7, size=M).astype(float)          # many exact ties
        cut = float(rng.integers(-6, 8))
        union = np.concatenate([c0 + sel.topk_pages(U[c0:c0 + C], k) for c0 in range(0, M, C)])
        assert np.all(np.diff(union) > 0)                     # page order
        count = sum(int(np.count_nonzero(U[c0:c0 + C] >= cut)) for c0 in range(0, M, C))
        keep = max(1, min(k, count))
        got = union[sel.topk_pages(U[union], keep)]
        want = sel.topk_pages(U, keep)
        np.testing.assert_array_equal(got, want)
        assert count == int(np.count_nonzero(U >= cut))
