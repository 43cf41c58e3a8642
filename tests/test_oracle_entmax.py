"""Pins of the oracle's alpha-entmax against what the mathematics fixes.

Source: "EntmaxKV: Support-Aware Decoding for Entmax Attention", section 2.2
(alpha-entmax; exact zeros) and section 2.1 (softmax); alpha = 2 is sparsemax
(Martins and Astudillo 2016), and alpha-entmax is the maximiser of
p.s + H^T_alpha(p) over the simplex (Peters et al. 2019), both cited there.
"""

import itertools
import os

import numpy as np
import pytest
from scipy.optimize import brentq, minimize

from oracle import entmax as em

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split(";")]


@pytest.mark.parametrize("row", list(_rows("entmax_worked.txt")))
def test_worked_examples(row):
    alpha = float(row[0])
    s = np.array([float(v) for v in row[1].split(",")])
    p_exp = np.array([eval(v) for v in row[2].split(",")])
    tau_exp = eval(row[3])
    p, tau, k = em.entmax(s, alpha)
    np.testing.assert_allclose(p, p_exp, rtol=0, atol=1e-13)
    assert abs(tau - tau_exp) < 1e-13
    assert k == int(np.count_nonzero(p_exp > 0))
    if alpha > 1:
        p2, tau2, _ = em.entmax(s, alpha, method="bisect")
        np.testing.assert_allclose(p2, p_exp, rtol=0, atol=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
def test_sum_to_one_exact_zeros(alpha):
    rng = np.random.default_rng(11)
    for n in (1, 2, 7, 64, 1000):
        s = rng.normal(size=n) * 3
        p, tau, k = em.entmax(s, alpha)
        assert abs(p.sum() - 1.0) < 1e-12
        x = (alpha - 1) * s
        assert np.all(p[x <= tau] == 0.0)          # exact zeros off the support
        assert np.all(p[x > tau] > 0.0)
        assert k == np.count_nonzero(p)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_sort_equals_bisection(alpha):
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(1, 257))
        s = rng.normal(size=n) * rng.uniform(0.1, 6)
        if trial % 5 == 0:
            s = np.round(s, 1)                      # plenty of ties
        t1, k1 = em.threshold_sort((alpha - 1) * s, alpha)
        t2, k2 = em.threshold_bisect((alpha - 1) * s, alpha)
        assert abs(t1 - t2) <= 1e-12 * max(1.0, abs(t1))
        assert k1 == k2


def _brute_force(x, beta):
    """Enumerate every support S; solve sum_S (x - tau)^beta = 1 for
    tau < min_S x by a bracketed root finder; keep the self-consistent ones."""
    n = x.size
    hits = []
    for m in range(1, n + 1):
        for S in itertools.combinations(range(n), m):
            xs = x[list(S)]
            lo_end = xs.min()
            f = lambda t: np.sum((xs - t) ** beta) - 1.0  # noqa: E731
            if f(lo_end) > 0:
                continue                               # no root below min_S x
            a = xs.max() - 1.0                         # f(a) >= 0: the top term alone is 1
            if f(lo_end) == 0:
                tau = lo_end
            elif f(a) <= 0:                            # only the top term (up to rounding)
                tau = a
            else:
                tau = brentq(f, a, lo_end, xtol=1e-15, rtol=1e-15)
            rest = np.delete(x, list(S))
            if xs.min() > tau and (rest.size == 0 or tau >= rest.max()):
                hits.append((set(S), tau))
    return hits


@pytest.mark.parametrize("alpha", [1.5, 2.0, 4.0 / 3.0, 1.25])
def test_brute_force_supports(alpha):
    rng = np.random.default_rng(17)
    beta = 1.0 / (alpha - 1.0)
    for _ in range(12):
        n = int(rng.integers(1, 10))
        s = rng.normal(size=n) * rng.uniform(0.5, 4)
        x = (alpha - 1) * s
        hits = _brute_force(x, beta)
        assert len(hits) == 1, "exactly one support is self-consistent"
        S, tau = hits[0]
        p, t, k = em.entmax(s, alpha)
        assert set(np.flatnonzero(p > 0)) == S
        assert abs(t - tau) < 1e-10


def _tsallis_argmax(s, alpha):
    """argmax_{p in simplex} p.s + (1/(alpha(alpha-1))) sum(p - p^alpha), by SLSQP."""
    n = s.size

    def negobj(p):
        pp = np.clip(p, 0, None)
        return -(pp @ s + np.sum(pp - pp ** alpha) / (alpha * (alpha - 1)))

    cons = ({"type": "eq", "fun": lambda p: p.sum() - 1.0},)
    best = None
    for start in (np.full(n, 1.0 / n), np.eye(n)[int(np.argmax(s))] * 0.9 + 0.1 / n):
        r = minimize(negobj, start, method="SLSQP", bounds=[(0, 1)] * n, constraints=cons,
                     options={"ftol": 1e-15, "maxiter": 2000})
        if best is None or r.fun < best.fun:
            best = r
    return np.clip(best.x, 0, None)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25, 3.0])
def test_variational_definition(alpha):
    rng = np.random.default_rng(23)
    for _ in range(6):
        n = int(rng.integers(2, 7))
        s = rng.normal(size=n) * 2
        p_ref = _tsallis_argmax(s, alpha)
        p, _, _ = em.entmax(s, alpha)
        np.testing.assert_allclose(p, p_ref, atol=2e-5)


def test_sparsemax_is_simplex_projection():
    """alpha = 2: the Euclidean projection of s onto the simplex."""
    rng = np.random.default_rng(29)
    for _ in range(20):
        n = int(rng.integers(2, 9))
        s = rng.normal(size=n)
        r = minimize(lambda p: np.sum((p - s) ** 2), np.full(n, 1.0 / n), method="SLSQP",
                     bounds=[(0, 1)] * n, constraints=({"type": "eq", "fun": lambda p: p.sum() - 1},),
                     options={"ftol": 1e-15, "maxiter": 500})
        p, _, _ = em.entmax(s, 2.0)
        np.testing.assert_allclose(p, r.x, atol=1e-6)


def test_alpha_to_one_approaches_softmax():
    rng = np.random.default_rng(31)
    s = rng.normal(size=50)
    ps, _ = em.softmax(s)
    errs = []
    for alpha in (1.1, 1.01, 1.001):
        p, _, _ = em.entmax(s, alpha)
        errs.append(np.abs(p - ps).max())
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 2e-3


def test_softmax_dense_and_logpartition():
    s = np.array([0.5, -1.0, 2.0])
    p, lse = em.softmax(s)
    assert np.all(p > 0)
    assert abs(lse - np.log(np.sum(np.exp(s)))) < 1e-14
    p2, lse2, k = em.entmax(s, 1.0)
    assert k == 3 and np.allclose(p, p2)


def test_invalid_slots_get_zero():
    s = np.array([1.0, -np.inf, 0.5])
    p, _, k = em.entmax(s, 1.5)
    assert p[1] == 0.0 and abs(p.sum() - 1) < 1e-12
