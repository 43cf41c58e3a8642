"""Pins of the oracle's sparse decode against the page's propositions.

Source: "EntmaxKV: Support-Aware Decoding for Entmax Attention":
  * Proposition 3.1 (section 3.1, proof Appendix C.1): ||o - o~|| <= 2 B delta,
    attained by the construction of the proof;
  * Proposition 3.2 (section 3.2, proof Appendix C.2): a kept set containing
    the entmax support gives delta = 0 and o~ = o exactly;
  * Appendix B.2: selecting pages whose upper-bounded score clears a
    conservative threshold cannot miss support;
  * section 3.2 / Appendix E.2.2 Table 3: softmax keeps positive mass
    everywhere, so any truncation drops mass and its support recall equals
    coverage.
"""

import os

import numpy as np
import pytest

from oracle import decode as dec
from oracle import entmax as em
from oracle import paged as pg
from oracle import select as sel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(seed, n=600, G=2, H=4, d=16, scale=2.0):
    rng = np.random.default_rng(seed)
    K = rng.normal(size=(n, G, d))
    V = rng.normal(size=(n, G, d))
    q = rng.normal(size=(H, d)) * scale
    return q, K, V


@pytest.mark.parametrize("alpha", [1.5, 2.0, 4.0 / 3.0])
def test_prop32_superset_of_support_is_exact(alpha):
    q, K, V = _problem(1)
    n = K.shape[0]
    G = K.shape[1]
    r = q.shape[0] // G
    full = dec.decode(q, K, V, None, alpha)
    rng = np.random.default_rng(2)
    for g in range(G):
        hs = slice(g * r, (g + 1) * r)
        support = np.flatnonzero((full["p"][hs] > 0).any(axis=0))
        extra = rng.choice(n, 50, replace=False)
        keep = np.union1d(support, extra)
        sp = dec.decode(q[hs], K[:, g:g + 1], V[:, g:g + 1], keep, alpha)
        fl = dec.decode(q[hs], K[:, g:g + 1], V[:, g:g + 1], None, alpha)
        np.testing.assert_allclose(sp["out"], fl["out"], atol=1e-12)
        for i, h in enumerate(range(hs.start, hs.stop)):
            delta = dec.dropped_mass_from_tau(fl["s"][i][keep], fl["tau"][i], alpha)
            assert abs(delta) < 1e-12
            assert abs(sp["tau"][i] - fl["tau"][i]) < 1e-12


@pytest.mark.parametrize("alpha", [1.0, 1.5, 2.0])
def test_prop31_error_bound(alpha):
    q, K, V = _problem(3)
    n = K.shape[0]
    full = dec.decode(q, K[:, :1], V[:, :1], None, alpha)
    B = np.linalg.norm(V[:, 0], axis=1).max()
    rng = np.random.default_rng(4)
    for _ in range(30):
        keep = np.sort(rng.choice(n, int(rng.integers(1, n)), replace=False))
        sp = dec.decode(q, K[:, :1], V[:, :1], keep, alpha)
        for h in range(q.shape[0]):
            delta = 1.0 - full["p"][h][keep].sum()
            err = np.linalg.norm(full["out"][h] - sp["out"][h])
            assert err <= 2 * B * delta + 1e-12
            # the kept probabilities only grow under re-normalisation (tau~ <= tau)
            assert np.all(sp["p"][h] >= full["p"][h][keep] - 1e-15)


def test_prop31_bound_is_attained():
    """Values B u on the kept tokens and -B u on the dropped ones give
    o = (1 - 2 delta) B u and o~ = B u: the gap is exactly 2 B delta."""
    rng = np.random.default_rng(5)
    n, d = 40, 6
    s = rng.normal(size=n)
    p, _ = em.softmax(s)
    keep = np.arange(25)
    u = rng.normal(size=d)
    u /= np.linalg.norm(u)
    Bn = 1.7
    Vv = np.where(np.isin(np.arange(n), keep)[:, None], Bn * u[None, :], -Bn * u[None, :])
    o = p @ Vv
    pk, _ = em.softmax(s[keep])
    o_t = pk @ Vv[keep]
    delta = 1.0 - p[keep].sum()
    assert abs(np.linalg.norm(o - o_t) - 2 * Bn * delta) < 1e-12


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_b2_superset_selection_from_box_bounds(alpha):
    """Pages whose box score clears a conservative threshold contain every
    support token: rho = 1 and delta = 0."""
    rng = np.random.default_rng(6)
    n, d, P = 2000, 16, 16
    K = rng.normal(size=(n, 1, d))
    K[rng.choice(n, 12, replace=False), 0, :] += 3.0 * np.ones(d) / np.sqrt(d)
    V = rng.normal(size=(n, 1, d))
    q = (rng.normal(size=(1, d)) + 2.0 * np.ones(d) / np.sqrt(d)) * 2
    full = dec.decode(q, K, V, None, alpha)
    kmin, kmax, _, _ = pg.page_stats(K, P)
    _, U = pg.box_scores(q, kmin, kmax)
    for eps in (0.0, 0.05, 0.5):
        tau_hat = full["tau"][0] - eps                    # conservative estimate
        pages = np.flatnonzero((alpha - 1) * U[0] > tau_hat)
        keep = dec.tokens_of_pages(pages, n, P)
        sp = dec.decode(q, K, V, keep, alpha)
        m = dec.metrics(full, sp, n)
        assert m["rho"][0] == 1.0 and abs(m["delta"][0]) < 1e-12
        assert m["R"][0] < 1e-12


def _table3_rows():
    with open(os.path.join(GOLDEN, "table3_softmax_recall.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split(";")]


@pytest.mark.parametrize("row", list(_table3_rows()))
def test_softmax_topk_recall_equals_coverage(row):
    coverage, rho_printed = float(row[1]), float(row[2])
    assert rho_printed == coverage
    n = 1280                                   # 80 pages: every printed coverage is whole pages
    q, K, V = _problem(7, n=n, G=1, H=2)
    full = dec.decode(q, K, V, None, 1.0)
    kmin, kmax, _, _ = pg.page_stats(K, 16)
    _, U = pg.box_scores(q, kmin, kmax)
    pages = sel.topk_pages(U[0], int(round(coverage * n / 16)))
    sp = dec.decode(q, K, V, dec.tokens_of_pages(pages, n, 16), 1.0)
    m = dec.metrics(full, sp, n)
    np.testing.assert_allclose(m["rho"], coverage, rtol=0, atol=1e-15)
    assert abs(m["coverage"] - coverage) < 1e-12
    assert np.all(m["delta"] > 0)                        # softmax truncation drops mass


def test_tiny_workload_support_calibration():
    """The tiny workload's planted shift yields a group support union of 10..40
    tokens holding at least half of the planted keys (recipe of the tiny
    CPU-checkable workload; see tests/golden/calibrate_tiny.py)."""
    from sparse_long_context_ekv_amd import workloads as W
    wl = W.make_workload(W.CONFIGS[1], "cpu")
    q, kc, vc, pt, n = W.host_sequence(wl, 0)
    K = pg.gather_logical(kc, pt, n)
    V = pg.gather_logical(vc, pt, n)
    res = dec.decode(q, K, V, None, 1.5)
    union = (res["p"] > 0).any(axis=0)
    planted = wl.planted[0]["mask"][0].numpy()
    assert 10 <= union.sum() <= 40
    assert 2 * (union & planted).sum() >= planted.sum()


def test_generator_is_deterministic():
    from sparse_long_context_ekv_amd import workloads as W
    cfg = W.CONFIGS[2].scaled(seq_len=3000)
    a = W.make_workload(cfg, "cpu")
    b = W.make_workload(cfg, "cpu")
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.page_table, b.page_table)]:
        assert x.dtype == y.dtype and bool((x.view(-1) == y.view(-1)).all())


def test_generator_sentinel_and_layout():
    """Slots past a sequence end hold the sentinel; valid tokens are finite
    normals; the page table is a permutation of physical pages."""
    from sparse_long_context_ekv_amd import workloads as W
    cfg = W.CONFIGS[2].scaled(seq_len=1000, batch=2)
    wl = W.make_workload(cfg, "cpu")
    P = cfg.page_size
    M = (1000 + P - 1) // P
    last = wl.page_table[0, M - 1].item()
    tail = wl.k_cache[last, :, 1000 - (M - 1) * P:, :].float()
    assert bool((tail == W.SENTINEL).all())
    used = wl.page_table[:, :M].reshape(-1).tolist()
    assert sorted(used) == list(range(wl.num_phys))


@pytest.mark.parametrize("alpha", [4.0 / 3.0, 1.5, 2.0, 3.0])
def test_threshold_of_a_subset_is_a_lower_bound(alpha):
    """For any subset T of the tokens, sum_T [x - tau]_+^beta <= sum_all, so
    the threshold solving the equation on T is at most the full threshold:
    entmax over the tokens of any pages gives a conservative estimate for
    the Appendix B.2 rule."""
    rng = np.random.default_rng(31)
    for trial in range(40):
        n = int(rng.integers(2, 400))
        s = rng.normal(size=n) * rng.uniform(0.2, 4.0)
        _, tau_full, _ = em.entmax(s, alpha)
        T = rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False)
        _, tau_t, _ = em.entmax(s[T], alpha)
        assert tau_t <= tau_full + 1e-12


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_superset_selector_pipeline_is_exact(alpha):
    """Appendix B.2 end to end with a lower bound from a first pass: entmax
    over the top-k0 pages by box score gives tau_lo <= tau per head; pages with
    (alpha-1) U > min_h tau_lo then hold every support token of every head of
    the group, so rho = 1, delta = 0 and the output equals the full-cache
    output (Proposition 3.2)."""
    for seed in range(4):
        q, K, V = _problem(seed, n=900, G=2, H=4, d=16, scale=2.0)
        n, P, G = K.shape[0], 16, 2
        H = q.shape[0]
        r = H // G
        full = dec.decode(q, K, V, None, alpha)
        kmin, kmax, _, _ = pg.page_stats(K, P)
        _, U = pg.box_scores(q, kmin, kmax)
        M = U.shape[1]
        for g in range(G):
            hs = slice(g * r, (g + 1) * r)
            first = sel.topk_pages(U[g], 2)
            toks = dec.tokens_of_pages(first, n, P)
            tau_lo = dec.decode(q[hs], K[:, g:g + 1], V[:, g:g + 1], toks, alpha)["tau"]
            assert np.all(tau_lo <= full["tau"][hs] + 1e-12)
            pages = sel.superset_pages(U[g], tau_lo, alpha, M)
            keep = dec.tokens_of_pages(pages, n, P)
            sp = dec.decode(q[hs], K[:, g:g + 1], V[:, g:g + 1], keep, alpha)
            sub_full = {"p": full["p"][hs], "out": full["out"][hs]}
            m = dec.metrics(sub_full, sp, n)
            assert np.all(m["rho"] == 1.0) and np.all(np.abs(m["delta"]) < 1e-12)
            assert np.all(m["R"] < 1e-10)
