"""Hand-computed pins of the oracle's token scores and decode output.

Source: "EntmaxKV: Support-Aware Decoding for Entmax Attention", section 2.1
(s_j = q.k_j/sqrt(d), o = sum_j p_j v_j), section 4.1 (sparse decode over
the candidate tokens), Appendix E.1 (dropped mass); GQA head-to-group map of
"EntroPrefill" section 2.1 Eq. (1) with consecutive heads per group (R1).
"""

import numpy as np

from oracle import decode as dec
from oracle import paged as pg


def test_token_score_by_hand():
    q = np.array([[1.0, 2.0, 3.0, 4.0]])
    K = np.array([[[1.0, 0.0, -1.0, 2.0]]])            # [n=1][G=1][d=4]
    # (1*1 + 2*0 + 3*(-1) + 4*2) / sqrt(4) = 6 / 2 = 3
    assert pg.token_scores(q, K)[0, 0] == 3.0


def test_heads_read_their_own_group():
    # H = 4, G = 2: heads 0,1 read group 0; heads 2,3 read group 1.
    q = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.0], [0.0, 1.0]])
    K = np.array([[[2.0, 0.0], [0.0, 4.0]]])           # one token; group 0 = (2,0), group 1 = (0,4)
    s = pg.token_scores(q, K) * np.sqrt(2.0)
    np.testing.assert_array_equal(s[:, 0], [2.0, 0.0, 0.0, 4.0])


def test_decode_output_by_hand():
    """1.5-entmax over two tokens, then the weighted value sum.

    q = (2, 0), keys e1, e2, d = 2: s = (sqrt 2, 0), x = s/2 = (a, 0) with
    a = sqrt(2)/2.  Both tokens in the support: (a - tau)^2 + tau^2 = 1 gives
    tau = (a - sqrt(2 - a^2))/2, p = ((a - tau)^2, tau^2).
    """
    q = np.array([[2.0, 0.0]])
    K = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    V = np.array([[[1.0, 2.0]], [[3.0, 4.0]]])
    a = np.sqrt(2.0) / 2
    tau = (a - np.sqrt(2 - a * a)) / 2
    p = np.array([(a - tau) ** 2, tau ** 2])
    res = dec.decode(q, K, V, None, 1.5)
    np.testing.assert_allclose(res["p"][0], p, atol=1e-15)
    np.testing.assert_allclose(res["out"][0], p[0] * np.array([1.0, 2.0]) + p[1] * np.array([3.0, 4.0]), atol=1e-14)
    assert abs(res["tau"][0] - tau) < 1e-15 and res["support"][0] == 2


def test_decode_uses_group_values():
    """Each head mixes its own group's values: with one token per sequence
    the output is exactly that token's value in the head's group."""
    q = np.ones((4, 3))
    K = np.zeros((1, 2, 3))
    V = np.array([[[1.0, 2.0, 3.0], [-1.0, -2.0, -3.0]]])
    res = dec.decode(q, K, V, None, 1.5)
    np.testing.assert_array_equal(res["out"], [[1, 2, 3], [1, 2, 3], [-1, -2, -3], [-1, -2, -3]])


def test_tokens_of_pages_partial_tail():
    np.testing.assert_array_equal(dec.tokens_of_pages([0, 2], 37, 16), list(range(16)) + list(range(32, 37)))


def test_dropped_mass_two_ways():
    """delta from the full-cache threshold equals 1 - sum of the full-cache
    probabilities over the kept tokens."""
    rng = np.random.default_rng(3)
    n, d = 500, 8
    K = rng.normal(size=(n, 1, d))
    V = rng.normal(size=(n, 1, d))
    q = rng.normal(size=(2, d)) * 3
    for alpha in (1.0, 1.5, 2.0):
        full = dec.decode(q, K, V, None, alpha)
        keep = np.sort(rng.choice(n, 300, replace=False))
        for h in range(2):
            d1 = dec.dropped_mass_from_tau(full["s"][h][keep], full["tau"][h], alpha)
            d2 = 1.0 - full["p"][h][keep].sum()
            assert abs(d1 - d2) < 1e-12


def test_metrics_by_hand():
    full = {"p": np.array([[0.5, 0.3, 0.2, 0.0]]), "out": np.array([[1.0, 0.0]])}
    sparse = {"tokens": np.array([0, 3]), "out": np.array([[0.0, 1.0]])}
    m = dec.metrics(full, sparse, 4)
    assert abs(m["delta"][0] - 0.5) < 1e-15          # kept mass 0.5
    assert abs(m["rho"][0] - 1.0 / 3.0) < 1e-15      # support {0,1,2}, kept {0}
    assert abs(m["R"][0] - np.sqrt(2.0)) < 1e-15
    assert m["coverage"] == 0.5
