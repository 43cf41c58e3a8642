"""Hand-worked pins of the oracle functions that the GPU parity tests lean
on most: the Gaussian page rule (reading R10 of the lost Eq. (21) of
"EntmaxKV: Support-Aware Decoding for Entmax Attention", section 4.3, pooled
over the group's heads by the maximum, reading R5) and the per-group
composition of page selection and sparse decode (section 4.1: each KV
group's heads attend over the tokens of that group's own page set).

Every expected value below is worked out by hand in the comments from the
stated inputs (dyadic numbers, so the arithmetic is exact in binary), and
none is computed by the function under test.  Each case is built so that a
plausible slip gives a different answer:
  * (mu - theta)/sigma**2 instead of (mu - theta)/sigma,
  * the mean (or the minimum) over the group's heads instead of the maximum,
  * theta = tau_hat instead of tau_hat/(alpha - 1), or theta dropped,
  * the sign of the margin flipped,
  * ">" instead of ">=" at exactly t = -z,
  * a group reading another group's heads, pages or tokens.
"""

import math
import os
import re

import numpy as np
import pytest
from scipy.special import erfcx

from oracle import decode as dec
from oracle import select as sel

# ---------------------------------------------------------------------------
# Gaussian margins and page rule, r = 2 heads, alpha = 3/2 (theta = 2 tau_hat)
# ---------------------------------------------------------------------------
ALPHA = 1.5
TAU_HAT = np.array([0.5, 1.0])          # theta = tau_hat / (alpha - 1) = [1.0, 2.0]
MU = np.array([[0.0, 0.5, 1.0, -2.0],    # head 0
               [1.5, 0.0, 2.5, 1.0]])    # head 1
SIG = np.array([[0.5, 2.0, 1.0, 0.25],
                [0.25, 1.0, 0.5, 0.5]])
# head 0: mu - 1.0 = [-1.0, -0.5, 0.0, -3.0]; / sigma = [-2.0, -0.25, 0.0, -12.0]
# head 1: mu - 2.0 = [-0.5, -2.0, 0.5, -1.0]; / sigma = [-2.0, -2.0, 1.0, -2.0]
# max over heads:                                      [-2.0, -0.25, 1.0, -2.0]
WANT_T = np.array([-2.0, -0.25, 1.0, -2.0])


def test_gauss_margins_two_heads_by_hand():
    t = sel.gauss_margins(MU, SIG, TAU_HAT, ALPHA)
    np.testing.assert_array_equal(t, WANT_T)           # exact: dyadic inputs


def test_gauss_select_at_exactly_minus_z():
    # z = 2: pages 0 and 3 sit exactly at t = -2 = -z and are kept (t >= -z).
    np.testing.assert_array_equal(sel.gauss_select(MU, SIG, TAU_HAT, ALPHA, 2.0, cap=4), [0, 1, 2, 3])
    # Just below: only t = 1 and t = -0.25 reach -1.99.
    np.testing.assert_array_equal(sel.gauss_select(MU, SIG, TAU_HAT, ALPHA, 1.99, cap=4), [1, 2])


def test_gauss_select_discriminates_plausible_slips():
    got = sel.gauss_select(MU, SIG, TAU_HAT, ALPHA, 2.0, cap=4)
    np.testing.assert_array_equal(got, [0, 1, 2, 3])
    # Slip (mu - theta)/sigma^2: head 0 -> [-4, -0.125, 0, -48], head 1 ->
    # [-8, -2, 2, -4]; max [-4, -0.125, 2, -4] keeps only {1, 2} at z = 2.
    # Slip "mean over heads": [-2, -1.125, 0.5, -7] keeps {0, 1, 2}.
    # Slip "min over heads": [-2, -2, 0, -12] keeps {0, 1, 2}.
    # All differ from {0, 1, 2, 3}.
    # The cap ranks by margin, ties to the lower page: t = [-2, -0.25, 1, -2]
    # ranks page 2, page 1, then page 0 before page 3.
    np.testing.assert_array_equal(sel.gauss_select(MU, SIG, TAU_HAT, ALPHA, 2.0, cap=2), [1, 2])
    np.testing.assert_array_equal(sel.gauss_select(MU, SIG, TAU_HAT, ALPHA, 2.0, cap=3), [0, 1, 2])
    # With cap = 2 the other slips pick differently:
    # flipped sign (theta - mu)/sigma: max [2, 2, 0, 12] -> top 2 {0, 3};
    # theta dropped (mu/sigma): max [6, 0.25, 5, 2] -> top 2 {0, 2};
    # theta = tau_hat (not divided by alpha - 1): head 0 (mu - 0.5)/sigma =
    # [-1, 0, 0.5, -10], head 1 (mu - 1)/sigma = [2, -1, 3, 0], max
    # [2, 0, 3, 0] -> top 2 {0, 2}.


def test_gauss_select_keeps_one_page_when_none_qualifies():
    # z = 0: no page has t >= 0 except page 2 (t = 1); with z = -1.5 none
    # does, and the single best page (page 2) is kept.
    np.testing.assert_array_equal(sel.gauss_select(MU, SIG, TAU_HAT, ALPHA, 0.0, cap=4), [2])
    np.testing.assert_array_equal(sel.gauss_select(MU, SIG, TAU_HAT, ALPHA, -1.5, cap=4), [2])


def test_gauss_margins_zero_sigma_by_hand():
    # sigma = 0: +inf when mu > theta, -inf when mu <= theta (a token exactly
    # at the threshold has probability 0).  alpha = 2: theta = tau_hat.
    mu = np.array([[1.0, 3.0, 2.0],
                   [0.0, 0.0, 5.0]])
    sig = np.array([[0.0, 0.0, 0.0],
                    [0.0, 1.0, 0.0]])
    t = sel.gauss_margins(mu, sig, np.array([2.0, 1.0]), 2.0)
    # head 0 (theta 2): [-inf, +inf, -inf (mu == theta)]
    # head 1 (theta 1): [-inf, (0 - 1)/1 = -1, +inf]
    np.testing.assert_array_equal(t, [-np.inf, np.inf, np.inf])


# ---------------------------------------------------------------------------
# Two KV groups, r = 2 heads each, page size 2, d = 2: each group must select
# its own page and its heads must attend over that page's tokens of their own
# group.
# ---------------------------------------------------------------------------
S2 = math.sqrt(2.0)
Q = np.array([[2.0, 0.0],      # heads 0, 1 -> group 0
              [1.0, 0.0],
              [0.0, 2.0],      # heads 2, 3 -> group 1
              [0.0, 1.0]])
# K[token][group][channel]; page 0 = tokens 0, 1; page 1 = tokens 2, 3.
K = np.array([[[3.0, 0.0], [0.0, -1.0]],
              [[2.5, 0.0], [0.0, 0.0]],
              [[0.0, 0.0], [0.0, 2.5]],
              [[-1.0, 0.0], [0.0, 3.0]]])
V = np.array([[[1.0, 0.0], [9.0, 9.0]],
              [[0.0, 1.0], [8.0, 8.0]],
              [[5.0, 5.0], [1.0, 2.0]],
              [[7.0, 7.0], [3.0, 4.0]]])


def test_two_group_topk_selection_by_hand():
    # Box scores (1/sqrt 2) sum_i max(q_i kmax_i, q_i kmin_i):
    # group 0, page 0: kmax [3, 0], kmin [2.5, 0]; head 0 -> 6/sqrt2,
    #   head 1 -> 3/sqrt2; pooled 6/sqrt2.  page 1: kmax [0, 0], kmin [-1, 0]:
    #   heads 0, 1 -> 0.  Group 0 keeps page 0.
    # group 1, page 0: kmax [0, 0], kmin [0, -1]: 0.  page 1: kmax [0, 3],
    #   kmin [0, 2.5]: head 2 -> 6/sqrt2.  Group 1 keeps page 1.
    res = dec.select_pages(Q, K, 4, 2, 2, "topk", 2.0, 1)
    np.testing.assert_allclose(res["U"], [[6 / S2, 0.0], [0.0, 6 / S2]], rtol=1e-15, atol=1e-15)
    assert [list(s) for s in res["sel"]] == [[0], [1]]


def test_two_group_gauss_selection_by_hand():
    # Single-token pages (P = 1) have sigma = 0, and then Eq. (18) is the exact
    # entmax equation, so a page is kept iff its token is in the sparsemax
    # (alpha = 2) support of some head of the group.
    # Head 0 over group 0's keys: s = q.k/sqrt2 = [3 sqrt2, 2.5 sqrt2, 0, -sqrt2];
    #   top two differ by sqrt2/2 < 1, third is 0 < tau = (5.5 sqrt2 - 1)/2:
    #   support {0, 1}.  Head 1 (half the scores): {0, 1} likewise.
    # Group 1 (heads 2, 3): s = [-sqrt2, 0, 2.5 sqrt2, 3 sqrt2] (head 2):
    #   support {2, 3}.
    res = dec.select_pages(Q, K, 4, 1, 2, "gauss", 2.0, 4, z=3.0)
    np.testing.assert_allclose(res["tau_hat"][0], (5.5 * S2 - 1.0) / 2.0, rtol=1e-12)
    np.testing.assert_allclose(res["tau_hat"][2], (5.5 * S2 - 1.0) / 2.0, rtol=1e-12)
    assert [list(s) for s in res["sel"]] == [[0, 1], [2, 3]]


def test_two_group_sparse_decode_by_hand():
    # sparsemax (alpha = 2) over each group's own page.  For two tokens whose
    # scores differ by c < 1: p = ((1 + c)/2, (1 - c)/2).
    # head 0: s = [3 sqrt2, 2.5 sqrt2], c = sqrt2/2 -> p0 = (1 + a)/2, a = sqrt2/2
    # head 1: s = [3/sqrt2, 2.5/sqrt2], c = sqrt2/4 -> b = sqrt2/4
    # head 2 over group 1's page 1: s = [2.5 sqrt2, 3 sqrt2] (reversed)
    # head 3: s = [2.5/sqrt2, 3/sqrt2]
    # tau (x units) = (s_0 + s_1 - 1)/2.
    a, b = S2 / 2.0, S2 / 4.0
    out = dec.sparse_decode_groups(Q, K, V, 4, 2, [np.array([0]), np.array([1])], 2.0)
    p = {0: ((1 + a) / 2, (1 - a) / 2), 1: ((1 + b) / 2, (1 - b) / 2),
         2: ((1 - a) / 2, (1 + a) / 2), 3: ((1 - b) / 2, (1 + b) / 2)}
    # group 0 values of tokens 0, 1: [1, 0], [0, 1]; group 1 values of tokens 2, 3: [1, 2], [3, 4]
    want = np.array([[p[0][0], p[0][1]],
                     [p[1][0], p[1][1]],
                     [p[2][0] * 1 + p[2][1] * 3, p[2][0] * 2 + p[2][1] * 4],
                     [p[3][0] * 1 + p[3][1] * 3, p[3][0] * 2 + p[3][1] * 4]])
    np.testing.assert_allclose(out["out"], want, rtol=1e-14, atol=1e-14)
    want_tau = [(5.5 * S2 - 1) / 2, (5.5 / S2 - 1) / 2, (5.5 * S2 - 1) / 2, (5.5 / S2 - 1) / 2]
    np.testing.assert_allclose(out["tau"], want_tau, rtol=1e-14)
    np.testing.assert_array_equal(out["support"], [2, 2, 2, 2])
    assert [list(t) for t in out["tokens_per_group"]] == [[0, 1], [2, 3]]


def test_two_group_pipeline_by_hand():
    # select_pages + sparse_decode_groups end to end equal the hand results.
    res = dec.select_pages(Q, K, 4, 2, 2, "topk", 2.0, 1)
    out = dec.sparse_decode_groups(Q, K, V, 4, 2, res["sel"], 2.0)
    a = S2 / 2.0
    np.testing.assert_allclose(out["out"][0], [(1 + a) / 2, (1 - a) / 2], rtol=1e-14)
    np.testing.assert_allclose(out["out"][2], [(1 - a) / 2 + 3 * (1 + a) / 2, (1 - a) + 2 * (1 + a)], rtol=1e-14)


# ---------------------------------------------------------------------------
# The Mills-ratio table of the GPU's Gaussian threshold kernel
# ---------------------------------------------------------------------------
SELECT_HIP = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "sparse_long_context_ekv_amd", "csrc", "select.hip")


def _mills_table():
    src = open(SELECT_HIP).read()
    k = float(re.search(r"kMillsK\s*=\s*([0-9.eE+-]+)f", src).group(1))
    body = re.search(r"kMillsC\[\d+\]\s*=\s*\{(.*?)\};", src, flags=re.S).group(1)
    c = [float(v.strip().rstrip("f")) for v in body.split(",") if v.strip()]
    return np.float32(k), np.asarray(c, dtype=np.float32)


def test_mills_ratio_table_matches_erfcx():
    """The committed fp32 coefficients: R(x) ~ t h(t), t = 1/(1 + K x), with
    R(x) = Q(x)/phi(x) = sqrt(pi/2) erfcx(x/sqrt2); relative error at most
    3.2e-7 over x in [0, 40] (Horner in float64 on the fp32 table)."""
    k, c = _mills_table()
    assert len(c) == 12
    x = np.concatenate([np.linspace(0.0, 12.0, 120001), np.linspace(12.0, 40.0, 2801)])
    t = 1.0 / (1.0 + float(k) * x)
    h = np.zeros_like(t)
    for ci in c[::-1].astype(np.float64):
        h = h * t + ci
    want = math.sqrt(math.pi / 2.0) * erfcx(x / math.sqrt(2.0))
    err = np.abs(t * h / want - 1.0)
    assert float(err.max()) <= 3.2e-7, float(err.max())


@pytest.mark.parametrize("x", [0.0, 1.0, 3.0, 10.0])
def test_mills_ratio_table_upper_tail_values(x):
    """Q(x) = phi(x) R(x) against the normal tail at a few points."""
    from scipy.special import ndtr
    k, c = _mills_table()
    t = 1.0 / (1.0 + float(k) * x)
    h = 0.0
    for ci in c[::-1].astype(np.float64):
        h = h * t + ci
    phi = math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    q = phi * t * h
    want = float(ndtr(-x))
    assert abs(q / want - 1.0) <= 3.2e-7
