"""GPU parity of ekv_select on its own, against the fp64 oracle, at page
counts and row counts that reach every kernel variant (one level: keys in
registers at 4..64 keys per thread, and the global-memory path beyond 65536
pages; two levels, chunk + merge, for few rows of more than 8192 pages), with
ragged and empty sequences and exact ties.  Selection rules: "EntmaxKV: Support-Aware Decoding
for Entmax Attention" section 4.3 (top-k page selection; Gaussian-aware
selection with the threshold of Appendix C.2 Eq. (18)); the Gaussian page rule
is this library's reading of the lost Eq. (21)."""

import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_ekv_amd import ekv
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

P = 16


def _shape(B, G, R, MP):
    return ekv.make_shape(B, G * R, G, 128, MP, 1, "bf16", "f32")


def _run_select(sh, selector, lens, alpha, budget, z, score=None, mu=None, sigma=None):
    B, G, HQ = sh.batch, sh.num_kv_groups, sh.num_q_heads
    sel = torch.full((B, G, budget), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, G), -7, dtype=torch.int32, device="cuda")
    th = torch.full((B, HQ), 7.0, device="cuda") if selector == ekv.SEL_GAUSS else None
    ws = torch.empty(ekv.select_workspace_bytes(sh, selector, alpha, budget, z), dtype=torch.uint8, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ekv.select(sh, selector, sl, alpha, budget, z, score, mu, sigma, sel, cnt, th, ws)
    H.sync()
    return sel.cpu().numpy(), cnt.cpu().numpy(), (None if th is None else th.cpu().numpy().astype(np.float64))


def _check_rows(sel, cnt, b, g, want, keys, budget):
    c = int(cnt[b, g])
    row = sel[b, g]
    assert c == len(want), (b, g, c, len(want))
    assert np.all(row[c:] == -1)
    assert np.all(np.diff(row[:c]) > 0)
    return H.compare_selection(row[:c], want, keys, len(want))


@pytest.mark.parametrize("MP", [300, 5000, 9000, 20000, 40000, 65536, 70000])
def test_topk_select_sizes(MP):
    print(f"[case] topk MP={MP}", flush=True)
    B, G, budget = 3, 2, 128
    lens = [MP * P, (MP // 2) * P + 5, 37]
    rng = np.random.default_rng(MP)
    score = rng.standard_normal((B, G, MP)).astype(np.float32)
    sel, cnt, _ = _run_select(_shape(B, G, 1, MP), ekv.SEL_TOPK, lens, 1.5, budget, 3.0,
                              score=torch.from_numpy(score).cuda())
    for b in range(B):
        M = (lens[b] + P - 1) // P
        for g in range(G):
            U = score[b, g, :M].astype(np.float64)
            want = oracle.select.topk_pages(U, budget)
            _check_rows(sel, cnt, b, g, want, U, budget)


@pytest.mark.parametrize("MP", [3000, 20000, 70000])
def test_topk_select_exact_ties(MP):
    """Integer-valued scores: many exact ties, broken toward the lower page
    index; fp32 and fp64 agree exactly, so the selection must be identical."""
    print(f"[case] ties MP={MP}", flush=True)
    B, G, budget = 2, 2, 200
    lens = [MP * P, MP * P - 3]
    rng = np.random.default_rng(7 + MP)
    score = rng.integers(-20, 21, size=(B, G, MP)).astype(np.float32)
    sel, cnt, _ = _run_select(_shape(B, G, 1, MP), ekv.SEL_TOPK, lens, 1.5, budget, 3.0,
                              score=torch.from_numpy(score).cuda())
    for b in range(B):
        M = (lens[b] + P - 1) // P
        for g in range(G):
            want = oracle.select.topk_pages(score[b, g, :M].astype(np.float64), budget)
            c = int(cnt[b, g])
            np.testing.assert_array_equal(sel[b, g, :c], want)


def test_topk_select_empty_and_short():
    B, G, budget, MP = 3, 2, 64, 100
    lens = [0, 40 * P - 1, 100 * P]
    score = torch.randn(B, G, MP, generator=torch.Generator().manual_seed(3)).cuda()
    sel, cnt, _ = _run_select(_shape(B, G, 1, MP), ekv.SEL_TOPK, lens, 1.5, budget, 3.0, score=score)
    assert np.all(cnt[0] == 0) and np.all(sel[0] == -1)
    for g in range(G):
        assert cnt[1, g] == 40
        np.testing.assert_array_equal(sel[1, g, :40], np.arange(40))
        assert np.all(sel[1, g, 40:] == -1)
        assert cnt[2, g] == budget


@pytest.mark.parametrize("MP,alpha", [(600, 1.5), (8192, 1.5), (8192, 2.0), (8192, 4.0 / 3.0), (20000, 1.5),
                                      (70000, 1.5)])
def test_gauss_select_sizes(MP, alpha):
    """tau_hat against the oracle's fp64 Eq. (18) root; the page rule
    against the oracle's margins computed from the GPU's own tau_hat."""
    print(f"[case] gauss MP={MP} alpha={alpha}", flush=True)
    B, G, R, budget, z = 2, 2, 4, 256, 3.0
    lens = [MP * P - 9, (MP // 3) * P]
    rng = np.random.default_rng(MP + int(alpha * 10))
    mu = (rng.standard_normal((B, G * R, MP)) * 0.25).astype(np.float32)
    sg = (0.8 + 0.4 * rng.random((B, G * R, MP))).astype(np.float32)
    sg[:, :, ::97] = 0.0                      # some zero-variance pages
    sel, cnt, th = _run_select(_shape(B, G, R, MP), ekv.SEL_GAUSS, lens, alpha, budget, z,
                               mu=torch.from_numpy(mu).cuda(), sigma=torch.from_numpy(sg).cuda())
    for b in range(B):
        n = lens[b]
        M = (n + P - 1) // P
        n_p = oracle.paged.page_valid_counts(n, P)
        for h in range(G * R):
            m64, s64 = mu[b, h, :M].astype(np.float64), sg[b, h, :M].astype(np.float64)
            want = oracle.select.gauss_tau_hat(m64, s64, n_p, alpha)
            assert H.tau_close(th[b, h], want), (b, h, th[b, h], want)
        for g in range(G):
            hs = slice(g * R, (g + 1) * R)
            m64, s64 = mu[b, hs, :M].astype(np.float64), sg[b, hs, :M].astype(np.float64)
            t = oracle.select.gauss_margins(m64, s64, th[b, hs], alpha)
            want = oracle.select.gauss_select(m64, s64, th[b, hs], alpha, z, budget)
            c = int(cnt[b, g])
            row = sel[b, g]
            assert c == len(want) or np.any(np.abs(t + z) < 1e-4 * z)
            assert np.all(row[c:] == -1) and np.all(np.diff(row[:c]) > 0)
            if c == len(want):
                H.compare_selection(row[:c], want, t, len(want))


@pytest.mark.parametrize("MP", [20000, 70000])
def test_topk_select_one_level_many_rows(MP):
    """256 (sequence, group) rows: enough rows for one block per row, so the
    one-level kernels run (keys in registers up to 65536 pages, the
    global-memory kernel beyond); fewer rows of this length take the
    two-level chunk + merge path covered above."""
    print(f"[case] topk one-level MP={MP}", flush=True)
    B, G, budget = 128, 2, 128
    lens = [MP * P - (b % 7) * 5 for b in range(B)]
    rng = np.random.default_rng(MP + 11)
    score = rng.standard_normal((B, G, MP)).astype(np.float32)
    score[::3, :, ::50] = 1.5                 # exact ties among high scores
    sel, cnt, _ = _run_select(_shape(B, G, 1, MP), ekv.SEL_TOPK, lens, 1.5, budget, 3.0,
                              score=torch.from_numpy(score).cuda())
    for b in range(0, B, 9):
        M = (lens[b] + P - 1) // P
        for g in range(G):
            U = score[b, g, :M].astype(np.float64)
            want = oracle.select.topk_pages(U, budget)
            _check_rows(sel, cnt, b, g, want, U, budget)


@pytest.mark.parametrize("MP,theta,lo,hi", [(20000, 0.5, -20, 21), (70000, 995.5, -1000, 1001),
                                            (9000, 1e9, -5, 5)])
def test_superset_select_two_level(MP, theta, lo, hi):
    """Superset rule ([EKV] Appendix B.2) on few long rows (two-level path):
    integer box scores and a threshold halfway between integers, so the GPU's
    slightly lowered threshold (it may only add pages) keeps the same pages;
    the cap ranks by score with ties to the lower page.  Cases: more
    qualifying pages than the cap, fewer, and none (one page kept)."""
    print(f"[case] superset MP={MP} theta={theta}", flush=True)
    B, G, budget, alpha = 2, 3, 200, 1.5
    lens = [MP * P, MP * P - 17]
    rng = np.random.default_rng(MP + 5)
    score = rng.integers(lo, hi, size=(B, G, MP)).astype(np.float32)
    sh = _shape(B, G, 1, MP)
    sel = torch.full((B, G, budget), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, G), -7, dtype=torch.int32, device="cuda")
    tau_lo = torch.full((B, G), theta * (alpha - 1.0), dtype=torch.float32, device="cuda")
    ws = torch.empty(ekv.select_workspace_bytes(sh, ekv.SEL_SUPERSET, alpha, budget, 3.0), dtype=torch.uint8,
                     device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ekv.select(sh, ekv.SEL_SUPERSET, sl, alpha, budget, 3.0, torch.from_numpy(score).cuda(), None, None, sel, cnt,
               tau_lo, ws)
    H.sync()
    sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        M = (lens[b] + P - 1) // P
        for g in range(G):
            want = oracle.select.superset_pages(score[b, g, :M].astype(np.float64),
                                                np.array([theta * (alpha - 1.0)]), alpha, budget)
            c = int(cnt[b, g])
            assert c == len(want), (b, g, c, len(want))
            np.testing.assert_array_equal(sel[b, g, :c], want)
            assert np.all(sel[b, g, c:] == -1)


def test_two_level_select_empty_and_short_rows():
    """Few long rows (two-level path) beside an empty row and rows shorter
    than one chunk or than the budget."""
    print("[case] two-level empty/short", flush=True)
    B, G, budget, MP = 4, 2, 128, 20000
    lens = [0, MP * P, 100 * P - 3, 4100 * P]
    rng = np.random.default_rng(404)
    score = rng.standard_normal((B, G, MP)).astype(np.float32)
    sel, cnt, _ = _run_select(_shape(B, G, 1, MP), ekv.SEL_TOPK, lens, 1.5, budget, 3.0,
                              score=torch.from_numpy(score).cuda())
    assert np.all(cnt[0] == 0) and np.all(sel[0] == -1)
    for b in range(1, B):
        M = (lens[b] + P - 1) // P
        for g in range(G):
            U = score[b, g, :M].astype(np.float64)
            want = oracle.select.topk_pages(U, budget)
            _check_rows(sel, cnt, b, g, want, U, budget)


def test_gauss_select_one_level_global_kernel():
    """256 (sequence, group) rows of 70000 pages in Gaussian mode: the
    one-level global-memory selection kernel and the threshold kernel
    without LDS staging (rows past its LDS capacity); sampled rows against
    the oracle."""
    print("[case] gauss one-level global", flush=True)
    B, G, R, MP, budget, z, alpha = 64, 4, 4, 70000, 256, 3.0, 1.5
    lens = [MP * P - 11 * (b % 5) for b in range(B)]
    rng = np.random.default_rng(70001)
    mu = (rng.standard_normal((B, G * R, MP)) * 0.25).astype(np.float32)
    sg = (0.8 + 0.4 * rng.random((B, G * R, MP))).astype(np.float32)
    sel, cnt, th = _run_select(_shape(B, G, R, MP), ekv.SEL_GAUSS, lens, alpha, budget, z,
                               mu=torch.from_numpy(mu).cuda(), sigma=torch.from_numpy(sg).cuda())
    for b in (0, B - 1):
        n = lens[b]
        M = (n + P - 1) // P
        n_p = oracle.paged.page_valid_counts(n, P)
        for h in range(G * R):
            want = oracle.select.gauss_tau_hat(mu[b, h, :M].astype(np.float64), sg[b, h, :M].astype(np.float64),
                                               n_p, alpha)
            assert H.tau_close(th[b, h], want), (b, h, th[b, h], want)
        for g in range(G):
            hs = slice(g * R, (g + 1) * R)
            m64, s64 = mu[b, hs, :M].astype(np.float64), sg[b, hs, :M].astype(np.float64)
            t = oracle.select.gauss_margins(m64, s64, th[b, hs], alpha)
            want = oracle.select.gauss_select(m64, s64, th[b, hs], alpha, z, budget)
            c = int(cnt[b, g])
            row = sel[b, g]
            assert c == len(want) or np.any(np.abs(t + z) < 1e-4 * z)
            assert np.all(row[c:] == -1) and np.all(np.diff(row[:c]) > 0)
            if c == len(want):
                H.compare_selection(row[:c], want, t, len(want))


def test_superset_select_one_level_global_kernel():
    """The superset rule on 256 rows of 70000 pages (one-level global-memory
    kernel); integer box scores and a threshold halfway between integers, as
    in the two-level case; sampled rows against the oracle."""
    print("[case] superset one-level global", flush=True)
    B, G, budget, alpha, MP, theta = 128, 2, 200, 1.5, 70000, 995.5
    lens = [MP * P - 7 * (b % 3) for b in range(B)]
    rng = np.random.default_rng(70002)
    score = rng.integers(-1000, 1001, size=(B, G, MP)).astype(np.float32)
    sh = _shape(B, G, 1, MP)
    sel = torch.full((B, G, budget), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, G), -7, dtype=torch.int32, device="cuda")
    tau_lo = torch.full((B, G), theta * (alpha - 1.0), dtype=torch.float32, device="cuda")
    ws = torch.empty(ekv.select_workspace_bytes(sh, ekv.SEL_SUPERSET, alpha, budget, 3.0), dtype=torch.uint8,
                     device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ekv.select(sh, ekv.SEL_SUPERSET, sl, alpha, budget, 3.0, torch.from_numpy(score).cuda(), None, None, sel, cnt,
               tau_lo, ws)
    H.sync()
    sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    for b in range(0, B, 17):
        M = (lens[b] + P - 1) // P
        for g in range(G):
            want = oracle.select.superset_pages(score[b, g, :M].astype(np.float64),
                                                np.array([theta * (alpha - 1.0)]), alpha, budget)
            c = int(cnt[b, g])
            assert c == len(want), (b, g, c, len(want))
            np.testing.assert_array_equal(sel[b, g, :c], want)
            assert np.all(sel[b, g, c:] == -1)


@pytest.mark.parametrize("G,R", [(4, 2), (1, 8)])
def test_gauss_select_two_level_group_sizes(G, R):
    """Two-level Gaussian selection with 2 and 8 query heads per KV group."""
    print(f"[case] gauss two-level G={G} R={R}", flush=True)
    B, MP, budget, z, alpha = 2, 20000, 256, 3.0, 1.5
    lens = [MP * P - 5, 12345 * P]
    rng = np.random.default_rng(100 * G + R)
    mu = (rng.standard_normal((B, G * R, MP)) * 0.25).astype(np.float32)
    sg = (0.8 + 0.4 * rng.random((B, G * R, MP))).astype(np.float32)
    sel, cnt, th = _run_select(_shape(B, G, R, MP), ekv.SEL_GAUSS, lens, alpha, budget, z,
                               mu=torch.from_numpy(mu).cuda(), sigma=torch.from_numpy(sg).cuda())
    for b in range(B):
        n = lens[b]
        M = (n + P - 1) // P
        for g in range(G):
            hs = slice(g * R, (g + 1) * R)
            m64, s64 = mu[b, hs, :M].astype(np.float64), sg[b, hs, :M].astype(np.float64)
            t = oracle.select.gauss_margins(m64, s64, th[b, hs], alpha)
            want = oracle.select.gauss_select(m64, s64, th[b, hs], alpha, z, budget)
            c = int(cnt[b, g])
            row = sel[b, g]
            assert c == len(want) or np.any(np.abs(t + z) < 1e-4 * z)
            assert np.all(row[c:] == -1) and np.all(np.diff(row[:c]) > 0)
            if c == len(want):
                H.compare_selection(row[:c], want, t, len(want))
