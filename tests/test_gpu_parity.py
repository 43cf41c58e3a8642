"""GPU parity of every stage of the decode step against the fp64 oracle, on
seeded workloads small enough for the oracle (several pages and tiles, ragged
tails, a sequence shorter than the budget, an empty sequence), through the C
ABI.  Source of each stage: "EntmaxKV: Support-Aware Decoding for Entmax
Attention" sections 4.1-4.3 and Appendix C.2."""

import functools

import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_ekv_amd import ekv
from sparse_long_context_ekv_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

P = 16


@functools.lru_cache(maxsize=None)
def workload(name):
    print(f"[workload] {name}", flush=True)
    if name == "tiny":
        return W.make_workload(W.CONFIGS[1], "cuda")
    if name == "llama-ragged":
        return W.make_workload(W.CONFIGS[2].scaled(batch=3), "cuda", seq_lens=[5000, 2053, 37])
    if name == "gauss-ragged":
        return W.make_workload(W.CONFIGS[3].scaled(batch=2), "cuda", seq_lens=[8197, 3001])
    if name == "tiny-ragged":
        return W.make_workload(W.CONFIGS[1].scaled(batch=2), "cuda", seq_lens=[1500, 37])
    if name == "with-empty":
        return W.make_workload(W.CONFIGS[2].scaled(batch=3), "cuda", seq_lens=[700, 0, 1601])
    if name == "flat":
        # nearly equal keys: the entmax support covers most selected tokens
        # (thousands per head), past what the decode keeps in LDS at once
        wl = W.make_workload(W.CONFIGS[2].scaled(batch=2), "cuda", seq_lens=[3000, 2400])
        g = torch.Generator(device="cuda").manual_seed(11)
        wl.k_cache.copy_((torch.randn(wl.k_cache.shape, generator=g, device="cuda") * 0.02).to(wl.k_cache.dtype))
        return wl
    if name == "long-with-empty":
        # an empty sequence beside rows of several candidate chunks
        return W.make_workload(W.CONFIGS[2].scaled(batch=3), "cuda", seq_lens=[9000, 0, 37])
    if name == "flat-long":
        # flat keys over several 4096-slot candidate chunks: in the full-cache
        # path every chunk has more threshold candidates than it may hand over,
        # so the threshold kernel compacts them itself
        wl = W.make_workload(W.CONFIGS[2].scaled(batch=2), "cuda", seq_lens=[12000, 5000])
        g = torch.Generator(device="cuda").manual_seed(12)
        wl.k_cache.copy_((torch.randn(wl.k_cache.shape, generator=g, device="cuda") * 0.02).to(wl.k_cache.dtype))
        return wl
    raise KeyError(name)


def _shape(wl, stat="f32"):
    c = wl.cfg
    return ekv.make_shape(c.batch, c.num_q_heads, c.num_kv_groups, c.head_dim, wl.max_pages, wl.num_phys,
                          c.kv_dtype, stat)


def _stats(wl, stat="f32"):
    c = wl.cfg
    NP, G, D = wl.num_phys, c.num_kv_groups, c.head_dim
    sdt = ekv.STAT_TORCH_DTYPE[stat]
    st = dict(kmin=torch.full((NP, G, D), 7.0, dtype=wl.k_cache.dtype, device="cuda"),
              kmax=torch.full((NP, G, D), 7.0, dtype=wl.k_cache.dtype, device="cuda"),
              kmean=torch.full((NP, G, D), 7.0).to(sdt).to("cuda"),
              kvar=torch.full((NP, G, D), 7.0).to(sdt).to("cuda"))
    ekv.build_page_stats(_shape(wl, stat), wl.k_cache, wl.page_table, wl.seq_lens, **st)
    return st


@pytest.mark.parametrize("name", ["tiny", "llama-ragged", "gauss-ragged"])
def test_page_stats(name):
    wl = workload(name)
    st = _stats(wl)
    H.sync()
    for b in range(wl.cfg.batch):
        q, K, V, n = H.seq_logical(wl, b)
        kmin, kmax, mean, var = oracle.paged.page_stats(K, P)
        rows = H.phys_rows(wl, b)
        np.testing.assert_array_equal(H.to_np(st["kmin"][rows]), kmin)       # bit-exact
        np.testing.assert_array_equal(H.to_np(st["kmax"][rows]), kmax)
        np.testing.assert_allclose(H.to_np(st["kmean"][rows]), mean, rtol=1e-6, atol=2e-6)
        np.testing.assert_allclose(H.to_np(st["kvar"][rows]), var, rtol=1e-6, atol=1e-6 * np.abs(var).max())


def test_page_stats_bf16_storage():
    """bf16 mean/var are the fp32 statistics rounded to nearest even."""
    wl = workload("gauss-ragged")
    st32 = _stats(wl, "f32")
    st16 = _stats(wl, "bf16")
    H.sync()
    for key in ("kmean", "kvar"):
        want = st32[key].to(torch.bfloat16)
        assert torch.equal(st16[key].view(torch.int16), want.view(torch.int16))


def test_page_stats_fp8_storage():
    """FP8 E4M3 mean/var are the fp32 statistics rounded to nearest even
    (oracle.paged.round_fp8_e4m3 applied to the fp32 statistics), code for
    code."""
    wl = workload("gauss-ragged")
    st32 = _stats(wl, "f32")
    st8 = _stats(wl, "fp8")
    H.sync()
    for key in ("kmean", "kvar"):
        want = oracle.paged.round_fp8_e4m3(H.to_np(st32[key]))
        got = st8[key].cpu().to(torch.float64).numpy()          # exact up-cast, on the host
        np.testing.assert_array_equal(got, want)


def test_page_stats_fp8_storage_d64():
    """The same on d = 64 with fp32 keys (each lane's slice of a statistic
    is then one 4-byte word), and Gaussian moments on the stored values."""
    wl = workload("tiny")
    c = wl.cfg
    st32 = _stats(wl, "f32")
    st8 = _stats(wl, "fp8")
    mu = torch.empty(c.batch, c.num_q_heads, wl.max_pages, device="cuda")
    sg = torch.empty_like(mu)
    ekv.score_pages(_shape(wl, "fp8"), ekv.SEL_GAUSS, wl.q, wl.page_table, wl.seq_lens, kmean=st8["kmean"],
                    kvar=st8["kvar"], mu=mu, sigma=sg)
    H.sync()
    for key in ("kmean", "kvar"):
        want = oracle.paged.round_fp8_e4m3(H.to_np(st32[key]))
        np.testing.assert_array_equal(st8[key].cpu().to(torch.float64).numpy(), want)
    q = H.to_np(wl.q[0])
    mean, var = _stored_stats_logical(st8, wl, 0)
    omu, osg = oracle.paged.gauss_moments(q, mean, var)
    M = omu.shape[1]
    np.testing.assert_allclose(H.to_np(mu[0, :, :M]), omu, rtol=1e-5, atol=1e-5 * np.abs(omu).max())
    np.testing.assert_allclose(H.to_np(sg[0, :, :M]), osg, rtol=1e-5, atol=1e-5 * np.abs(osg).max())


def _stored_stats_logical(st, wl, b):
    """The stored mean/var of sequence b, up-cast exactly, in logical page order."""
    rows = H.phys_rows(wl, b)
    return (st["kmean"].cpu().to(torch.float64).numpy()[rows], st["kvar"].cpu().to(torch.float64).numpy()[rows])


def test_page_stats_page_list():
    """Only the listed logical pages are (re)written."""
    wl = workload("llama-ragged")
    sh = _shape(wl)
    full = _stats(wl)
    c = wl.cfg
    part = {k: torch.zeros_like(v) for k, v in full.items()}
    picks = [(0, 0), (0, 312), (1, 128), (2, 2), (2, 50)]       # (2, 50) is past the end: skipped
    # entries that name no page of the batch are skipped too: negative ones
    # (which would divide to sequence 0 and a negative page) and b >= B
    bad = [-1, -(wl.max_pages - 1), -wl.max_pages - 5, c.batch * wl.max_pages, c.batch * wl.max_pages + 7]
    lst = torch.tensor([b * wl.max_pages + p for b, p in picks] + bad, dtype=torch.int32, device="cuda")
    ekv.build_page_stats(sh, wl.k_cache, wl.page_table, wl.seq_lens, page_list=lst, **part)
    H.sync()
    written = set()
    for b, p in picks:
        if p < (wl.seq_lens_host[b] + P - 1) // P:
            written.add(int(wl.page_table[b, p]))
    for k in part:
        for r in range(wl.num_phys):
            if r in written:
                assert torch.equal(part[k][r], full[k][r])
            else:
                assert bool((part[k][r] == 0).all())
    assert c.num_kv_groups == 8


@pytest.mark.parametrize("name", ["tiny", "llama-ragged"])
def test_box_scores(name):
    wl = workload(name)
    c = wl.cfg
    st = _stats(wl)
    score = torch.full((c.batch, c.num_kv_groups, wl.max_pages), -7.0, device="cuda")
    ekv.score_pages(_shape(wl), ekv.SEL_TOPK, wl.q, wl.page_table, wl.seq_lens, kmin=st["kmin"],
                    kmax=st["kmax"], score=score)
    H.sync()
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        kmin, kmax, _, _ = oracle.paged.page_stats(K, P)
        _, U = oracle.paged.box_scores(q, kmin, kmax)
        M = U.shape[1]
        got = H.to_np(score[b, :, :M])
        np.testing.assert_allclose(got, U, rtol=1e-5, atol=1e-5 * np.abs(U).max())
        assert bool((score[b, :, M:] == -7.0).all())                   # past the end: untouched


@pytest.mark.parametrize("name", ["tiny", "llama-ragged"])
def test_per_head_box_scores(name):
    """The optional per-head box scores of top-k scoring: u_{h,p} against the
    oracle, their maximum over a group's heads against the pooled score, -inf
    at a page whose table entry lies outside the cache, nothing written past
    a sequence's last page."""
    wl = workload(name)
    c = wl.cfg
    st = _stats(wl)
    pt = wl.page_table.clone()
    pt[0, 1] = -3                                                     # outside the cache
    score = torch.full((c.batch, c.num_kv_groups, wl.max_pages), -7.0, device="cuda")
    hs = torch.full((c.batch, c.num_q_heads, wl.max_pages), -7.0, device="cuda")
    ekv.score_pages(_shape(wl), ekv.SEL_TOPK, wl.q, pt, wl.seq_lens, kmin=st["kmin"], kmax=st["kmax"], score=score,
                    head_score=hs)
    H.sync()
    r = c.num_q_heads // c.num_kv_groups
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        kmin, kmax, _, _ = oracle.paged.page_stats(K, P)
        u, U = oracle.paged.box_scores(q, kmin, kmax)
        M = u.shape[1]
        got = H.to_np(hs[b, :, :M])
        pooled = H.to_np(score[b, :, :M])
        keep = np.ones(M, dtype=bool)
        if b == 0 and M > 1:
            assert np.all(got[:, 1] == -np.inf) and np.all(pooled[:, 1] == -np.inf)
            keep[1] = False
        np.testing.assert_allclose(got[:, keep], u[:, keep], rtol=1e-5, atol=1e-5 * np.abs(u).max())
        gmax = got.reshape(c.num_kv_groups, r, M).max(axis=1)
        np.testing.assert_allclose(gmax[:, keep], pooled[:, keep], rtol=1e-5, atol=1e-5 * np.abs(U).max())
        assert bool((hs[b, :, M:] == -7.0).all())                      # past the end: untouched


def test_scores_with_bad_table_entries():
    """A page inside a sequence whose page-table entry lies outside [0, NP)
    is never read: its box score is -inf and its moments are mu = -inf,
    sigma = 0 (a point mass below every threshold).  Every other entry is
    bitwise the same as with the intact table."""
    wl = workload("llama-ragged")
    c = wl.cfg
    st = _stats(wl)
    sh = _shape(wl)
    bad_pt = wl.page_table.clone()
    bad = [(0, 3, -3), (0, 200, wl.num_phys), (1, 5, wl.num_phys + 7), (2, 0, -1)]
    for b, p, v in bad:
        bad_pt[b, p] = v
    outs = {}
    for name, pt in (("ok", wl.page_table), ("bad", bad_pt)):
        score = torch.full((c.batch, c.num_kv_groups, wl.max_pages), 5.0, device="cuda")
        mu = torch.full((c.batch, c.num_q_heads, wl.max_pages), 5.0, device="cuda")
        sg = torch.full_like(mu, 5.0)
        ekv.score_pages(sh, ekv.SEL_TOPK, wl.q, pt, wl.seq_lens, kmin=st["kmin"], kmax=st["kmax"], score=score)
        ekv.score_pages(sh, ekv.SEL_GAUSS, wl.q, pt, wl.seq_lens, kmean=st["kmean"], kvar=st["kvar"], mu=mu,
                        sigma=sg)
        H.sync()
        outs[name] = (score, mu, sg)
    s_ok, mu_ok, sg_ok = outs["ok"]
    s_bad, mu_bad, sg_bad = outs["bad"]
    keep = torch.ones_like(s_ok, dtype=torch.bool)
    keep_h = torch.ones_like(mu_ok, dtype=torch.bool)
    for b, p, _ in bad:
        assert bool((s_bad[b, :, p] == -float("inf")).all())
        assert bool((mu_bad[b, :, p] == -float("inf")).all()) and bool((sg_bad[b, :, p] == 0).all())
        keep[b, :, p] = False
        keep_h[b, :, p] = False
    assert torch.equal(s_bad[keep], s_ok[keep])
    assert torch.equal(mu_bad[keep_h], mu_ok[keep_h]) and torch.equal(sg_bad[keep_h], sg_ok[keep_h])


@pytest.mark.parametrize("stat", ["f32", "bf16", "fp8"])
def test_gauss_moments(stat):
    wl = workload("gauss-ragged")
    c = wl.cfg
    st = _stats(wl, stat)
    mu = torch.empty(c.batch, c.num_q_heads, wl.max_pages, device="cuda")
    sg = torch.empty_like(mu)
    ekv.score_pages(_shape(wl, stat), ekv.SEL_GAUSS, wl.q, wl.page_table, wl.seq_lens, kmean=st["kmean"],
                    kvar=st["kvar"], mu=mu, sigma=sg)
    H.sync()
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        _, _, mean, var = oracle.paged.page_stats(K, P)
        if stat != "f32":
            # scoring checked on the stored 16- or 8-bit statistics themselves
            # (their rounding from the fp32 statistics has its own tests above)
            mean, var = _stored_stats_logical(st, wl, b)
        omu, osg = oracle.paged.gauss_moments(q, mean, var)
        M = omu.shape[1]
        tol = 1e-5
        np.testing.assert_allclose(H.to_np(mu[b, :, :M]), omu, rtol=tol, atol=tol * np.abs(omu).max())
        np.testing.assert_allclose(H.to_np(sg[b, :, :M]), osg, rtol=tol, atol=tol * np.abs(osg).max())


@pytest.mark.parametrize("heads,groups,dim,stat", [(8, 8, 128, "bf16"), (16, 8, 128, "fp8"), (64, 8, 128, "bf16"),
                                                   (32, 8, 64, "bf16"), (32, 8, 64, "fp8"), (12, 6, 128, "bf16"),
                                                   (8, 1, 64, "fp8")])
def test_gauss_moments_16bit_shapes(heads, groups, dim, stat):
    """bf16 queries over 16-bit / FP8 statistics take the matrix-core moments
    kernel: every r (1, 2, 8 heads per group), d = 64, group counts that
    split the block 4, 2 or 1 ways, a ragged batch whose lengths end inside
    a 16-page tile, and one page-table entry outside the cache (mu = -inf,
    sigma = 0 there); against the oracle on the stored statistics at 1e-5."""
    cfg = W.CONFIGS[3].scaled(batch=3, num_q_heads=heads, num_kv_groups=groups, head_dim=dim)
    wl = W.make_workload(cfg, "cuda", seq_lens=[1111, 4099, 37])
    c = wl.cfg
    st = _stats(wl, stat)
    pt = wl.page_table.clone()
    pt[1, 7] = wl.num_phys + 5                       # outside the cache
    mu = torch.empty(c.batch, c.num_q_heads, wl.max_pages, device="cuda")
    sg = torch.empty_like(mu)
    ekv.score_pages(_shape(wl, stat), ekv.SEL_GAUSS, wl.q, pt, wl.seq_lens, kmean=st["kmean"], kvar=st["kvar"],
                    mu=mu, sigma=sg)
    H.sync()
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        mean, var = _stored_stats_logical(st, wl, b)
        omu, osg = oracle.paged.gauss_moments(q, mean, var)
        M = omu.shape[1]
        gmu, gsg = H.to_np(mu[b, :, :M]), H.to_np(sg[b, :, :M])
        if b == 1:
            assert np.all(gmu[:, 7] == -np.inf) and np.all(gsg[:, 7] == 0.0)
            keep = np.ones(M, dtype=bool)
            keep[7] = False
            gmu, gsg, omu, osg = gmu[:, keep], gsg[:, keep], omu[:, keep], osg[:, keep]
        tol = 1e-5
        np.testing.assert_allclose(gmu, omu, rtol=tol, atol=tol * np.abs(omu).max())
        np.testing.assert_allclose(gsg, osg, rtol=tol, atol=tol * np.abs(osg).max())


@pytest.mark.parametrize("name", ["tiny", "llama-ragged"])
def test_topk_selection(name):
    wl = workload(name)
    c = wl.cfg
    dec = ekv.Decoder(wl, "topk", 1.5, c.budget_pages)
    dec.build_stats()
    dec.score()
    dec.select()
    H.sync()
    exact = 0
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        kmin, kmax, _, _ = oracle.paged.page_stats(K, P)
        _, U = oracle.paged.box_scores(q, kmin, kmax)
        for g in range(c.num_kv_groups):
            want = oracle.select.topk_pages(U[g], c.budget_pages)
            cnt = int(dec.buf.sel_count[b, g])
            row = dec.buf.sel_pages[b, g].cpu().numpy()
            assert cnt == len(want)
            assert np.all(row[cnt:] == -1) and np.all(np.diff(row[:cnt]) > 0)
            exact += H.compare_selection(row[:cnt], want, U[g], len(want))
    assert exact >= 1


def test_gauss_threshold_and_selection():
    wl = workload("gauss-ragged")
    c = wl.cfg
    cap = 64
    dec = ekv.Decoder(wl, "gauss", 1.5, cap, z=c.z)
    dec.build_stats()
    dec.score()
    dec.select()
    H.sync()
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        res = oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "gauss", 1.5, cap, z=c.z)
        th = H.to_np(dec.buf.tau_hat[b])
        for h in range(c.num_q_heads):
            assert H.tau_close(th[h], res["tau_hat"][h]), (h, th[h], res["tau_hat"][h])
            assert abs(oracle.select.gauss_F(th[h], res["mu"][h], res["sigma"][h], res["n_p"], 1.5)) < 1e-3
        for g in range(c.num_kv_groups):
            t = res["margins"][g]
            want = res["sel"][g]
            cnt = int(dec.buf.sel_count[b, g])
            got = dec.buf.sel_pages[b, g, :cnt].cpu().numpy()
            assert np.all(dec.buf.sel_pages[b, g, cnt:].cpu().numpy() == -1)
            near_z = np.any(np.abs(t + c.z) < 1e-3 * max(1.0, c.z))
            if not near_z and len(want) < cap:
                np.testing.assert_array_equal(got, want)
            else:
                H.compare_selection(got, want, t, len(want), rel=1e-3)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_gauss_selection_fp8_statistics(alpha):
    """The Gaussian selector on FP8 E4M3 page mean/variance: threshold and
    page set against the oracle run on the same stored statistics."""
    wl = workload("gauss-ragged")
    c = wl.cfg
    cap = 64
    dec = ekv.Decoder(wl, "gauss", alpha, cap, z=c.z, stat_dtype="fp8")
    dec.build_stats()
    dec.score()
    dec.select()
    H.sync()
    r = c.num_q_heads // c.num_kv_groups
    for b in range(c.batch):
        q = H.to_np(wl.q[b])
        n = wl.seq_lens_host[b]
        mean, var = _stored_stats_logical(dec.stats, wl, b)
        mu, sg = oracle.paged.gauss_moments(q, mean, var)
        n_p = oracle.paged.page_valid_counts(n, P)
        th = np.array([oracle.select.gauss_tau_hat(mu[h], sg[h], n_p, alpha) for h in range(c.num_q_heads)])
        got_th = H.to_np(dec.buf.tau_hat[b])
        for h in range(c.num_q_heads):
            assert H.tau_close(got_th[h], th[h]), (b, h, got_th[h], th[h])
        for g in range(c.num_kv_groups):
            hs = slice(g * r, (g + 1) * r)
            t = oracle.select.gauss_margins(mu[hs], sg[hs], th[hs], alpha)
            want = oracle.select.gauss_select(mu[hs], sg[hs], th[hs], alpha, c.z, cap)
            cnt = int(dec.buf.sel_count[b, g])
            got = dec.buf.sel_pages[b, g, :cnt].cpu().numpy()
            H.compare_selection(got, want, t, len(want), rel=1e-3)


def _oracle_sel_tensor(sels, B, G, budget):
    t = torch.full((B, G, budget), -1, dtype=torch.int32)
    cnt = torch.zeros(B, G, dtype=torch.int32)
    for b in range(B):
        for g in range(G):
            s = sels[b][g]
            t[b, g, :len(s)] = torch.as_tensor(s, dtype=torch.int32)
            cnt[b, g] = len(s)
    return t.cuda(), cnt.cuda()


def _run_decode(wl, alpha, sel=None, cnt=None, stride=0, tau_ref=None, tau_hint=None):
    c = wl.cfg
    sh = _shape(wl)
    out = torch.empty(c.batch, c.num_q_heads, c.head_dim, device="cuda")
    tau = torch.empty(c.batch, c.num_q_heads, device="cuda")
    sup = torch.empty(c.batch, c.num_q_heads, dtype=torch.int32, device="cuda")
    delta = torch.empty_like(tau) if tau_ref is not None else None
    supref = torch.empty_like(sup) if tau_ref is not None else None
    ws = torch.empty(ekv.decode_workspace_bytes(sh, sel is not None, stride, alpha), dtype=torch.uint8, device="cuda")
    ekv.entmax_decode(sh, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, sel, cnt, stride, alpha,
                      out, tau, ws, support=sup, delta=delta, tau_ref=tau_ref, support_ref=supref, tau_hint=tau_hint)
    H.sync()
    return out, tau, sup, delta, supref


def _support_slack(s_row, tau, alpha):
    if alpha == 1.0:
        return 0
    x = (alpha - 1.0) * s_row
    return int(np.count_nonzero(np.abs(x - tau) < 1e-5 * max(1.0, abs(tau))))


@pytest.mark.parametrize("name,alpha", [("tiny", 1.5), ("tiny", 2.0), ("tiny", 1.0), ("tiny", 4.0 / 3.0),
                                        ("tiny", 3.0), ("llama-ragged", 1.5), ("llama-ragged", 1.0),
                                        ("llama-ragged", 2.0), ("llama-ragged", 4.0 / 3.0), ("llama-ragged", 3.0),
                                        ("flat-long", 1.5), ("long-with-empty", 1.5), ("long-with-empty", 1.0)])
def test_full_cache_decode(name, alpha):
    """Full-cache decode (every token) against the oracle: the streamed
    candidate path, several candidate lists per head on the longer rows
    (llama-ragged: 5000 tokens), and the threshold kernel's list-reading
    fallback when a head has more than 8192 candidates (flat-long); an empty
    sequence gives out 0, tau -inf and support 0 (entmax over no token is
    undefined)."""
    wl = workload(name)
    c = wl.cfg
    out, tau, sup, _, _ = _run_decode(wl, alpha)
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        if n == 0:
            assert bool((out[b] == 0).all()) and bool((tau[b] == -float("inf")).all())
            assert bool((sup[b] == 0).all())
            continue
        ref = oracle.decode.decode(q, K, V, None, alpha)
        assert np.abs(H.to_np(out[b]) - ref["out"]).max() <= H.OUT_ATOL
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau[b, h]), ref["tau"][h])
            slack = _support_slack(ref["s"][h], ref["tau"][h], alpha)
            assert abs(int(sup[b, h]) - int(ref["support"][h])) <= slack


@pytest.mark.parametrize("name,alpha", [("tiny", 1.5), ("tiny", 2.0), ("tiny", 1.0), ("tiny", 4.0 / 3.0),
                                        ("tiny", 3.0), ("llama-ragged", 1.5), ("llama-ragged", 1.0),
                                        ("llama-ragged", 2.0), ("gauss-ragged", 1.5), ("flat", 1.5), ("flat", 2.0),
                                        ("flat", 4.0 / 3.0), ("llama-ragged-wide", 1.5), ("llama-ragged-wide", 1.0),
                                        ("llama-ragged-wide", 2.0)])
def test_sparse_decode_on_oracle_selection(name, alpha):
    """Decode over a given selection (the oracle's top-k), with the dropped
    mass measured against the full-cache threshold.  "llama-ragged-wide"
    selects 300 pages (4800 slots) per group: past the fused kernel's 4096
    slots, so it takes the general path (and, for entmax, the multi-block
    threshold-candidate compaction) with a selection."""
    wl = workload("llama-ragged" if name == "llama-ragged-wide" else name)
    c = wl.cfg
    budget = {"gauss-ragged": 64, "flat": 256, "llama-ragged-wide": 300}.get(name, c.budget_pages)
    sels, fulls = [], []
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        res = oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", alpha, budget)
        sels.append(res["sel"])
    sel, cnt = _oracle_sel_tensor(sels, c.batch, c.num_kv_groups, budget)
    _, tau_full, sup_full, _, _ = _run_decode(wl, alpha)
    out, tau, sup, delta, supref = _run_decode(wl, alpha, sel, cnt, budget, tau_ref=tau_full)
    r = c.num_q_heads // c.num_kv_groups
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels[b], alpha)
        full = oracle.decode.decode(q, K, V, None, alpha)
        assert np.abs(H.to_np(out[b]) - sp["out"]).max() <= H.OUT_ATOL
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau[b, h]), sp["tau"][h])
            toks = sp["tokens_per_group"][h // r]
            d_or = oracle.decode.dropped_mass_from_tau(full["s"][h][toks], full["tau"][h], alpha)
            assert abs(float(delta[b, h]) - d_or) <= H.DELTA_ATOL
            s_sel = full["s"][h][toks]
            assert abs(int(sup[b, h]) - int(sp["support"][h])) <= _support_slack(s_sel, sp["tau"][h], alpha)
            # support recall rho: full-cache support tokens inside the selection
            rho = oracle.decode.metrics(full, {"tokens": toks, "out": sp["out"]}, n)["rho"][h]
            kept_or = int(round(rho * max(int(np.count_nonzero(full["p"][h] > 0)), 1)))
            assert abs(int(supref[b, h]) - kept_or) <= _support_slack(s_sel, full["tau"][h], alpha), (b, h)
            if alpha == 1.0:
                assert int(supref[b, h]) == len(toks)          # softmax: rho is the coverage
            assert int(supref[b, h]) <= int(sup_full[b, h]) + _support_slack(full["s"][h], full["tau"][h], alpha)


@pytest.mark.parametrize("heads,groups,dim,alpha", [(8, 8, 128, 1.5), (16, 8, 64, 1.5), (64, 8, 128, 1.5),
                                                    (32, 8, 64, 2.0), (12, 6, 128, 4.0 / 3.0), (8, 1, 64, 1.5),
                                                    (8, 8, 128, 1.0), (16, 8, 64, 1.0), (64, 8, 128, 1.0),
                                                    (32, 8, 128, 1.0)])
def test_decode_shapes_bf16(heads, groups, dim, alpha):
    """bf16 keys at every r (1, 2, 4, 8) and d = 64: the matrix-core logits
    of the fused path (on the oracle's top-k selection) and the matrix-core
    candidate stream of the full-cache path, against the oracle; a ragged
    batch with a sequence ending inside a page.  alpha = 1: the one-pass
    softmax, over the selection and over the whole cache."""
    cfg = W.CONFIGS[3].scaled(batch=3, num_q_heads=heads, num_kv_groups=groups, head_dim=dim)
    wl = W.make_workload(cfg, "cuda", seq_lens=[1499, 37, 2900])
    c = wl.cfg
    budget = 48
    sels = []
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sels.append(oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", alpha, budget)["sel"])
    sel, cnt = _oracle_sel_tensor(sels, c.batch, c.num_kv_groups, budget)
    out_s, tau_s, sup_s, _, _ = _run_decode(wl, alpha, sel, cnt, budget)
    out_f, tau_f, sup_f, _, _ = _run_decode(wl, alpha)
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels[b], alpha)
        full = oracle.decode.decode(q, K, V, None, alpha)
        assert np.abs(H.to_np(out_s[b]) - sp["out"]).max() <= H.OUT_ATOL, b
        assert np.abs(H.to_np(out_f[b]) - full["out"]).max() <= H.OUT_ATOL, b
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau_s[b, h]), sp["tau"][h]), (b, h)
            assert H.tau_close(float(tau_f[b, h]), full["tau"][h]), (b, h)
            assert abs(int(sup_f[b, h]) - int(full["support"][h])) <= _support_slack(full["s"][h], full["tau"][h],
                                                                                      alpha)


@pytest.mark.parametrize("name", ["tiny", "llama-ragged"])
def test_pipeline_end_to_end(name):
    wl = workload(name)
    c = wl.cfg
    dec = ekv.Decoder(wl, "topk", 1.5, c.budget_pages)
    dec.build_stats()
    dec.step()
    H.sync()
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        res = oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", 1.5, c.budget_pages)
        same = all(np.array_equal(dec.buf.sel_pages[b, g, :int(dec.buf.sel_count[b, g])].cpu().numpy(), res["sel"][g])
                   for g in range(c.num_kv_groups))
        assert same, "selection differs on a separated cutoff"
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, res["sel"], 1.5)
        assert np.abs(H.to_np(dec.buf.out[b]) - sp["out"]).max() <= H.OUT_ATOL


def test_empty_sequence_and_short_sequence():
    wl = workload("with-empty")
    c = wl.cfg
    dec = ekv.Decoder(wl, "topk", 1.5, c.budget_pages)
    dec.build_stats()
    dec.step()
    H.sync()
    assert bool((dec.buf.sel_count[1] == 0).all())
    assert bool((dec.buf.sel_pages[1] == -1).all())
    assert bool((dec.buf.out[1] == 0).all()) and bool(torch.isinf(dec.buf.tau[1]).all())
    assert bool((dec.buf.support[1] == 0).all())
    # 700 tokens = 44 pages < budget 128: every page is selected.
    assert bool((dec.buf.sel_count[0] == 44).all())
    q, K, V, n = H.seq_logical(wl, 0)
    ref = oracle.decode.decode(q, K, V, None, 1.5)
    assert np.abs(H.to_np(dec.buf.out[0]) - ref["out"]).max() <= H.OUT_ATOL


@pytest.mark.parametrize("alpha", [1.5, 1.0])
def test_full_cache_many_sequences(alpha):
    """Full-cache decode of a batch of 300 ragged sequences (past the 256
    that the streamed path orders by length inside each block: the one-block
    ordering kernel runs), with empty and one-token sequences among them;
    sampled sequences against the oracle (entmax and the one-pass softmax)."""
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(1, 700, size=300)]
    lens[3], lens[100], lens[299] = 0, 1, 2500
    cfg = W.CONFIGS[2].scaled(batch=300)
    wl = W.make_workload(cfg, "cuda", seq_lens=lens)
    c = wl.cfg
    out, tau, sup, _, _ = _run_decode(wl, alpha)
    for b in (0, 3, 100, 157, 298, 299):
        q, K, V, n = H.seq_logical(wl, b)
        if n == 0:
            assert bool((out[b] == 0).all()) and bool((tau[b] == -float("inf")).all())
            continue
        ref = oracle.decode.decode(q, K, V, None, alpha)
        assert np.abs(H.to_np(out[b]) - ref["out"]).max() <= H.OUT_ATOL
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau[b, h]), ref["tau"][h])


@pytest.mark.parametrize("name,alpha", [("llama-ragged", 1.5), ("llama-ragged", 2.0), ("long-with-empty", 1.5),
                                        ("llama-ragged", 1.0)])
def test_full_cache_bitwise_reproducible(name, alpha):
    """The streamed full-cache path shares its running max between a block's
    waves through an atomic, so the candidate lists may hold other extra
    entries from run to run; the results must not change, bit for bit."""
    wl = workload(name)
    first = _run_decode(wl, alpha)
    for _ in range(3):
        again = _run_decode(wl, alpha)
        for a, b in zip(first[:3], again[:3]):
            assert torch.equal(a, b)


def test_softmax_large_logits():
    """Softmax over logits in the hundreds (the query scaled by 40): every
    block's sums are taken relative to its running max and the merge
    rescales them, so nothing overflows; against the oracle, full cache
    and over a selection."""
    base = workload("llama-ragged")
    wl = W.Workload(cfg=base.cfg, q=(base.q.float() * 40.0).to(base.q.dtype), k_cache=base.k_cache,
                    v_cache=base.v_cache, page_table=base.page_table, seq_lens=base.seq_lens,
                    seq_lens_host=base.seq_lens_host, max_pages=base.max_pages, num_phys=base.num_phys, planted={})
    c = wl.cfg
    budget = 40
    sels = []
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sels.append(oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", 1.0, budget)["sel"])
    sel, cnt = _oracle_sel_tensor(sels, c.batch, c.num_kv_groups, budget)
    out_f, tau_f, sup_f, _, _ = _run_decode(wl, 1.0)
    out_s, tau_s, _, _, _ = _run_decode(wl, 1.0, sel, cnt, budget)
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        full = oracle.decode.decode(q, K, V, None, 1.0)
        assert float(np.abs(full["s"]).max()) > 100.0
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels[b], 1.0)
        assert np.abs(H.to_np(out_f[b]) - full["out"]).max() <= H.OUT_ATOL, b
        assert np.abs(H.to_np(out_s[b]) - sp["out"]).max() <= H.OUT_ATOL, b
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau_f[b, h]), full["tau"][h]), (b, h)
            assert H.tau_close(float(tau_s[b, h]), sp["tau"][h]), (b, h)
            assert int(sup_f[b, h]) == n


@pytest.mark.parametrize("name", ["llama-ragged", "tiny-ragged"])
@pytest.mark.parametrize("alpha", [1.0, 1.5, 2.0])
def test_nan_outside_the_sequences(name, alpha):
    """Cache slots that belong to no token hold NaN: the unused tail of every
    sequence's last page and an unreferenced physical page 0 (the page the
    kernels read in place of one past a range).  Decode over the whole cache
    and over a selection that includes each last page must not see them
    (bf16 keys: llama-ragged; fp32 keys: tiny-ragged)."""
    base = workload(name)
    c = base.cfg
    nan = float("nan")
    kc = torch.full((base.num_phys + 1,) + tuple(base.k_cache.shape[1:]), nan, dtype=base.k_cache.dtype, device="cuda")
    vc = torch.full_like(kc, nan)
    kc[1:] = base.k_cache
    vc[1:] = base.v_cache
    pt = base.page_table + 1
    for b, n in enumerate(base.seq_lens_host):
        M = (n + P - 1) // P
        if n % P:
            last = int(pt[b, M - 1])
            kc[last, :, n % P:] = nan
            vc[last, :, n % P:] = nan
    wl = W.Workload(cfg=c, q=base.q, k_cache=kc, v_cache=vc, page_table=pt, seq_lens=base.seq_lens,
                    seq_lens_host=base.seq_lens_host, max_pages=base.max_pages, num_phys=base.num_phys + 1,
                    planted={})
    stride = 48
    sels = []
    for b, n in enumerate(base.seq_lens_host):
        M = (n + P - 1) // P
        pages = sorted(set(range(min(M, stride - 1))) | ({M - 1} if M else set()))
        sels.append([np.array(pages, dtype=np.int64) for _ in range(c.num_kv_groups)])
    sel, cnt = _oracle_sel_tensor(sels, c.batch, c.num_kv_groups, stride)
    out_f, tau_f, _, _, _ = _run_decode(wl, alpha)
    out_s, tau_s, _, _, _ = _run_decode(wl, alpha, sel, cnt, stride)
    assert bool(torch.isfinite(out_f).all()) and bool(torch.isfinite(out_s).all())
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(base, b)
        full = oracle.decode.decode(q, K, V, None, alpha)
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels[b], alpha)
        assert np.abs(H.to_np(out_f[b]) - full["out"]).max() <= H.OUT_ATOL, b
        assert np.abs(H.to_np(out_s[b]) - sp["out"]).max() <= H.OUT_ATOL, b
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau_f[b, h]), full["tau"][h]), (b, h)
            assert H.tau_close(float(tau_s[b, h]), sp["tau"][h]), (b, h)


@pytest.mark.parametrize("name,alpha,budget", [("llama-ragged", 1.0, 40), ("llama-ragged", 1.5, 40),
                                               ("llama-ragged", 2.0, 300), ("llama-ragged", 1.0, 300),
                                               ("tiny-ragged", 1.0, 40), ("tiny-ragged", 1.5, 40)])
def test_decode_skips_invalid_selected_pages(name, alpha, budget):
    """Selections that name pages outside the sequence (-1, the page count,
    beyond it) and a selected page whose table entry lies outside the cache:
    those contribute no token; the rest decode as the oracle does on the valid
    pages (fused and one-pass paths at 40 pages, the streamed paths at 300)."""
    base = workload(name)
    c = base.cfg
    stride = budget + 3
    pt = base.page_table.clone()
    sels, bad = [], None
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(base, b)
        sels.append(oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", alpha, budget)["sel"])
    bad = int(sels[0][0][0])                              # page of sequence 0 with an unreadable table entry
    pt[0, bad] = -5
    wl = W.Workload(cfg=c, q=base.q, k_cache=base.k_cache, v_cache=base.v_cache, page_table=pt,
                    seq_lens=base.seq_lens, seq_lens_host=base.seq_lens_host, max_pages=base.max_pages,
                    num_phys=base.num_phys, planted={})
    given, valid = [], []
    for b in range(c.batch):
        M = (base.seq_lens_host[b] + P - 1) // P
        given.append([np.concatenate([sg, np.array([-1, M, M + 7], dtype=np.int64)]) for sg in sels[b]])
        valid.append([sg[sg != bad] if b == 0 else sg for sg in sels[b]])
    sel, cnt = _oracle_sel_tensor(given, c.batch, c.num_kv_groups, stride)
    out, tau, sup, _, _ = _run_decode(wl, alpha, sel, cnt, stride)
    assert bool(torch.isfinite(out).all())
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(base, b)
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, valid[b], alpha)
        assert np.abs(H.to_np(out[b]) - sp["out"]).max() <= H.OUT_ATOL, b
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau[b, h]), sp["tau"][h]), (b, h)


@pytest.mark.parametrize("alpha,budget", [(1.0, 40), (1.5, 40), (2.0, 300)])
def test_decode_page_named_twice(alpha, budget):
    """A selection that names a page twice decodes over its tokens twice, as
    the oracle does over the same page list (fused or one-pass at 40 pages,
    streamed at 300)."""
    wl = workload("llama-ragged")
    c = wl.cfg
    stride = budget + 3
    sels = []
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sg = oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", alpha, budget)["sel"]
        sels.append([np.concatenate([x, x[:3]]) for x in sg])
    sel, cnt = _oracle_sel_tensor(sels, c.batch, c.num_kv_groups, stride)
    out, tau, _, _, _ = _run_decode(wl, alpha, sel, cnt, stride)
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels[b], alpha)
        assert np.abs(H.to_np(out[b]) - sp["out"]).max() <= H.OUT_ATOL, b
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau[b, h]), sp["tau"][h]), (b, h)


def test_bitwise_reproducible():
    wl = workload("llama-ragged")
    dec = ekv.Decoder(wl, "topk", 1.5, wl.cfg.budget_pages)
    dec.build_stats()
    dec.step()
    H.sync()
    a = (dec.buf.out.clone(), dec.buf.tau.clone(), dec.buf.sel_pages.clone(), dec.buf.score.clone())
    dec.step()
    H.sync()
    b = (dec.buf.out, dec.buf.tau, dec.buf.sel_pages, dec.buf.score)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    # score entries past a sequence's last page are never written: compare
    # only the written ones (the rest hold whatever the buffer held).
    for bb, n in enumerate(wl.seq_lens_host):
        M = (n + P - 1) // P
        assert torch.equal(a[3][bb, :, :M], b[3][bb, :, :M])


def test_physical_placement_invariance():
    """Same logical cache at other physical pages: identical results, bit for bit."""
    wl = workload("llama-ragged")
    dec = ekv.Decoder(wl, "topk", 1.5, wl.cfg.budget_pages)
    dec.build_stats()
    dec.step()
    H.sync()
    perm = torch.randperm(wl.num_phys, generator=torch.Generator().manual_seed(5)).cuda()
    wl2 = W.Workload(cfg=wl.cfg, q=wl.q, k_cache=torch.empty_like(wl.k_cache), v_cache=torch.empty_like(wl.v_cache),
                     page_table=perm[wl.page_table.long()].to(torch.int32), seq_lens=wl.seq_lens,
                     seq_lens_host=wl.seq_lens_host, max_pages=wl.max_pages, num_phys=wl.num_phys, planted={})
    wl2.k_cache[perm] = wl.k_cache
    wl2.v_cache[perm] = wl.v_cache
    dec2 = ekv.Decoder(wl2, "topk", 1.5, wl.cfg.budget_pages)
    dec2.build_stats()
    dec2.step()
    H.sync()
    assert torch.equal(dec.buf.out, dec2.buf.out)
    assert torch.equal(dec.buf.sel_pages, dec2.buf.sel_pages)


@pytest.mark.parametrize("name,alpha", [("llama-ragged", 1.5), ("llama-ragged", 2.0), ("llama-ragged", 4.0 / 3.0),
                                        ("llama-ragged-wide", 1.5), ("llama-ragged-wide", 2.0),
                                        ("llama-ragged-wide", 4.0 / 3.0)])
def test_decode_threshold_hint(name, alpha):
    """Decode with a start for the threshold iteration (the hand-off of the
    selection's threshold estimate to decode, "EntmaxKV" section 4.4): hints
    left of the root, at it, right of it, at and past the largest score,
    +-inf and NaN all give the oracle's threshold, support and output on the
    selected tokens.  "llama-ragged-wide" (300 pages) takes the general path."""
    wl = workload("llama-ragged")
    c = wl.cfg
    budget = 300 if name == "llama-ragged-wide" else c.budget_pages
    sels = []
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sels.append(oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", alpha, budget)["sel"])
    sel, cnt = _oracle_sel_tensor(sels, c.batch, c.num_kv_groups, budget)
    ref = []
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        ref.append(oracle.decode.sparse_decode_groups(q, K, V, n, P, sels[b], alpha))
    # per-head x range over the selected tokens, from the oracle
    r = c.num_q_heads // c.num_kv_groups
    xmax = torch.zeros(c.batch, c.num_q_heads, dtype=torch.float64)
    tau_or = torch.zeros(c.batch, c.num_q_heads, dtype=torch.float64)
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        for h in range(c.num_q_heads):
            toks = ref[b]["tokens_per_group"][h // r]
            s_h = oracle.paged.token_scores(q[h:h + 1], K[:, h // r:h // r + 1, :], toks)[0]
            xmax[b, h] = (alpha - 1.0) * s_h.max()
            tau_or[b, h] = ref[b]["tau"][h]
    hints = {
        "left": 0.5 * (xmax - 1.0 + tau_or), "root": tau_or, "right": 0.5 * (tau_or + xmax),
        "near_max": xmax - 1e-3, "max": xmax, "past_max": xmax + 5.0, "+inf": torch.full_like(xmax, float("inf")),
        "-inf": torch.full_like(xmax, -float("inf")), "nan": torch.full_like(xmax, float("nan")),
    }
    base_out, base_tau, base_sup, _, _ = _run_decode(wl, alpha, sel, cnt, budget)
    for hname, hv in hints.items():
        print(f"[case] {name} alpha={alpha} hint={hname}", flush=True)
        out, tau, sup, _, _ = _run_decode(wl, alpha, sel, cnt, budget, tau_hint=hv.float().cuda())
        for b in range(c.batch):
            assert np.abs(H.to_np(out[b]) - ref[b]["out"]).max() <= H.OUT_ATOL, (hname, b)
            for h in range(c.num_q_heads):
                assert H.tau_close(float(tau[b, h]), ref[b]["tau"][h]), (hname, b, h, float(tau[b, h]), ref[b]["tau"][h])
        # the same threshold as without a hint, up to fp32 rounding
        np.testing.assert_allclose(H.to_np(tau), H.to_np(base_tau), rtol=2e-6, atol=2e-6)
        np.testing.assert_allclose(H.to_np(out), H.to_np(base_out), rtol=0, atol=2e-5)
        assert int((sup - base_sup).abs().max()) <= 1


@pytest.mark.parametrize("alpha", [4.0 / 3.0, 1.5, 2.0])
def test_gaussian_step_with_threshold_hint(alpha):
    """The Gaussian-selector step as bench times it: decode starts from the
    selection's threshold estimate tau_hat; output and threshold against the
    oracle's decode on the GPU's selection, and equal (to rounding) to the
    same decode started without the estimate."""
    wl = workload("gauss-ragged")
    c = wl.cfg
    cap = 64
    dec = ekv.Decoder(wl, "gauss", alpha, cap, z=c.z)
    dec.build_stats()
    dec.step()
    H.sync()
    out_h, tau_h = dec.buf.out.clone(), dec.buf.tau.clone()
    nohint = ekv.Decoder(wl, "gauss", alpha, cap, z=c.z, tau_hint=False)
    nohint.stats = dec.stats
    nohint.score()
    nohint.select()
    nohint.decode()
    H.sync()
    assert torch.equal(nohint.buf.sel_pages, dec.buf.sel_pages)
    np.testing.assert_allclose(H.to_np(tau_h), H.to_np(nohint.buf.tau), rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(H.to_np(out_h), H.to_np(nohint.buf.out), rtol=0, atol=2e-5)
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sels = [dec.buf.sel_pages[b, g, :int(dec.buf.sel_count[b, g])].cpu().numpy() for g in range(c.num_kv_groups)]
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels, alpha)
        assert np.abs(H.to_np(out_h[b]) - sp["out"]).max() <= H.OUT_ATOL
        for h in range(c.num_q_heads):
            assert H.tau_close(float(tau_h[b, h]), sp["tau"][h]), (b, h)
