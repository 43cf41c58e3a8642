"""GPU tests of ekv_append_kv: one token per sequence per call written
through the page table, with the statistics of its page refreshed ("EntmaxKV:
Support-Aware Decoding for Entmax Attention" section 4.2 for what a page's
metadata is).  After any number of appends the statistics must equal a
rebuild from the cache bit for bit, and the oracle's statistics of the grown
sequences to the usual tolerances."""

import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_ekv_amd import ekv
from sparse_long_context_ekv_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

P = 16


def _stats_buffers(wl, stat):
    c = wl.cfg
    NP, G, D = wl.num_phys, c.num_kv_groups, c.head_dim
    sdt = ekv.STAT_TORCH_DTYPE[stat]
    return dict(kmin=torch.full((NP, G, D), 7.0, dtype=wl.k_cache.dtype, device="cuda"),
                kmax=torch.full((NP, G, D), 7.0, dtype=wl.k_cache.dtype, device="cuda"),
                kmean=torch.full((NP, G, D), 7.0).to(sdt).to("cuda"),
                kvar=torch.full((NP, G, D), 7.0).to(sdt).to("cuda"))


def _bits(t):
    """Storage bits of a tensor, for bit-for-bit comparison."""
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16) if t.element_size() == 2 else t


def _grown_workload(base, extra, cfg):
    """Sequences generated `extra` tokens longer than `base`, then cut back to
    `base`: the pages an append will fill are mapped and hold stale data."""
    wl = W.make_workload(cfg, "cuda", seq_lens=[n + extra for n in base])
    wl.seq_lens.copy_(torch.tensor(base, dtype=torch.int32))
    wl.seq_lens_host = list(base)
    return wl


@pytest.mark.parametrize("stat", ["f32", "bf16", "fp8"])
def test_append_matches_rebuild_and_oracle(stat):
    T = 20
    base = [5000, 2048, 0, 37]            # mid-page, page boundary, empty, short
    cfg = W.CONFIGS[2].scaled(batch=len(base))
    wl = _grown_workload(base, T, cfg)
    c = wl.cfg
    B, G, D = c.batch, c.num_kv_groups, c.head_dim
    sh = ekv.make_shape(B, c.num_q_heads, G, D, wl.max_pages, wl.num_phys, c.kv_dtype, stat)
    st = _stats_buffers(wl, stat)
    ekv.build_page_stats(sh, wl.k_cache, wl.page_table, wl.seq_lens, **st)
    k_before = wl.k_cache.clone()
    gen = torch.Generator(device="cuda").manual_seed(9)
    new_lens = torch.empty_like(wl.seq_lens)
    ks, vs = [], []
    for _ in range(T):
        kn = torch.randn(B, G, D, generator=gen, device="cuda").to(wl.k_cache.dtype)
        vn = torch.randn(B, G, D, generator=gen, device="cuda").to(wl.k_cache.dtype)
        ekv.append_kv(sh, kn, vn, wl.page_table, wl.seq_lens, wl.k_cache, wl.v_cache, new_lens=new_lens, **st)
        wl.seq_lens.copy_(new_lens)
        ks.append(kn)
        vs.append(vn)
    H.sync()
    assert wl.seq_lens.cpu().tolist() == [n + T for n in base]
    wl.seq_lens_host = [n + T for n in base]
    fresh = _stats_buffers(wl, stat)
    ekv.build_page_stats(sh, wl.k_cache, wl.page_table, wl.seq_lens, **fresh)
    H.sync()
    K_new = torch.stack(ks, dim=1).double().cpu().numpy()     # [B][T][G][D]
    V_new = torch.stack(vs, dim=1).double().cpu().numpy()
    for b in range(B):
        rows = H.phys_rows(wl, b)
        for key in st:                                          # bit for bit against a rebuild
            assert torch.equal(_bits(st[key])[rows], _bits(fresh[key])[rows]), (b, key)
        q, K, V, n = H.seq_logical(wl, b)
        np.testing.assert_array_equal(K[base[b]:], K_new[b])   # appended tokens stored exactly
        np.testing.assert_array_equal(V[base[b]:], V_new[b])
        pre = H.seq_tokens_f64(k_before, wl, b, np.arange(base[b])) if base[b] else np.zeros((0, G, D))
        np.testing.assert_array_equal(K[:base[b]], pre)         # earlier tokens untouched
        kmin, kmax, mean, var = oracle.paged.page_stats(K, P)
        np.testing.assert_array_equal(H.to_np(st["kmin"][rows]), kmin)
        np.testing.assert_array_equal(H.to_np(st["kmax"][rows]), kmax)
        if stat == "f32":
            np.testing.assert_allclose(H.to_np(st["kmean"][rows]), mean, rtol=1e-6, atol=2e-6)
            np.testing.assert_allclose(H.to_np(st["kvar"][rows]), var, rtol=1e-5, atol=1e-5)


def test_append_skips_full_sequences_and_then_decodes():
    """A sequence with no mapped page left is untouched (its length is
    returned unchanged); a decode step on the grown cache matches the oracle."""
    base = [64 * 16, 300]                 # the first sequence fills all 64 of its pages
    cfg = W.CONFIGS[1].scaled(batch=2)
    wl = W.make_workload(cfg, "cuda", seq_lens=[base[0], base[1] + 1])
    wl.seq_lens.copy_(torch.tensor(base, dtype=torch.int32))
    wl.seq_lens_host = list(base)
    c = wl.cfg
    B, G, D = c.batch, c.num_kv_groups, c.head_dim
    assert wl.max_pages == 64
    sh = ekv.make_shape(B, c.num_q_heads, G, D, wl.max_pages, wl.num_phys, c.kv_dtype, "f32")
    dec = ekv.Decoder(wl, "topk", 1.5, 8)
    dec.build_stats()
    kc, vc = wl.k_cache.clone(), wl.v_cache.clone()
    kn = torch.randn(B, G, D, device="cuda", generator=torch.Generator(device="cuda").manual_seed(4))
    vn = torch.randn(B, G, D, device="cuda", generator=torch.Generator(device="cuda").manual_seed(5))
    new_lens = torch.empty_like(wl.seq_lens)
    ekv.append_kv(sh, kn, vn, wl.page_table, wl.seq_lens, wl.k_cache, wl.v_cache, new_lens=new_lens, **dec.stats)
    H.sync()
    assert new_lens.cpu().tolist() == [base[0], base[1] + 1]
    rows0 = H.phys_rows(wl, 0)
    assert torch.equal(wl.k_cache[rows0], kc[rows0]) and torch.equal(wl.v_cache[rows0], vc[rows0])
    wl.seq_lens.copy_(new_lens)
    wl.seq_lens_host = new_lens.cpu().tolist()
    dec.step()
    H.sync()
    for b in range(B):
        q, K, V, n = H.seq_logical(wl, b)
        res = oracle.decode.select_pages(q, K, n, P, G, "topk", 1.5, 8)
        for g in range(G):
            cnt = int(dec.buf.sel_count[b, g])
            kmin, kmax, _, _ = oracle.paged.page_stats(K, P)
            _, U = oracle.paged.box_scores(q, kmin, kmax)
            H.compare_selection(dec.buf.sel_pages[b, g, :cnt].cpu().numpy(), res["sel"][g], U[g], len(res["sel"][g]))
        sels = [dec.buf.sel_pages[b, g, :int(dec.buf.sel_count[b, g])].cpu().numpy() for g in range(G)]
        sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels, 1.5)
        assert np.abs(H.to_np(dec.buf.out[b]) - sp["out"]).max() <= H.OUT_ATOL
