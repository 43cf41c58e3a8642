"""ekv_entmax_decode_noalloc (the decode on the library's static per-GPU
scratch, for callers that cannot allocate) against ekv_entmax_decode with a
caller workspace, through the C ABI: two calls in a row on the same GPU,
the second on a smaller input, each equal bit for bit to the workspace
entry point on the same inputs (same kernels, same arithmetic), and both
within the decode tolerances of the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_ekv_amd import ekv
from sparse_long_context_ekv_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

P = 16


def _shape(wl):
    c = wl.cfg
    return ekv.make_shape(c.batch, c.num_q_heads, c.num_kv_groups, c.head_dim, wl.max_pages, wl.num_phys,
                          c.kv_dtype, "f32")


def _oracle_selection(wl, budget, alpha):
    c = wl.cfg
    sels = []
    for b in range(c.batch):
        q, K, V, n = H.seq_logical(wl, b)
        sels.append(oracle.decode.select_pages(q, K, n, P, c.num_kv_groups, "topk", alpha, budget)["sel"])
    t = torch.full((c.batch, c.num_kv_groups, budget), -1, dtype=torch.int32)
    cnt = torch.zeros(c.batch, c.num_kv_groups, dtype=torch.int32)
    for b in range(c.batch):
        for g in range(c.num_kv_groups):
            t[b, g, :len(sels[b][g])] = torch.as_tensor(sels[b][g], dtype=torch.int32)
            cnt[b, g] = len(sels[b][g])
    return sels, t.cuda(), cnt.cuda()


def _both(wl, alpha, sel, cnt, stride):
    """(noalloc outputs, workspace outputs), each (out, tau, support)."""
    c = wl.cfg
    sh = _shape(wl)
    res = []
    for which in ("noalloc", "workspace"):
        out = torch.full((c.batch, c.num_q_heads, c.head_dim), 9.0, device="cuda")
        tau = torch.full((c.batch, c.num_q_heads), 9.0, device="cuda")
        sup = torch.full((c.batch, c.num_q_heads), -9, dtype=torch.int32, device="cuda")
        if which == "noalloc":
            ekv.entmax_decode_noalloc(sh, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, sel, cnt,
                                      stride, alpha, out, tau, support=sup)
        else:
            nb = ekv.decode_workspace_bytes(sh, sel is not None, stride, alpha)
            assert nb <= ekv.NOALLOC_SCRATCH_BYTES
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            ekv.entmax_decode(sh, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, sel, cnt, stride,
                              alpha, out, tau, ws, support=sup)
        H.sync()
        res.append((out, tau, sup))
    return res


@pytest.mark.parametrize("alpha", [1.5, 1.0])
def test_noalloc_decode_matches_workspace_decode(alpha):
    big = W.make_workload(W.CONFIGS[2].scaled(batch=3), "cuda", seq_lens=[5000, 2053, 37])
    small = W.make_workload(W.CONFIGS[2].scaled(batch=1), "cuda", seq_lens=[700])
    for name, wl, budget in (("3 sequences, 128 pages", big, 128), ("1 sequence, 16 pages", small, 16)):
        print(f"[case] noalloc alpha={alpha} {name}", flush=True)
        sels, sel, cnt = _oracle_selection(wl, budget, alpha)
        (o1, t1, s1), (o2, t2, s2) = _both(wl, alpha, sel, cnt, budget)
        assert torch.equal(o1, o2) and torch.equal(t1, t2) and torch.equal(s1, s2)
        for b in range(wl.cfg.batch):
            q, K, V, n = H.seq_logical(wl, b)
            sp = oracle.decode.sparse_decode_groups(q, K, V, n, P, sels[b], alpha)
            assert np.abs(H.to_np(o1[b]) - sp["out"]).max() <= H.OUT_ATOL
            for h in range(wl.cfg.num_q_heads):
                assert H.tau_close(float(t1[b, h]), sp["tau"][h])


def test_noalloc_full_cache_softmax():
    """Full-cache softmax on the static scratch (bf16 keys: the one-pass path;
    fp32 keys: the logits path), second call smaller than the first, equal
    bit for bit to the decode with a workspace."""
    wl = W.make_workload(W.CONFIGS[2].scaled(batch=2), "cuda", seq_lens=[9000, 1234])
    small = W.make_workload(W.CONFIGS[1], "cuda")
    for name, w in (("softmax, full cache, 2 sequences", wl), ("softmax, full cache, tiny", small)):
        print(f"[case] noalloc {name}", flush=True)
        (o1, t1, s1), (o2, t2, s2) = _both(w, 1.0, None, None, 0)
        assert torch.equal(o1, o2) and torch.equal(t1, t2) and torch.equal(s1, s2)
        for b in range(w.cfg.batch):
            q, K, V, n = H.seq_logical(w, b)
            ref = oracle.decode.decode(q, K, V, None, 1.0)
            assert np.abs(H.to_np(o1[b]) - ref["out"]).max() <= H.OUT_ATOL


def test_noalloc_full_cache_decode_and_oversize_rejection():
    """Full-cache decode on the static scratch (second call smaller than the
    first), and a decode larger than the scratch turned away with
    EKV_ERR_WORKSPACE before anything is enqueued."""
    wl = W.make_workload(W.CONFIGS[2].scaled(batch=2), "cuda", seq_lens=[9000, 1234])
    small = W.make_workload(W.CONFIGS[1], "cuda")
    for name, w in (("full cache, 2 sequences", wl), ("full cache, tiny", small)):
        print(f"[case] noalloc {name}", flush=True)
        (o1, t1, s1), (o2, t2, s2) = _both(w, 1.5, None, None, 0)
        assert torch.equal(o1, o2) and torch.equal(t1, t2) and torch.equal(s1, s2)
    c = wl.cfg
    sh = ekv.make_shape(64, c.num_q_heads, c.num_kv_groups, c.head_dim, 8192, wl.num_phys, c.kv_dtype, "f32")
    out = torch.empty(1, device="cuda")
    with pytest.raises(ekv.EkvError) as err:
        ekv.entmax_decode_noalloc(sh, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, None, None, 0,
                                  1.5, out, out)
    assert err.value.status == ekv.ERR_WORKSPACE
