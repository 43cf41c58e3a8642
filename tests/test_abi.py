"""The C ABI without a GPU: the library loads, exports every function that
include/ekv.h declares, rejects bad arguments on the host before any HIP
call, and answers workspace queries.  (Compute calls need a GPU and live in
the gpu-marked tests.)"""

import ctypes
import os
import re

import pytest

from sparse_long_context_ekv_amd import ekv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ekv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ekv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ekv.LIB_PATH):
        pytest.fail("libekv.so is not built (run python -m sparse_long_context_ekv_amd.build)")
    return ekv.load()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("ekv_build_page_stats", "ekv_score_pages", "ekv_select", "ekv_entmax_decode", "ekv_append_kv"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.ekv_abi_version() == 6


def _shape(**kw):
    base = dict(batch=2, num_q_heads=32, num_kv_groups=8, head_dim=128, max_pages_per_seq=64,
                num_phys_pages=128, kv_dtype="bf16", stat_dtype="f32")
    base.update(kw)
    return ekv.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=30), ekv.ERR_INVALID_ARG),          # not a multiple of G
    (dict(num_q_heads=24), ekv.ERR_UNSUPPORTED),          # r = 3
    (dict(head_dim=96), ekv.ERR_UNSUPPORTED),
    (dict(page_size=8), ekv.ERR_UNSUPPORTED),
    (dict(batch=0), ekv.ERR_INVALID_ARG),
    (dict(num_kv_groups=32, num_q_heads=32), ekv.ERR_UNSUPPORTED),
])
def test_shape_validation(lib, kw, status):
    page_size = kw.pop("page_size", 16)
    sh = _shape(**kw)
    sh.page_size = page_size
    n = ctypes.c_size_t(0)
    st = lib.ekv_entmax_decode(ctypes.byref(sh), None, None, None, None, None, None, None, 0, 1.5, None, None,
                               None, None, None, None, None, None, ctypes.byref(n), None)
    assert st == status
    assert lib.ekv_last_error().decode() != ""


def test_bad_dtype_rejected(lib):
    sh = _shape()
    sh.kv_dtype = 7
    with pytest.raises(ekv.EkvError) as e:
        ekv.decode_workspace_bytes(sh, False, 0)
    assert e.value.status == ekv.ERR_UNSUPPORTED


def test_null_required_pointers_rejected_before_launch(lib):
    sh = _shape()
    st = lib.ekv_build_page_stats(ctypes.byref(sh), None, None, None, None, 0, None, None, None, None, None)
    assert st == ekv.ERR_INVALID_ARG
    st = lib.ekv_build_page_stats(ctypes.byref(sh), 8, 8, 8, None, 0, 8, None, None, None, None)
    assert st == ekv.ERR_INVALID_ARG                       # kmin without kmax
    st = lib.ekv_score_pages(ctypes.byref(sh), ekv.SEL_TOPK, 8, 8, 8, None, None, None, None, None, None, None, None,
                             None)
    assert st == ekv.ERR_INVALID_ARG
    st = lib.ekv_score_pages(ctypes.byref(sh), 5, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, None, None)
    assert st == ekv.ERR_INVALID_ARG
    assert lib.ekv_score_pages(None, 0, 8, 8, 8, 8, 8, 8, 8, 8, 8, 8, None, None) == ekv.ERR_INVALID_ARG


def test_select_argument_checks(lib):
    sh = _shape()
    n = ctypes.c_size_t(0)
    assert lib.ekv_select(ctypes.byref(sh), ekv.SEL_TOPK, None, 1.5, 0, 3.0, None, None, None, None, None,
                          None, None, ctypes.byref(n), None) == ekv.ERR_INVALID_ARG      # budget 0
    assert lib.ekv_select(ctypes.byref(sh), ekv.SEL_GAUSS, None, 1.7, 8, 3.0, None, None, None, None, None,
                          None, None, ctypes.byref(n), None) == ekv.ERR_UNSUPPORTED      # alpha 1.7
    assert lib.ekv_select(ctypes.byref(sh), ekv.SEL_GAUSS, None, 1.0, 8, 3.0, None, None, None, None, None,
                          None, None, ctypes.byref(n), None) == ekv.ERR_INVALID_ARG      # softmax + Gaussian
    assert lib.ekv_select(ctypes.byref(sh), ekv.SEL_TOPK, None, 1.5, 8, 3.0, None, None, None, None, None,
                          None, None, None, None) == ekv.ERR_INVALID_ARG                 # no size pointer
    assert lib.ekv_select(ctypes.byref(sh), ekv.SEL_SUPERSET, None, 1.0, 8, 3.0, None, None, None, None, None,
                          None, None, ctypes.byref(n), None) == ekv.ERR_INVALID_ARG      # superset needs alpha > 1
    assert lib.ekv_select(ctypes.byref(sh), 3, None, 1.5, 8, 3.0, None, None, None, None, None,
                          None, None, ctypes.byref(n), None) == ekv.ERR_INVALID_ARG      # unknown selector


def test_superset_select_needs_thresholds(lib):
    """EKV_SEL_SUPERSET reads per-head lower bounds from tau_hat: a NULL
    tau_hat is rejected before anything is launched."""
    sh = _shape()
    need = ekv.select_workspace_bytes(sh, ekv.SEL_SUPERSET, 1.5, 8)
    assert need == ekv.select_workspace_bytes(sh, ekv.SEL_TOPK, 1.5, 8)
    n = ctypes.c_size_t(need)
    st = lib.ekv_select(ctypes.byref(sh), ekv.SEL_SUPERSET, 8, 1.5, 8, 3.0, 8, None, None, 8, 8, None, 256,
                        ctypes.byref(n), None)
    assert st == ekv.ERR_INVALID_ARG
    assert b"tau_hat" in lib.ekv_last_error()


def test_select_workspace_query(lib):
    sh = _shape()
    need_topk = ekv.select_workspace_bytes(sh, ekv.SEL_TOPK, 1.5, 8)
    need_gauss = ekv.select_workspace_bytes(sh, ekv.SEL_GAUSS, 1.5, 8)
    assert need_topk >= 2 * 8 * 64 * 4 and need_topk % 256 == 0
    assert need_gauss > need_topk
    assert ekv.select_workspace_bytes(sh, ekv.SEL_TOPK, 1.5, 8) == need_topk     # idempotent
    n = ctypes.c_size_t(need_topk - 1)
    st = lib.ekv_select(ctypes.byref(sh), ekv.SEL_TOPK, 8, 1.5, 8, 3.0, 8, None, None, 8, 8, None, 256,
                        ctypes.byref(n), None)
    assert st == ekv.ERR_WORKSPACE


def test_decode_workspace_query_and_checks(lib):
    sh = _shape()
    sparse = ekv.decode_workspace_bytes(sh, True, 16)
    full = ekv.decode_workspace_bytes(sh, False, 0)
    assert 0 < sparse < full
    assert ekv.decode_workspace_bytes(sh, True, 16) == sparse
    n = ctypes.c_size_t(sparse - 1)
    st = lib.ekv_entmax_decode(ctypes.byref(sh), 8, 8, 8, 8, 8, 8, 8, 16, 1.5, None, None, 8, 8, None, None, None, 256,
                               ctypes.byref(n), None)
    assert st == ekv.ERR_WORKSPACE
    n = ctypes.c_size_t(sparse)
    st = lib.ekv_entmax_decode(ctypes.byref(sh), 8, 8, 8, 8, 8, 8, 8, 16, 1.5, None, None, 8, 8, None, 8, None, 256,
                               ctypes.byref(n), None)
    assert st == ekv.ERR_INVALID_ARG                       # delta without tau_ref
    st = lib.ekv_entmax_decode(ctypes.byref(sh), 8, 8, 8, 8, 8, 8, 8, 16, 1.5, None, None, 8, 8, None, None, 8, 256,
                               ctypes.byref(n), None)
    assert st == ekv.ERR_INVALID_ARG                       # support_ref without tau_ref
    st = lib.ekv_entmax_decode(ctypes.byref(sh), 8, 8, 8, 8, 8, 8, 8, 16, 0.5, None, None, 8, 8, None, None, None, 256,
                               ctypes.byref(n), None)
    assert st == ekv.ERR_INVALID_ARG                       # alpha < 1
    st = lib.ekv_entmax_decode(ctypes.byref(sh), 8, 8, 8, 8, 8, 8, 8, 16, 1.5, None, None, 8, 8, None, None, None, 300,
                               ctypes.byref(n), None)
    assert st == ekv.ERR_INVALID_ARG                       # misaligned workspace
    st = lib.ekv_entmax_decode(ctypes.byref(sh), 8, 8, 8, 8, 8, 8, None, 16, 1.5, None, None, 8, 8, None, None, None, 256,
                               ctypes.byref(n), None)
    assert st == ekv.ERR_INVALID_ARG                       # sel_pages without sel_count


def test_append_argument_checks(lib):
    """ekv_append_kv rejects missing buffers, unpaired statistics and an
    output length array that aliases the input lengths, before launching."""
    sh = _shape()
    a = ctypes.byref(sh)
    assert lib.ekv_append_kv(a, None, 8, 8, 8, 8, 8, None, None, None, None, None, None) == ekv.ERR_INVALID_ARG
    assert lib.ekv_append_kv(a, 8, 8, 8, 8, 8, 8, 8, None, None, None, None, None) == ekv.ERR_INVALID_ARG
    assert lib.ekv_append_kv(a, 8, 8, 8, 8, 8, 8, None, None, 8, None, None, None) == ekv.ERR_INVALID_ARG
    st = lib.ekv_append_kv(a, 8, 8, 8, 1024, 8, 8, None, None, None, None, 1024, None)
    assert st == ekv.ERR_INVALID_ARG and b"alias" in lib.ekv_last_error()
    assert lib.ekv_append_kv(None, 8, 8, 8, 8, 8, 8, None, None, None, None, None, None) == ekv.ERR_INVALID_ARG


def test_noalloc_decode_rejects_before_any_gpu_call(lib):
    """ekv_entmax_decode_noalloc validates like ekv_entmax_decode and turns
    away, on the host, a decode whose scratch need exceeds the static
    per-GPU array (nothing is enqueued, so this runs without a GPU)."""
    sh = _shape(batch=64, max_pages_per_seq=8192, num_phys_pages=8192)
    need = ekv.decode_workspace_bytes(sh, False, 0, 1.5)          # full cache: logits of every token
    assert need > ekv.NOALLOC_SCRATCH_BYTES
    st = lib.ekv_entmax_decode_noalloc(ctypes.byref(sh), 8, 8, 8, 8, 8, None, None, 0, 1.5, None, None, 8, 8, None,
                                       None, None, None)
    assert st == ekv.ERR_WORKSPACE
    assert "scratch" in lib.ekv_last_error().decode()
    small = _shape()
    assert ekv.decode_workspace_bytes(small, True, 16, 1.5) <= ekv.NOALLOC_SCRATCH_BYTES
    st = lib.ekv_entmax_decode_noalloc(ctypes.byref(small), 8, 8, 8, 8, 8, 8, 8, 16, 0.5, None, None, 8, 8, None,
                                       None, None, None)
    assert st == ekv.ERR_INVALID_ARG                       # alpha < 1
    st = lib.ekv_entmax_decode_noalloc(ctypes.byref(small), 8, 8, 8, 8, 8, 8, None, 16, 1.5, None, None, 8, 8, None,
                                       None, None, None)
    assert st == ekv.ERR_INVALID_ARG                       # sel_pages without sel_count
    st = lib.ekv_entmax_decode_noalloc(ctypes.byref(small), None, 8, 8, 8, 8, 8, 8, 16, 1.5, None, None, 8, 8, None,
                                       None, None, None)
    assert st == ekv.ERR_INVALID_ARG                       # q missing
    st = lib.ekv_entmax_decode_noalloc(ctypes.byref(small), 8, 8, 8, 8, 8, 8, 8, 16, 1.5, None, None, 8, 8, None,
                                       8, None, None)
    assert st == ekv.ERR_INVALID_ARG                       # delta without tau_ref


def test_probe_read_validation(lib):
    """The streaming-read probe rejects bad sizes and launch shapes on the host."""
    sink = 64
    assert lib.ekv_probe_read(4096, 4095, None, 8, 16, sink, None) == ekv.ERR_INVALID_ARG
    assert lib.ekv_probe_read(4096, 0, None, 8, 16, sink, None) == ekv.ERR_INVALID_ARG
    assert lib.ekv_probe_read(4100, 8192, None, 8, 16, sink, None) == ekv.ERR_INVALID_ARG    # misaligned
    assert lib.ekv_probe_read(4096, 8192, None, 3, 16, sink, None) == ekv.ERR_UNSUPPORTED
    assert lib.ekv_probe_read(4096, 8192, None, 8, 0, sink, None) == ekv.ERR_INVALID_ARG
    assert lib.ekv_probe_read(None, 8192, None, 8, 16, sink, None) == ekv.ERR_INVALID_ARG
