"""Thin ctypes binding of libekv (include/ekv.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory (tensors) and the stream
(``torch.cuda.current_stream()``).  If the library has not been built,
``load()`` raises; there is no fallback implementation.

Names follow the C ABI: ``build_page_stats``, ``score_pages``, ``select``,
``entmax_decode``.  ``Decoder`` wires them into one decode step over a
workload's buffers (score -> select -> decode).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libekv.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16, FP8_E4M3 = 0, 1, 2
SEL_TOPK, SEL_GAUSS, SEL_SUPERSET = 0, 1, 2
_STATUS = {0: "EKV_OK", 1: "EKV_ERR_INVALID_ARG", 2: "EKV_ERR_UNSUPPORTED", 3: "EKV_ERR_WORKSPACE", 4: "EKV_ERR_HIP"}
SYMBOLS = ("ekv_build_page_stats", "ekv_append_kv", "ekv_score_pages", "ekv_select", "ekv_entmax_decode",
           "ekv_entmax_decode_noalloc", "ekv_probe_read", "ekv_last_error", "ekv_abi_version")
NOALLOC_SCRATCH_BYTES = 32 << 20      # EKV_NOALLOC_SCRATCH_BYTES


class EkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_groups", "head_dim", "page_size",
        "max_pages_per_seq", "num_phys_pages", "kv_dtype", "stat_dtype")]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_szp = ctypes.POINTER(ctypes.c_size_t)


def load(path: str | None = None):
    """Open libekv.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} not built: run `python -m sparse_long_context_ekv_amd.build`")
    lib = ctypes.CDLL(p)
    sp = ctypes.POINTER(Shape)
    lib.ekv_build_page_stats.argtypes = [sp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.ekv_append_kv.argtypes = [sp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.ekv_score_pages.argtypes = [sp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.ekv_select.argtypes = [sp, _i32, _vp, _f32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _szp, _vp]
    lib.ekv_entmax_decode.argtypes = [sp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _szp, _vp]
    lib.ekv_entmax_decode_noalloc.argtypes = [sp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _vp,
                                              _vp, _vp, _vp, _vp, _vp, _vp]
    lib.ekv_probe_read.argtypes = [_vp, ctypes.c_size_t, _vp, _i32, _i32, _vp, _vp]
    for name in ("ekv_build_page_stats", "ekv_append_kv", "ekv_score_pages", "ekv_select", "ekv_entmax_decode",
                 "ekv_entmax_decode_noalloc", "ekv_probe_read"):
        getattr(lib, name).restype = ctypes.c_int
    lib.ekv_last_error.restype = ctypes.c_char_p
    lib.ekv_last_error.argtypes = []
    lib.ekv_abi_version.restype = ctypes.c_int32
    lib.ekv_abi_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def _check(st: int):
    if st != OK:
        raise EkvError(st, load().ekv_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# torch storage dtype of page mean/variance per statistics dtype name
STAT_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def make_shape(batch, num_q_heads, num_kv_groups, head_dim, max_pages_per_seq, num_phys_pages,
               kv_dtype="bf16", stat_dtype="f32", page_size=16) -> Shape:
    dt = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, F32: F32, BF16: BF16, FP8_E4M3: FP8_E4M3}
    return Shape(batch, num_q_heads, num_kv_groups, head_dim, page_size, max_pages_per_seq,
                 num_phys_pages, dt[kv_dtype], dt[stat_dtype])


# ------------------------------------------------------------ entry points --
def build_page_stats(shape, k_cache, page_table, seq_lens, kmin=None, kmax=None, kmean=None,
                     kvar=None, page_list=None, stream=None):
    n_list = 0 if page_list is None else int(page_list.numel())
    _check(load().ekv_build_page_stats(ctypes.byref(shape), _ptr(k_cache), _ptr(page_table), _ptr(seq_lens),
                                       _ptr(page_list), n_list, _ptr(kmin), _ptr(kmax), _ptr(kmean),
                                       _ptr(kvar), _stream(stream)))


def append_kv(shape, k_new, v_new, page_table, seq_lens, k_cache, v_cache, kmin=None, kmax=None, kmean=None,
              kvar=None, new_lens=None, stream=None):
    _check(load().ekv_append_kv(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(page_table), _ptr(seq_lens),
                                _ptr(k_cache), _ptr(v_cache), _ptr(kmin), _ptr(kmax), _ptr(kmean), _ptr(kvar),
                                _ptr(new_lens), _stream(stream)))


def score_pages(shape, selector, q, page_table, seq_lens, kmin=None, kmax=None, kmean=None, kvar=None,
                score=None, mu=None, sigma=None, stream=None, head_score=None):
    _check(load().ekv_score_pages(ctypes.byref(shape), int(selector), _ptr(q), _ptr(page_table), _ptr(seq_lens),
                                  _ptr(kmin), _ptr(kmax), _ptr(kmean), _ptr(kvar), _ptr(score), _ptr(mu),
                                  _ptr(sigma), _ptr(head_score), _stream(stream)))


def select_workspace_bytes(shape, selector, alpha=1.5, budget_pages=1, z=3.0) -> int:
    n = ctypes.c_size_t(0)
    _check(load().ekv_select(ctypes.byref(shape), int(selector), None, float(alpha), int(budget_pages), float(z),
                             None, None, None, None, None, None, None, ctypes.byref(n), None))
    return n.value


def select(shape, selector, seq_lens, alpha, budget_pages, z, score, mu, sigma, sel_pages, sel_count,
           tau_hat, workspace, stream=None):
    n = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check(load().ekv_select(ctypes.byref(shape), int(selector), _ptr(seq_lens), float(alpha), int(budget_pages),
                             float(z), _ptr(score), _ptr(mu), _ptr(sigma), _ptr(sel_pages), _ptr(sel_count),
                             _ptr(tau_hat), _ptr(workspace), ctypes.byref(n), _stream(stream)))


def decode_workspace_bytes(shape, sparse: bool, sel_stride: int, alpha: float = 1.5) -> int:
    n = ctypes.c_size_t(0)
    dummy = 1 if sparse else None
    _check(load().ekv_entmax_decode(ctypes.byref(shape), None, None, None, None, None, dummy, dummy,
                                    int(sel_stride), float(alpha), None, None, None, None, None, None, None, None,
                                    ctypes.byref(n), None))
    return n.value


def entmax_decode(shape, q, k_cache, v_cache, page_table, seq_lens, sel_pages, sel_count, sel_stride, alpha,
                  out, tau, workspace, support=None, delta=None, tau_ref=None, support_ref=None, tau_hint=None,
                  stream=None):
    n = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _check(load().ekv_entmax_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                    _ptr(seq_lens), _ptr(sel_pages), _ptr(sel_count), int(sel_stride),
                                    float(alpha), _ptr(tau_hint), _ptr(tau_ref), _ptr(out), _ptr(tau), _ptr(support),
                                    _ptr(delta), _ptr(support_ref), _ptr(workspace), ctypes.byref(n),
                                    _stream(stream)))


def entmax_decode_noalloc(shape, q, k_cache, v_cache, page_table, seq_lens, sel_pages, sel_count, sel_stride,
                          alpha, out, tau, support=None, delta=None, tau_ref=None, support_ref=None, tau_hint=None,
                          stream=None):
    """ekv_entmax_decode_noalloc: the same decode on the library's static
    per-GPU scratch (no workspace argument, no allocation)."""
    _check(load().ekv_entmax_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(page_table), _ptr(seq_lens), _ptr(sel_pages), _ptr(sel_count),
                                            int(sel_stride), float(alpha), _ptr(tau_hint), _ptr(tau_ref), _ptr(out),
                                            _ptr(tau),
                                            _ptr(support), _ptr(delta), _ptr(support_ref), _stream(stream)))


def probe_read(buf, order=None, unroll=8, blocks=2048, sink=None, stream=None):
    """ekv_probe_read over the bytes of tensor `buf` (4 KiB chunks, linear or
    in the chunk order of the int32 tensor `order`)."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(load().ekv_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(order), int(unroll), int(blocks),
                                 _ptr(sink), _stream(stream)))


# ------------------------------------------------------------- one step ----
@dataclass
class StepBuffers:
    score: torch.Tensor | None
    mu: torch.Tensor | None
    sigma: torch.Tensor | None
    sel_pages: torch.Tensor
    sel_count: torch.Tensor
    tau_hat: torch.Tensor | None
    out: torch.Tensor
    tau: torch.Tensor
    support: torch.Tensor
    ws_select: torch.Tensor
    ws_decode: torch.Tensor


class Decoder:
    """Buffers and calls for one decode step of a workload:
    ekv_score_pages -> ekv_select -> ekv_entmax_decode, all on one stream.

    selector "topk" | "gauss" | "superset".  "superset" (alpha > 1) scores
    pages by box bounds, decodes over the top `first_pages` pages to get a
    threshold no larger than the full-cache one (the threshold of any token
    subset is), then selects every page whose box bound clears it
    (EKV_SEL_SUPERSET) and decodes on that set; with budget_pages at least the
    number of qualifying pages the result is exact."""

    def __init__(self, wl, selector: str, alpha: float, budget_pages: int, z: float = 3.0,
                 stat_dtype: str = "f32", first_pages: int = 8, tau_hint: bool = True):
        c = wl.cfg
        dev = wl.k_cache.device
        self.wl = wl
        # Gaussian selector: hand its threshold estimate to decode as the start
        # of the threshold iteration, with the selected pages.
        self.use_hint = bool(tau_hint)
        self.superset = selector == "superset"
        self.selector = SEL_GAUSS if selector == "gauss" else SEL_TOPK
        self.alpha = float(alpha)
        self.budget = int(budget_pages)
        self.z = float(z)
        self.shape = make_shape(c.batch, c.num_q_heads, c.num_kv_groups, c.head_dim, wl.max_pages, wl.num_phys,
                                c.kv_dtype, stat_dtype)
        B, H, G, D, MP, NP = c.batch, c.num_q_heads, c.num_kv_groups, c.head_dim, wl.max_pages, wl.num_phys
        kvdt = wl.k_cache.dtype
        sdt = STAT_TORCH_DTYPE[stat_dtype]
        self.stats = {}
        if self.selector == SEL_TOPK:
            self.stats["kmin"] = torch.empty(NP, G, D, dtype=kvdt, device=dev)
            self.stats["kmax"] = torch.empty(NP, G, D, dtype=kvdt, device=dev)
        else:
            self.stats["kmean"] = torch.empty(NP, G, D, dtype=sdt, device=dev)
            self.stats["kvar"] = torch.empty(NP, G, D, dtype=sdt, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.buf = StepBuffers(
            score=torch.empty(B, G, MP, **f32) if self.selector == SEL_TOPK else None,
            mu=torch.empty(B, H, MP, **f32) if self.selector == SEL_GAUSS else None,
            sigma=torch.empty(B, H, MP, **f32) if self.selector == SEL_GAUSS else None,
            sel_pages=torch.empty(B, G, self.budget, dtype=torch.int32, device=dev),
            sel_count=torch.empty(B, G, dtype=torch.int32, device=dev),
            tau_hat=torch.empty(B, H, **f32) if self.selector == SEL_GAUSS else None,
            out=torch.empty(B, H, D, **f32),
            tau=torch.empty(B, H, **f32),
            support=torch.empty(B, H, dtype=torch.int32, device=dev),
            ws_select=torch.empty(select_workspace_bytes(self.shape, self.selector, self.alpha, self.budget, self.z),
                                  dtype=torch.uint8, device=dev),
            ws_decode=torch.empty(decode_workspace_bytes(self.shape, True, self.budget, self.alpha),
                                  dtype=torch.uint8, device=dev),
        )
        self.first = None
        if self.superset:
            k0 = int(first_pages)
            self.first = {
                "pages": k0,
                "sel": torch.empty(B, G, k0, dtype=torch.int32, device=dev),
                "cnt": torch.empty(B, G, dtype=torch.int32, device=dev),
                "out": torch.empty(B, H, D, **f32),
                "tau": torch.empty(B, H, **f32),
                "ws": torch.empty(decode_workspace_bytes(self.shape, True, k0, self.alpha), dtype=torch.uint8,
                                  device=dev),
            }

    def build_stats(self, stream=None):
        wl = self.wl
        build_page_stats(self.shape, wl.k_cache, wl.page_table, wl.seq_lens, stream=stream, **self.stats)

    def score(self, stream=None):
        wl, b = self.wl, self.buf
        score_pages(self.shape, self.selector, wl.q, wl.page_table, wl.seq_lens, score=b.score, mu=b.mu,
                    sigma=b.sigma, stream=stream, **self.stats)

    def select(self, stream=None):
        b = self.buf
        if self.superset:
            wl, f = self.wl, self.first
            select(self.shape, SEL_TOPK, wl.seq_lens, self.alpha, f["pages"], self.z, b.score, None, None,
                   f["sel"], f["cnt"], None, b.ws_select, stream=stream)
            entmax_decode(self.shape, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, f["sel"],
                          f["cnt"], f["pages"], self.alpha, f["out"], f["tau"], f["ws"], stream=stream)
            select(self.shape, SEL_SUPERSET, wl.seq_lens, self.alpha, self.budget, self.z, b.score, None, None,
                   b.sel_pages, b.sel_count, f["tau"], b.ws_select, stream=stream)
            return
        select(self.shape, self.selector, self.wl.seq_lens, self.alpha, self.budget, self.z, b.score, b.mu,
               b.sigma, b.sel_pages, b.sel_count, b.tau_hat, b.ws_select, stream=stream)

    def decode(self, stream=None, tau_ref=None, delta=None, support_ref=None):
        wl, b = self.wl, self.buf
        hint = b.tau_hat if (self.use_hint and self.selector == SEL_GAUSS and not self.superset) else None
        entmax_decode(self.shape, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, b.sel_pages,
                      b.sel_count, self.budget, self.alpha, b.out, b.tau, b.ws_decode, support=b.support,
                      delta=delta, tau_ref=tau_ref, support_ref=support_ref, tau_hint=hint, stream=stream)

    def step(self, stream=None):
        self.score(stream)
        self.select(stream)
        self.decode(stream)


class FullDecoder:
    """Full-cache alpha-entmax decode (every page selected): the baseline
    the sparse step is compared with, and the source of tau_ref for delta."""

    def __init__(self, wl, alpha: float, stat_dtype: str = "f32"):
        c = wl.cfg
        dev = wl.k_cache.device
        self.wl = wl
        self.alpha = float(alpha)
        self.shape = make_shape(c.batch, c.num_q_heads, c.num_kv_groups, c.head_dim, wl.max_pages, wl.num_phys,
                                c.kv_dtype, stat_dtype)
        f32 = dict(dtype=torch.float32, device=dev)
        self.out = torch.empty(c.batch, c.num_q_heads, c.head_dim, **f32)
        self.tau = torch.empty(c.batch, c.num_q_heads, **f32)
        self.support = torch.empty(c.batch, c.num_q_heads, dtype=torch.int32, device=dev)
        self.ws = torch.empty(decode_workspace_bytes(self.shape, False, 0, self.alpha), dtype=torch.uint8, device=dev)

    def run(self, stream=None):
        wl = self.wl
        entmax_decode(self.shape, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, None, None, 0,
                      self.alpha, self.out, self.tau, self.ws, support=self.support, stream=stream)
