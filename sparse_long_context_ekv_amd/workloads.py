"""Seeded synthetic decode workloads in the paged GQA layout.

This module only draws inputs.  It contains none of the attention method's
arithmetic and is the one piece of code that the HIP path's tests and the
fp64 oracle's tests share.

Layout produced (the one the library's header documents):
    q           [B][H_Q][d]              KV dtype
    k_cache     [num_phys][G][P][d]      KV dtype
    v_cache     [num_phys][G][P][d]      KV dtype
    page_table  [B][max_pages]           int32 logical page -> physical page
    seq_lens    [B]                      int32

Recipe (per sequence b, generator seeded with 1_000_003 * config_id + b):
  * q_h ~ N(0, I) * q_scale, rounded to the KV dtype;  u_g is the unit vector
    along the sum of the r rounded queries of group g.
  * keys and values ~ N(0, I).
  * "points": in every group, n_planted distinct token positions get
    k += gamma_g * u_g, gamma_g chosen so that the mean over the group's heads
    of the planted score shift gamma_g (q_h . u_g)/sqrt(d) equals
    shift_sigmas * mean_h(||q_h|| / sqrt(d)).
  * "runs": runs of run_len contiguous tokens starting at uniform random
    offsets, covering about run_frac of the sequence, get k += run_shift * u_g
    (clustered support).
  * keys/values rounded to the KV dtype (round-to-nearest-even).
  * Logical pages are placed at physical pages given by one seeded permutation
    of all the batch's pages.  Slots past the end of a sequence's last page
    hold a large finite sentinel so that any read of them shows up.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

SENTINEL = 32768.0   # exactly representable in bf16 and fp32


@dataclass(frozen=True)
class WorkloadConfig:
    cid: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_groups: int
    head_dim: int
    seq_len: int | None          # fixed length, or None for log-uniform lengths
    kv_dtype: str                # "f32" | "bf16"
    q_scale: float
    planting: str                # "points" | "runs"
    alphas: tuple = (1.5,)
    selector: str = "topk"       # "topk" | "gauss"
    budget_pages: int = 128
    z: float = 3.0
    page_size: int = 16
    n_planted: int = 0           # per group ("points"); ignored if density set
    density: float | None = None
    shift_sigmas: float = 5.0
    run_len: int = 64
    run_frac: float = 0.05
    run_shift: float = 2.0
    len_range: tuple = (4096, 262144)
    seed_base: int | None = None
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return self.cid if self.seed_base is None else self.seed_base

    def scaled(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


# The five workloads, in order.  shift_sigmas of the first was picked from the
# ladder 1.0, 1.25, ..., 8.0 as the first value for which the fp64 1.5-entmax
# support of the group (union over its heads) holds 10..40 tokens and at least
# half of the planted keys (tests/golden/calibrate_tiny.py).
CONFIGS = {
    1: WorkloadConfig(1, "tiny-cpu-checkable", 1, 4, 1, 64, 4096, "f32", 3.0, "points",
                      alphas=(1.5,), selector="topk", budget_pages=32, n_planted=8,
                      shift_sigmas=3.0),
    2: WorkloadConfig(2, "llama3-8b-layer-32k", 1, 32, 8, 128, 32768, "bf16", 2.5, "points",
                      alphas=(1.5,), selector="topk", budget_pages=128, n_planted=64),
    3: WorkloadConfig(3, "batched-128k-clustered", 16, 32, 8, 128, 131072, "bf16", 1.0, "runs",
                      alphas=(1.5,), selector="gauss", budget_pages=256, z=3.0),
    4: WorkloadConfig(4, "extreme-1m", 1, 32, 8, 128, 1048576, "bf16", 2.5, "points",
                      alphas=(1.5,), selector="topk", budget_pages=256, n_planted=256),
    5: WorkloadConfig(5, "ragged-alpha-sweep", 64, 32, 8, 128, None, "bf16", 2.5, "points",
                      alphas=(1.0, 1.5, 2.0), selector="topk", budget_pages=128,
                      density=0.001),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def seq_lengths(cfg: WorkloadConfig) -> list[int]:
    if cfg.seq_len is not None:
        return [int(cfg.seq_len)] * cfg.batch
    g = torch.Generator().manual_seed(7919 * cfg.seed + 1)
    lo, hi = cfg.len_range
    u = torch.rand(cfg.batch, generator=g, dtype=torch.float64)
    return [int(round(math.exp(math.log(lo) + float(x) * (math.log(hi) - math.log(lo))))) for x in u]


@dataclass
class Workload:
    cfg: WorkloadConfig
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    seq_lens_host: list
    max_pages: int
    num_phys: int
    planted: dict

    @property
    def shape(self) -> dict:
        c = self.cfg
        return dict(batch=c.batch, num_q_heads=c.num_q_heads, num_kv_groups=c.num_kv_groups,
                    head_dim=c.head_dim, page_size=c.page_size, max_pages_per_seq=self.max_pages,
                    num_phys_pages=self.num_phys, kv_dtype=c.kv_dtype)


def _group_directions(qb: torch.Tensor, G: int) -> torch.Tensor:
    H, d = qb.shape
    r = H // G
    s = qb.float().reshape(G, r, d).sum(dim=1)
    return s / s.norm(dim=1, keepdim=True)


def make_workload(cfg: WorkloadConfig, device="cpu", seq_lens: list[int] | None = None) -> Workload:
    """Draw the workload on ``device`` (device tensors are the source of truth;
    host copies for the oracle are taken from them)."""
    B, H, G, d, P = cfg.batch, cfg.num_q_heads, cfg.num_kv_groups, cfg.head_dim, cfg.page_size
    dt = torch_dtype(cfg.kv_dtype)
    lens = list(seq_lens) if seq_lens is not None else seq_lengths(cfg)
    assert len(lens) == B
    pages = [(n + P - 1) // P for n in lens]
    max_pages = max(max(pages), 1)
    num_phys = max(sum(pages), 1)
    gperm = torch.Generator().manual_seed(104729 * cfg.seed + 3)
    perm = torch.randperm(num_phys, generator=gperm).to(torch.int32)
    page_table = torch.zeros(B, max_pages, dtype=torch.int32)
    off = 0
    for b in range(B):
        page_table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    k_cache = torch.empty(num_phys, G, P, d, dtype=dt, device=device)
    v_cache = torch.empty(num_phys, G, P, d, dtype=dt, device=device)
    q = torch.empty(B, H, d, dtype=dt, device=device)
    planted = {}
    for b in range(B):
        n, M = lens[b], pages[b]
        gen = torch.Generator(device=device).manual_seed(1_000_003 * cfg.seed + b)
        qb = (torch.randn(H, d, generator=gen, device=device) * cfg.q_scale).to(dt)
        q[b] = qb
        u = _group_directions(qb, G)                                   # [G][d]
        K = torch.randn(M * P, G, d, generator=gen, device=device)
        V = torch.randn(M * P, G, d, generator=gen, device=device)
        if n > 0:
            mask = torch.zeros(G, n, dtype=torch.bool, device=device)
            shift = torch.zeros(G, device=device)
            if cfg.planting == "points":
                k_pl = cfg.n_planted if cfg.density is None else max(1, int(round(cfg.density * n)))
                k_pl = min(k_pl, n)
                r = H // G
                qf = qb.float().reshape(G, r, d)
                sig = (qf.norm(dim=2) / math.sqrt(d)).mean(dim=1)            # [G]
                proj = ((qf * u[:, None, :]).sum(dim=2) / math.sqrt(d)).mean(dim=1)
                shift = cfg.shift_sigmas * sig / proj
                for g in range(G):
                    pos = torch.randperm(n, generator=gen, device=device)[:k_pl]
                    mask[g, pos] = True
            elif cfg.planting == "runs":
                n_runs = max(1, int(round(cfg.run_frac * n / cfg.run_len)))
                shift = torch.full((G,), cfg.run_shift, device=device)
                for g in range(G):
                    starts = torch.randint(0, max(n - cfg.run_len, 0) + 1, (n_runs,),
                                           generator=gen, device=device)
                    idx = (starts[:, None] + torch.arange(cfg.run_len, device=device)[None, :]).reshape(-1)
                    mask[g, idx.clamp(max=n - 1)] = True
            else:
                raise ValueError(cfg.planting)
            for g in range(G):
                idx = mask[g].nonzero().squeeze(1)
                K[idx, g, :] += shift[g] * u[g]
            planted[b] = {"mask": mask.cpu(), "gamma": shift.cpu()}
        if n < M * P:
            K[n:] = SENTINEL
            V[n:] = SENTINEL
        Kp = K.to(dt).reshape(M, P, G, d).permute(0, 2, 1, 3)
        Vp = V.to(dt).reshape(M, P, G, d).permute(0, 2, 1, 3)
        phys = page_table[b, :M].long().to(device)
        k_cache[phys] = Kp
        v_cache[phys] = Vp
        del K, V, Kp, Vp
    return Workload(cfg=cfg, q=q, k_cache=k_cache, v_cache=v_cache,
                    page_table=page_table.to(device), seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
                    seq_lens_host=lens, max_pages=max_pages, num_phys=num_phys, planted=planted)


def host_sequence(wl: Workload, b: int):
    """Host float64 copies needed by the oracle for sequence b:
    (q [H][d], k_cache, v_cache restricted to b's physical pages re-indexed,
    page_table row, n).  Only b's pages are copied."""
    import numpy as np
    n = wl.seq_lens_host[b]
    P = wl.cfg.page_size
    M = (n + P - 1) // P
    phys = wl.page_table[b, :M].long()
    kc = wl.k_cache[phys].float().cpu().numpy().astype(np.float64)
    vc = wl.v_cache[phys].float().cpu().numpy().astype(np.float64)
    q = wl.q[b].float().cpu().numpy().astype(np.float64)
    return q, kc, vc, np.arange(M, dtype=np.int64), n
