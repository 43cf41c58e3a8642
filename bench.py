#!/usr/bin/env python3
"""Decode-step benchmark of the sparse alpha-entmax paged decode path.

One step = page scoring + candidate selection + sparse entmax decode for the
whole batch, one layer (page statistics are built once, before timing, as
they are per page and not per step).  Default workload: batch 16, 32 query
heads over 8 KV groups, head dim 128, 128K-token context per sequence,
clustered support, 1.5-entmax, Gaussian-aware selector capped at 256 pages.

Timing follows the pages' protocol ("EntmaxKV", Appendix E.1, "Decoding
efficiency": warm-ups, then the median of timed steps): W untimed warm-up
steps, then K steps bracketed by torch.cuda.synchronize(), each between two
HIP events on the launch stream; steps/s = 1 / median step time.  When one
step's bytes fit in the 256 MB Infinity Cache (the 1M-token and 32K
workloads), each timed step follows a read of a 512 MiB buffer outside its
events, so that it reads from HBM and not from what the previous step left
in the cache (--flush auto|on|off).

Prints ONE JSON line: steps/s (value), ms per step, the step's algorithmic
bytes and GB/s, the dominant kernel's roofline entry (bytes read per launch
over its event-timed launch, against 8 TB/s and against the read bandwidth
this chip achieves for the same access pattern, measured by the library's
streaming-read probe), the full-cache entmax step for comparison, the
selection's quality (dropped mass, support recall, coverage), and the fp64
oracle timed on the host cores on a bounded sample (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--workload N] [--alpha A]
                    [--selector topk|gauss|superset] [--stat-dtype f32|bf16|fp8]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 * 2**20
METRIC = "decode attn steps/s + achieved HBM GB/s, 1.5-entmax, GQA 32/8, 128K ctx"
STAT_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def n_pages(wl):
    P = wl.cfg.page_size
    return sum((n + P - 1) // P for n in wl.seq_lens_host)


def step_bytes(wl, stat_kind, e_stat, sel_count, support):
    """Algorithmic bytes one step must move (the method's own traffic), as
    (read, written): page statistics of every page ("box": min/max in the KV
    dtype; "gauss": mean/var in the statistics dtype) and its page-table
    entry, the selected K tiles, the V rows of the support (union over a
    group's heads, bounded below by the largest per-head support), the
    queries; written: the outputs."""
    c = wl.cfg
    G, D, H, P = c.num_kv_groups, c.head_dim, c.num_q_heads, c.page_size
    e_kv = 2 if c.kv_dtype == "bf16" else 4
    pages = n_pages(wl)
    meta = pages * G * 2 * D * (e_stat if stat_kind == "gauss" else e_kv) + pages * 4
    k_sel = int(sel_count.sum().item()) * P * D * e_kv
    r = H // G
    sup = support.view(c.batch, G, r).max(dim=2).values
    v_sup = int(sup.sum().item()) * D * e_kv
    q = c.batch * H * D * e_kv
    outs = c.batch * H * (D + 1) * 4
    return {"page_stats": meta, "selected_k": k_sel, "support_v": v_sup, "q": q,
            "read_total": meta + k_sel + v_sup + q, "written": outs}


def score_kernel_bytes(wl, stat_kind, e_stat):
    """(read, written) bytes of one score-kernel launch: statistics of every
    page of every group, page-table entries and queries in; one fp32 per
    (page, group) (box) or two per (page, head) (Gaussian) out."""
    c = wl.cfg
    G, D, H = c.num_kv_groups, c.head_dim, c.num_q_heads
    e_kv = 2 if c.kv_dtype == "bf16" else 4
    pages = n_pages(wl)
    if stat_kind == "gauss":
        return pages * G * 2 * D * e_stat + pages * 4 + c.batch * H * D * e_kv, pages * H * 2 * 4
    return pages * G * 2 * D * e_kv + pages * 4 + c.batch * H * D * e_kv, pages * G * 4


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gauss_score_kernel_traffic_batched-128k-clustered.md")


def measured_traffic(workload, stat_kind, stat_dtype):
    """HBM bytes per launch of the Gaussian score kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a plain copy of known
    size), or None when the workload differs or the kernel's sources changed
    since the counters were taken."""
    import hashlib
    if workload != "batched-128k-clustered" or stat_kind != "gauss" or stat_dtype != "f32" \
            or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if ": " in line and not line.startswith(("#", "|")):
            k, v = line.split(": ", 1)
            kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in kv["sources"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != kv["source_sha256"]:
            return None
        return {"read": int(kv["hbm_read_bytes_per_launch"]), "written": int(kv["hbm_write_bytes_per_launch"])}
    except (KeyError, OSError, ValueError):
        return None


class Flusher:
    """Evicts the Infinity Cache by reading a 512 MiB buffer (twice the
    cache) with the streaming-read probe.  A read, not a write: dirty lines
    left by a write would be written back during the next step and slow it."""

    def __init__(self, on):
        import torch
        from sparse_long_context_ekv_amd import ekv
        self.on = on
        self.ekv = ekv
        self.buf = torch.ones(2 * MALL_BYTES, dtype=torch.uint8, device="cuda") if on else None
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def __call__(self):
        if self.on:
            self.ekv.probe_read(self.buf, sink=self.sink)


def timed_steps(step, steps, stream, flush, inner=None):
    """K steps, each between two HIP events on the launch stream (with the
    optional cache-evicting read before it, outside its events), bracketed by
    synchronize().  With `inner` = (first, rest), events also bracket the
    first part of each step (the score kernel), for its launch time.
    Returns (step ms list, inner ms list or None, wall seconds)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, m, b in ev:
        flush()
        a.record(stream)
        if inner is None:
            step()
        else:
            inner[0]()
            m.record(stream)
            inner[1]()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, _, b in ev]
    ims = [a.elapsed_time(m) for a, m, _ in ev] if inner is not None else None
    return ms, ims, wall


def back_to_back(step, steps):
    """Throughput of K steps enqueued back to back with nothing between them."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def probe_bandwidth(reps=5):
    """Read bandwidth the chip achieves with the library's streaming-read
    probe over a 1 GiB buffer (four times the Infinity Cache), read in 4 KiB
    chunks front to back ("linear") and in a seeded random chunk order
    ("gather_4k"); the best median over a few launch shapes."""
    import torch
    from sparse_long_context_ekv_amd import ekv
    nbytes = 1 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    nch = nbytes // 4096
    g = torch.Generator(device="cuda").manual_seed(4242)
    order = torch.randperm(nch, generator=g, device="cuda").to(torch.int32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for name, ordr in (("linear", None), ("gather_4k", order)):
        best = None
        for unroll in (4, 8):
            for blocks in (1024, 2048, 4096):
                ekv.probe_read(buf, ordr, unroll, blocks, sink)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
                for a, b in ev:
                    a.record(stream)
                    ekv.probe_read(buf, ordr, unroll, blocks, sink)
                    b.record(stream)
                torch.cuda.synchronize()
                ms = statistics.median([a.elapsed_time(b) for a, b in ev])
                gbps = nbytes / (ms * 1e-3) / 1e9
                if best is None or gbps > best[0]:
                    best = (gbps, unroll, blocks)
        out[name] = {"gbps": round(best[0], 1), "unroll": best[1], "blocks": best[2]}
    del buf, order
    torch.cuda.synchronize()
    return out


def cpu_baseline(wl, selector, alpha, budget, z, nseq, stat_round=None):
    """The fp64 oracle on a bounded sample of sequences, same stages as the
    timed GPU step (statistics precomputed, untimed)."""
    import numpy as np
    import oracle
    from sparse_long_context_ekv_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    cores = len(os.sched_getaffinity(0))
    c = wl.cfg
    P, G, H = c.page_size, c.num_kv_groups, c.num_q_heads
    r = H // G
    B = c.batch
    lens = wl.seq_lens_host
    if len(set(lens)) == 1:
        picks = sorted(set([0, B - 1] + list(range(1, B - 1))[: max(0, nseq - 2)]))[:nseq]
    else:
        # ragged batch: sequences at evenly spaced length quantiles, longest included
        order = sorted(range(B), key=lambda i: lens[i])
        k = max(1, min(nseq, B))
        picks = sorted({order[round((B - 1) * (j + 1) / k)] for j in range(k)})
    times = []
    for b in picks:
        q, kc, vc, pt, n = W.host_sequence(wl, b)
        K = oracle.paged.gather_logical(kc, pt, n)
        V = oracle.paged.gather_logical(vc, pt, n)
        kmin, kmax, mean, var = oracle.paged.page_stats(K, P)
        if stat_round is not None:
            mean, var = stat_round(mean), stat_round(var)
        n_p = oracle.paged.page_valid_counts(n, P)
        t0 = time.perf_counter()
        if selector == "gauss":
            mu, sg = oracle.paged.gauss_moments(q, mean, var)
            th = np.array([oracle.select.gauss_tau_hat(mu[h], sg[h], n_p, alpha) for h in range(H)])
            sel = [oracle.select.gauss_select(mu[g * r:(g + 1) * r], sg[g * r:(g + 1) * r], th[g * r:(g + 1) * r],
                                              alpha, z, budget) for g in range(G)]
        else:
            _, U = oracle.paged.box_scores(q, kmin, kmax)
            sel = [oracle.select.topk_pages(U[g], budget) for g in range(G)]
        oracle.decode.sparse_decode_groups(q, K, V, n, P, sel, alpha)
        times.append(time.perf_counter() - t0)
        log(f"oracle sequence {b}: {times[-1]:.2f} s")
    per_seq = statistics.mean(times)
    # one step = the whole batch: the sample's time per token times the batch's tokens
    step_s = sum(times) * sum(lens) / sum(lens[b] for b in picks)
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(picks)} of {B} sequences (b={picks}, {sum(lens[b] for b in picks)} of {sum(lens)} "
                      f"tokens), fp64 numpy/scipy oracle ({selector} selection + sparse decode, page statistics "
                      f"precomputed); sample time scaled by the batch's token count = one step",
            "blas_threads": blas, "seconds_per_sequence": per_seq}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--alpha", type=float, default=None, help="default: 1.5 where the workload has it")
    ap.add_argument("--selector", default=None, choices=["topk", "gauss", "superset"],
                    help="default: the workload's own; superset = the exact (App. B.2) selector")
    ap.add_argument("--budget", type=int, default=None,
                    help="pages per (sequence, group); default: the workload's (superset: every page)")
    ap.add_argument("--stat-dtype", default="f32", choices=["f32", "bf16", "fp8"])
    ap.add_argument("--flush", default="auto", choices=["auto", "on", "off"],
                    help="evict the Infinity Cache before each timed step (auto: when a step's bytes fit in it)")
    ap.add_argument("--cpu-seqs", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many bytes "
                         "(a kernel of known traffic for scaling hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the library runs on one GPU only (the decode path is not sharded); "
                                   "--gpus must be 1", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    from sparse_long_context_ekv_amd import ekv
    from sparse_long_context_ekv_amd import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)
    ekv.load()

    cfg = W.CONFIGS[args.workload]
    alpha = args.alpha if args.alpha is not None else (1.5 if 1.5 in cfg.alphas else cfg.alphas[0])
    selector = args.selector or cfg.selector
    z = cfg.z
    log(f"workload {cfg.name}: drawing inputs on the GPU")
    t0 = time.time()
    wl = W.make_workload(cfg, "cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s: {wl.num_phys} physical pages")
    budget = args.budget or (wl.max_pages if selector == "superset" else cfg.budget_pages)
    stat_kind = "gauss" if selector == "gauss" else "box"
    e_stat = STAT_BYTES[args.stat_dtype]

    dec = ekv.Decoder(wl, selector, alpha, budget, z=z, stat_dtype=args.stat_dtype)
    dec.build_stats()
    torch.cuda.synchronize()
    log("page statistics built")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dec.step()
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps done")

    sk_read, sk_written = score_kernel_bytes(wl, stat_kind, e_stat)
    flush_on = args.flush == "on" or (args.flush == "auto" and sk_read < 2 * MALL_BYTES)
    flush = Flusher(flush_on)

    step_ms, _, wall = timed_steps(dec.step, args.steps, stream, flush)
    med = statistics.median(step_ms)
    log(f"{args.steps} timed steps: median {med:.4f} ms (events{', after a cache-evicting read' if flush_on else ''}), "
        f"wall {wall * 1e3 / args.steps:.4f} ms/step")
    # the score kernel's launch time, from events around it inside each step
    _, score_ms, _ = timed_steps(None, args.steps, stream, flush, inner=(dec.score, lambda: (dec.select(), dec.decode())))
    sk_us = statistics.mean(score_ms) * 1e3
    b2b = back_to_back(dec.step, args.steps)
    log(f"score kernel {sk_us:.1f} us (mean); back to back {b2b * 1e3:.4f} ms/step")

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {args.copy_bytes} bytes done")

    sb = step_bytes(wl, stat_kind, e_stat, dec.buf.sel_count, dec.buf.support)
    achieved = sk_read / (sk_us * 1e-6) / 1e9
    kernel = "gauss_score_kernel" if stat_kind == "gauss" else "box_score_kernel"
    roofline = {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                "basis": "algorithmic bytes read per launch / mean event-timed launch",
                "bytes_read_per_launch": sk_read, "bytes_written_per_launch": sk_written,
                "achieved_read_write": round((sk_read + sk_written) / (sk_us * 1e-6) / 1e9, 1),
                "frac_read_write": round((sk_read + sk_written) / (sk_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                "avg_launch_us": round(sk_us, 2)}
    tr = measured_traffic(cfg.name, stat_kind, args.stat_dtype)
    if tr is not None:
        roofline["traffic"] = tr["read"] + tr["written"]
        roofline["traffic_read"] = tr["read"]
        roofline["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    if not args.no_probe:
        pr = probe_bandwidth()
        roofline["achievable"] = pr
        roofline["achievable_gbps"] = pr["gather_4k"]["gbps"]
        roofline["frac_of_achievable"] = round(achieved / pr["gather_4k"]["gbps"], 4)
        log(f"streaming-read probe: linear {pr['linear']['gbps']} GB/s, 4 KiB gather {pr['gather_4k']['gbps']} GB/s")

    step_gbps = sb["read_total"] / (med * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(1e3 / med, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "context": cfg.seq_len, "num_q_heads": cfg.num_q_heads,
                   "num_kv_groups": cfg.num_kv_groups, "head_dim": cfg.head_dim, "page_size": cfg.page_size,
                   "alpha": alpha, "selector": selector, "budget_pages": budget, "z": z,
                   "kv_dtype": cfg.kv_dtype, "stat_dtype": args.stat_dtype},
        "timing": "median of K event-timed steps after W warm-ups (HIP events on the launch stream, between "
                  "steps); value = 1 / median" + ("; each step after a 512 MiB read that evicts the "
                                                 "Infinity Cache" if flush_on else ""),
        "cache_flushed": flush_on,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "back_to_back": {"steps_per_s": round(1.0 / b2b, 3), "ms_per_step": round(b2b * 1e3, 4),
                         "note": "K steps enqueued with nothing between them, no cache eviction"},
        "hbm_gbps": round(step_gbps, 1),
        "step_bytes": sb,
        "step_roofline": {"bytes_read": sb["read_total"], "achieved": round(step_gbps, 1),
                          "frac": round(step_gbps / PEAK_HBM_GBPS, 4)},
        "roofline": roofline,
    }

    if selector == "gauss":
        # The adaptive budget before the cap: the pages the Gaussian rule
        # admits per (sequence, group) with no cap (a selection with budget = MP).
        c = cfg
        unc = ekv.Decoder(wl, "gauss", alpha, wl.max_pages, z=z, stat_dtype=args.stat_dtype)
        unc.stats = dec.stats
        unc.buf.mu, unc.buf.sigma = dec.buf.mu, dec.buf.sigma
        dec.score()
        unc.select()
        torch.cuda.synchronize()
        cnt = unc.buf.sel_count.double()
        result["adaptive_budget"] = {
            "uncapped_pages_mean": round(float(cnt.mean()), 2), "uncapped_pages_min": int(cnt.min()),
            "uncapped_pages_max": int(cnt.max()), "cap_pages": budget,
            "rows_at_cap": int((cnt >= budget).sum()), "rows": int(cnt.numel()),
            "uncapped_coverage": round(float(cnt.sum()) * c.page_size / (c.num_kv_groups * sum(wl.seq_lens_host)), 5)}
        del unc
        torch.cuda.synchronize()

    def time_full(runner, reps=5):
        runner()
        torch.cuda.synchronize()
        ms, _, _ = timed_steps(runner, reps, stream, flush)
        return statistics.median(ms)

    if not args.no_full:
        # Full-cache baselines on the same inputs: entmax (same alpha) and softmax.
        full = ekv.FullDecoder(wl, alpha)
        full_ms = time_full(full.run)
        delta = torch.empty_like(dec.buf.tau)
        supref = torch.empty_like(dec.buf.support)
        dec.step()
        dec.decode(tau_ref=full.tau, delta=delta, support_ref=supref)
        torch.cuda.synchronize()
        rho = (supref.double() / full.support.double().clamp(min=1.0)).flatten()
        P = cfg.page_size
        cov = float(dec.buf.sel_count.sum().item()) * P / (cfg.num_kv_groups * sum(wl.seq_lens_host))
        rel = ((dec.buf.out - full.out).norm(dim=2) / full.out.norm(dim=2)).flatten()
        result["full_cache"] = {"ms_per_step": round(full_ms, 4), "speedup_sparse_over_full": round(full_ms / med, 3)}
        result["quality"] = {"coverage": round(cov, 5), "delta_mean": float(delta.mean()),
                             "delta_max": float(delta.max()), "rho_mean": float(rho.mean()),
                             "rho_min": float(rho.min()), "R_mean": float(rel.mean()), "R_max": float(rel.max())}
        if selector == "superset":
            result["quality"]["rows_cut_by_budget"] = int((dec.buf.sel_count >= budget).sum())
        full_tau = full.tau.clone()
        del full
        if alpha != 1.0:
            soft = ekv.FullDecoder(wl, 1.0)
            soft_ms = time_full(soft.run)
            result["full_cache_softmax"] = {"ms_per_step": round(soft_ms, 4),
                                            "speedup_sparse_over_full": round(soft_ms / med, 3)}
            del soft
        torch.cuda.synchronize()
        log(f"full-cache entmax {full_ms:.3f} ms per step")

    if not args.no_variants and selector == "gauss" and args.stat_dtype == "f32" and args.workload == 3:
        # Same step with the page mean/variance stored in bf16 (half the
        # statistics bytes) and in FP8 E4M3 (a quarter); reported beside the
        # fp32 headline, not as it.
        result["variants"] = {}
        for sd, note in (("bf16", "page mean/variance stored as bf16 (fp32 accumulation); min/max unaffected"),
                         ("fp8", "page mean/variance stored as OCP FP8 E4M3 (round to nearest even, "
                                 "saturating at 448); min/max unaffected")):
            dv = ekv.Decoder(wl, selector, alpha, budget, z=z, stat_dtype=sd)
            dv.build_stats()
            for _ in range(max(args.warmup // 2, 3)):
                dv.step()
            torch.cuda.synchronize()
            ms, _, _ = timed_steps(dv.step, args.steps, stream, flush)
            _, sms, _ = timed_steps(None, args.steps, stream, flush, inner=(dv.score, lambda: (dv.select(), dv.decode())))
            skv = statistics.mean(sms) * 1e3
            rd, _ = score_kernel_bytes(wl, "gauss", STAT_BYTES[sd])
            m = statistics.median(ms)
            entry = {"value": round(1e3 / m, 3), "unit": "steps/s", "ms_per_step": round(m, 4),
                     "score_kernel_us": round(skv, 2), "score_kernel_read_gbps": round(rd / (skv * 1e-6) / 1e9, 1),
                     "note": note}
            if not args.no_full:
                dlt = torch.empty_like(dv.buf.tau)
                dv.decode(tau_ref=full_tau, delta=dlt)
                torch.cuda.synchronize()
                entry["quality"] = {"coverage": round(float(dv.buf.sel_count.sum().item()) * cfg.page_size /
                                                      (cfg.num_kv_groups * sum(wl.seq_lens_host)), 5),
                                    "delta_mean": float(dlt.mean()), "delta_max": float(dlt.max())}
            result["variants"][f"{sd}_page_mean_var"] = entry
            del dv
            torch.cuda.synchronize()

    if not args.no_cpu_baseline and selector != "superset":
        rnd = None
        if args.stat_dtype == "bf16":
            rnd = lambda a: torch.from_numpy(a).float().to(torch.bfloat16).double().numpy()  # noqa: E731
        elif args.stat_dtype == "fp8":
            import numpy as np
            import oracle
            rnd = lambda a: oracle.paged.round_fp8_e4m3(np.asarray(a, dtype=np.float32))  # noqa: E731
        result["cpu_baseline"] = cpu_baseline(wl, selector, alpha, budget, z, args.cpu_seqs, rnd)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
