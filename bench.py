#!/usr/bin/env python3
"""Decode-step benchmark of the sparse alpha-entmax paged decode path.

One step = page scoring + candidate selection + sparse entmax decode for the
whole batch, one layer (page statistics are built once, before timing, as
they are per page and not per step).  Default workload: batch 16, 32 query
heads over 8 KV groups, head dim 128, 128K-token context per sequence,
clustered support, 1.5-entmax, Gaussian-aware selector capped at 256 pages.

Prints ONE JSON line: steps/s (value), ms per step, achieved GB/s of the
step's algorithmic bytes, the dominant kernel's roofline entry (HIP-event
time on the launch stream), the full-cache entmax step for comparison, the
dropped mass / coverage of the selection, and the fp64 oracle timed on the
host cores on a bounded sample (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--workload N]
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
METRIC = "decode attn steps/s + achieved HBM GB/s, 1.5-entmax, GQA 32/8, 128K ctx"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def step_bytes(wl, selector, stat_bytes, sel_count, support, q_bytes):
    """Algorithmic bytes one step must move (the method's own traffic):
    page statistics of every page, the selected K tiles, the V rows of the
    support (union over a group's heads, bounded below by the largest
    per-head support), the queries, page-table entries and outputs."""
    c = wl.cfg
    G, D, H, P = c.num_kv_groups, c.head_dim, c.num_q_heads, c.page_size
    e_kv = 2 if c.kv_dtype == "bf16" else 4
    pages = sum((n + P - 1) // P for n in wl.seq_lens_host)
    per_page_stats = 2 * D * (stat_bytes if selector == "gauss" else e_kv)
    meta = pages * G * per_page_stats + pages * 4
    k_sel = int(sel_count.sum().item()) * P * D * e_kv
    r = H // G
    sup = support.view(c.batch, G, r).max(dim=2).values
    v_sup = int(sup.sum().item()) * D * e_kv
    q = c.batch * H * D * q_bytes
    outs = c.batch * H * D * 4
    return meta, k_sel, v_sup, q + outs


def score_kernel_bytes(wl, selector, stat_bytes):
    c = wl.cfg
    G, D, H, P = c.num_kv_groups, c.head_dim, c.num_q_heads, c.page_size
    e_kv = 2 if c.kv_dtype == "bf16" else 4
    pages = sum((n + P - 1) // P for n in wl.seq_lens_host)
    if selector == "gauss":
        rd = pages * G * 2 * D * stat_bytes + pages * 4 + c.batch * H * D * e_kv
        wr = pages * H * 2 * 4
    else:
        rd = pages * G * 2 * D * e_kv + pages * 4 + c.batch * H * D * e_kv
        wr = pages * G * 4
    return rd + wr


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gauss_score_kernel_traffic_batched-128k-clustered.md")


def measured_traffic(workload, stat_dtype):
    """HBM bytes per launch of the Gaussian score kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a plain copy of known
    size), or None when the workload differs or the kernel's sources changed
    since the counters were taken."""
    import hashlib
    if workload != "batched-128k-clustered" or stat_dtype != "f32" or not os.path.exists(TRAFFIC_FILE):
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
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def timed_steps(dec, steps, stream):
    """The timed steps, then the same number of instrumented ones.

    The timed steps run back to back with nothing between them, bracketed by
    torch.cuda.synchronize(): their wall time gives steps/s.  HIP events go
    only into a second, instrumented pass (events on the launch stream around
    the score call and around each step), because on this runtime an event
    recorded between two kernels drains the queue: about 6 us inside a step
    and 10 us between steps, which would be charged to the step.  Returns the
    timed wall seconds and the instrumented per-step and score-kernel times
    (ms)."""
    import torch
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        dec.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b2, c2 in ev:
        a.record(stream)
        dec.score()
        b2.record(stream)
        dec.select()
        dec.decode()
        c2.record(stream)
    torch.cuda.synchronize()
    return wall, [a.elapsed_time(c2) for a, _, c2 in ev], [a.elapsed_time(b2) for a, b2, _ in ev]


def cpu_baseline(wl, selector, alpha, budget, z, nseq, stat_round=None):
    """The fp64 oracle on a bounded sample of sequences, same stages as the
    timed GPU step (statistics precomputed, untimed)."""
    import numpy as np
    import oracle
    from sparse_long_context_ekv_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
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
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(picks)} of {B} sequences (b={picks}, {sum(lens[b] for b in picks)} of {sum(lens)} "
                      f"tokens), fp64 numpy/scipy oracle, same stages as the GPU step (page statistics "
                      f"precomputed); sample time scaled by the batch's token count = one step",
            "seconds_per_sequence": per_seq}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--stat-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--cpu-seqs", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--flush-mall", action="store_true",
                    help="also time steps that each follow a 512 MiB read, which evicts the 256 MB Infinity "
                         "Cache (for workloads whose per-step bytes fit in it); reported as mall_flushed")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many bytes "
                         "(a kernel of known traffic for scaling hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
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
    alpha = 1.5 if 1.5 in cfg.alphas else cfg.alphas[0]
    selector, budget, z = cfg.selector, cfg.budget_pages, cfg.z
    log(f"workload {cfg.name}: drawing inputs on the GPU")
    t0 = time.time()
    wl = W.make_workload(cfg, "cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s: {wl.num_phys} physical pages")

    dec = ekv.Decoder(wl, selector, alpha, budget, z=z, stat_dtype=args.stat_dtype)
    dec.build_stats()
    torch.cuda.synchronize()
    log("page statistics built")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dec.step()
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps done")

    wall, step_ms, score_ms = timed_steps(dec, args.steps, stream)
    log(f"{args.steps} timed steps: {wall * 1e3 / args.steps:.3f} ms/step wall; instrumented pass: "
        f"median event {statistics.median(step_ms):.3f} ms, score kernel {statistics.mean(score_ms) * 1e3:.1f} us")

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {args.copy_bytes} bytes done")

    stat_bytes = 4 if args.stat_dtype == "f32" else 2
    e_kv = 2 if cfg.kv_dtype == "bf16" else 4
    meta, k_sel, v_sup, small = step_bytes(wl, selector, stat_bytes, dec.buf.sel_count, dec.buf.support, e_kv)
    total_bytes = meta + k_sel + v_sup + small
    ms_per_step = wall * 1e3 / args.steps
    sk_bytes = score_kernel_bytes(wl, selector, stat_bytes)
    sk_us = statistics.mean(score_ms) * 1e3
    achieved = sk_bytes / (sk_us * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(args.steps / wall, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "context": cfg.seq_len, "num_q_heads": cfg.num_q_heads,
                   "num_kv_groups": cfg.num_kv_groups, "head_dim": cfg.head_dim, "page_size": cfg.page_size,
                   "alpha": alpha, "selector": selector, "budget_pages": budget, "z": z,
                   "kv_dtype": cfg.kv_dtype, "stat_dtype": args.stat_dtype},
        "hbm_gbps": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_bytes": {"page_stats": meta, "selected_k": k_sel, "support_v": v_sup, "q_and_out": small,
                       "total": total_bytes},
        "median_event_ms_per_step": round(statistics.median(step_ms), 4),
        "event_timing": "HIP events on the launch stream over a second, instrumented pass of the same "
                        "number of steps (median step; mean score-kernel launch)",
        "roofline": {"kernel": "gauss_score_kernel" if selector == "gauss" else "box_score_kernel",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(cfg.name, args.stat_dtype) if selector == "gauss" else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "bytes_per_launch": sk_bytes, "avg_launch_us": round(sk_us, 2)},
    }

    if args.flush_mall:
        # Each step follows a read of a 512 MiB buffer (outside its events), so
        # nothing it reads can come from the Infinity Cache left by the
        # previous step.  A read, not a write: evicting dirty lines would be
        # written back during the step and slow it instead.
        junk = torch.ones(128 * 2**20, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b2, c2 in fe:
            junk.sum()
            a.record(stream)
            dec.score()
            b2.record(stream)
            dec.select()
            dec.decode()
            c2.record(stream)
        torch.cuda.synchronize()
        del junk
        f_step = statistics.median([a.elapsed_time(c2) for a, _, c2 in fe])
        f_score = statistics.mean([a.elapsed_time(b2) for a, b2, _ in fe]) * 1e3
        result["mall_flushed"] = {"median_event_ms_per_step": round(f_step, 4), "score_kernel_us": round(f_score, 2),
                                  "score_kernel_gbps": round(sk_bytes / (f_score * 1e-6) / 1e9, 1),
                                  "note": "each step after a 512 MiB read; HIP events around each step"}
        log(f"after a cache-evicting read: median step {f_step:.4f} ms (events), score kernel {f_score:.1f} us")

    # Quality of the selection: dropped mass against the full-cache threshold.
    def time_full(runner, reps=5):
        runner()
        torch.cuda.synchronize()
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b2 in fe:
            a.record(stream)
            runner()
            b2.record(stream)
        torch.cuda.synchronize()
        return statistics.median([a.elapsed_time(b2) for a, b2 in fe])

    if not args.no_full:
        # Full-cache baselines on the same inputs: entmax (same alpha) and softmax.
        full = ekv.FullDecoder(wl, alpha)
        full_ms = time_full(full.run)
        delta = torch.empty_like(dec.buf.tau)
        supref = torch.empty_like(dec.buf.support)
        dec.decode(tau_ref=full.tau, delta=delta, support_ref=supref)
        torch.cuda.synchronize()
        rho = (supref.double() / full.support.double().clamp(min=1.0)).flatten()
        P = cfg.page_size
        cov = float(dec.buf.sel_count.sum().item()) * P / (cfg.num_kv_groups * sum(wl.seq_lens_host))
        rel = ((dec.buf.out - full.out).norm(dim=2) / full.out.norm(dim=2)).flatten()
        result["full_cache"] = {"ms_per_step": round(full_ms, 4),
                                "speedup_sparse_over_full": round(full_ms / ms_per_step, 3)}
        result["quality"] = {"coverage": round(cov, 5), "delta_mean": float(delta.mean()),
                             "delta_max": float(delta.max()), "rho_mean": float(rho.mean()),
                             "rho_min": float(rho.min()), "R_mean": float(rel.mean()), "R_max": float(rel.max())}
        full_tau = full.tau.clone()
        del full
        soft = ekv.FullDecoder(wl, 1.0)
        soft_ms = time_full(soft.run)
        result["full_cache_softmax"] = {"ms_per_step": round(soft_ms, 4),
                                        "speedup_sparse_over_full": round(soft_ms / ms_per_step, 3)}
        del soft
        torch.cuda.synchronize()
        log(f"full-cache entmax {full_ms:.3f} ms, softmax {soft_ms:.3f} ms per step")

    if not args.no_variants and selector == "gauss" and args.stat_dtype == "f32":
        # Same step with the page mean/variance stored in bf16 (half the
        # statistics bytes) and in FP8 E4M3 (a quarter); reported beside the
        # fp32 headline, not as it.
        result["variants"] = {}
        for sd, nbytes, note in (("bf16", 2, "page mean/variance stored as bf16 (fp32 accumulation); min/max unaffected"),
                                 ("fp8", 1, "page mean/variance stored as OCP FP8 E4M3 (round to nearest even, "
                                            "saturating at 448); min/max unaffected")):
            dv = ekv.Decoder(wl, selector, alpha, budget, z=z, stat_dtype=sd)
            dv.build_stats()
            for _ in range(max(args.warmup // 2, 3)):
                dv.step()
            torch.cuda.synchronize()
            wallv, _, skv_ms = timed_steps(dv, args.steps, stream)
            skv = statistics.mean(skv_ms) * 1e3
            bv = score_kernel_bytes(wl, selector, nbytes)
            entry = {"value": round(args.steps / wallv, 3), "unit": "steps/s",
                     "ms_per_step": round(wallv * 1e3 / args.steps, 4),
                     "score_kernel_us": round(skv, 2), "score_kernel_gbps": round(bv / (skv * 1e-6) / 1e9, 1),
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

    if not args.no_cpu_baseline:
        rnd = None
        if args.stat_dtype == "bf16":
            rnd = lambda a: torch.from_numpy(a).float().to(torch.bfloat16).double().numpy()  # noqa: E731
        result["cpu_baseline"] = cpu_baseline(wl, selector, alpha, budget, z, args.cpu_seqs, rnd)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
