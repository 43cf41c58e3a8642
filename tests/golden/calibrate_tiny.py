"""Pick the planted-key shift of the tiny CPU-checkable workload.

Walks the ladder 1.0, 1.25, ..., 8.0 (in units of the mean per-head score
standard deviation ||q_h||/sqrt(d)) and prints the first value for which the
fp64 oracle's full-cache 1.5-entmax support, counted over the union of the
group's four heads (the token set one page selection per group has to
cover), holds between 10 and 40 tokens and contains at least half of the
planted keys.  A per-head count cannot reach 10 at this query scale: with
score spread ||q||/sqrt(d) = 3 the top tokens are too far apart for more
than about 8 of them to share a 1.5-entmax support.  Uses only the input
generator and the oracle; the value it prints is written into the workload
table by hand.

    python tests/golden/calibrate_tiny.py
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
from sparse_long_context_ekv_amd import workloads as W  # noqa: E402


def support_sizes(shift: float):
    """(per-head support sizes, union size, planted keys in the union, planted)."""
    cfg = W.CONFIGS[1].scaled(shift_sigmas=shift)
    wl = W.make_workload(cfg, "cpu")
    q, kc, vc, pt, n = W.host_sequence(wl, 0)
    K = oracle.paged.gather_logical(kc, pt, n)
    V = oracle.paged.gather_logical(vc, pt, n)
    res = oracle.decode.decode(q, K, V, None, 1.5)
    union = (res["p"] > 0).any(axis=0)
    planted = wl.planted[0]["mask"][0].numpy()
    return ([int(x) for x in res["support"]], int(union.sum()),
            int((union & planted).sum()), int(planted.sum()))


def main():
    for shift in np.arange(1.0, 8.0 + 1e-9, 0.25):
        per_head, uni, hit, npl = support_sizes(float(shift))
        ok = 10 <= uni <= 40 and 2 * hit >= npl
        print(f"shift={shift:.2f} per-head={per_head} union={uni} planted-in-union={hit}/{npl}"
              f" {'OK' if ok else ''}")
        if ok:
            print(f"chosen shift_sigmas = {shift:.2f}")
            return
    print("no ladder value fits")


if __name__ == "__main__":
    main()
