"""Plain fp64 CPU oracle for support-aware sparse alpha-entmax paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP library (no kernels, headers, helpers or constants) and
imports nothing from it.

Source of every step: the web page "EntmaxKV: Support-Aware Decoding for
Entmax Attention" (Duarte, Couceiro, Treviso; arXiv 2605.21649), abbreviated
[EKV] below, plus the GQA notation of "EntroPrefill: Renyi-Guided Context
Pruning" section 2.1 Eq. (1) for the head-to-group map.  Each function cites
the section, equation or appendix it follows.  Where the page text is damaged
or silent, the reading taken is named (R1..R14) at the function that takes it.

Everything is numpy/scipy in float64.  Inputs stored in bf16 or fp32 are
up-cast exactly before any arithmetic.

Modules
-------
entmax   alpha-entmax threshold (sort-based exact and bisection), softmax
paged    logical gather through the page table, page statistics, box scores,
         Gaussian score moments
select   top-k page selection, Gaussian threshold estimate, Gaussian page rule
decode   sparse / full-cache decode, dropped mass and the quality metrics
"""

from . import entmax, paged, select, decode  # noqa: F401
