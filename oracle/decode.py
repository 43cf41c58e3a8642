"""Sparse and full-cache alpha-entmax decode, dropped mass and quality metrics
in float64 (oracle; test infrastructure only).

[EKV] = "EntmaxKV: Support-Aware Decoding for Entmax Attention".

The EntmaxKV step ([EKV] section 4.1): page candidates C_page(q) give the
token candidates C_tok(q) (the valid tokens of the selected pages);

    p~ = alpha-entmax({s_j(q) : j in C_tok}),   o~ = sum_{j in C_tok} p~_j v_j.

Full-cache decode is the same with C_tok = every token ([EKV] section 2.1).
Quality metrics follow [EKV] Appendix E.1 "Approximation quality":
dropped mass delta = 1 - sum_{j in C_tok} p_j (p the full-cache
distribution, section 3.1), support recall rho = |S and C_tok| / |S|
(a count), relative error R = ||o - o~|| / ||o||, coverage |C_tok| / n.
"""

from __future__ import annotations

import numpy as np

from . import entmax as _em
from . import paged as _pg
from . import select as _sel


def tokens_of_pages(pages, n: int, page_size: int) -> np.ndarray:
    """Valid token indices of the given logical pages, in page order."""
    out = []
    for p in np.asarray(pages, dtype=np.int64):
        out.append(np.arange(p * page_size, min((p + 1) * page_size, n)))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, tokens, alpha: float):
    """alpha-entmax attention of every head over the given tokens.

    q: [H][d]; K, V: [n][G][d] logical order; tokens: index array (None = all).
    Returns dict with out [H][d], tau [H] (x units; log-partition for
    alpha = 1), support [H] (nonzero count), p [H][len(tokens)], s [H][len].
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    n, G, _ = K.shape
    r = H // G
    if tokens is None:
        tokens = np.arange(n)
    tokens = np.asarray(tokens, dtype=np.int64)
    s = _pg.token_scores(q, K, tokens)
    Vt = np.asarray(V[tokens], dtype=np.float64)
    out = np.empty((H, d))
    tau = np.empty(H)
    sup = np.empty(H, dtype=np.int64)
    P = np.empty_like(s)
    for h in range(H):
        p, t, k = _em.entmax(s[h], alpha)
        P[h] = p
        out[h] = p @ Vt[:, h // r, :]
        tau[h] = t
        sup[h] = k
    return {"out": out, "tau": tau, "support": sup, "p": P, "s": s, "tokens": tokens}


def dropped_mass_from_tau(s_sel: np.ndarray, tau_ref: float, alpha: float) -> float:
    """delta = 1 - sum_{j in C_tok} p_j, written with the full-cache threshold:
    p_j = [(alpha-1) s_j - tau_ref]_+^beta (alpha > 1) or exp(s_j - tau_ref)
    (alpha = 1, tau_ref the full log-partition)."""
    s_sel = np.asarray(s_sel, dtype=np.float64)
    s_sel = s_sel[np.isfinite(s_sel)]
    if alpha == 1.0:
        return float(1.0 - np.sum(np.exp(s_sel - tau_ref)))
    beta = 1.0 / (alpha - 1.0)
    return float(1.0 - np.sum(np.maximum((alpha - 1.0) * s_sel - tau_ref, 0.0) ** beta))


def metrics(full: dict, sparse: dict, n: int) -> dict:
    """delta, rho, R per head and coverage, against the full-cache result."""
    tok = sparse["tokens"]
    keep = np.zeros(n, dtype=bool)
    keep[tok] = True
    pf = full["p"]                       # [H][n] over all tokens in order
    delta = 1.0 - pf[:, keep].sum(axis=1)
    S = pf > 0
    rho = (S & keep[None, :]).sum(axis=1) / np.maximum(S.sum(axis=1), 1)
    num = np.linalg.norm(full["out"] - sparse["out"], axis=1)
    den = np.linalg.norm(full["out"], axis=1)
    return {"delta": delta, "rho": rho, "R": num / den, "coverage": tok.size / n}


def select_pages(q, K, n, page_size, num_groups, selector, alpha, budget_pages,
                 z=3.0, stat_round=None):
    """Page statistics, page scores and per-group selection for one sequence.

    stat_round: optional callable applied to mean/var before scoring (used
    when the statistics are stored at reduced precision, reading R4).
    Returns dict with per-group selections and the intermediate stages.
    """
    q = np.asarray(q, dtype=np.float64)
    H = q.shape[0]
    r = H // num_groups
    kmin, kmax, mean, var = _pg.page_stats(K, page_size)
    n_p = _pg.page_valid_counts(n, page_size)
    res = {"kmin": kmin, "kmax": kmax, "mean": mean, "var": var, "n_p": n_p}
    sel = []
    if selector == "topk":
        u, U = _pg.box_scores(q, kmin, kmax)
        res.update(u=u, U=U)
        for g in range(num_groups):
            sel.append(_sel.topk_pages(U[g], budget_pages))
    elif selector == "gauss":
        if stat_round is not None:
            mean, var = stat_round(mean), stat_round(var)
        mu, sig = _pg.gauss_moments(q, mean, var)
        tau_hat = np.array([_sel.gauss_tau_hat(mu[h], sig[h], n_p, alpha) for h in range(H)])
        res.update(mu=mu, sigma=sig, tau_hat=tau_hat)
        margins = []
        for g in range(num_groups):
            hs = slice(g * r, (g + 1) * r)
            margins.append(_sel.gauss_margins(mu[hs], sig[hs], tau_hat[hs], alpha))
            sel.append(_sel.gauss_select(mu[hs], sig[hs], tau_hat[hs], alpha, z, budget_pages))
        res["margins"] = np.stack(margins)
    else:
        raise ValueError(selector)
    res["sel"] = sel
    return res


def sparse_decode_groups(q, K, V, n, page_size, sel, alpha):
    """Decode each group's heads over the tokens of that group's own page
    selection (one page set per KV group, reading R5).  Returns the same
    fields as ``decode`` stacked over heads, plus per-group token lists."""
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    G = len(sel)
    r = H // G
    out = np.empty((H, d))
    tau = np.empty(H)
    sup = np.empty(H, dtype=np.int64)
    toks = []
    for g in range(G):
        tk = tokens_of_pages(sel[g], n, page_size)
        toks.append(tk)
        Kg = K[:, g:g + 1, :]
        Vg = V[:, g:g + 1, :]
        res = decode(q[g * r:(g + 1) * r], Kg, Vg, tk, alpha)
        out[g * r:(g + 1) * r] = res["out"]
        tau[g * r:(g + 1) * r] = res["tau"]
        sup[g * r:(g + 1) * r] = res["support"]
    return {"out": out, "tau": tau, "support": sup, "tokens_per_group": toks}
