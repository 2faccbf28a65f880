"""Oracle acceptance rules: greedy longest prefix and modified rejection sampling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Greedy rule, "SpecDec-Context-Scaling 项目解读" (richardf123.github.io),
section 3 and section 3.1: the verify block's row j predicts the token after
draft d_j, so d_1 is checked against the logits saved before the round
(saved_next), d_(j+1) against rows[j-1], and rows[k-1] is only used on full
acceptance.  The longest matching prefix d_1..d_m is committed together with
the target's own token at position m+1; on full acceptance the bonus token
comes from rows[k-1] (the "bonus-aware" variant of section 3; the standard
variant without bonus is a flag).

Stochastic rule, the wmrh.cn explainer section 2.2 and "mini-infer系统实战-13"
(smarter.xin), section on modified rejection sampling: accept a draft x with
probability min(1, p(x)/q(x)); on the first rejection resample from
norm(max(0, p - q)) and stop; if all k pass, sample a bonus token from the
distribution of the last verify row.  The guards follow the mini-infer page's
sampler: q(x) + 1e-10 in the ratio, a strict ``u < ratio`` test, and a
fallback to p when the residual mass is <= 1e-10.

Sampling is by inverse CDF: the smallest index i whose running sum (float64,
index order) exceeds u times the total.  Argmax ties go to the lowest index.
"""
from __future__ import annotations

import numpy as np

RATIO_EPS = 1e-10
RESIDUAL_EPS = 1e-10


def argmax_lowest(logits: np.ndarray) -> int:
    """Index of the maximum; the lowest such index on ties."""
    return int(np.argmax(np.asarray(logits)))


def top2_margin(logits: np.ndarray) -> float:
    a = np.partition(np.asarray(logits, dtype=np.float64), -2)[-2:]
    return float(a[1] - a[0])


def greedy_accept(verify_argmax, drafts, bonus: bool = True):
    """Longest-prefix greedy acceptance on target argmax tokens.

    verify_argmax: k+1 ints [argmax(saved_next), argmax(rows[0]), ...,
    argmax(rows[k-1])]; entry j is the target's choice at the position of
    draft j (0-based), entry k the bonus choice.
    Returns (m, committed): m accepted drafts, then the target's token at
    position m (replacement, or the bonus when m == k and bonus is on).
    """
    drafts = [int(d) for d in drafts]
    v = [int(a) for a in verify_argmax]
    k = len(drafts)
    if len(v) != k + 1:
        raise ValueError("need k+1 verify choices")
    m = 0
    while m < k and drafts[m] == v[m]:
        m += 1
    if m < k:
        return m, drafts[:m] + [v[m]]
    return k, drafts + ([v[k]] if bonus else [])


def greedy_accept_logits(saved_next: np.ndarray, rows: np.ndarray, drafts, bonus: bool = True):
    """greedy_accept with the argmax taken from logits (saved_next [V], rows [k, V])."""
    v = [argmax_lowest(saved_next)] + [argmax_lowest(r) for r in rows]
    return greedy_accept(v, drafts, bonus)


def softmax(logits: np.ndarray) -> np.ndarray:
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def sample_inverse_cdf(weights: np.ndarray, u: float) -> int:
    """Smallest i with sum(weights[:i+1]) > u * sum(weights) (float64, index order)."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    i = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(i, c.shape[0] - 1)


def accept_ratio(p: np.ndarray, q: np.ndarray, x: int) -> float:
    return min(1.0, float(p[x]) / (float(q[x]) + RATIO_EPS))


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    return np.maximum(0.0, np.asarray(p, np.float64) - np.asarray(q, np.float64))


def stochastic_accept(p_rows, q_rows, drafts, u_accept, u_resample: float, bonus: bool = True):
    """Modified rejection sampling over one round.

    p_rows: k+1 target distributions; p_rows[j] is the target's distribution
    at draft j's position, p_rows[k] the bonus distribution.
    q_rows: k draft distributions (q_rows[j] is what drafts[j] was drawn from).
    u_accept: k uniforms for the accept tests; u_resample: one uniform for the
    residual (or bonus) sample.
    Returns (m, committed, info) with info = per-draft ratios and the reason
    the round stopped.
    """
    drafts = [int(d) for d in drafts]
    k = len(drafts)
    ratios = []
    for j in range(k):
        a = accept_ratio(p_rows[j], q_rows[j], drafts[j])
        ratios.append(a)
        if u_accept[j] < a:
            continue
        w = residual(p_rows[j], q_rows[j])
        s = float(w.sum())
        src = w if s > RESIDUAL_EPS else np.asarray(p_rows[j], np.float64)
        c = sample_inverse_cdf(src, u_resample)
        return j, drafts[:j] + [c], {"ratios": ratios, "stop": "reject", "residual_mass": s}
    if not bonus:
        return k, drafts, {"ratios": ratios, "stop": "full"}
    c = sample_inverse_cdf(p_rows[k], u_resample)
    return k, drafts + [c], {"ratios": ratios, "stop": "bonus"}
