"""Oracle acceptance rules: greedy longest prefix, the relaxed (Delta-logit)
variant, and modified rejection sampling with temperature and post-acceptance
truncation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Greedy rule, "SpecDec-Context-Scaling 项目解读" (richardf123.github.io),
section 3 and section 3.1: the verify block's row j predicts the token after
draft d_j, so d_1 is checked against the logits saved before the round
(saved_next), d_(j+1) against rows[j-1], and rows[k-1] is only used on full
acceptance.  The longest matching prefix d_1..d_m is committed together with
the target's own token at position m+1; on full acceptance the bonus token
comes from rows[k-1] (the "bonus-aware" variant of section 3; the standard
variant without bonus is a flag).

Relaxed rule, same page, section 7.2: a draft passes when its target logit
is within Delta of the target's top-1 logit at that position.  The rest of
the round (first failure -> the target's own token, bonus on full
acceptance) is the greedy rule's.  The output is no longer the target's
greedy decode.

Stochastic rule, the wmrh.cn explainer, section 2.2: a draft x drawn from q
is kept with probability min(1, p(x) / q(x)); at the first rejection a token
is drawn from norm(max(0, p - q)) and the round stops; when all k drafts are
kept a bonus token is drawn from the last verify row.  Written here as
vectors: the k ratios at once, then the first index whose uniform is not
below its ratio.  Numerical guards are this project's choices: 1e-10 added
to q(x) in the ratio (a draft with q(x) = 0 cannot have been drawn, so only
rounding reaches it), a strict ``u < ratio`` test, and p itself as the
resampling distribution when the residual mass is <= 1e-10 (rejection then
happened through rounding alone, where p ~ q).

Temperature and truncation, the wmrh.cn explainer, sections 3.3, 4.2 and 8:
draft and target use the same temperature T (p = softmax(z / T)); the
accept/reject step runs on the tempered, untruncated distributions; top-k /
top-p truncation is applied afterwards, to the distribution the round's last
token is drawn from (the residual on a rejection, the bonus row on full
acceptance).  With top_k = 0 (off) and top_p = 1 the round's output follows
the tempered target distribution exactly.

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


def relaxed_accept(logit_rows, drafts, delta: float, bonus: bool = True):
    """Delta-logit relaxed acceptance.

    logit_rows: k+1 target logit rows, row j at draft j's position, row k the
    bonus position.  Draft j passes when max(row_j) - row_j[d_j] <= delta,
    evaluated in the rows' own floating-point type.  Returns (m, committed).
    """
    drafts = [int(d) for d in drafts]
    k = len(drafts)
    if len(logit_rows) != k + 1:
        raise ValueError("need k+1 logit rows")
    m = 0
    while m < k:
        row = np.asarray(logit_rows[m])
        gap = row[argmax_lowest(row)] - row[drafts[m]]
        if not gap <= row.dtype.type(delta):
            break
        m += 1
    if m < k:
        return m, drafts[:m] + [argmax_lowest(logit_rows[m])]
    return k, drafts + ([argmax_lowest(logit_rows[k])] if bonus else [])


def softmax(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """softmax(z / T) in float64."""
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def sample_inverse_cdf(weights: np.ndarray, u: float) -> int:
    """Smallest i with sum(weights[:i+1]) > u * sum(weights) (float64, index order)."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    i = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(i, c.shape[0] - 1)


def cdf_margin(weights: np.ndarray, u: float, i: int) -> float:
    """How far u * total lies from the CDF steps that bound index i, relative to the total
    (a sample whose margin is small may flip under a small change of the weights)."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    t = u * c[-1]
    lo = c[i - 1] if i > 0 else 0.0
    return float(min(abs(t - lo), abs(t - c[i])) / c[-1])


def truncate(weights: np.ndarray, top_k: int = 0, top_p: float = 1.0) -> np.ndarray:
    """Top-k, then top-p, truncation of non-negative weights (not renormalised).

    Entries are ranked by weight, larger first, ties by lower index.  top_k
    keeps the first top_k of that order (0: all).  top_p then keeps the
    shortest leading run of the survivors whose mass reaches top_p times the
    survivors' mass (1: all).  Dropped entries get weight 0.
    """
    w = np.asarray(weights, dtype=np.float64)
    order = np.lexsort((np.arange(w.shape[0]), -w))      # weight desc, index asc
    n = w.shape[0] if top_k <= 0 else min(int(top_k), w.shape[0])
    keep = order[:n]
    if top_p < 1.0:
        c = np.cumsum(w[keep])
        n2 = int(np.searchsorted(c, top_p * c[-1], side="left")) + 1
        keep = keep[:min(n2, keep.shape[0])]
    out = np.zeros_like(w)
    out[keep] = w[keep]
    return out


def accept_ratio(p: np.ndarray, q: np.ndarray, x: int) -> float:
    return min(1.0, float(p[x]) / (float(q[x]) + RATIO_EPS))


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    return np.maximum(0.0, np.asarray(p, np.float64) - np.asarray(q, np.float64))


def stochastic_accept(p_rows, q_rows, drafts, u_accept, u_resample: float, bonus: bool = True,
                      top_k: int = 0, top_p: float = 1.0):
    """Modified rejection sampling over one round.

    p_rows: k+1 target distributions; p_rows[j] is the target's distribution
    at draft j's position, p_rows[k] the bonus distribution.
    q_rows: k draft distributions (q_rows[j] is what drafts[j] was drawn from).
    u_accept: k uniforms for the accept tests; u_resample: one uniform for the
    residual (or bonus) sample.  top_k / top_p truncate that last sample's
    distribution only.
    Returns (m, committed, info); info holds the ratios of the drafts examined,
    the uniforms, the reason the round stopped, the residual mass and the
    (truncated, unnormalised) weights the last token was drawn from.
    """
    drafts = [int(d) for d in drafts]
    k = len(drafts)
    P = np.asarray(p_rows, dtype=np.float64)
    Q = np.asarray(q_rows, dtype=np.float64)
    if P.shape[0] != k + 1 or Q.shape[0] != k:
        raise ValueError("need k+1 target rows and k draft rows")
    j = np.arange(k)
    p_d, q_d = P[j, drafts], Q[j, drafts]
    ratios = np.minimum(1.0, p_d / (q_d + RATIO_EPS))
    kept = np.asarray(u_accept, dtype=np.float64)[:k] < ratios
    m = k if kept.all() else int(np.argmin(kept))          # first index that fails
    info = {"ratios": [float(r) for r in ratios[:min(m + 1, k)]],
            "u_accept": [float(u) for u in np.asarray(u_accept)[:k]], "u_resample": float(u_resample),
            "sample_weights": None}
    if m < k:
        w = residual(P[m], Q[m])
        s = float(w.sum())
        full = w if s > RESIDUAL_EPS else P[m]
        src = truncate(full, top_k, top_p)
        c = sample_inverse_cdf(src, u_resample)
        info.update(stop="reject", residual_mass=s, sample_weights=src, source_weights=full)
        return m, drafts[:m] + [c], info
    if not bonus:
        info.update(stop="full")
        return k, drafts, info
    src = truncate(P[k], top_k, top_p)
    c = sample_inverse_cdf(src, u_resample)
    info.update(stop="bonus", sample_weights=src, source_weights=P[k])
    return k, drafts + [c], info
