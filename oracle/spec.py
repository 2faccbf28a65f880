"""Oracle speculative rounds and autoregressive decoding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Round, "SpecDec-Context-Scaling 项目解读" (richardf123.github.io), section 3
and section 3.2 (schedule "A", the page's literal form): with t committed
positions in the cache, take k drafts, forward them as one block at
positions t..t+k-1 (appending their K/V), decide m by the acceptance rule,
trim every cache to t+m, then forward the round's last committed token
through every cache so each reaches t+m+1.  The invariant checked after
every round is: cache length == prompt length + committed tokens.

Schedule "B" folds the target's one-token repair forward into the next
round's verify block: the block is [pending, d_1..d_k] (k+1 rows), its row 0
plays the role of saved_next, and the caches hold every committed token but
the pending one.  The committed tokens are the same as under "A".  The
one-forward-per-round form follows the merged verify-and-advance design of
"mini-infer系统实战-13" (smarter.xin), section "v2".

Draft provision per workload:
* table: d_j = table[n0 + j - 1], n0 = tokens generated so far;
* model: an independent draft decoder runs its k one-token steps on its own
  cache (tokens overridden by the table) and is trimmed / repaired like the
  target (the two-cache API of the SpecDec page, section 2.2);
* noisy_self: q_j = softmax(z_j + noise[n0 + j - 1]) with z_1 = saved_next and
  z_j (j > 1) from one-token target steps on the shared cache; d_j ~ q_j;
* q4_self: the substitute draft (4-bit linears, shared embedding / LM head /
  norms, shared cache; "SubSpec" summary, sections 4.1.1-4.1.3): d_1 =
  argmax(saved_next), then D-1 one-token draft steps; the verify overwrites
  the draft's K/V.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import accept as acc
from . import philox
from .model import OracleCache, OracleWeights, forward, prefill


@dataclass
class SpecTrace:
    tokens: list = field(default_factory=list)       # committed tokens (truncated to n_new)
    m: list = field(default_factory=list)            # accepted drafts per round
    drafts: list = field(default_factory=list)       # drafts per round
    lengths: list = field(default_factory=list)      # (target len, draft len) after each round
    target_calls: int = 0
    draft_calls: int = 0
    rounds: int = 0
    stops: list = field(default_factory=list)
    margins: list = field(default_factory=list)      # stochastic: (accept, sample) closest calls per round
    cache: object = None        # target cache at the end of the run
    draft_cache: object = None  # independent draft's cache, if any


def ar_greedy(w: OracleWeights, prompt, n_new: int, chunk: int = 2048, max_len: int | None = None):
    """Plain greedy decoding: x_{t+1} = argmax p(x | x_1..t), one step per token.

    "SpecDec-Context-Scaling 项目解读", section 1 (the autoregressive baseline).
    Returns (tokens, per-step logits).
    """
    prompt = np.asarray(prompt)
    cache = OracleCache(w.shape, max_len or prompt.shape[0] + n_new + 1)
    logits = prefill(w, cache, prompt, chunk)
    out, all_logits = [], []
    for i in range(n_new):
        all_logits.append(logits)
        tok = acc.argmax_lowest(logits)
        out.append(tok)
        if i + 1 < n_new:
            logits = forward(w, cache, [tok])[0]
    return out, np.stack(all_logits)


def spec_greedy(w: OracleWeights, prompt, n_new: int, k: int, table=None, schedule: str = "A",
                bonus: bool = True, draft_w: OracleWeights | None = None,
                q4_draft_w: OracleWeights | None = None, chunk: int = 2048, max_len: int | None = None,
                check_invariant: bool = True, relax_delta: float | None = None) -> SpecTrace:
    """Greedy speculative decoding, schedule A or B (see the module docstring).

    relax_delta: None for the exact greedy rule, else the Delta of the relaxed
    rule ("SpecDec-Context-Scaling 项目解读", section 7.2), which then decides
    every round on the target's logit rows.
    """
    prompt = np.asarray(prompt)
    P = prompt.shape[0]
    cap = max_len or (P + n_new + 2 * k + 2)
    tc = OracleCache(w.shape, cap)
    dc = OracleCache(draft_w.shape, cap) if draft_w is not None else None
    tr = SpecTrace()
    if schedule == "A":
        saved = prefill(w, tc, prompt, chunk)
        d_saved = prefill(draft_w, dc, prompt, chunk) if dc is not None else None
        pending = None
    elif schedule == "B":
        if not bonus:
            raise ValueError("schedule B needs the bonus token")
        prefill(w, tc, prompt[:-1], chunk) if P > 1 else None
        if dc is not None:
            d_saved = prefill(draft_w, dc, prompt, chunk)
        pending = int(prompt[-1])
        saved = None
    else:
        raise ValueError(schedule)

    committed = []
    while len(committed) < n_new:
        n0 = len(committed)
        t = tc.length
        # ---- draft provision -------------------------------------------------
        if q4_draft_w is not None:
            if schedule == "B":
                raise ValueError("q4 draft uses schedule A here")
            drafts = [acc.argmax_lowest(saved)]
            for j in range(1, k):
                dl = forward(q4_draft_w, tc, [drafts[-1]])[0]
                tr.draft_calls += 1
                drafts.append(acc.argmax_lowest(dl))
            tc.trim(t)  # the verify block rewrites the draft's positions
        else:
            drafts = [int(x) for x in table[n0:n0 + k]]
            if dc is not None:
                for j in range(k):
                    forward(draft_w, dc, [drafts[j]])
                    tr.draft_calls += 1
        # ---- verify ------------------------------------------------------------
        if schedule == "A":
            rows = forward(w, tc, drafts)
            tr.target_calls += 1
            logit_rows = [saved] + list(rows)
        else:
            rows = forward(w, tc, [pending] + drafts)
            tr.target_calls += 1
            logit_rows = list(rows)
        if relax_delta is None:
            m, com = acc.greedy_accept([acc.argmax_lowest(r) for r in logit_rows], drafts, bonus)
        else:
            m, com = acc.relaxed_accept(logit_rows, drafts, relax_delta, bonus)
        # ---- trim + repair ------------------------------------------------------
        if schedule == "A":
            if m < k or bonus:
                tc.trim(t + m)
                saved = forward(w, tc, [com[-1]])[0]
                tr.target_calls += 1
            else:
                saved = rows[k - 1]
        else:
            tc.trim(t + 1 + m)
            pending = com[-1]
        if dc is not None:
            # draft cache: after its k steps it holds d_1..d_k from the round start
            d_t = dc.length - k
            dc.trim(d_t + m)
            if m < k or bonus:
                forward(draft_w, dc, [com[-1]])
                tr.draft_calls += 1
        committed += com
        tr.m.append(m)
        tr.drafts.append(drafts)
        tr.rounds += 1
        tr.lengths.append((tc.length, dc.length if dc is not None else None))
        if check_invariant:
            expect = P + len(committed) - (1 if schedule == "B" else 0)
            assert tc.length == expect, (tc.length, expect)
            if dc is not None:
                assert dc.length == P + len(committed), (dc.length, P + len(committed))
    tr.tokens = committed[:n_new]
    tr.cache, tr.draft_cache = tc, dc
    return tr


def draft_sample(q_logit_row, seed: int, rnd: int, slot: int, temperature: float = 1.0) -> int:
    """The noisy self-draft's token for slot j of round rnd: drawn from
    softmax(q_logit_row / T) by inverse CDF with the Philox uniform of
    (round rnd, slot j, draft stream)."""
    u = philox.uniform(seed, rnd, slot, philox.STREAM_DRAFT)
    return acc.sample_inverse_cdf(acc.softmax(q_logit_row, temperature), u)


def draft_samples(q_logits, seed: int, rnd: int, temperature: float = 1.0):
    """draft_sample over the k draft logit rows of one round."""
    return [draft_sample(z, seed, rnd, j, temperature) for j, z in enumerate(q_logits)]


def round_uniforms(seed: int, rnd: int, k: int):
    """The accept uniforms u_1..u_k and the resample / bonus uniform of round rnd."""
    ua = [philox.uniform(seed, rnd, j, philox.STREAM_ACCEPT) for j in range(k)]
    return ua, philox.uniform(seed, rnd, 0, philox.STREAM_RESAMPLE)


def stochastic_round(saved, rows, q_logits, drafts, seed: int, rnd: int, bonus: bool = True,
                     temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0, uniforms=None):
    """One round of modified rejection sampling on given logits (schedule A).

    saved: the target's logits at draft 1's position (saved_next, [V]);
    rows: the k verify rows ([k, V]; rows[j] sits at draft j+2's position,
    rows[k-1] is the bonus position); q_logits: the k draft logit rows the
    drafts were drawn from; drafts: the k draft tokens.  The target rows are
    p_1 = softmax(saved / T), p_(j+1) = softmax(rows[j] / T), the draft rows
    q_j = softmax(q_logits[j] / T) (wmrh.cn explainer, sections 2.2 and 8).
    uniforms: (u_accept[k], u_resample) to inject, else the Philox stream of
    round rnd.  Returns stochastic_accept's (m, committed, info).
    """
    k = len(drafts)
    rows = np.asarray(rows)
    if rows.shape[0] != k or len(q_logits) != k:
        raise ValueError("need k verify rows and k draft rows")
    p_rows = [acc.softmax(saved, temperature)] + [acc.softmax(r, temperature) for r in rows]
    q_rows = [acc.softmax(z, temperature) for z in q_logits]
    ua, ur = uniforms if uniforms is not None else round_uniforms(seed, rnd, k)
    return acc.stochastic_accept(p_rows, q_rows, drafts, ua, ur, bonus, top_k, top_p)


def spec_stochastic(w: OracleWeights, prompt, n_new: int, k: int, noise: np.ndarray, seed: int,
                    chunk: int = 2048, max_len: int | None = None, bonus: bool = True, temperature: float = 1.0,
                    top_k: int = 0, top_p: float = 1.0) -> SpecTrace:
    """Modified rejection sampling with the noisy self-draft, schedule A.

    tr.margins[r] is round r's pair of closest calls: the smallest distance of
    an accept uniform from its threshold, and the smallest distance (relative
    to the total) of a sampling uniform from the CDF steps around the index it
    picked.

    Round r at n0 committed tokens: z_1 = saved_next, z_j (j > 1) the target's
    one-token step on d_(j-1) over the shared cache; the draft logits are
    z_j + noise[n0 + j - 1] (0-based: noise[n0 + j] for slot j); the cache is
    rewound to t before the k-row verify.  Without the bonus a fully accepted
    round commits the k drafts only, keeps the cache at t + k and takes the
    last verify row as the next saved_next (no repair forward).
    """
    prompt = np.asarray(prompt)
    P = prompt.shape[0]
    tc = OracleCache(w.shape, max_len or (P + n_new + 2 * k + 2))
    saved = prefill(w, tc, prompt, chunk)
    tr = SpecTrace()
    committed = []
    rnd = 0
    while len(committed) < n_new:
        n0 = len(committed)
        t = tc.length
        z = saved
        drafts, q_logits, s_margin = [], [], 1.0
        for j in range(k):
            ql = np.asarray(z, np.float64) + noise[n0 + j]
            d = draft_sample(ql, seed, rnd, j, temperature)
            s_margin = min(s_margin, acc.cdf_margin(acc.softmax(ql, temperature),
                                                    philox.uniform(seed, rnd, j, philox.STREAM_DRAFT), d))
            drafts.append(d)
            q_logits.append(ql)
            if j + 1 < k:
                z = forward(w, tc, [d])[0]
                tr.draft_calls += 1
        tc.trim(t)
        rows = forward(w, tc, drafts)
        tr.target_calls += 1
        m, com, info = stochastic_round(saved, rows, q_logits, drafts, seed, rnd, bonus, temperature, top_k, top_p)
        a_margin = min([1.0] + [abs(u - a) for u, a in zip(info["u_accept"], info["ratios"])])
        if info["sample_weights"] is not None:
            s_margin = min(s_margin, acc.cdf_margin(info["sample_weights"], info["u_resample"], com[-1]))
        tr.margins.append((a_margin, s_margin))
        if m == k and not bonus:
            saved = rows[k - 1]
        else:
            tc.trim(t + m)
            saved = forward(w, tc, [com[-1]])[0]
            tr.target_calls += 1
        committed += com
        tr.m.append(m)
        tr.drafts.append(drafts)
        tr.stops.append(info["stop"])
        tr.rounds += 1
        rnd += 1
        tr.lengths.append((tc.length, None))
        assert tc.length == P + len(committed)
    tr.tokens = committed[:n_new]
    tr.cache = tc
    return tr
