"""Pins of the oracle's stochastic round (stochastic_round, spec_stochastic), of the
relaxed Delta-logit rule and of post-acceptance truncation (CPU only).

Round rule: the wmrh.cn explainer, section 2.2 (min(1, p/q), residual
norm(max(0, p - q)), bonus on full acceptance), with temperature and
truncation ordered as in its sections 3.3, 4.2 and 8.  Relaxed rule:
"SpecDec-Context-Scaling 项目解读", section 7.2.  Each test is chosen so that
a plausible slip fails it: a target row shifted by one, a noise row taken at
the wrong generated index, truncation applied before the accept test, a
temperature applied to one side only.
"""
import numpy as np
import pytest
from scipy import stats

from block_verify_amd.shapes import TINY
from block_verify_amd.synth import make_noise
from oracle import accept as acc
from oracle.model import OracleWeights
from oracle.spec import draft_sample, spec_greedy, spec_stochastic, stochastic_round, ar_greedy

N_NEW, K = 16, 4
LOG = np.log


@pytest.fixture(scope="module")
def tw(tiny_weights):
    return OracleWeights(TINY, tiny_weights)


# ---------------------------------------------------------------------------
# hand-built rounds with injected uniforms (V = 4, k = 2)
# ---------------------------------------------------------------------------
P1 = np.array([0.1, 0.2, 0.3, 0.4])      # target at draft 1's position (saved_next)
P2 = np.array([0.25, 0.25, 0.25, 0.25])  # target at draft 2's position (rows[0])
P3 = np.array([0.7, 0.1, 0.1, 0.1])      # bonus row (rows[1])
Q1 = np.array([0.4, 0.1, 0.4, 0.1])
Q2 = np.array([0.1, 0.1, 0.1, 0.7])
DRAFTS = [2, 3]


def _hand(u_accept, u_res, **kw):
    return stochastic_round(LOG(P1), LOG(np.stack([P2, P3])), [LOG(Q1), LOG(Q2)], DRAFTS, seed=0, rnd=0,
                            uniforms=(u_accept, u_res), **kw)


@pytest.mark.parametrize("u_accept,u_res,kw,m,committed", [
    # ratio_1 = 0.3 / 0.4 = 0.75, ratio_2 = 0.25 / 0.7 = 0.357; bonus from P3: cumsum .7 .8 .9 1
    ([0.74, 0.30], 0.50, {}, 2, [2, 3, 0]),
    ([0.74, 0.30], 0.99, {}, 2, [2, 3, 3]),
    # u_1 = 0.76 >= 0.75 rejects d_1: residual max(0, P1 - Q1) = [0, .1, 0, .3] -> [0, .25, 0, .75]
    ([0.76, 0.00], 0.20, {}, 0, [1]),
    ([0.76, 0.00], 0.30, {}, 0, [3]),
    # d_2 rejected (u_2 = 0.36 >= 0.357): residual max(0, P2 - Q2) = [.15, .15, .15, 0] / .45
    ([0.10, 0.36], 0.50, {}, 1, [2, 1]),
    # no bonus: a fully accepted round commits the drafts only
    ([0.74, 0.30], 0.50, {"bonus": False}, 2, [2, 3]),
    # truncation acts on the post-acceptance sample only: top-1 of the residual is token 3
    ([0.76, 0.00], 0.20, {"top_k": 1}, 0, [3]),
    # ... and of the bonus row: top_p 0.5 of P3 keeps token 0 alone
    ([0.74, 0.30], 0.99, {"top_p": 0.5}, 2, [2, 3, 0]),
    # top_p 0.75 of P3 keeps tokens 0 and 1 (.7 + .1 reaches .75): u = .99 of [.7, .1] -> 1
    ([0.74, 0.30], 0.99, {"top_p": 0.75}, 2, [2, 3, 1]),
    # the accept test itself never sees the truncation: u_1 = 0.74 still passes with top_k = 1
    ([0.74, 0.30], 0.50, {"top_k": 1}, 2, [2, 3, 0]),
    # temperature 0.5 on both sides: p1 ~ P1^2 -> .3/.3 * ... ratio_1 = (.09/.30) / (.16/.34) = 0.6375
    ([0.63, 0.00], 0.50, {"temperature": 0.5}, 2, [2, 3, 0]),
    # ... u_1 = 0.64 rejects: tempered residual [0, .104, 0, .504], u = .9 lands on token 3
    ([0.64, 0.00], 0.90, {"temperature": 0.5}, 0, [3]),
])
def test_hand_built_round(u_accept, u_res, kw, m, committed):
    got_m, got, _ = _hand(u_accept, u_res, **kw)
    assert (got_m, got) == (m, committed)


def test_hand_built_round_tempered_residual():
    """T = 0.5: p1 = P1^2 / .30, q1 = Q1^2 / .34; residual is positive at tokens 1 and 3 only."""
    p = P1 ** 2 / (P1 ** 2).sum()
    q = Q1 ** 2 / (Q1 ** 2).sum()
    r = np.maximum(0, p - q)
    assert np.all((r > 0) == np.array([False, True, False, True]))
    split = r[1] / r.sum()    # u below this picks token 1, above it token 3
    assert _hand([0.9, 0.0], split - 1e-9, temperature=0.5)[1] == [1]
    assert _hand([0.9, 0.0], split + 1e-9, temperature=0.5)[1] == [3]


# ---------------------------------------------------------------------------
# truncation against a brute-force search of its definition
# ---------------------------------------------------------------------------
def _truncate_brute(w, top_k, top_p):
    w = np.asarray(w, float)
    ranked = sorted(range(len(w)), key=lambda i: (-w[i], i))
    if top_k > 0:
        ranked = ranked[:top_k]
    if top_p < 1.0:
        total = sum(w[i] for i in ranked)
        for n in range(1, len(ranked) + 1):      # the shortest leading run reaching top_p of the mass
            if sum(w[i] for i in ranked[:n]) >= top_p * total:
                ranked = ranked[:n]
                break
    out = np.zeros_like(w)
    out[ranked] = w[ranked]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_truncate_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    w = rng.dirichlet(np.ones(24) * 0.5)
    w[rng.choice(24, 5, replace=False)] = 0.0
    w[3] = w[7]                                   # a tie: the lower index ranks first
    for top_k in (0, 1, 2, 7, 24, 40):
        for top_p in (1.0, 0.99, 0.5, 0.1, 1e-6):
            np.testing.assert_array_equal(acc.truncate(w, top_k, top_p), _truncate_brute(w, top_k, top_p))


def test_truncate_tie_order():
    w = np.array([0.2, 0.3, 0.2, 0.3])
    np.testing.assert_array_equal(acc.truncate(w, top_k=3), [0.2, 0.3, 0.0, 0.3])
    np.testing.assert_array_equal(acc.truncate(w, top_k=1), [0.0, 0.3, 0.0, 0.0])


# ---------------------------------------------------------------------------
# laws of the round through stochastic_round
# ---------------------------------------------------------------------------
def _chain(V, seed):
    rng = np.random.default_rng(seed)
    return rng.dirichlet(np.ones(V) * 0.7, size=V), rng.dirichlet(np.ones(V) * 0.7, size=V)


def _chain_round(P, Q, x0, k, rnd, seed, temperature=1.0, **kw):
    """One round on a Markov chain: target p(. | prev) = P[prev], draft q = Q[prev];
    the round's logits are the chain's log-probabilities scaled by T, so the
    tempered distributions are the chain's own."""
    T = temperature
    q_logits, drafts, prev = [], [], x0
    for j in range(k):
        ql = T * LOG(Q[prev])
        d = draft_sample(ql, seed, rnd, j, T)
        q_logits.append(ql)
        drafts.append(d)
        prev = d
    rows = np.stack([T * LOG(P[d]) for d in drafts])
    return stochastic_round(T * LOG(P[x0]), rows, q_logits, drafts, seed, rnd, temperature=T, **kw)


@pytest.mark.parametrize("temperature", [1.0, 0.6])
def test_markov_chain_joint_two_tokens(temperature):
    """The first two emitted tokens follow the target chain (joint chi-square, p > 1e-3).

    A round whose target rows were shifted by one (d_1 checked against P[d_1])
    or whose temperature reached only one side breaks this law.
    """
    V, k, x0, n = 4, 3, 0, 30000
    P, Q = _chain(V, 21)
    rng = np.random.default_rng(7)
    counts = np.zeros((V, V))
    for rnd in range(n):
        m, com, _ = _chain_round(P, Q, x0, k, rnd, seed=3, temperature=temperature)
        a = com[0]
        b = com[1] if len(com) >= 2 else int(rng.choice(V, p=P[a]))   # the next round starts at a
        counts[a, b] += 1
    _, pval = stats.chisquare(counts.ravel(), (n * P[x0][:, None] * P).ravel())
    assert pval > 1e-3


def test_first_token_law_with_truncation():
    """k = 1: the first token's law is min(p, q) + (1 - sum min(p, q)) * the truncated,
    renormalised residual (accept on the full distributions, truncate afterwards)."""
    V, n = 6, 30000
    P, Q = _chain(V, 5)
    p, q = P[0], Q[0]
    r = acc.truncate(np.maximum(0, p - q), top_k=2)
    law = np.minimum(p, q) + (1 - np.minimum(p, q).sum()) * r / r.sum()
    first = np.zeros(V)
    for rnd in range(n):
        _, com, _ = _chain_round(P, Q, 0, 1, rnd, seed=9, top_k=2)
        first[com[0]] += 1
    keep = law > 0
    assert first[~keep].sum() == 0
    _, pval = stats.chisquare(first[keep], n * law[keep])
    assert pval > 1e-3


def test_low_temperature_reduces_to_greedy():
    """As T -> 0 both distributions become one-hot: the round keeps a draft iff it is the
    target's argmax, replaces the first other one by the argmax, and the bonus is the
    last row's argmax (the greedy rule of "SpecDec-Context-Scaling 项目解读", section 3)."""
    rng = np.random.default_rng(2)
    V, k = 32, 4
    for trial in range(40):
        saved = rng.standard_normal(V)
        rows = rng.standard_normal((k, V))
        # a top-1 margin of 5 makes softmax(z / T) exactly one-hot in float64 at T = 1e-3
        saved[rng.integers(V)] += 5.0
        rows[np.arange(k), rng.integers(0, V, k)] += 5.0
        drafts = [int(acc.argmax_lowest(saved))] + [int(acc.argmax_lowest(r)) for r in rows[:k - 1]]
        for j in rng.choice(k, rng.integers(0, k + 1), replace=False):
            drafts[j] = int(rng.integers(0, V))
        q_logits = [np.where(np.arange(V) == d, 50.0, 0.0) for d in drafts]
        m, com, _ = stochastic_round(saved, rows, q_logits, drafts, seed=3, rnd=trial, temperature=1e-3)
        assert (m, com) == acc.greedy_accept_logits(saved, rows, drafts)


# ---------------------------------------------------------------------------
# spec_stochastic on the tiny decoder
# ---------------------------------------------------------------------------
def test_zero_noise_accepts_every_draft(tw, tiny_prompt):
    """With no noise the draft distribution is the target's own: every draft is kept and
    every round ends with a bonus token (k + 1 tokens per round)."""
    noise = np.zeros((N_NEW + 2 * K, TINY.vocab))
    tr = spec_stochastic(tw, tiny_prompt, N_NEW, K, noise, seed=3)
    assert tr.m == [K] * tr.rounds and tr.stops == ["bonus"] * tr.rounds
    assert tr.rounds == -(-N_NEW // (K + 1))


def test_zero_noise_no_bonus_commits_k_per_round(tw, tiny_prompt):
    noise = np.zeros((N_NEW + 2 * K, TINY.vocab))
    tr = spec_stochastic(tw, tiny_prompt, N_NEW, K, noise, seed=3, bonus=False)
    assert tr.m == [K] * tr.rounds and tr.stops == ["full"] * tr.rounds
    assert tr.rounds == -(-N_NEW // K)


def test_noise_row_follows_generated_index(tw, tiny_prompt):
    """A noise row with one large spike makes the draft at that generated index the spiked
    token: slot j of the round at n0 reads noise[n0 + j]."""
    rng = np.random.default_rng(11)
    spikes = rng.integers(0, TINY.vocab, N_NEW + 2 * K)
    noise = np.zeros((N_NEW + 2 * K, TINY.vocab))
    noise[np.arange(noise.shape[0]), spikes] = 60.0
    tr = spec_stochastic(tw, tiny_prompt, N_NEW, K, noise, seed=3)
    n0 = 0
    for m, drafts, stop in zip(tr.m, tr.drafts, tr.stops):
        assert list(drafts) == [int(s) for s in spikes[n0:n0 + K]]
        n0 += m + (0 if stop == "full" else 1)


def test_spec_stochastic_rounds_replay_through_round_function(tw, tiny_prompt):
    """Temperature 0.8, top-k 40: the job keeps the cache invariant, and its committed
    tokens use only the vocabulary."""
    noise = make_noise(N_NEW + 2 * K, TINY.vocab)
    tr = spec_stochastic(tw, tiny_prompt, N_NEW, K, noise, seed=3, temperature=0.8, top_k=40)
    assert len(tr.tokens) == N_NEW and all(0 <= t < TINY.vocab for t in tr.tokens)
    assert tr.cache.length == len(tiny_prompt) + sum(m + (0 if s == "full" else 1) for m, s in zip(tr.m, tr.stops))


# ---------------------------------------------------------------------------
# relaxed (Delta-logit) acceptance
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("delta,m,committed", [
    (0.0, 1, [2, 1]),          # exact: d_2 = 3 is not row 1's top-1 (token 1)
    (0.5, 2, [2, 3, 0]),       # gap of d_2 = 0.4 <= 0.5, then the bonus argmax of row 2
    (0.39, 1, [2, 1]),
    (10.0, 2, [2, 3, 0]),
])
def test_relaxed_golden(delta, m, committed):
    rows = [np.array([0.0, 1.0, 3.0, 2.0]),    # top-1 is token 2 = d_1
            np.array([0.0, 2.0, 0.5, 1.6]),    # top-1 token 1; d_2 = 3 trails by 0.4
            np.array([5.0, 1.0, 1.0, 1.0])]    # bonus row
    assert acc.relaxed_accept(rows, [2, 3], delta) == (m, committed)


def test_relaxed_gap_is_taken_in_the_rows_precision():
    row = np.array([1.0, 1.0 + 2 ** -23], np.float32)
    assert acc.relaxed_accept([row, row], [0], 2 ** -23)[0] == 1
    assert acc.relaxed_accept([row, row], [0], 2 ** -24)[0] == 0


def test_relaxed_large_delta_accepts_everything_and_zero_is_greedy(tw, tiny_prompt):
    ar, _ = ar_greedy(tw, tiny_prompt, N_NEW + K + 1)
    table = np.array(ar) * 0 + 7            # every draft is token 7
    tr = spec_greedy(tw, tiny_prompt, N_NEW, K, table=table, relax_delta=1e9)
    assert tr.m[:-1] == [K] * (tr.rounds - 1)
    from block_verify_amd.synth import make_draft_table
    table = make_draft_table(np.array(ar), TINY.vocab, 0.4)
    for sched in ("A", "B"):
        tr = spec_greedy(tw, tiny_prompt, N_NEW, K, table=table, relax_delta=0.0, schedule=sched)
        assert tr.tokens == ar[:N_NEW]
