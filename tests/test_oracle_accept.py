"""Pins of the oracle's acceptance rules and of its Philox generator (CPU only)."""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import accept as acc
from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load("greedy_accept_cases.json"), ids=lambda c: c["name"][:40])
def test_greedy_golden(case):
    m, com = acc.greedy_accept(case["v"], case["drafts"], case["bonus"])
    assert m == case["m"]
    assert com == case["committed"]


def test_greedy_from_logits_uses_saved_next_for_d1():
    V, k = 8, 4
    saved = np.zeros(V); saved[3] = 1.0
    rows = np.zeros((k, V))
    for j, t in enumerate([4, 5, 6, 7]):
        rows[j, t] = 1.0
    m, com = acc.greedy_accept_logits(saved, rows, [3, 4, 5, 6])
    assert (m, com) == (4, [3, 4, 5, 6, 7])
    # shifted drafts (what an off-by-one verifier would expect) are rejected at once
    m, com = acc.greedy_accept_logits(saved, rows, [4, 5, 6, 7])
    assert (m, com) == (0, [3])


def test_argmax_ties_take_lowest_index():
    assert acc.argmax_lowest(np.array([0.0, 2.0, 1.0, 2.0])) == 1


@pytest.mark.parametrize("case", _load("stochastic_accept_cases.json"), ids=lambda c: c["name"][:40])
def test_stochastic_golden(case):
    p = [np.array(r) for r in case["p"]]
    q = [np.array(r) for r in case["q"]]
    m, com, _ = acc.stochastic_accept(p, q, case["drafts"], case["u_accept"], case["u_resample"])
    assert m == case["m"]
    assert com == case["committed"]


def test_inverse_cdf_never_picks_zero_weight():
    w = np.array([0.0, 0.0, 0.3, 0.0, 0.7, 0.0])
    for u in np.linspace(0, 0.9999999, 1001):
        assert w[acc.sample_inverse_cdf(w, u)] > 0


def _round_trials(p_rows, q_rows, n, rng):
    """Run n independent rounds with drafts drawn from q; return (m, committed) lists."""
    k = len(q_rows)
    out = []
    for _ in range(n):
        drafts = [int(rng.choice(len(q), p=q)) for q in q_rows]
        ua = rng.random(k)
        ur = rng.random()
        m, com, _ = acc.stochastic_accept(p_rows, q_rows, drafts, ua, ur)
        out.append((m, com))
    return out


def test_accept_probability_is_overlap_mass():
    """P(accept d_1) = sum_x min(p(x), q(x)) (the overlap mass of the explainer, section 2.2)."""
    rng = np.random.default_rng(0)
    p = np.array([0.05, 0.3, 0.0, 0.15, 0.2, 0.1, 0.15, 0.05])
    q = np.array([0.2, 0.1, 0.1, 0.2, 0.1, 0.1, 0.05, 0.15])
    n = 60000
    res = _round_trials([p, p], [q], n, rng)
    acc_rate = np.mean([m == 1 for m, _ in res])
    expect = np.minimum(p, q).sum()
    assert abs(acc_rate - expect) < 4.5 * np.sqrt(expect * (1 - expect) / n)


@pytest.mark.parametrize("k", [1, 3])
def test_chi_square_first_token_follows_p(k):
    """The first emitted token of a round is distributed as p_1 (Leviathan-style theorem)."""
    rng = np.random.default_rng(10 + k)
    V = 8
    p_rows = [rng.dirichlet(np.ones(V)) for _ in range(k + 1)]
    p_rows[0][2] = 0.0
    p_rows[0] /= p_rows[0].sum()
    q_rows = [rng.dirichlet(np.ones(V)) for _ in range(k)]
    q_rows[0][5] = 0.0
    q_rows[0] /= q_rows[0].sum()
    n = 40000
    res = _round_trials(p_rows, q_rows, n, rng)
    first = np.bincount([com[0] for _, com in res], minlength=V)
    keep = p_rows[0] > 0
    assert first[~keep].sum() == 0
    _, pval = stats.chisquare(first[keep], n * p_rows[0][keep])
    assert pval > 1e-3


def test_chi_square_markov_chain_joint_two_tokens():
    """Sequential target p(x_n | x_(n-1)): the first two emitted tokens follow the target chain.

    The round's p rows are P[x0], P[d_1], ..., so a wrong row alignment (for
    example checking d_1 against P[d_1]) breaks this joint law.
    """
    rng = np.random.default_rng(21)
    V, k, x0 = 4, 3, 0
    P = rng.dirichlet(np.ones(V) * 0.7, size=V)
    Q = rng.dirichlet(np.ones(V) * 0.7, size=V)
    n = 40000
    counts = np.zeros((V, V))
    for _ in range(n):
        prev, drafts, q_rows = x0, [], []
        for _ in range(k):
            d = int(rng.choice(V, p=Q[prev]))
            drafts.append(d)
            q_rows.append(Q[prev])
            prev = d
        p_rows = [P[x0]] + [P[d] for d in drafts]
        m, com, _ = acc.stochastic_accept(p_rows, q_rows, drafts, rng.random(k), rng.random())
        a = com[0]
        if len(com) >= 2:
            b = com[1]
        else:
            b = int(rng.choice(V, p=P[a]))   # next round would start from the target at a
        counts[a, b] += 1
    expect = n * P[x0][:, None] * P
    _, pval = stats.chisquare(counts.ravel(), expect.ravel())
    assert pval > 1e-3


def test_q_equal_p_always_accepts():
    rng = np.random.default_rng(4)
    p = rng.dirichlet(np.ones(16))
    res = _round_trials([p, p, p], [p, p], 2000, rng)
    assert all(m == 2 for m, _ in res)


def test_one_hot_q_accepts_with_probability_p_of_draft():
    rng = np.random.default_rng(5)
    p = np.array([0.1, 0.6, 0.3])
    q = np.array([0.0, 0.0, 1.0])
    n = 20000
    res = _round_trials([p, p], [q], n, rng)
    rate = np.mean([m == 1 for m, _ in res])
    assert abs(rate - 0.3) < 4.5 * np.sqrt(0.3 * 0.7 / n)
    # on rejection the residual is p without the draft, renormalised: token 2 never appears
    rejected = [com[0] for m, com in res if m == 0]
    assert 2 not in rejected


def test_residual_fallback_to_p_when_mass_vanishes():
    p = np.array([0.5, 0.5])
    q = np.array([0.5, 0.5])
    # force a rejection with u above the ratio (ratio just below 1)
    m, com, info = acc.stochastic_accept([p, p], [q], [0], [0.9999999999], 0.75)
    assert m == 0 and info["residual_mass"] <= acc.RESIDUAL_EPS
    assert com == [1]


# ---------------------------------------------------------------------------
# Philox4x64-10
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("key,counter", [((3, 0), 0), ((3, 0), 41), ((0, 0), 0),
                                         ((0xDEADBEEF12345678, 0x0123456789ABCDEF), 123456789)])
def test_philox_matches_numpy_bitgenerator(key, counter):
    """numpy.random.Philox is an independent Philox4x64-10; it increments the counter before use."""
    k = key[0] | (key[1] << 64)
    bg = np.random.Philox(key=k, counter=counter)
    raw = [int(x) for x in bg.random_raw(8)]
    ours = list(philox.philox4x64_10((counter + 1, 0, 0, 0), key)) + \
        list(philox.philox4x64_10((counter + 2, 0, 0, 0), key))
    assert ours == raw


def test_philox_counter_words_all_matter():
    base = philox.philox4x64_10((1, 2, 3, 4), (3, 0))
    for i in range(4):
        c = [1, 2, 3, 4]
        c[i] += 1
        assert philox.philox4x64_10(c, (3, 0)) != base


def test_philox_uniform24_range_and_uniformity():
    u = np.array([philox.uniform(3, r, j, s) for r in range(400) for j in range(8) for s in range(3)])
    assert u.min() >= 0 and u.max() < 1
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))
    hist = np.histogram(u, bins=16, range=(0, 1))[0]
    _, pval = stats.chisquare(hist)
    assert pval > 1e-3
