"""Pins of the oracle's speculative rounds on the tiny decoder (CPU only).

Greedy speculative decoding is lossless: with any drafts its committed
tokens equal plain greedy decoding ("SpecDec-Context-Scaling 项目解读",
section 8, the algorithmic-correctness layer).  The cache invariant
(length == committed tokens, no rejected token left) is the page's section
3.2; it is asserted inside every round and checked here against a fresh
prefill.
"""
import numpy as np
import pytest

from block_verify_amd.shapes import SEED_DRAFT, TINY, SEED_NOISE
from block_verify_amd.synth import make_draft_table, make_noise, make_weights, quantize_q4g64
from oracle import q4
from oracle.model import OracleCache, OracleWeights, prefill
from oracle.spec import ar_greedy, spec_greedy, spec_stochastic

N_NEW, K = 16, 4


@pytest.fixture(scope="module")
def tw(tiny_weights):
    return OracleWeights(TINY, tiny_weights)


@pytest.fixture(scope="module")
def ar(tw, tiny_prompt):
    toks, _ = ar_greedy(tw, tiny_prompt, N_NEW + K + 1)
    return toks


@pytest.mark.parametrize("c", [0.0, 0.4, 1.0])
@pytest.mark.parametrize("schedule", ["A", "B"])
def test_spec_table_drafts_equal_ar(tw, tiny_prompt, ar, c, schedule):
    table = make_draft_table(np.array(ar), TINY.vocab, c)
    tr = spec_greedy(tw, tiny_prompt, N_NEW, K, table=table, schedule=schedule)
    assert tr.tokens == ar[:N_NEW]
    if c == 0.0:
        assert all(m == K for m in tr.m[:-1])
    if c == 1.0:
        assert all(m == 0 for m in tr.m)


def test_spec_no_bonus_equal_ar(tw, tiny_prompt, ar):
    table = make_draft_table(np.array(ar), TINY.vocab, 0.2)
    tr = spec_greedy(tw, tiny_prompt, N_NEW, K, table=table, bonus=False)
    assert tr.tokens == ar[:N_NEW]


def test_acceptance_matches_corruption_rate(tw, tiny_prompt, ar):
    """With table drafts, draft j is accepted iff it was not corrupted (and its prefix was)."""
    table = make_draft_table(np.array(ar), TINY.vocab, 0.4)
    tr = spec_greedy(tw, tiny_prompt, N_NEW, K, table=table)
    n0 = 0
    for m, d in zip(tr.m, tr.drafts):
        ok = [table[n0 + j] == ar[n0 + j] for j in range(K)]
        expect = next((j for j in range(K) if not ok[j]), K)
        assert m == expect
        n0 += m + 1


def test_cache_after_spec_equals_fresh_prefill(tw, tiny_prompt, ar):
    table = make_draft_table(np.array(ar), TINY.vocab, 0.4)
    P = len(tiny_prompt)
    for schedule in ("A", "B"):
        tr = spec_greedy(tw, tiny_prompt, N_NEW, K, table=table, schedule=schedule)
        c = tr.cache
        full = list(tiny_prompt) + list(ar[:c.length - P])
        ref = OracleCache(TINY, c.max_len)
        prefill(tw, ref, full)
        assert c.length == ref.length
        for l in range(TINY.n_layers):
            np.testing.assert_allclose(c.k[l][:, :c.length], ref.k[l][:, :c.length], atol=1e-10)
            np.testing.assert_allclose(c.v[l][:, :c.length], ref.v[l][:, :c.length], atol=1e-10)


def test_spec_with_independent_draft_model(tw, tiny_prompt, ar):
    """Config-3 form: a second decoder with its own cache, tokens overridden by the table."""
    dw = OracleWeights(TINY, make_weights(TINY, SEED_DRAFT))
    table = make_draft_table(np.array(ar), TINY.vocab, 0.5)
    for schedule in ("A", "B"):
        tr = spec_greedy(tw, tiny_prompt, N_NEW, K, table=table, draft_w=dw, schedule=schedule)
        assert tr.tokens == ar[:N_NEW]
        assert tr.draft_calls == sum(K + 1 for _ in tr.m)


def _q4_weights(shape, tensors):
    """Substitute draft: 4-bit linears, bf16 embedding / LM head / norms shared."""
    out = list(tensors)
    for i, (name, _, kind) in enumerate(shape.tensor_specs()):
        if kind == "linear" and name != "lm_head":
            packed, s, z = quantize_q4g64(tensors[i])
            out[i] = q4.dequantize(packed, s, z)
    return OracleWeights(shape, out)


def test_spec_with_q4_substitute_draft_is_lossless(tw, tiny_weights, tiny_prompt, ar):
    qw = _q4_weights(TINY, tiny_weights)
    tr = spec_greedy(tw, tiny_prompt, N_NEW, 8, q4_draft_w=qw)
    assert tr.tokens == ar[:N_NEW]
    assert all(m >= 1 for m in tr.m)   # d_1 = argmax(saved_next) always passes


def test_stochastic_rounds_keep_invariant(tw, tiny_prompt):
    noise = make_noise(N_NEW + K, TINY.vocab, SEED_NOISE)
    tr = spec_stochastic(tw, tiny_prompt, N_NEW, K, noise, seed=3)
    assert len(tr.tokens) == N_NEW
    assert tr.rounds == len(tr.m)
    assert all(0 <= t < TINY.vocab for t in tr.tokens)
