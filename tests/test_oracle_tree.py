"""Pins of the oracle's draft tree (oracle/tree.py) on the tiny decoder (CPU only).

"SubSpec" summary, section 4.2 (tree construction by cumulative sharpened draft
probability, k x D nodes) and the tree-causal verify; a single chain must
reduce to the block verify of "SpecDec-Context-Scaling 项目解读", section 3.
"""
import numpy as np
import pytest

from block_verify_amd.shapes import SEED_DRAFT, TINY
from block_verify_amd.synth import make_weights
from oracle import accept as acc
from oracle import tree
from oracle.model import OracleCache, OracleWeights, forward, prefill
from oracle.spec import ar_greedy

P = 64


@pytest.fixture(scope="module")
def tw(tiny_weights):
    return OracleWeights(TINY, tiny_weights)


@pytest.fixture(scope="module")
def base(tw, tiny_prompt):
    c = OracleCache(TINY, 256)
    prefill(tw, c, tiny_prompt[:P])
    return c


def test_chain_tree_equals_block_forward(tw, base):
    toks = [5, 77, 4095, 0, 1234]
    a, b = base.clone(), base.clone()
    lt = tree.tree_forward(tw, a, toks, [-1, 0, 1, 2, 3])
    lb = forward(tw, b, toks)
    np.testing.assert_allclose(lt, lb, rtol=0, atol=1e-12)
    for l in range(TINY.n_layers):
        np.testing.assert_array_equal(a.k[l][:, :a.length], b.k[l][:, :b.length])


def test_every_node_equals_the_forward_of_its_path(tw, base):
    """Brute force: each row of a branching tree equals the last row of a plain causal
    forward of its root-to-node path (the mask admits exactly the ancestors, the position
    is the depth)."""
    toks = [9, 100, 200, 300, 400, 500, 600, 700]
    pars = [-1, 0, 0, 1, 1, 2, 4, 6]
    lt = tree.tree_forward(tw, base.clone(), toks, pars)
    for i in range(len(toks)):
        path, j = [], i
        while j >= 0:
            path.append(toks[j])
            j = pars[j]
        ref = forward(tw, base.clone(), path[::-1])[-1]
        np.testing.assert_allclose(lt[i], ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("argmax,path,committed", [
    ([10, 0, 0, 0, 0, 0], [], [10]),                 # no child of the root carries 10
    ([1, 3, 0, 0, 0, 0], [1], [1, 3]),               # root -> row 1 (token 1); its children carry 4, 5
    ([1, 5, 0, 0, 7, 0], [1, 4], [1, 5, 7]),         # root -> 1 -> row 4 (token 5), a leaf: bonus 7
    ([2, 0, 6, 0, 0, 0], [2], [2, 6]),               # row 2 (token 2) has no child with token 6: commit 6
    ([2, 0, 9, 0, 0, 0], [2, 5], [2, 9, 0]),         # row 2 -> row 5 (token 9)
])
def test_tree_accept_golden(argmax, path, committed):
    # rows: 0 root; 1 (token 1) and 2 (token 2) children of the root; 3 (token 4) and 4 (token 5)
    # children of row 1; 5 (token 9) child of row 2
    toks = [7, 1, 2, 4, 5, 9]
    pars = [-1, 0, 0, 1, 1, 2]
    assert tree.tree_accept_greedy(toks, pars, argmax) == (path, committed)


def test_chain_accept_equals_block_greedy():
    rng = np.random.default_rng(3)
    for _ in range(50):
        k = int(rng.integers(1, 6))
        drafts = list(rng.integers(0, 4, k))
        v = list(rng.integers(0, 4, k + 1))
        path, com = tree.tree_accept_greedy([99] + drafts, [-1] + list(range(k)), v)
        m, com2 = acc.greedy_accept(v, drafts)
        assert (len(path), com) == (m, com2)


def test_compact_keeps_root_and_path(tw, base):
    toks = [9, 100, 200, 300, 400, 500]
    pars = [-1, 0, 0, 2, 2, 4]
    c = base.clone()
    t = c.length
    tree.tree_forward(tw, c, toks, pars)
    tree.compact(c, t, [2, 4, 5])
    ref = base.clone()
    forward(tw, ref, [9, 200, 400, 500])
    assert c.length == ref.length == t + 4
    for l in range(TINY.n_layers):
        np.testing.assert_allclose(c.k[l][:, :c.length], ref.k[l][:, :ref.length], atol=1e-10)
        np.testing.assert_allclose(c.v[l][:, :c.length], ref.v[l][:, :ref.length], atol=1e-10)


def test_tree_shape_and_top_k_selection(tw, base):
    """k x D nodes; each step's k leaves are the k best (leaf, token) pairs by cumulative
    sharpened probability, checked by brute force over every leaf path's plain forward."""
    k, D = 3, 3
    dw = OracleWeights(TINY, make_weights(TINY, SEED_DRAFT))
    toks, pars = tree.build_draft_tree(dw, base, 17, k, D)
    assert len(toks) == 1 + k * D and base.length == P
    assert pars[1:1 + k] == [0] * k
    score = {0: 1.0}
    level = [0]
    for s in range(D):
        cand = []
        for leaf in level:
            path, j = [], leaf
            while j >= 0:
                path.append(toks[j])
                j = pars[j]
            z = forward(dw, base.clone(), path[::-1])[-1]
            p = acc.softmax(z, tree.SHARPEN_T)
            cand += [(score[leaf] * p[x], leaf, x) for x in range(TINY.vocab)]
        cand.sort(key=lambda c: (-c[0], c[1], c[2]))
        rows = list(range(1 + k * s, 1 + k * (s + 1)))
        assert [(pars[r], toks[r]) for r in rows] == [(c[1], c[2]) for c in cand[:k]]
        for r, c in zip(rows, cand[:k]):
            score[r] = c[0]
        level = rows


def test_single_branch_tree_is_the_draft_greedy_chain(tw, base):
    dw = OracleWeights(TINY, make_weights(TINY, SEED_DRAFT))
    toks, pars = tree.build_draft_tree(dw, base, 17, 1, 4)
    assert pars == [-1, 0, 1, 2, 3]
    c = base.clone()
    lg = forward(dw, c, [17])[0]
    chain = []
    for _ in range(4):
        chain.append(acc.argmax_lowest(lg))
        lg = forward(dw, c, [chain[-1]])[0]
    assert toks[1:] == chain


def test_tree_speculation_is_lossless(tw, tiny_prompt):
    ar, _ = ar_greedy(tw, tiny_prompt[:P], 12)
    dw = OracleWeights(TINY, make_weights(TINY, SEED_DRAFT))
    toks, ms, _ = tree.spec_tree_greedy(tw, dw, tiny_prompt[:P], 12, k=2, depth=3)
    assert toks == ar
    # the target as its own draft: every round takes a whole path of depth D
    toks, ms, _ = tree.spec_tree_greedy(tw, tw, tiny_prompt[:P], 12, k=2, depth=3)
    assert toks == ar and all(m == 3 for m in ms[:-1])
