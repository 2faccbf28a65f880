"""GPU parity of the draft-tree verify and its greedy acceptance ("SubSpec" summary,
section 4.2) on the tiny decoder, through the C ABI (specdec_tree_verify,
specdec_tree_accept), against the oracle (oracle/tree.py)."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_logits_close, bf16_bits_to_f64, say, to_np

pytestmark = pytest.mark.gpu

P = 128
TOKS = [9, 100, 200, 300, 400, 500, 600, 700, 800, 900]
PARS = [-1, 0, 0, 1, 1, 2, 4, 6, 3, 5]


@pytest.fixture(scope="module")
def env():
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import TINY, SEED_TARGET
    from block_verify_amd.synth import make_prompt, make_weights
    from oracle.model import OracleCache, OracleWeights, prefill
    w = make_weights(TINY, SEED_TARGET)
    prompt = make_prompt(TINY.vocab, P)
    ow = OracleWeights(TINY, w)
    oc = OracleCache(TINY, 512)
    prefill(ow, oc, prompt)
    return dict(b=b, S=TINY, w=w, model=b.Model(TINY, w), prompt=prompt, ow=ow, oc=oc)


def _cache(env, max_len=512):
    b, S = env["b"], env["S"]
    c, ws = b.Cache(S, max_len), b.Workspace(S, max_len)
    b.prefill(env["model"], c, torch.from_numpy(env["prompt"]).cuda(), ws)
    return c, ws


def _tree(env, c, ws, toks, pars):
    b, S = env["b"], env["S"]
    n = len(toks)
    t = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    p = torch.from_numpy(np.asarray(pars, np.int32)).cuda()
    lg = torch.empty((n, S.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(n, dtype=torch.int32, device="cuda")
    b.tree_verify(env["model"], c, t, p, ws, logits=lg, argmax=am)
    return t, p, lg, am


def test_chain_tree_is_the_block_verify_bit_for_bit(env):
    b = env["b"]
    toks = TOKS[:6]
    c1, w1 = _cache(env)
    _, _, lt, at = _tree(env, c1, w1, toks, [-1, 0, 1, 2, 3, 4])
    c2, w2 = _cache(env)
    lb = torch.empty_like(lt)
    ab = torch.empty_like(at)
    b.decode_step(env["model"], c2, torch.from_numpy(np.asarray(toks, np.int32)).cuda(), w2, logits=lb, argmax=ab)
    assert torch.equal(lt.view(torch.int32), lb.view(torch.int32)) and torch.equal(at, ab)
    k1, v1 = c1.kv()
    k2, v2 = c2.kv()
    assert torch.equal(k1[:, :, :P + 6], k2[:, :, :P + 6]) and torch.equal(v1[:, :, :P + 6], v2[:, :, :P + 6])


def test_branching_tree_logits_and_kv_against_oracle(env):
    from oracle.tree import tree_forward
    c, ws = _cache(env)
    _, _, lg, am = _tree(env, c, ws, TOKS, PARS)
    oc = env["oc"].clone()
    ol = tree_forward(env["ow"], oc, TOKS, PARS)
    g = to_np(lg)
    assert_logits_close(g, ol, "tiny tree verify")
    assert np.array_equal(to_np(am), g.argmax(axis=1))
    assert c.length() == P + len(TOKS) and ws.error_bits() == 0
    kk, vv = c.kv()
    for l in range(env["S"].n_layers):
        gk = bf16_bits_to_f64(to_np(kk[l][:, P:P + len(TOKS)]))
        gv = bf16_bits_to_f64(to_np(vv[l][:, P:P + len(TOKS)]))
        for g_, o_ in ((gk, oc.k[l][:, P:P + len(TOKS)]), (gv, oc.v[l][:, P:P + len(TOKS)])):
            assert np.abs(g_ - o_).max() <= 1e-2 * np.abs(o_).max()


def test_each_node_matches_the_forward_of_its_path(env):
    """Every row of the tree against the GPU's own causal forward of its root-to-node path
    (same kernels; only the keys' slots differ, so within a float tolerance)."""
    b = env["b"]
    c, ws = _cache(env)
    _, _, lg, _ = _tree(env, c, ws, TOKS, PARS)
    g = to_np(lg)
    for i in range(len(TOKS)):
        path, j = [], i
        while j >= 0:
            path.append(TOKS[j])
            j = PARS[j]
        cp, wp = _cache(env)
        lp = torch.empty((len(path), env["S"].vocab), dtype=torch.float32, device="cuda")
        b.decode_step(env["model"], cp, torch.from_numpy(np.asarray(path[::-1], np.int32)).cuda(), wp, logits=lp)
        np.testing.assert_allclose(g[i], to_np(lp)[-1], rtol=0, atol=2e-5)


def test_accept_and_compaction(env):
    """The path and committed tokens equal the oracle rule on the GPU's argmax; the cache
    keeps the root and moves the path's K/V (bit copies of the tree forward's rows)."""
    from oracle.tree import tree_accept_greedy
    b, S = env["b"], env["S"]
    c, ws = _cache(env)
    # make the tree agree with the target where it can: each row's first child carries its
    # parent's argmax (set in row order, so the parent's ancestors are final when it is read)
    toks, pars = list(TOKS), list(PARS)
    for i in range(1, len(toks)):
        if i == min(j for j in range(len(toks)) if pars[j] == pars[i]):
            _, _, _, am0 = _tree(env, c, ws, toks, pars)
            toks[i] = int(to_np(am0)[pars[i]])
            c.trim(P, ws)
    t, p, lg, amt = _tree(env, c, ws, toks, pars)
    k0, v0 = (x.clone() for x in c.kv())
    out = torch.zeros(len(toks), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    b.tree_accept(c, t, p, amt, out, cnt, err)
    path, com = tree_accept_greedy(toks, pars, list(to_np(amt)))
    n = int(cnt.item())
    assert n == len(com) and [int(x) for x in to_np(out)[:n]] == com and int(err.item()) == 0
    assert c.length() == P + 1 + len(path) and path == [1, 3, 8]
    k1, v1 = c.kv()
    rows = [P] + [P + i for i in path]
    for dst, src in enumerate(rows):
        assert torch.equal(k1[:, :, P + dst], k0[:, :, src]) and torch.equal(v1[:, :, P + dst], v0[:, :, src])
    say(f"tree accept: path {path}, committed {com}")


def test_invalid_parent_is_flagged(env):
    c, ws = _cache(env)
    _tree(env, c, ws, [1, 2, 3], [-1, 2, 0])
    assert ws.error_bits() & env["b"].DERR_TREE


def test_tree_job_is_lossless(env):
    """Rounds with trees from the oracle's builder (k = 2, D = 3, sharpening 0.2) verified
    and accepted on the GPU commit the GPU's greedy decode.  The draft is the target with
    N(0, 0.005) added to its LM head, so that paths of every length occur."""
    from oracle.model import OracleCache, OracleWeights, forward, prefill
    from oracle.tree import build_draft_tree
    b, S = env["b"], env["S"]
    n_new = 16
    # GPU greedy AR
    c, ws = _cache(env)
    toks = torch.zeros(n_new + 2, dtype=torch.int32, device="cuda")
    lg = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    c2, w2 = b.Cache(S, 512), b.Workspace(S, 512)
    b.prefill(env["model"], c2, torch.from_numpy(env["prompt"]).cuda(), w2, logits=lg, argmax=toks[0:1])
    for i in range(n_new):
        b.decode_step(env["model"], c2, toks[i:i + 1], w2, logits=lg, argmax=toks[i + 1:i + 2])
    ar = [int(x) for x in to_np(toks)]
    # tree job, schedule-B layout: prompt[:-1] cached, prompt[-1] pending
    dt = [bf16_bits_to_f64(t) for t in env["w"]]
    head = [i for i, (name, _, _) in enumerate(S.tensor_specs()) if name == "lm_head"][0]
    dt[head] = dt[head] + np.random.default_rng(5).normal(0, 0.005, dt[head].shape)
    dw = OracleWeights(S, dt)
    oc = OracleCache(S, 512)
    prefill(dw, oc, env["prompt"][:-1])
    gc, gw = b.Cache(S, 512), b.Workspace(S, 512)
    b.prefill(env["model"], gc, torch.from_numpy(env["prompt"][:-1]).cuda(), gw)
    pending, committed, ms = int(env["prompt"][-1]), [], []
    out = torch.zeros(32, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    while len(committed) < n_new:
        tt, pp = build_draft_tree(dw, oc, pending, 2, 3)
        t, p, _, am = _tree(env, gc, gw, tt, pp)
        b.tree_accept(gc, t, p, am, out[:len(tt)], cnt, err)
        n = int(cnt.item())
        com = [int(x) for x in to_np(out)[:n]]
        forward(dw, oc, [pending] + com[:-1])    # the draft's own cache follows the committed tokens
        committed += com
        ms.append(n - 1)
        pending = com[-1]
        assert gc.length() == P - 1 + len(committed)
    assert committed[:n_new] == ar[:n_new] and int(err.item()) == 0 and gw.error_bits() == 0
    assert sum(ms) >= 4 and min(ms) < 3
    say(f"tree job: {len(ms)} rounds, accepted per round {ms}")
