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
    dw = noisy_head(TINY, w)
    return dict(b=b, S=TINY, w=w, model=b.Model(TINY, w), prompt=prompt, ow=ow, oc=oc, draft_w=dw,
                draft=b.Model(TINY, dw))


def noisy_head(S, w, sd=0.005, seed=5):
    """The target's weights with N(0, sd) added to the LM head, rounded to bf16: a draft
    that shares the target's cache and agrees with it often but not always."""
    head = [i for i, (name, _, _) in enumerate(S.tensor_specs()) if name == "lm_head"][0]
    out = list(w)
    h = bf16_bits_to_f64(w[head]) + np.random.default_rng(seed).normal(0, sd, w[head].shape)
    out[head] = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out


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
    N(0, 0.005) added to its LM head (rounded to bf16), so that paths of every length occur."""
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
    dw = OracleWeights(S, env["draft_w"])
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


def _greedy_ar(env, n_new):
    b, S = env["b"], env["S"]
    toks = torch.zeros(n_new + 2, dtype=torch.int32, device="cuda")
    lg = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    c, w = b.Cache(S, 512), b.Workspace(S, 512)
    b.prefill(env["model"], c, torch.from_numpy(env["prompt"]).cuda(), w, logits=lg, argmax=toks[0:1])
    for i in range(n_new):
        b.decode_step(env["model"], c, toks[i:i + 1], w, logits=lg, argmax=toks[i + 1:i + 2])
    return [int(x) for x in to_np(toks)]


def _deep_tree(rng, levels, width):
    """A tree of `width` nodes a level: each node's parent is a random node of the level above."""
    pars, level = [-1], [0]
    for _ in range(levels):
        nxt = []
        for _ in range(width):
            pars.append(int(rng.choice(level)))
            nxt.append(len(pars) - 1)
        level = nxt
    return pars


def test_deep_tree_verify_in_passes_against_oracle(env):
    """97 nodes (three passes of 32 and one of 1) against the oracle's tree-causal forward."""
    from oracle.tree import tree_forward
    rng = np.random.default_rng(97)
    pars = _deep_tree(rng, 24, 4)
    toks = [int(x) for x in rng.integers(0, env["S"].vocab, len(pars))]
    c, ws = _cache(env)
    _, _, lg, am = _tree(env, c, ws, toks, pars)
    ol = tree_forward(env["ow"], env["oc"].clone(), toks, pars)
    g = to_np(lg)
    assert_logits_close(g, ol, "tiny deep tree verify (97 nodes)")
    assert np.array_equal(to_np(am), g.argmax(axis=1)) and c.length() == P + len(toks) and ws.error_bits() == 0


def test_deep_chain_equals_block_passes(env):
    """A 40-node chain: the same kernels as causal blocks of 32 and 8 rows, bit for bit."""
    b = env["b"]
    toks = [int(x) for x in np.random.default_rng(40).integers(0, env["S"].vocab, 40)]
    c1, w1 = _cache(env)
    _, _, lt, at = _tree(env, c1, w1, toks, [-1] + list(range(39)))
    c2, w2 = _cache(env)
    lb = torch.empty_like(lt)
    t = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    b.decode_step(env["model"], c2, t[:32], w2, logits=lb[:32])
    b.decode_step(env["model"], c2, t[32:], w2, logits=lb[32:])
    assert torch.equal(lt.view(torch.int32), lb.view(torch.int32))


def test_deep_accept_moves_long_paths(env):
    """Two nodes a level over 40 levels, the target's greedy token always on the second:
    a 40-node path from nodes 2, 4, ..., 80, so the compaction moves runs of 32 and 8."""
    from oracle.tree import tree_accept_greedy
    b, S = env["b"], env["S"]
    ar = _greedy_ar(env, 41)
    toks, pars = [int(env["prompt"][-1])], [-1]
    c, ws = _cache(env)
    c.trim(P - 1, ws)   # the root is the prompt's last token: pending again
    prev = 0
    for lv in range(40):
        toks += [(ar[lv] + 1) % S.vocab, ar[lv]]
        pars += [prev, prev]
        prev = len(toks) - 1
    t, p, lg, am = _tree(env, c, ws, toks, pars)
    kk, vv = c.kv()
    k0, v0 = kk.clone(), vv.clone()
    out = torch.zeros(len(toks), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    root = torch.zeros(1, dtype=torch.int32, device="cuda")
    log = torch.zeros(1 + 64, dtype=torch.int32, device="cuda")
    b.tree_accept(c, t, p, am, out, cnt, err, root=root, log=log)
    path, com = tree_accept_greedy(toks, pars, list(to_np(am)))
    assert path == list(range(2, 81, 2)) and com == ar[:41]
    assert int(cnt.item()) == 41 and [int(x) for x in to_np(out)[:41]] == com and int(root.item()) == ar[40]
    assert int(log[0].item()) == 41 and [int(x) for x in to_np(log)[1:42]] == com and int(err.item()) == 0
    t0 = P - 1
    assert c.length() == t0 + 41
    k1, v1 = c.kv()
    for dst, src in enumerate([0] + path):
        assert torch.equal(k1[:, :, t0 + dst], k0[:, :, t0 + src]) and torch.equal(v1[:, :, t0 + dst], v0[:, :, t0 + src])


def _draft_tree(env, c, ws, k, D, T=0.2, draft=None, root=None):
    b = env["b"]
    n = 1 + k * D
    root = torch.tensor([int(env["prompt"][-1]) if root is None else root], dtype=torch.int32, device="cuda")
    toks = torch.zeros(n, dtype=torch.int32, device="cuda")
    pars = torch.zeros(n, dtype=torch.int32, device="cuda")
    sc = torch.zeros(n, dtype=torch.float32, device="cuda")
    b.tree_draft(draft or env["draft"], c, root, k, D, toks, pars, sc, ws, temperature=T)
    return toks, pars, sc


def _check_construction(env, c, ws, toks, pars, sc, k, D, T=0.2, draft=None):
    """Replays the oracle's selection rule on the draft's own logits of the GPU's tree
    (a draft tree forward of the whole tree); near-ties (relative score gap below 1e-5
    at the k-th place) are counted, not compared.  Returns the number of near-ties."""
    from oracle.tree import select_children
    b, S = env["b"], env["S"]
    t0 = c.length()
    n = 1 + k * D
    lg = torch.empty((n, S.vocab), dtype=torch.float32, device="cuda")
    b.tree_verify(draft or env["draft"], c, toks, pars, ws, logits=lg)
    c.trim(t0, ws)
    z = to_np(lg).astype(np.float64)
    gt, gp, gs = [int(x) for x in to_np(toks)], [int(x) for x in to_np(pars)], to_np(sc).astype(np.float64)
    score = {0: 1.0}
    leaves, ties = [0], 0
    for s in range(D):
        cand = select_children(leaves, [z[l] for l in leaves], score, k + 1, T)
        rows = list(range(1 + k * s, 1 + k * (s + 1)))
        if len(cand) > k and cand[k - 1][0] - cand[k][0] <= 1e-5 * cand[k - 1][0]:
            ties += 1
            break   # the GPU may take either side of a near-tie: later steps differ
        for r, (s_, leaf, tok) in zip(rows, cand[:k]):
            assert (gp[r], gt[r]) == (leaf, tok), f"step {s} node {r}"
            assert abs(gs[r] - np.log(s_)) <= 1e-3 + 1e-4 * abs(np.log(s_)), f"score of node {r}"
            score[r] = s_
        leaves = rows
    return ties


def test_tree_draft_follows_the_selection_rule(env):
    c, ws = _cache(env)
    c.trim(P - 1, ws)
    toks, pars, sc = _draft_tree(env, c, ws, 3, 4)
    assert c.length() == P - 1 and ws.error_bits() == 0
    ties = _check_construction(env, c, ws, toks, pars, sc, 3, 4)
    say(f"tree draft k=3 D=4: tokens {[int(x) for x in to_np(toks)]}, parents {[int(x) for x in to_np(pars)]}, "
        f"near-ties {ties}")
    assert ties == 0


def test_deep_tree_draft_k6_d48(env):
    """The pages' deep construction (k = 6, D = 48: 289 nodes): shape, monotone scores,
    the selection rule at every step, then the target's verify of all 289 nodes against
    the oracle and the acceptance against the oracle rule."""
    from oracle.tree import tree_accept_greedy, tree_forward
    b = env["b"]
    k, D = 6, 48
    c, ws = _cache(env)
    ar = _greedy_ar(env, 2)
    toks, pars, sc = _draft_tree(env, c, ws, k, D, root=ar[0])
    gp, gs = [int(x) for x in to_np(pars)], to_np(sc)
    for s in range(1, D):
        assert all(1 + k * (s - 1) <= gp[r] < 1 + k * s for r in range(1 + k * s, 1 + k * (s + 1)))
    assert all(gs[i] <= gs[gp[i]] + 1e-6 for i in range(1, len(gp)))
    ties = _check_construction(env, c, ws, toks, pars, sc, k, D)
    say(f"deep tree draft: near-ties {ties}")
    lg = torch.empty((len(gp), env["S"].vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(len(gp), dtype=torch.int32, device="cuda")
    b.tree_verify(env["model"], c, toks, pars, ws, logits=lg, argmax=am)
    oc = env["oc"].clone()
    gt = [int(x) for x in to_np(toks)]
    ol = tree_forward(env["ow"], oc, gt, gp)
    assert_logits_close(to_np(lg), ol, "tiny 289-node tree verify")
    out = torch.zeros(len(gp), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    b.tree_accept(c, toks, pars, am, out, cnt, err)
    path, com = tree_accept_greedy(gt, gp, list(to_np(am)))
    assert int(cnt.item()) == len(com) and [int(x) for x in to_np(out)[:len(com)]] == com
    assert len(path) >= 1 and c.length() == P + 1 + len(path) and ws.error_bits() == 0 and int(err.item()) == 0
    say(f"289-node tree: path {path}")


@pytest.fixture(scope="module")
def q4draft(env):
    from block_verify_amd.synth import make_q4_draft
    b, S = env["b"], env["S"]
    return b.Model(S, make_q4_draft(S, env["w"]), weight_format=b.W_Q4G64, share=env["model"])


def test_q4_tree_draft_follows_the_selection_rule(env, q4draft):
    """The 4-bit substitute builds with k = 6 leaves a step."""
    c, ws = _cache(env)
    c.trim(P - 1, ws)
    toks, pars, sc = _draft_tree(env, c, ws, 6, 3, draft=q4draft)
    assert c.length() == P - 1 and ws.error_bits() == 0
    ties = _check_construction(env, c, ws, toks, pars, sc, 6, 3, draft=q4draft)
    say(f"q4 tree draft k=6 D=3: near-ties {ties}")
    assert ties == 0


@pytest.mark.parametrize("k,D,q4", [(2, 3, False), (4, 6, False), (6, 4, True)])
def test_gpu_built_tree_job_is_lossless(env, q4draft, k, D, q4):
    """Rounds of construction (the noisy-head draft on the shared cache), verify and
    acceptance, all on the GPU with the job log and the next root on the device, commit
    the GPU's greedy decode."""
    b, S = env["b"], env["S"]
    n_new = 24
    ar = _greedy_ar(env, n_new)
    c, ws = _cache(env)
    c.trim(P - 1, ws)
    n = 1 + k * D
    root = torch.tensor([int(env["prompt"][-1])], dtype=torch.int32, device="cuda")
    toks = torch.zeros(n, dtype=torch.int32, device="cuda")
    pars = torch.zeros(n, dtype=torch.int32, device="cuda")
    sc = torch.zeros(n, dtype=torch.float32, device="cuda")
    am = torch.zeros(n, dtype=torch.int32, device="cuda")
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    log = torch.zeros(1 + 128, dtype=torch.int32, device="cuda")
    rounds, ms = 0, []
    while int(log[0].item()) < n_new:
        b.tree_draft(q4draft if q4 else env["draft"], c, root, k, D, toks, pars, sc, ws)
        b.tree_verify(env["model"], c, toks, pars, ws, argmax=am)
        b.tree_accept(c, toks, pars, am, out, cnt, err, root=root, log=log)
        rounds += 1
        ms.append(int(cnt.item()) - 1)
    got = [int(x) for x in to_np(log)[1:1 + int(log[0].item())]]
    assert got[:n_new] == ar[:n_new] and int(err.item()) == 0 and ws.error_bits() == 0
    assert c.length() == P - 1 + len(got)
    say(f"GPU-built tree job k={k} D={D} {'4-bit' if q4 else 'noisy-head'} draft: {rounds} rounds, "
        f"accepted per round {ms}")
    assert sum(ms) > 0


def test_tree_argument_checks(env):
    b = env["b"]
    c, ws = _cache(env)
    root = torch.zeros(1, dtype=torch.int32, device="cuda")
    big = torch.zeros(600, dtype=torch.int32, device="cuda")
    sc = torch.zeros(600, dtype=torch.float32, device="cuda")
    with pytest.raises(b.SpecdecError):
        b.tree_draft(env["draft"], c, root, 0, 3, big, big, sc, ws)
    with pytest.raises(b.SpecdecError):
        b.tree_draft(env["draft"], c, root, 6, 90, big, big, sc, ws)   # 541 nodes
    with pytest.raises(b.SpecdecError):
        b.tree_draft(env["draft"], c, root, 2, 3, big, big, sc, ws, temperature=0.0)
    with pytest.raises(b.SpecdecError):
        b.tree_verify(env["model"], c, big[:513], big[:513], ws)
    assert c.length() == P


def test_largest_tree_and_single_node(env):
    """SPECDEC_MAX_TREE = 512 nodes (a chain of 200 nodes, then a fan of the rest under
    node 150, so the ancestor masks use their last word) against the oracle's tree
    forward and acceptance; then a tree of the root alone (no path, one committed token)."""
    from oracle.tree import tree_accept_greedy, tree_forward
    b, S = env["b"], env["S"]
    n = b.MAX_TREE
    pars = [-1] + list(range(199)) + [150] * (n - 200)
    toks = [int(x) for x in np.random.default_rng(512).integers(0, S.vocab, n)]
    c, ws = b.Cache(S, 1024), b.Workspace(S, 1024)
    b.prefill(env["model"], c, torch.from_numpy(env["prompt"]).cuda(), ws)
    t, p, lg, am = _tree(env, c, ws, toks, pars)
    oc = _oracle_cache(env, 1024)
    ol = tree_forward(env["ow"], oc, toks, pars)
    assert_logits_close(to_np(lg), ol, "tiny 512-node tree verify")
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    b.tree_accept(c, t, p, am, out, cnt, err)
    path, com = tree_accept_greedy(toks, pars, list(to_np(am)))
    assert int(cnt.item()) == len(com) and c.length() == P + 1 + len(path) and ws.error_bits() == 0
    # the root alone
    c.trim(P, ws)
    t1, p1, lg1, am1 = _tree(env, c, ws, [toks[0]], [-1])
    b.tree_accept(c, t1, p1, am1, out[:1], cnt, err)
    assert int(cnt.item()) == 1 and int(out[0].item()) == int(am1[0].item()) and c.length() == P + 1
    assert int(err.item()) == 0


def _oracle_cache(env, max_len):
    from oracle.model import OracleCache
    oc = OracleCache(env["S"], max_len)
    src = env["oc"]
    for l in range(env["S"].n_layers):
        oc.k[l][:, :P] = src.k[l][:, :P]
        oc.v[l][:, :P] = src.v[l][:, :P]
    oc.length = P
    return oc
