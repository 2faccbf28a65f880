"""GPU parity on seeded random decoder shapes (one or two layers).

Every launch path of the forward depends on the shape: the k-split of each
product, the row-group forms of gate/up, the attention's query tiles per
workgroup, the grid padding and the merge form (by cache capacity).  Each case
draws a shape within the library's documented limits (head dim 64 or 128, up
to 8 query heads per kv head, hidden up to 4096, multiples of 32), a prompt
length, a pass of 1..32 rows and a cache capacity, then checks

- the pass against the oracle forward (logit tolerance of the parity bar);
- the pass against the same rows in single-row steps, bit for bit (batch
  invariance across every launch form);

and the 4-bit cases the same against the oracle with the dequantised weights.
Greedy rounds on random shapes (k up to 16, so verify passes of up to 17
rows) must commit the GPU's own greedy AR decode token for token.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_logits_close, q4_oracle_weights, say, to_np

pytestmark = pytest.mark.gpu


def _case(seed, q4=False):
    rng = np.random.default_rng(seed)
    while True:
        hd = int(rng.choice([64, 128]))
        nkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 6, 7, 8]))
        H = int(rng.choice([256, 512, 768, 896, 1024, 1536, 2048]))
        F = 32 * int(rng.integers(8, 160))
        V = 16 * int(rng.integers(64, 512))
        L = int(rng.choice([1, 2]))
        qd = nkv * G * hd
        ok = qd % 32 == 0 and qd <= 4096
        if q4:
            ok = ok and H % 64 == 0 and F % 64 == 0 and qd % 64 == 0
        if ok:
            break
    P = int(rng.integers(1, 300))
    M = int(rng.integers(1, 33))
    cap = max(int(rng.choice([P + M, P + M + 7, 512, 3072, 3136, 4200])), P + M)
    chunk = int(rng.integers(1, 33))
    return dict(L=L, H=H, F=F, V=V, nq=nkv * G, nkv=nkv, hd=hd, P=P, M=M, cap=cap, chunk=chunk, seed=seed)


def _run(c, q4):
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import ModelShape
    from block_verify_amd.synth import make_prompt, make_q4_draft, make_weights
    from oracle.model import OracleCache, OracleWeights, forward, prefill
    S = ModelShape(f"rand{c['seed']}", c["L"], c["H"], c["nq"], c["nkv"], c["hd"], c["F"], c["V"])
    say(f"random shape {c} q4={q4}")
    w = make_weights(S, 1000 + c["seed"])
    model = b.Model(S, w)
    ow = OracleWeights(S, w)
    if q4:
        qt = make_q4_draft(S, w)
        model = b.Model(S, qt, weight_format=b.W_Q4G64, share=model)
        ow = q4_oracle_weights(S, w, qt)
    prompt = make_prompt(S.vocab, c["P"], seed=2000 + c["seed"])
    toks = np.random.default_rng(3000 + c["seed"]).integers(0, S.vocab, c["M"]).astype(np.int32)
    pt, t = torch.from_numpy(prompt).cuda(), torch.from_numpy(toks).cuda()
    M, cap = c["M"], c["cap"]
    c1, w1 = b.Cache(S, cap), b.Workspace(S, cap)
    b.prefill(model, c1, pt, w1, chunk=c["chunk"])
    lb = torch.empty((M, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(model, c1, t, w1, logits=lb)
    assert w1.error_bits() == 0 and c1.length() == c["P"] + M
    c2, w2 = b.Cache(S, cap), b.Workspace(S, cap)
    b.prefill(model, c2, pt, w2)
    ls = torch.empty((M, S.vocab), dtype=torch.float32, device="cuda")
    for i in range(M):
        b.decode_step(model, c2, t[i:i + 1], w2, logits=ls[i])
    assert w2.error_bits() == 0
    assert torch.equal(lb.view(torch.int32), ls.view(torch.int32)), "a pass differs from single-row steps"
    oc = OracleCache(S, cap)
    prefill(ow, oc, prompt)
    assert_logits_close(to_np(lb), forward(ow, oc, toks), f"random shape {c}")


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_bf16(seed):
    _run(_case(seed), q4=False)


@pytest.mark.parametrize("seed", range(100, 108))
def test_random_shape_q4(seed):
    _run(_case(seed, q4=True), q4=True)


@pytest.mark.parametrize("seed", range(200, 208))
def test_random_shape_rounds_commit_gpu_ar(seed):
    """Greedy rounds on a random shape (draft table corrupted with a random
    rate, k in 1..16, schedule A or B, a random capacity margin): the committed
    tokens equal the GPU's greedy AR decode token for token, and the cache
    length equals prompt + committed after the job."""
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import ModelShape
    from block_verify_amd.synth import make_draft_table, make_prompt, make_weights
    c = _case(seed)
    rng = np.random.default_rng(5000 + seed)
    k = int(rng.integers(1, 17))
    schedule = int(rng.integers(0, 2))
    corrupt = float(rng.choice([0.0, 0.3, 0.6, 1.0]))
    n_new = int(rng.integers(8, 41))
    S = ModelShape(f"rr{seed}", c["L"], c["H"], c["nq"], c["nkv"], c["hd"], c["F"], c["V"])
    say(f"random rounds {c} k={k} schedule={'AB'[schedule]} c={corrupt} n={n_new}")
    w = make_weights(S, 4000 + seed)
    model = b.Model(S, w)
    prompt = make_prompt(S.vocab, c["P"], seed=6000 + seed)
    max_len = c["P"] + n_new + 2 * (k + 2) + int(rng.integers(0, 200))
    # greedy AR on the GPU, one step at a time
    cache, ws = b.Cache(S, max_len), b.Workspace(S, max_len)
    n_ar = n_new + k + 1
    toks = torch.zeros(n_ar + 1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(model, cache, torch.from_numpy(prompt).cuda(), ws, logits=scratch, argmax=toks[0:1])
    for i in range(n_ar - 1):
        b.decode_step(model, cache, toks[i:i + 1], ws, logits=scratch, argmax=toks[i + 1:i + 2])
    ar = [int(x) for x in to_np(toks)[:n_ar]]
    table = make_draft_table(np.array(ar), S.vocab, corrupt, seed=7000 + seed)
    r = b.Round(model, k, schedule=schedule, table=table, max_len=max_len)
    r.prefill(prompt)
    st, got = r.run(n_new)
    assert list(got[:n_new]) == ar[:n_new]
    assert r.tcache.length() == c["P"] + st.n_committed - (1 if schedule == 1 else 0)
    assert r.ws.error_bits() == 0


@pytest.mark.parametrize("seed", range(300, 306))
def test_random_shape_stochastic_rounds_match_oracle_rule(seed):
    """Modified rejection sampling on a random shape and vocabulary (noisy
    self-draft, k in 1..8, schedule A, a random temperature, top-k / top-p and
    bonus setting): every round's draft samples and accept / resample / bonus
    decisions, replayed by the oracle on the GPU's own logits, agree (up to
    counted boundary cases), and the cache length equals prompt + committed."""
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import ModelShape
    from block_verify_amd.synth import make_noise, make_prompt, make_weights
    from gpu_helpers import check_stochastic_round
    c = _case(seed)
    rng = np.random.default_rng(8000 + seed)
    k = int(rng.integers(1, 9))
    kw = dict(temperature=float(rng.choice([1.0, 0.7, 1.3])), bonus=bool(rng.integers(0, 2)))
    if rng.integers(0, 2):
        kw["top_k"] = int(rng.choice([1, 5, 50]))
    if rng.integers(0, 2):
        kw["top_p"] = float(rng.choice([0.5, 0.9]))
    n_new = int(rng.integers(8, 25))
    S = ModelShape(f"rs{seed}", 1, c["H"], c["nq"], c["nkv"], c["hd"], c["F"], c["V"])
    say(f"random stochastic {c} k={k} {kw} n={n_new}")
    w = make_weights(S, 9000 + seed)
    model = b.Model(S, w)
    prompt = make_prompt(S.vocab, c["P"], seed=9500 + seed)
    max_len = c["P"] + n_new + 2 * (k + 2) + 64
    noise = float(rng.choice([1.0, 0.2])) * make_noise(n_new + 2 * k + 2, S.vocab, seed=9700 + seed)
    r = b.Round(model, k, mode=b.STOCHASTIC, draft_source=b.DRAFT_NOISY_SELF, noise=noise, seed=seed,
                max_len=max_len, **kw)
    r.prefill(prompt)
    r.reset(n_new)
    V = S.vocab
    exempt, n0, rounds = 0, 0, 0
    while n0 < n_new:
        saved = to_np(r.debug_view(0)).copy()
        st0, _ = r.read_state()
        r.step()
        st, toks = r.read_state()
        rows = to_np(r.debug_view(1)).reshape(k + 1, V)[:k].copy()
        qz = to_np(r.debug_view(2)).reshape(k, V).copy()
        drafts = [int(x) for x in to_np(r.debug_view(3, torch.int32))[:k]]
        com = [int(x) for x in toks[n0:st.n_committed]]
        exempt += check_stochastic_round(saved, rows, qz, drafts, st.m_last, com, seed, st0.round, kw["bonus"],
                                         kw["temperature"], kw.get("top_k", 0), kw.get("top_p", 1.0))
        assert r.tcache.length() == c["P"] + st.n_committed
        n0 = st.n_committed
        rounds += 1
    assert r.ws.error_bits() == 0
    say(f"  {rounds} rounds, {exempt} boundary exemptions")
    assert exempt <= 1


@pytest.mark.parametrize("seed", range(400, 406))
def test_random_shape_trees_match_oracle(seed):
    """A random draft tree (1..64 nodes, each parent an earlier node) on a random
    shape and cache capacity: the tree verify's logits against the oracle's
    tree forward, its argmax against its logits, and the cache length after
    the tree; passes of up to 32 rows with the ancestor mask."""
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import ModelShape
    from block_verify_amd.synth import make_prompt, make_weights
    from oracle.model import OracleCache, OracleWeights, prefill
    from oracle.tree import tree_forward
    c = _case(seed)
    rng = np.random.default_rng(10000 + seed)
    n = int(rng.integers(1, 65))
    pars = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
    S = ModelShape(f"rt{seed}", c["L"], c["H"], c["nq"], c["nkv"], c["hd"], c["F"], c["V"])
    toks = rng.integers(0, S.vocab, n).astype(np.int32)
    say(f"random tree {c} n={n}")
    w = make_weights(S, 11000 + seed)
    model = b.Model(S, w)
    prompt = make_prompt(S.vocab, c["P"], seed=12000 + seed)
    cap = max(c["cap"], c["P"] + n)
    cache, ws = b.Cache(S, cap), b.Workspace(S, cap)
    b.prefill(model, cache, torch.from_numpy(prompt).cuda(), ws)
    lg = torch.empty((n, S.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(n, dtype=torch.int32, device="cuda")
    b.tree_verify(model, cache, torch.from_numpy(toks).cuda(), torch.from_numpy(np.asarray(pars, np.int32)).cuda(),
                  ws, logits=lg, argmax=am)
    assert ws.error_bits() == 0 and cache.length() == c["P"] + n
    g = to_np(lg)
    assert np.array_equal(to_np(am), g.argmax(axis=1))
    ow = OracleWeights(S, w)
    oc = OracleCache(S, cap)
    prefill(ow, oc, prompt)
    assert_logits_close(g, tree_forward(ow, oc, toks, pars), f"random tree {c} n={n}")
