"""GPU parity at the full 1.5B shape and 2048-token context (the benchmark's workload).

The oracle runs its own float64 prefill of the same 2048 seeded prompt ids on
the host (tens of seconds), then the same verify blocks; sampled K/V entries
of the cache; the full 64-token job under schedules A and B against the GPU's
own greedy decode (bit for bit) and against the oracle (teacher-forced, exact
except where the oracle's top-2 margin is below 0.1).
"""
import time

import numpy as np
import pytest
import torch

from gpu_helpers import (MARGIN, assert_logits_close, bf16_bits_to_f64, check_stochastic_round, oracle_margin, say,
                         to_np)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

P, N_NEW, K, C = 2048, 64, 4, 0.46


@pytest.fixture(scope="module")
def big():
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_1_5B, SEED_TARGET
    from block_verify_amd.synth import make_prompt, make_weights
    from oracle.model import OracleCache, OracleWeights, prefill
    S = QWEN_1_5B
    t0 = time.time()
    w = make_weights(S, SEED_TARGET)
    model = b.Model(S, w)
    prompt = make_prompt(S.vocab, P)
    say(f"1.5B: weights + pack {time.time() - t0:.1f} s")
    max_len = P + 256
    cache = b.Cache(S, max_len)
    ws = b.Workspace(S, max_len)
    saved = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(model, cache, torch.from_numpy(prompt).cuda(), ws, logits=saved)
    torch.cuda.synchronize()
    t0 = time.time()
    ow = OracleWeights(S, w)
    oc = OracleCache(S, max_len)
    o_saved = prefill(ow, oc, prompt)
    say(f"1.5B: oracle float64 prefill of {P} tokens {time.time() - t0:.1f} s")
    return dict(b=b, S=S, w=w, model=model, prompt=prompt, cache=cache, ws=ws, saved=to_np(saved),
                ow=ow, oc=oc, o_saved=o_saved, max_len=max_len)


def test_prefill_saved_next_logits(big):
    assert big["cache"].length() == P
    assert_logits_close(big["saved"], big["o_saved"], "1.5B saved_next")
    assert big["ws"].error_bits() == 0


def test_kv_cache_sampled_entries(big):
    S = big["S"]
    kk, vv = big["cache"].kv()
    rng = np.random.default_rng(0)
    for l in rng.choice(S.n_layers, 6, replace=False):
        pos = rng.choice(P, 64, replace=False)
        pt = torch.from_numpy(pos).cuda()
        g = bf16_bits_to_f64(np.stack([to_np(kk[int(l)][:, pt, :]), to_np(vv[int(l)][:, pt, :])]))
        ok = np.stack([big["oc"].k[l][:, pos], big["oc"].v[l][:, pos]])
        scale = np.abs(ok).max()
        err = np.abs(g - ok).max()
        say(f"layer {l}: K/V max err {err:.3e} of scale {scale:.3f}")
        assert err <= 1e-2 * scale


@pytest.mark.parametrize("rows", [1, 4, 5, 9])
def test_verify_block_logits(big, rows):
    from oracle.model import forward
    b, S = big["b"], big["S"]
    toks = np.random.default_rng(100 + rows).integers(0, S.vocab, rows)
    logits = torch.empty((rows, S.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(rows, dtype=torch.int32, device="cuda")
    b.decode_step(big["model"], big["cache"], torch.from_numpy(toks.astype(np.int32)).cuda(), big["ws"],
                  logits=logits, argmax=am)
    assert big["cache"].length() == P + rows
    big["cache"].trim(P, big["ws"])
    oc = big["oc"].clone()
    ol = forward(big["ow"], oc, toks)
    g = to_np(logits)
    assert_logits_close(g, ol, f"1.5B verify rows={rows}")
    gam = to_np(am)
    assert np.array_equal(gam, g.argmax(axis=1))
    for i in range(rows):
        if oracle_margin(ol[i]) >= MARGIN:
            assert gam[i] == int(np.argmax(ol[i]))
    assert big["ws"].error_bits() == 0


def test_batch_invariance_full_size(big):
    b, S = big["b"], big["S"]
    toks = torch.from_numpy(np.array([11, 222, 3333, 44444, 151935], np.int32)).cuda()
    lb = torch.empty((5, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(big["model"], big["cache"], toks, big["ws"], logits=lb)
    big["cache"].trim(P, big["ws"])
    ls = torch.empty((5, S.vocab), dtype=torch.float32, device="cuda")
    for i in range(5):
        b.decode_step(big["model"], big["cache"], toks[i:i + 1], big["ws"], logits=ls[i])
    big["cache"].trim(P, big["ws"])
    assert torch.equal(lb.view(torch.int32), ls.view(torch.int32))


@pytest.fixture(scope="module")
def ar_tokens(big):
    b, S = big["b"], big["S"]
    n = N_NEW + K + 2
    toks = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    toks[0] = int(np.argmax(big["saved"]))
    scratch = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    for i in range(n - 1):
        b.decode_step(big["model"], big["cache"], toks[i:i + 1], big["ws"], logits=scratch, argmax=toks[i + 1:i + 2])
    big["cache"].trim(P, big["ws"])
    return [int(x) for x in to_np(toks)[:n]]


def test_gpu_ar_against_oracle_teacher_forced(big, ar_tokens):
    from oracle.model import forward
    oc = big["oc"].clone()
    toks = ar_tokens[:N_NEW]
    rows = np.concatenate([big["o_saved"][None], forward(big["ow"], oc, toks[:-1])])
    exempt = 0
    for i, t in enumerate(toks):
        a = int(np.argmax(rows[i]))
        if a != t:
            assert oracle_margin(rows[i]) < MARGIN, f"token {i}: gpu {t} oracle {a} margin {oracle_margin(rows[i])}"
            exempt += 1
    say(f"1.5B AR vs oracle: {N_NEW} tokens, {exempt} differ where the oracle top-2 margin < {MARGIN}")


@pytest.mark.parametrize("graph", [False, True])
@pytest.mark.parametrize("schedule", [0, 1])
def test_spec_job_equals_gpu_ar(big, ar_tokens, schedule, graph):
    """The benchmark's job (eager rounds, and the captured round replayed as HIP graphs as
    the benchmark times it) commits the GPU's greedy tokens."""
    from block_verify_amd.synth import make_draft_table
    b, S = big["b"], big["S"]
    table = make_draft_table(np.array(ar_tokens), S.vocab, C)
    r = b.Round(big["model"], K, schedule=schedule, table=table, max_len=big["max_len"])
    r.prefill(big["prompt"])
    if graph:
        r.capture()
    st, toks = r.run(N_NEW, graph=graph)
    assert list(toks[:N_NEW]) == ar_tokens[:N_NEW]
    assert r.tcache.length() == P + st.n_committed - (1 if schedule == 1 else 0)
    assert r.ws.error_bits() == 0
    # accepted drafts per round follow the table's corruption pattern exactly:
    # a round at n0 accepts the leading drafts that equal the greedy tokens
    n0, rounds, accepted = 0, 0, 0
    while n0 < N_NEW:
        m = 0
        while m < K and table[n0 + m] == ar_tokens[n0 + m]:
            m += 1
        n0 += m + 1
        rounds += 1
        accepted += m
    say(f"schedule {'AB'[schedule]}{' graph' if graph else ''}: {st.round} rounds, {st.accepted_total} drafts accepted")
    assert (st.round, st.accepted_total) == (rounds, accepted)


P4 = 4096


def test_stochastic_4k_rounds_match_oracle(big):
    """Modified rejection sampling at a 4096-token context (noisy self-draft, Philox seed 3):
    the first rounds' verify rows and saved_next against the oracle's float64 forward,
    every round's draft samples and decisions against the oracle rule on the GPU's logits."""
    import torch
    from block_verify_amd.synth import make_noise, make_prompt
    from oracle.model import OracleCache, forward, prefill
    b, S = big["b"], big["S"]
    V, seed = S.vocab, 3
    prompt = make_prompt(S.vocab, P4)
    noise = make_noise(N_NEW + 2 * K + 2, V)
    r = b.Round(big["model"], K, mode=b.STOCHASTIC, draft_source=b.DRAFT_NOISY_SELF, noise=noise, seed=seed,
                max_len=P4 + 256)
    r.prefill(prompt)
    r.reset(N_NEW)
    t0 = time.time()
    oc = OracleCache(S, P4 + 256)
    o_saved = prefill(big["ow"], oc, prompt)
    say(f"4K: oracle float64 prefill {time.time() - t0:.1f} s")
    exempt, n0, ms, checked = 0, 0, [], 0
    while n0 < N_NEW:
        saved = to_np(r.debug_view(0)).copy()
        st0, _ = r.read_state()
        teacher = st0.round < 3
        if teacher:
            assert_logits_close(saved, o_saved, f"4K round {st0.round} saved_next")
        r.step()
        st, toks = r.read_state()
        rows = to_np(r.debug_view(1)).reshape(K + 1, V)[:K].copy()
        qz = to_np(r.debug_view(2)).reshape(K, V).copy()
        drafts = to_np(r.debug_view(3, torch.int32))[:K].copy()
        assert np.array_equal(qz[0], (saved + noise[n0]).astype(np.float32))
        for j in range(1, K):
            assert np.array_equal(qz[j], (rows[j - 1] + noise[n0 + j]).astype(np.float32))
        com = toks[n0:st.n_committed]
        if teacher:
            ol = forward(big["ow"], oc.clone(), [int(x) for x in drafts])
            assert_logits_close(rows, ol, f"4K round {st0.round} verify rows")
            o_saved = forward(big["ow"], oc, [int(x) for x in com])[-1]
            checked += 1
        exempt += check_stochastic_round(saved, rows, qz, drafts, st.m_last, com, seed, st0.round)
        assert r.tcache.length() == P4 + st.n_committed
        ms.append(st.m_last)
        n0 = st.n_committed
    assert r.ws.error_bits() == 0
    say(f"4K stochastic: {len(ms)} rounds, accepted {ms}, {exempt} boundary exemptions, "
        f"{checked} rounds teacher-forced against the oracle")
    assert exempt <= 2


def test_tree_verify_and_accept_29_nodes(big):
    """A draft tree of 4 nodes a level over 7 levels (29 rows with the root, the shape of
    the context-aware tree with k = 4, D = 7) at 2K: logits against the oracle's
    tree-causal forward, the accepted path against the oracle rule on the GPU's argmax,
    and the compacted K/V as bit copies of the tree forward's rows."""
    from oracle.model import forward
    from oracle.tree import tree_accept_greedy, tree_forward
    b, S = big["b"], big["S"]
    rng = np.random.default_rng(29)
    pars, level = [-1], [0]
    for _ in range(7):
        nxt = []
        for _ in range(4):
            pars.append(int(rng.choice(level)))
            nxt.append(len(pars) - 1)
        level = nxt
    n = len(pars)
    toks = rng.integers(0, S.vocab, n).astype(np.int32)
    # the root's first child carries the root's argmax, so the path has at least one node
    oc0 = big["oc"].clone()
    toks[1] = int(np.argmax(forward(big["ow"], oc0, toks[:1])[0]))
    t, p = torch.from_numpy(toks).cuda(), torch.from_numpy(np.asarray(pars, np.int32)).cuda()
    lg = torch.empty((n, S.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(n, dtype=torch.int32, device="cuda")
    b.tree_verify(big["model"], big["cache"], t, p, big["ws"], logits=lg, argmax=am)
    kk, vv = big["cache"].kv()
    before = [(kk[l][:, P:P + n].clone(), vv[l][:, P:P + n].clone()) for l in (0, S.n_layers - 1)]
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    b.tree_accept(big["cache"], t, p, am, out, cnt, err)
    gam = to_np(am)
    path, com = tree_accept_greedy(toks, pars, list(gam))
    m = big["cache"].length() - P - 1
    after = [(kk[l][:, P:P + 1 + m].clone(), vv[l][:, P:P + 1 + m].clone()) for l in (0, S.n_layers - 1)]
    big["cache"].trim(P, big["ws"])
    ol = tree_forward(big["ow"], big["oc"].clone(), toks, pars)
    g = to_np(lg)
    assert_logits_close(g, ol, "1.5B tree verify (29 rows)")
    assert np.array_equal(gam, g.argmax(axis=1))
    exempt = sum(oracle_margin(ol[i]) < MARGIN for i in range(n))
    for i in range(n):
        if oracle_margin(ol[i]) >= MARGIN:
            assert gam[i] == int(np.argmax(ol[i]))
    assert m == len(path) >= 1 and int(cnt.item()) == len(com)
    assert [int(x) for x in to_np(out)[:len(com)]] == com and int(err.item()) == 0
    for (k0, v0), (k1, v1) in zip(before, after):
        for dst, src in enumerate([0] + path):
            assert torch.equal(k1[:, dst], k0[:, src]) and torch.equal(v1[:, dst], v0[:, src])
    assert big["ws"].error_bits() == 0
    say(f"1.5B tree: path {path}, committed {com}, {exempt} rows with oracle margin < {MARGIN}")


def test_q4_substitute_short_prompt(big):
    """The 4-bit substitute of the 1.5B shape (down projection split over three
    workgroups, five row groups a workgroup for gate/up) against the oracle with the
    dequantised weights on a 48-token prompt: saved_next and a 6-row block, then the same
    rows one at a time bit for bit."""
    from block_verify_amd.synth import make_q4_draft
    from oracle.model import OracleCache, forward, prefill
    from gpu_helpers import q4_oracle_weights
    b, S = big["b"], big["S"]
    qt = make_q4_draft(S, big["w"])
    qm = b.Model(S, qt, weight_format=b.W_Q4G64, share=big["model"])
    ow = q4_oracle_weights(S, big["w"], qt, cache=False)
    prompt = big["prompt"][:48]
    cache, ws = b.Cache(S, 128), b.Workspace(S, 128)
    saved = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(qm, cache, torch.from_numpy(prompt).cuda(), ws, logits=saved)
    oc = OracleCache(S, 128)
    o_saved = prefill(ow, oc, prompt)
    assert_logits_close(to_np(saved), o_saved, "1.5B q4 prefill saved_next")
    toks = np.random.default_rng(61).integers(0, S.vocab, 6).astype(np.int32)
    lg = torch.empty((6, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(qm, cache, torch.from_numpy(toks).cuda(), ws, logits=lg)
    assert_logits_close(to_np(lg), forward(ow, oc, toks), "1.5B q4 block rows=6")
    cache.trim(48, ws)
    ls = torch.empty_like(lg)
    for i in range(6):
        b.decode_step(qm, cache, torch.from_numpy(toks[i:i + 1]).cuda(), ws, logits=ls[i])
    assert torch.equal(lg.view(torch.int32), ls.view(torch.int32)) and ws.error_bits() == 0
