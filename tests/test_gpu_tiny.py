"""GPU parity on the tiny decoder: forward, cache, batch invariance, rounds, errors.

Every case calls the HIP path through the C ABI (block_verify_amd.lib) and
compares with the CPU oracle on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (MARGIN, assert_logits_close, bf16_bits_to_f64, check_stochastic_round, oracle_margin,
                         q4_oracle_weights, say, to_np, tokens_match_teacher_forced)

pytestmark = pytest.mark.gpu

P, N_NEW, K = 128, 16, 4


@pytest.fixture(scope="module")
def env():
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import TINY, SEED_TARGET
    from block_verify_amd.synth import make_prompt, make_weights
    from oracle.model import OracleWeights
    say("tiny: building model")
    w = make_weights(TINY, SEED_TARGET)
    model = b.Model(TINY, w)
    prompt = make_prompt(TINY.vocab, P)
    return dict(b=b, shape=TINY, w=w, model=model, prompt=prompt, ow=OracleWeights(TINY, w))


def _fresh(env, max_len=512):
    b = env["b"]
    cache = b.Cache(env["shape"], max_len)
    ws = b.Workspace(env["shape"], max_len)
    return cache, ws


def _gpu_prefill(env, cache, ws, tokens, chunk=32):
    b = env["b"]
    V = env["shape"].vocab
    t = torch.from_numpy(np.asarray(tokens, np.int32)).cuda()
    logits = torch.empty(V, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    lse = torch.empty(1, dtype=torch.float32, device="cuda")
    b.prefill(env["model"], cache, t, ws, chunk=chunk, logits=logits, argmax=am, lse=lse)
    return to_np(logits), int(to_np(am)[0]), float(to_np(lse)[0])


def _gpu_forward(env, cache, ws, tokens):
    b = env["b"]
    V = env["shape"].vocab
    M = len(tokens)
    t = torch.from_numpy(np.asarray(tokens, np.int32)).cuda()
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    am = torch.empty(M, dtype=torch.int32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    b.decode_step(env["model"], cache, t, ws, logits=logits, argmax=am, lse=lse)
    return to_np(logits), to_np(am), to_np(lse)


@pytest.mark.parametrize("chunk", [32, 7])
def test_prefill_logits_and_cache(env, chunk):
    from oracle.model import OracleCache, prefill
    say(f"tiny prefill chunk={chunk}")
    cache, ws = _fresh(env)
    logits, am, lse = _gpu_prefill(env, cache, ws, env["prompt"], chunk=chunk)
    assert cache.length() == P
    oc = OracleCache(env["shape"], 512)
    ol = prefill(env["ow"], oc, env["prompt"])
    assert_logits_close(logits, ol, "prefill logits")
    assert am == int(np.argmax(logits))
    ref_lse = np.log(np.sum(np.exp(logits.astype(np.float64) - logits.max()))) + logits.max()
    assert abs(lse - ref_lse) < 1e-4
    kk, vv = cache.kv()
    kk, vv = to_np(kk.contiguous()), to_np(vv.contiguous())
    for l in range(env["shape"].n_layers):
        gk = bf16_bits_to_f64(kk[l, :, :P])
        gv = bf16_bits_to_f64(vv[l, :, :P])
        for g, o, nm in ((gk, oc.k[l][:, :P], "K"), (gv, oc.v[l][:, :P], "V")):
            scale = np.abs(o).max()
            err = np.abs(g - o).max()
            say(f"layer {l} {nm}: max err {err:.3e} (scale {scale:.3f})")
            assert err <= 1e-2 * scale
    assert ws.error_bits() == 0


@pytest.mark.parametrize("rows", [1, 2, 4, 5, 8, 9, 16, 17, 32])
def test_block_forward_rows(env, rows):
    from oracle.model import OracleCache, forward, prefill
    say(f"tiny forward rows={rows}")
    cache, ws = _fresh(env)
    _gpu_prefill(env, cache, ws, env["prompt"])
    toks = np.random.default_rng(rows).integers(0, env["shape"].vocab, rows)
    logits, am, lse = _gpu_forward(env, cache, ws, toks)
    assert cache.length() == P + rows
    oc = OracleCache(env["shape"], 512)
    prefill(env["ow"], oc, env["prompt"])
    ol = forward(env["ow"], oc, toks)
    assert_logits_close(logits, ol, f"rows={rows}")
    assert np.array_equal(am, logits.argmax(axis=1))
    assert ws.error_bits() == 0


@pytest.mark.parametrize("rows", [1, 5, 9])
def test_long_cache_launch_shapes_give_the_same_logits(env, rows):
    """A long cache launches many more chunk workgroups (the grid padded so that
    a chunk's query-tile workgroups share an XCD) and merges them in the
    four-wave form instead of the one-wave form; the arithmetic of every tile
    and the merge's summation order are unchanged, so the logits equal those
    of a short cache bit for bit."""
    say(f"tiny long cache rows={rows}")
    toks = np.random.default_rng(100 + rows).integers(0, env["shape"].vocab, rows)
    out = []
    # 8 chunks, the last capacity of the one-wave merge (48 chunks), the first
    # of the eight-wave one (49), and a long cache
    for max_len in (512, 3072, 3136, 8448):
        cache, ws = _fresh(env, max_len)
        _gpu_prefill(env, cache, ws, env["prompt"])
        logits, am, lse = _gpu_forward(env, cache, ws, toks)
        assert cache.length() == P + rows and ws.error_bits() == 0
        out.append((logits, am, lse))
    for o in out[1:]:
        assert np.array_equal(out[0][0], o[0])
        assert np.array_equal(out[0][1], o[1]) and np.array_equal(out[0][2], o[2])


def test_batch_invariance_block_equals_single_steps(env):
    """Rows of an M=5 block equal five M=1 steps bit for bit (logits and cache)."""
    toks = np.array([5, 77, 4095, 0, 1234])
    c1, w1 = _fresh(env)
    c2, w2 = _fresh(env)
    _gpu_prefill(env, c1, w1, env["prompt"])
    _gpu_prefill(env, c2, w2, env["prompt"])
    lb, ab, sb = _gpu_forward(env, c1, w1, toks)
    singles = [_gpu_forward(env, c2, w2, toks[i:i + 1]) for i in range(5)]
    ls = np.concatenate([s[0] for s in singles])
    assert np.array_equal(lb.view(np.uint32), ls.view(np.uint32))
    assert np.array_equal(ab, np.concatenate([s[1] for s in singles]))
    n = P + len(toks)   # positions past the length were never written
    for a, b_ in zip(c1.kv(), c2.kv()):
        assert torch.equal(a[:, :, :n], b_[:, :, :n])
    # prefill in different chunkings gives the same cache bits too
    c3, w3 = _fresh(env)
    _gpu_prefill(env, c3, w3, env["prompt"], chunk=13)
    for a, b_ in zip(c1.kv(), c3.kv()):
        assert torch.equal(a[:, :, :P], b_[:, :, :P])


def _gpu_ar(env, n, max_len=512):
    """Greedy AR on the GPU: each step's argmax feeds the next step (device only)."""
    b = env["b"]
    cache, ws = _fresh(env, max_len)
    V = env["shape"].vocab
    toks = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    pt = torch.from_numpy(np.asarray(env["prompt"], np.int32)).cuda()
    logits = torch.empty(V, dtype=torch.float32, device="cuda")
    b.prefill(env["model"], cache, pt, ws, logits=logits, argmax=toks[0:1])
    scratch = torch.empty(V, dtype=torch.float32, device="cuda")
    for i in range(n - 1):
        b.decode_step(env["model"], cache, toks[i:i + 1], ws, logits=scratch, argmax=toks[i + 1:i + 2])
    return [int(x) for x in to_np(toks)[:n]]


@pytest.fixture(scope="module")
def gpu_ar(env):
    return _gpu_ar(env, N_NEW + K + 1)


def test_gpu_ar_matches_oracle_teacher_forced(env, gpu_ar):
    from oracle.model import full_recompute_logits
    seq = list(env["prompt"]) + gpu_ar
    ol = full_recompute_logits(env["ow"], seq)
    rows = ol[P - 1:P - 1 + len(gpu_ar)]
    exempt = tokens_match_teacher_forced(gpu_ar, rows)
    say(f"tiny AR: {len(gpu_ar)} tokens, {exempt} exempt by the top-2 margin rule")


@pytest.mark.parametrize("schedule", [0, 1])
@pytest.mark.parametrize("c", [0.0, 0.4, 1.0])
def test_spec_rounds_equal_gpu_ar(env, gpu_ar, schedule, c):
    from block_verify_amd.synth import make_draft_table
    b = env["b"]
    table = make_draft_table(np.array(gpu_ar), env["shape"].vocab, c)
    r = b.Round(env["model"], K, schedule=schedule, table=table, max_len=512)
    r.prefill(env["prompt"])
    for rep in range(2):
        st, toks = r.run(N_NEW)
        assert list(toks[:N_NEW]) == gpu_ar[:N_NEW]
        # the invariant: cache length == prompt + committed (minus the pending token under B)
        assert r.tcache.length() == P + st.n_committed - (1 if schedule == 1 else 0)
        assert r.ws.error_bits() == 0
    say(f"schedule {'AB'[schedule]} c={c}: rounds {st.round} accepted {st.accepted_total}")
    if c == 0.0:
        assert st.accepted_total >= (st.round - 1) * K
    if c == 1.0:
        assert st.accepted_total == 0


@pytest.mark.parametrize("schedule", [0, 1])
def test_graph_replay_commits_the_same_tokens(env, gpu_ar, schedule):
    """One captured round replayed as a HIP graph: same tokens, same cache length, several jobs in a row."""
    from block_verify_amd.synth import make_draft_table
    b = env["b"]
    table = make_draft_table(np.array(gpu_ar), env["shape"].vocab, 0.4)
    r = b.Round(env["model"], K, schedule=schedule, table=table, max_len=512)
    r.prefill(env["prompt"])
    r.capture()
    for rep in range(3):
        st, toks = r.run(N_NEW, graph=True)
        assert list(toks[:N_NEW]) == gpu_ar[:N_NEW]
        assert r.tcache.length() == P + st.n_committed - (1 if schedule == 1 else 0)
        # eager rounds interleaved with graph replays stay consistent
        st2, toks2 = r.run(N_NEW)
        assert list(toks2[:N_NEW]) == gpu_ar[:N_NEW]
    assert r.ws.error_bits() == 0


@pytest.mark.parametrize("schedule", [0, 1])
def test_timed_graph_replay_records_terms(env, gpu_ar, schedule):
    """With a ring of per-term events the round replays as four graphs with the
    events between them (without one, as a single graph): the same tokens, and
    five ordered timestamps per round."""
    import ctypes
    from block_verify_amd.synth import make_draft_table
    b = env["b"]
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    n_ev = 5 * (N_NEW + 1)
    evs = (ctypes.c_void_p * n_ev)()
    for i in range(n_ev):
        e = ctypes.c_void_p()
        assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0) == 0
        evs[i] = e.value
    table = make_draft_table(np.array(gpu_ar), env["shape"].vocab, 0.4)
    r = b.Round(env["model"], K, schedule=schedule, table=table, max_len=512, events=evs, n_events=n_ev)
    r.prefill(env["prompt"])
    r.capture()
    c0 = r.calls()
    st, toks = r.run(N_NEW, graph=True)
    torch.cuda.synchronize()
    assert list(toks[:N_NEW]) == gpu_ar[:N_NEW]
    assert r.calls() - c0 >= st.round
    for c in range(c0, r.calls()):
        base = (c % (N_NEW + 1)) * 5
        for i in range(4):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[base + i], evs[base + i + 1]) == 0
            assert ms.value >= 0.0
    assert r.ws.error_bits() == 0
    del r
    for i in range(n_ev):
        hip.hipEventDestroy(evs[i])


def test_spec_no_bonus(env, gpu_ar):
    from block_verify_amd.synth import make_draft_table
    b = env["b"]
    table = make_draft_table(np.array(gpu_ar), env["shape"].vocab, 0.1)
    r = b.Round(env["model"], K, bonus=False, table=table, max_len=512)
    r.prefill(env["prompt"])
    st, toks = r.run(N_NEW)
    assert list(toks[:N_NEW]) == gpu_ar[:N_NEW]
    assert r.tcache.length() == P + st.n_committed


def test_spec_accept_matches_oracle_rule_on_gpu_argmax(env, gpu_ar):
    """Accept decisions are exact on the GPU's own logits: replay the oracle rule per round."""
    from block_verify_amd.synth import make_draft_table
    from oracle.accept import greedy_accept
    b = env["b"]
    table = make_draft_table(np.array(gpu_ar), env["shape"].vocab, 0.4)
    r = b.Round(env["model"], K, table=table, max_len=512)
    r.prefill(env["prompt"])
    r.reset(N_NEW)
    n0 = 0
    while n0 < N_NEW:
        r.step()
        st, toks = r.read_state()
        drafts = [int(x) for x in table[n0:n0 + K]]
        v = [gpu_ar[n0 + j] for j in range(K + 1)]
        m, com = greedy_accept(v, drafts, True)
        assert st.m_last == m
        assert list(toks[n0:n0 + m + 1]) == com
        n0 = st.n_committed


def test_trim_and_capacity_errors_are_flagged_not_faults(env):
    b = env["b"]
    cache, ws = _fresh(env, max_len=140)
    _gpu_prefill(env, cache, ws, env["prompt"])
    cache.trim(130, ws)   # above the length (128): flagged, length unchanged
    assert ws.error_bits() & b.DERR_TRIM
    assert cache.length() == P
    ws2 = b.Workspace(env["shape"], 140)
    toks = np.arange(16)
    _gpu_forward(env, cache, ws2, toks)      # 128 + 16 > 140: flagged, cache writes skipped
    assert ws2.error_bits() & b.DERR_CAPACITY
    cache.trim(100, ws2)
    assert cache.length() == 100


def test_philox_matches_oracle_words():
    from block_verify_amd import lib as b
    from oracle.philox import philox4x64_10
    rng = np.random.default_rng(0)
    n = 4096
    ctr = rng.integers(0, 2 ** 63, (n, 4), dtype=np.int64).astype(np.uint64) * np.uint64(2) + np.uint64(1)
    ctr[:64, 1:] = 0
    ctr[:64, 0] = np.arange(64, dtype=np.uint64)
    key = rng.integers(0, 2 ** 63, (n, 2), dtype=np.int64).astype(np.uint64)
    key[:64] = [3, 0]
    got = b.philox4x64(ctr, key)
    for i in list(range(64)) + list(range(64, n, 97)):
        assert tuple(int(x) for x in got[i]) == philox4x64_10(ctr[i], key[i])


@pytest.mark.parametrize("schedule", [0, 1])
def test_draft_model_rounds_keep_both_caches(env, gpu_ar, schedule):
    """A separate draft model with its own cache: k draft steps per round (tokens from the
    table), both caches trimmed to t+m and repaired; the draft cache ends up holding the
    draft model's K/V of prompt + committed tokens."""
    from block_verify_amd.shapes import SEED_DRAFT
    from block_verify_amd.synth import make_draft_table, make_weights
    from oracle.model import OracleCache, OracleWeights, prefill
    b, S = env["b"], env["shape"]
    dw = make_weights(S, SEED_DRAFT)
    draft = b.Model(S, dw)
    table = make_draft_table(np.array(gpu_ar), S.vocab, 0.4)
    r = b.Round(env["model"], K, schedule=schedule, draft_source=b.DRAFT_MODEL, draft=draft, table=table,
                max_len=512)
    r.prefill(env["prompt"])
    for rep in range(2):
        st, toks = r.run(N_NEW)
        assert list(toks[:N_NEW]) == gpu_ar[:N_NEW]
        assert r.tcache.length() == P + st.n_committed - (1 if schedule == 1 else 0)
        assert r.dcache.length() == P + st.n_committed
        assert r.ws.error_bits() == 0 and r.dws.error_bits() == 0
    seq = list(env["prompt"]) + [int(x) for x in toks[:st.n_committed]]
    ow = OracleWeights(S, dw)
    oc = OracleCache(S, len(seq) + 8)
    prefill(ow, oc, seq)
    kk, vv = r.dcache.kv()
    n = len(seq)
    for l in range(S.n_layers):
        g = bf16_bits_to_f64(np.stack([to_np(kk[l][:, :n]), to_np(vv[l][:, :n])]))
        o = np.stack([oc.k[l][:, :n], oc.v[l][:, :n]])
        err = np.abs(g - o).max()
        say(f"draft cache layer {l}: max err {err:.3e} of {np.abs(o).max():.3f}")
        assert err <= 1e-2 * np.abs(o).max()


def test_stochastic_rounds_match_oracle_decisions(env):
    """Modified rejection sampling with the noisy self-draft (schedule A): per round, the
    noisy draft logits, the verify rows, the draft samples and the accept/resample/bonus
    decisions against the oracle on the GPU's own logits."""
    from block_verify_amd.synth import make_noise
    from oracle.model import OracleCache, forward, prefill
    b, S = env["b"], env["shape"]
    V, seed = S.vocab, 3
    noise = make_noise(N_NEW + 2 * K + 2, V)
    r = b.Round(env["model"], K, mode=b.STOCHASTIC, draft_source=b.DRAFT_NOISY_SELF, noise=noise, seed=seed,
                max_len=512)
    r.prefill(env["prompt"])
    r.reset(N_NEW)
    oc = OracleCache(S, 512)
    o_saved = prefill(env["ow"], oc, env["prompt"])
    exempt, n0, stops = 0, 0, []
    while n0 < N_NEW:
        saved = to_np(r.debug_view(0)).copy()
        st0, _ = r.read_state()
        assert_logits_close(saved, o_saved, f"round {st0.round} saved_next")
        r.step()
        st, toks = r.read_state()
        rows = to_np(r.debug_view(1)).reshape(K + 1, V)[:K].copy()
        qz = to_np(r.debug_view(2)).reshape(K, V).copy()
        drafts = to_np(r.debug_view(3, torch.int32))[:K].copy()
        # q_1 from saved_next, q_(j+1) from the M=1 step on d_j: equal bit for bit to verify row j plus noise
        assert np.array_equal(qz[0], (saved + noise[n0]).astype(np.float32))
        for j in range(1, K):
            assert np.array_equal(qz[j], (rows[j - 1] + noise[n0 + j]).astype(np.float32))
        ol = forward(env["ow"], oc.clone(), [int(x) for x in drafts])
        assert_logits_close(rows, ol, f"round {st0.round} verify rows")
        com = toks[n0:st.n_committed]
        assert len(com) == st.m_last + 1
        exempt += check_stochastic_round(saved, rows, qz, drafts, st.m_last, com, seed, st0.round)
        assert r.tcache.length() == P + st.n_committed
        stops.append(st.m_last)
        o_saved = forward(env["ow"], oc, [int(x) for x in com])[-1]
        n0 = st.n_committed
    assert r.ws.error_bits() == 0
    say(f"stochastic: {len(stops)} rounds, accepted per round {stops}, {exempt} boundary exemptions")
    assert exempt <= 1


def test_stochastic_job_is_deterministic_eager_and_graph(env):
    from block_verify_amd.synth import make_noise
    b, S = env["b"], env["shape"]
    noise = make_noise(N_NEW + 2 * K + 2, S.vocab)
    r = b.Round(env["model"], K, mode=b.STOCHASTIC, draft_source=b.DRAFT_NOISY_SELF, noise=noise, seed=3,
                max_len=512)
    r.prefill(env["prompt"])
    st, ref = r.run(N_NEW)
    r.capture()
    for rep in range(2):
        st2, toks = r.run(N_NEW, graph=True)
        assert list(toks) == list(ref) and st2.round == st.round
        st3, toks3 = r.run(N_NEW)
        assert list(toks3) == list(ref)
    r2 = b.Round(env["model"], K, mode=b.STOCHASTIC, draft_source=b.DRAFT_NOISY_SELF, noise=noise, seed=4,
                 max_len=512)
    r2.prefill(env["prompt"])
    _, other = r2.run(N_NEW)
    assert list(other[:N_NEW]) != list(ref[:N_NEW])
    assert r.ws.error_bits() == 0


@pytest.fixture(scope="module")
def q4env(env):
    from block_verify_amd.synth import make_q4_draft
    b, S = env["b"], env["shape"]
    qt = make_q4_draft(S, env["w"])
    qm = b.Model(S, qt, weight_format=b.W_Q4G64, share=env["model"])
    return dict(model=qm, ow=q4_oracle_weights(S, env["w"], qt))


@pytest.mark.parametrize("rows,chunk", [(1, 4), (3, 32), (9, 5), (32, 32)])
def test_q4_forward_matches_oracle(env, q4env, rows, chunk):
    """The 4-bit substitute model (shared bf16 embedding / LM head) against the oracle
    forward with the dequantised weights: prefill (in `chunk`-row passes) and a block of
    rows."""
    from oracle.model import OracleCache, forward, prefill
    b, S = env["b"], env["shape"]
    cache, ws = _fresh(env)
    t = torch.from_numpy(np.asarray(env["prompt"], np.int32)).cuda()
    saved = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(q4env["model"], cache, t, ws, chunk=chunk, logits=saved)
    oc = OracleCache(S, 512)
    o_saved = prefill(q4env["ow"], oc, env["prompt"])
    assert_logits_close(to_np(saved), o_saved, "q4 prefill saved_next")
    toks = np.random.default_rng(7 + rows).integers(0, S.vocab, rows)
    logits = torch.empty((rows, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(q4env["model"], cache, torch.from_numpy(toks.astype(np.int32)).cuda(), ws, logits=logits)
    assert_logits_close(to_np(logits), forward(q4env["ow"], oc, toks), f"q4 block rows={rows}")
    assert cache.length() == P + rows
    kk, vv = cache.kv()
    n = P + rows
    for l in range(S.n_layers):
        g = bf16_bits_to_f64(np.stack([to_np(kk[l][:, :n]), to_np(vv[l][:, :n])]))
        o = np.stack([oc.k[l][:, :n], oc.v[l][:, :n]])
        assert np.abs(g - o).max() <= 1e-2 * np.abs(o).max()
    assert ws.error_bits() == 0


def test_q4_batch_invariance_and_row_limit(env, q4env):
    """A row's 4-bit product does not depend on the pass: 17 rows at once (three column
    tiles) equal the same rows one at a time and in a pass of 8, bit for bit."""
    b, S = env["b"], env["shape"]
    cache, ws = _fresh(env)
    t = torch.from_numpy(np.asarray(env["prompt"], np.int32)).cuda()
    b.prefill(q4env["model"], cache, t, ws, chunk=32)
    toks = torch.from_numpy(np.random.default_rng(17).integers(0, S.vocab, 17).astype(np.int32)).cuda()
    lb = torch.empty((17, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(q4env["model"], cache, toks, ws, logits=lb)
    cache.trim(P, ws)
    ls = torch.empty((17, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(q4env["model"], cache, toks[:8], ws, logits=ls[:8])
    for i in range(8, 17):
        b.decode_step(q4env["model"], cache, toks[i:i + 1], ws, logits=ls[i])
    assert torch.equal(lb.view(torch.int32), ls.view(torch.int32))
    with pytest.raises(b.SpecdecError):
        b.decode_step(q4env["model"], cache, torch.zeros(33, dtype=torch.int32, device="cuda"), ws)


def test_q4_substitute_draft_rounds(env, q4env, gpu_ar):
    """Substitute-draft rounds on the shared cache (depth 8, schedule A): committed tokens equal
    greedy AR, d_1 = argmax(saved_next) is always accepted, and every 4-bit draft token is the
    oracle's argmax on the same prefix (teacher-forced) unless its top-2 margin is < 0.1."""
    from oracle.model import OracleCache, forward, prefill
    b, S = env["b"], env["shape"]
    D = 8
    r = b.Round(env["model"], D, draft_source=b.DRAFT_Q4_SELF, draft=q4env["model"], max_len=512)
    r.prefill(env["prompt"])
    st, toks = r.run(N_NEW)
    assert list(toks[:N_NEW]) == gpu_ar[:N_NEW]
    assert r.tcache.length() == P + st.n_committed
    assert r.ws.error_bits() == 0
    # per round, against the oracle on the shared (target-written) cache
    r.reset(N_NEW)
    oc = OracleCache(S, 512)
    prefill(env["ow"], oc, env["prompt"])
    n0, exempt, ms = 0, 0, []
    while n0 < N_NEW:
        r.step()
        st, toks = r.read_state()
        drafts = [int(x) for x in to_np(r.debug_view(3, torch.int32))[:D]]
        assert drafts[0] == gpu_ar[n0]
        assert st.m_last >= 1
        rows = forward(q4env["ow"], oc.clone(), drafts[:-1])
        for j in range(1, D):
            if int(np.argmax(rows[j - 1])) != drafts[j]:
                assert oracle_margin(rows[j - 1]) < MARGIN, f"round at {n0}: draft {j}"
                exempt += 1
        forward(env["ow"], oc, [int(x) for x in toks[n0:st.n_committed]])
        ms.append(st.m_last)
        n0 = st.n_committed
    say(f"q4 substitute draft: accepted per round {ms}, {exempt} draft tokens exempt by the margin rule")


def test_round_prefill_fits_a_tight_cache(env, gpu_ar):
    """A cache sized for the prompt and one job only (no spare margin) runs the job."""
    from block_verify_amd.synth import make_draft_table
    b = env["b"]
    table = make_draft_table(np.array(gpu_ar), env["shape"].vocab, 0.4)
    tight = P + N_NEW + 2 * (K + 1) + 2
    r = b.Round(env["model"], K, table=table, max_len=tight)
    r.prefill(env["prompt"])
    st, toks = r.run(N_NEW)
    assert list(toks[:N_NEW]) == gpu_ar[:N_NEW]
    with pytest.raises(b.SpecdecError):
        r.reset(N_NEW + 2 * (K + 1))


@pytest.mark.parametrize("schedule", [0, 1])
@pytest.mark.parametrize("k", [1, 16])
def test_spec_extreme_draft_counts(env, gpu_ar, schedule, k):
    """k = 1 and the maximum k = 16 (a 17-row verify under schedule B) commit the greedy tokens."""
    from block_verify_amd.synth import make_draft_table
    b = env["b"]
    n = 24
    ar = _gpu_ar(env, n + k + 2)
    table = make_draft_table(np.array(ar), env["shape"].vocab, 0.3)
    r = b.Round(env["model"], k, schedule=schedule, table=table, max_len=512)
    r.prefill(env["prompt"])
    st, toks = r.run(n)
    assert list(toks[:n]) == ar[:n]
    assert r.tcache.length() == P + st.n_committed - (1 if schedule == 1 else 0)
    assert r.ws.error_bits() == 0


@pytest.mark.parametrize("schedule,plen", [(0, 1), (1, 2)])
def test_spec_shortest_prompt(env, schedule, plen):
    """The shortest prompts each schedule takes (1 token for A, 2 for B, whose last one stays pending)."""
    from block_verify_amd.synth import make_draft_table
    b, S = env["b"], env["shape"]
    prompt = env["prompt"][:plen]
    cache, ws = _fresh(env)
    n = 12
    toks = torch.zeros(n + K + 3, dtype=torch.int32, device="cuda")
    scratch = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(env["model"], cache, torch.from_numpy(np.asarray(prompt, np.int32)).cuda(), ws, logits=scratch,
              argmax=toks[0:1])
    for i in range(n + K + 1):
        b.decode_step(env["model"], cache, toks[i:i + 1], ws, logits=scratch, argmax=toks[i + 1:i + 2])
    ar = [int(x) for x in to_np(toks)[:n + K + 2]]
    table = make_draft_table(np.array(ar), S.vocab, 0.4)
    r = b.Round(env["model"], K, schedule=schedule, table=table, max_len=128)
    r.prefill(prompt)
    st, got = r.run(n)
    assert list(got[:n]) == ar[:n]
    assert r.tcache.length() == plen + st.n_committed - (1 if schedule == 1 else 0)


def test_host_rejects_empty_and_oversized_inputs(env):
    b = env["b"]
    cache, ws = _fresh(env, max_len=64)
    with pytest.raises(b.SpecdecError):
        b.decode_step(env["model"], cache, torch.zeros(0, dtype=torch.int32, device="cuda"), ws)
    with pytest.raises(b.SpecdecError):
        b.decode_step(env["model"], cache, torch.zeros(33, dtype=torch.int32, device="cuda"), ws)
    with pytest.raises(b.SpecdecError):
        b.Round(env["model"], 17, table=np.zeros(64, np.int32), max_len=256)
    r = b.Round(env["model"], K, schedule=1, table=np.zeros(64, np.int32), max_len=256)
    with pytest.raises(b.SpecdecError):
        r.prefill(env["prompt"][:1])   # schedule B needs a pending token besides the prefix


def test_stochastic_zero_noise_accepts_every_draft(env):
    """q = p (no noise): min(1, p/q) = 1 up to rounding, so each round accepts all k drafts
    and adds a bonus token."""
    b, S = env["b"], env["shape"]
    noise = np.zeros((N_NEW + 2 * K + 2, S.vocab), np.float32)
    r = b.Round(env["model"], K, mode=b.STOCHASTIC, draft_source=b.DRAFT_NOISY_SELF, noise=noise, seed=3,
                max_len=512)
    r.prefill(env["prompt"])
    st, toks = r.run(N_NEW)
    assert st.accepted_total == K * st.round
    assert st.n_committed == (K + 1) * st.round
    assert r.ws.error_bits() == 0


@pytest.mark.parametrize("H,nq,hd,F", [(768, 12, 64, 4160), (1536, 12, 128, 2848), (2048, 16, 128, 4160)])
def test_gate_up_forms_give_the_same_bits(H, nq, hd, F):
    """Passes of 3 to 8 and of 17 to 32 rows run gate/up over several row
    groups per workgroup (activation tiles held in registers; one LDS slot per
    group for one column tile, two slots in turn for three or four), the
    other passes one row group per workgroup.  One-layer decoders whose
    k-split gives 3, 6 and 8 k-blocks a wave and 2 or 3 row groups a
    workgroup (one with a short last workgroup): a pass of 3, 8, 12 or 29 rows
    equals the same rows in single-row steps bit for bit, the 29-row pass on a
    long cache (head dims 64 and 128 through both merge forms) too, and the
    29-row pass matches the oracle."""
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import ModelShape
    from block_verify_amd.synth import make_prompt, make_weights
    from oracle.model import OracleCache, OracleWeights, forward, prefill
    S = ModelShape(f"gu{H}", 1, H, nq, 2, hd, F, 2048)
    say(f"gate/up forms H={H} F={F}")
    w = make_weights(S, 7)
    model = b.Model(S, w)
    prompt = make_prompt(S.vocab, 40, seed=8)
    pt = torch.from_numpy(prompt).cuda()
    for M in (3, 8, 12, 29):
        toks = np.random.default_rng(M).integers(0, S.vocab, M).astype(np.int32)
        t = torch.from_numpy(toks).cuda()
        c1, w1 = b.Cache(S, 128), b.Workspace(S, 128)
        c2, w2 = b.Cache(S, 128), b.Workspace(S, 128)
        b.prefill(model, c1, pt, w1)
        b.prefill(model, c2, pt, w2)
        lb = torch.empty((M, S.vocab), dtype=torch.float32, device="cuda")
        b.decode_step(model, c1, t, w1, logits=lb)
        ls = torch.empty((M, S.vocab), dtype=torch.float32, device="cuda")
        for i in range(M):
            b.decode_step(model, c2, t[i:i + 1], w2, logits=ls[i])
        assert torch.equal(lb.view(torch.int32), ls.view(torch.int32)), f"M={M}"
        assert w1.error_bits() == 0 and w2.error_bits() == 0
    # a long cache (more chunk workgroups, the eight-wave merge) gives the same bits
    c3, w3 = b.Cache(S, 8448), b.Workspace(S, 8448)
    b.prefill(model, c3, pt, w3)
    ll = torch.empty((M, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(model, c3, t, w3, logits=ll)
    assert torch.equal(lb.view(torch.int32), ll.view(torch.int32)) and w3.error_bits() == 0
    ow = OracleWeights(S, w)
    oc = OracleCache(S, 128)
    prefill(ow, oc, prompt)
    assert_logits_close(to_np(lb), forward(ow, oc, toks), f"H={H} pass of 29 rows")


def test_single_chunk_cache_gives_the_same_logits(env):
    """A cache of one attention chunk (capacity 48: one chunk workgroup per
    head and tile, a merge over one partial) gives the same logits, argmax and
    lse as a long cache, bit for bit, and the oracle's values."""
    from oracle.model import OracleCache, forward, prefill
    prompt = env["prompt"][:40]
    toks = np.random.default_rng(77).integers(0, env["shape"].vocab, 5)
    out = []
    for max_len in (48, 8448):
        cache, ws = _fresh(env, max_len)
        _gpu_prefill(env, cache, ws, prompt, chunk=13)
        logits, am, lse = _gpu_forward(env, cache, ws, toks)
        assert cache.length() == 45 and ws.error_bits() == 0
        out.append((logits, am, lse))
    for a, b_ in zip(out[0], out[1]):
        assert np.array_equal(a, b_)
    oc = OracleCache(env["shape"], 48)
    prefill(env["ow"], oc, prompt)
    assert_logits_close(out[0][0], forward(env["ow"], oc, toks), "one-chunk cache")
