"""GPU parity at an 8192-token context: the 1.5B-shape target with a 0.5B-shape
draft model on its own cache (k draft steps per round whose tokens the
corrupted-greedy table overrides; both caches trimmed and repaired).

The float64 oracle prefills the full 8192 tokens for both models (about a
minute each) and checks the target's saved_next and verify rows, and sampled
K/V of both caches; the job's committed tokens equal the GPU's own greedy
decode, and both cache lengths follow the invariant after every round.
"""
import time

import numpy as np
import pytest
import torch

from gpu_helpers import assert_logits_close, bf16_bits_to_f64, say, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1100)]

P, N_NEW, K, C = 8192, 64, 4, 0.51


@pytest.fixture(scope="module")
def ctx8k():
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_0_5B, QWEN_1_5B, SEED_DRAFT, SEED_TARGET
    from block_verify_amd.synth import make_prompt, make_weights
    S, D = QWEN_1_5B, QWEN_0_5B
    w, dw = make_weights(S, SEED_TARGET), make_weights(D, SEED_DRAFT)
    model, draft = b.Model(S, w), b.Model(D, dw)
    prompt = make_prompt(S.vocab, P)
    max_len = P + 256
    cache, ws = b.Cache(S, max_len), b.Workspace(S, max_len)
    saved = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    n = N_NEW + K + 2
    toks = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    b.prefill(model, cache, torch.from_numpy(prompt).cuda(), ws, logits=saved, argmax=toks[0:1])
    saved_np = to_np(saved).copy()
    scratch = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    for i in range(n - 1):
        b.decode_step(model, cache, toks[i:i + 1], ws, logits=scratch, argmax=toks[i + 1:i + 2])
    cache.trim(P, ws)
    ar = [int(x) for x in to_np(toks)[:n]]
    return dict(b=b, S=S, D=D, w=w, dw=dw, model=model, draft=draft, prompt=prompt, cache=cache, ws=ws,
                saved=saved_np, ar=ar, max_len=max_len)


def test_8k_target_against_oracle(ctx8k):
    from oracle.model import OracleCache, OracleWeights, forward, prefill
    b, S = ctx8k["b"], ctx8k["S"]
    t0 = time.time()
    ow = OracleWeights(S, ctx8k["w"])
    oc = OracleCache(S, ctx8k["max_len"])
    o_saved = prefill(ow, oc, ctx8k["prompt"])
    say(f"8K: oracle float64 prefill {time.time() - t0:.1f} s")
    assert_logits_close(ctx8k["saved"], o_saved, "8K saved_next")
    rows = 5
    toks = np.random.default_rng(8).integers(0, S.vocab, rows).astype(np.int32)
    lg = torch.empty((rows, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(ctx8k["model"], ctx8k["cache"], torch.from_numpy(toks).cuda(), ctx8k["ws"], logits=lg)
    assert_logits_close(to_np(lg), forward(ow, oc.clone(), toks), "8K verify rows")
    kk, vv = ctx8k["cache"].kv()
    rng = np.random.default_rng(1)
    for l in rng.choice(S.n_layers, 4, replace=False):
        pos = rng.choice(P, 60, replace=False)
        pt = torch.from_numpy(pos).cuda()
        g = bf16_bits_to_f64(np.stack([to_np(kk[int(l)][:, pt, :]), to_np(vv[int(l)][:, pt, :])]))
        o = np.stack([oc.k[l][:, pos], oc.v[l][:, pos]])
        err = np.abs(g - o).max()
        say(f"8K layer {l}: K/V max err {err:.3e} of {np.abs(o).max():.3f}")
        assert err <= 1e-2 * np.abs(o).max()
    ctx8k["cache"].trim(P, ctx8k["ws"])
    assert ctx8k["ws"].error_bits() == 0


@pytest.mark.parametrize("schedule", [0, 1])
def test_8k_draft_model_job(ctx8k, schedule):
    from block_verify_amd.synth import make_draft_table
    b, S = ctx8k["b"], ctx8k["S"]
    table = make_draft_table(np.array(ctx8k["ar"]), S.vocab, C)
    r = b.Round(ctx8k["model"], K, schedule=schedule, draft_source=b.DRAFT_MODEL, draft=ctx8k["draft"], table=table,
                max_len=ctx8k["max_len"])
    r.prefill(ctx8k["prompt"])
    r.reset(N_NEW)
    n0 = 0
    while n0 < N_NEW:
        r.step()
        st, got = r.read_state()
        assert r.tcache.length() == P + st.n_committed - (1 if schedule == 1 else 0)
        assert r.dcache.length() == P + st.n_committed
        n0 = st.n_committed
    assert list(got[:N_NEW]) == ctx8k["ar"][:N_NEW]
    assert r.ws.error_bits() == 0 and r.dws.error_bits() == 0
    say(f"8K schedule {'AB'[schedule]}: {st.round} rounds, {st.accepted_total} drafts accepted")
    if schedule == 0:
        ctx8k["dcache_after"] = (r, [int(x) for x in got[:st.n_committed]])


def test_8k_draft_cache_against_oracle(ctx8k):
    """The draft model's cache after the job holds its K/V of prompt + committed tokens."""
    from oracle.model import OracleCache, OracleWeights, prefill
    if "dcache_after" not in ctx8k:
        pytest.skip("needs the schedule-A job")
    r, com = ctx8k["dcache_after"]
    D = ctx8k["D"]
    seq = np.concatenate([ctx8k["prompt"], np.array(com, np.int32)])
    t0 = time.time()
    oc = OracleCache(D, len(seq) + 8)
    prefill(OracleWeights(D, ctx8k["dw"]), oc, seq)
    say(f"8K draft: oracle float64 prefill {time.time() - t0:.1f} s")
    kk, vv = r.dcache.kv()
    rng = np.random.default_rng(2)
    n = len(seq)
    for l in rng.choice(D.n_layers, 4, replace=False):
        pos = np.concatenate([rng.choice(P, 40, replace=False), np.arange(P, n)])
        pt = torch.from_numpy(pos).cuda()
        g = bf16_bits_to_f64(np.stack([to_np(kk[int(l)][:, pt, :]), to_np(vv[int(l)][:, pt, :])]))
        o = np.stack([oc.k[l][:, pos], oc.v[l][:, pos]])
        err = np.abs(g - o).max()
        say(f"8K draft layer {l}: K/V max err {err:.3e} of {np.abs(o).max():.3f}")
        assert err <= 1e-2 * np.abs(o).max()
