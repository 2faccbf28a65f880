"""GPU parity of the substitute-draft round at the 7B shape (28 layers, hidden 3584,
28 q / 4 kv heads of 128, FFN 18944, vocab 152064).

Values at the job's own 2048-token context come from stored oracle values
(tests/golden/qwen7b_2k_oracle.json, written by tests/golden/make_qwen7b_goldens.py,
which calls only the float64 oracle; ten minutes on the host, so it is not rerun
here): the prefill's saved_next, the 4-bit draft's step on the shared cache, and
an 8-row verify block over the oracle's own greedy tokens, each on 512 seeded
columns plus the row's top 8, and the argmax of every row (teacher forcing on
the oracle's tokens).  Over a 16-token prompt the oracle also runs here, on the
full vocabulary.  Properties at any size: committed tokens equal the GPU's own
greedy decode, d_1 = argmax(saved_next) is always accepted, the cache length
equals prompt + committed, and block rows equal single-row steps bit for bit.
"""
import json
import os
import time

import numpy as np
import pytest
import torch

from gpu_helpers import MARGIN, assert_logits_close, q4_oracle_weights, say, to_np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "qwen7b_2k_oracle.json")

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1100)]

P, N_NEW, D = 2048, 64, 8
P_SHORT = 16


@pytest.fixture(scope="module")
def m7():
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_7B, SEED_TARGET
    from block_verify_amd.synth import make_q4_draft, make_weights
    S = QWEN_7B
    t0 = time.time()
    w = make_weights(S, SEED_TARGET)
    say(f"7B: weights {time.time() - t0:.1f} s")
    t0 = time.time()
    qt = make_q4_draft(S, w)
    say(f"7B: 4-bit quantisation {time.time() - t0:.1f} s")
    model = b.Model(S, w)
    qmodel = b.Model(S, qt, weight_format=b.W_Q4G64, share=model)
    torch.cuda.synchronize()
    return dict(b=b, S=S, w=w, qt=qt, model=model, qmodel=qmodel)


@pytest.mark.parametrize("which", ["target", "q4"])
def test_7b_short_prompt_logits(m7, which):
    from block_verify_amd.synth import make_prompt
    from oracle.model import OracleCache, OracleWeights, forward, prefill
    b, S = m7["b"], m7["S"]
    prompt = make_prompt(S.vocab, P_SHORT, seed=21)
    model = m7["model"] if which == "target" else m7["qmodel"]
    cache = b.Cache(S, 64)
    ws = b.Workspace(S, 64)
    saved = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(model, cache, torch.from_numpy(prompt).cuda(), ws, chunk=32 if which == "target" else 4, logits=saved)
    rows = 4
    toks = np.random.default_rng(3).integers(0, S.vocab, rows).astype(np.int32)
    lg = torch.empty((rows, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(model, cache, torch.from_numpy(toks).cuda(), ws, logits=lg)
    t0 = time.time()
    ow = OracleWeights(S, m7["w"], cache=False) if which == "target" else q4_oracle_weights(S, m7["w"], m7["qt"], cache=False)
    oc = OracleCache(S, 64)
    o_saved = prefill(ow, oc, prompt)
    o_rows = forward(ow, oc, toks)
    say(f"7B {which}: oracle {time.time() - t0:.1f} s")
    assert_logits_close(to_np(saved), o_saved, f"7B {which} prefill saved_next")
    assert_logits_close(to_np(lg), o_rows, f"7B {which} block rows")
    assert ws.error_bits() == 0


def test_7b_batch_invariance_q4_and_target(m7):
    from block_verify_amd.synth import make_prompt
    b, S = m7["b"], m7["S"]
    prompt = make_prompt(S.vocab, 64, seed=22)
    for model, n in ((m7["model"], 8), (m7["qmodel"], 4)):
        cache = b.Cache(S, 128)
        ws = b.Workspace(S, 128)
        b.prefill(model, cache, torch.from_numpy(prompt).cuda(), ws, chunk=4)
        toks = torch.from_numpy(np.arange(n, dtype=np.int32) * 9973 + 17).cuda()
        lb = torch.empty((n, S.vocab), dtype=torch.float32, device="cuda")
        b.decode_step(model, cache, toks, ws, logits=lb)
        cache.trim(64, ws)
        ls = torch.empty((n, S.vocab), dtype=torch.float32, device="cuda")
        for i in range(n):
            b.decode_step(model, cache, toks[i:i + 1], ws, logits=ls[i])
        assert torch.equal(lb.view(torch.int32), ls.view(torch.int32))


def test_7b_substitute_job_equals_greedy_ar(m7):
    from block_verify_amd.synth import make_prompt
    b, S = m7["b"], m7["S"]
    prompt = make_prompt(S.vocab, P)
    max_len = P + 256
    cache = b.Cache(S, max_len)
    ws = b.Workspace(S, max_len)
    n = N_NEW + D + 2
    toks = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(m7["model"], cache, torch.from_numpy(prompt).cuda(), ws, logits=scratch, argmax=toks[0:1])
    for i in range(n - 1):
        b.decode_step(m7["model"], cache, toks[i:i + 1], ws, logits=scratch, argmax=toks[i + 1:i + 2])
    ar = [int(x) for x in to_np(toks)[:n]]
    r = b.Round(m7["model"], D, draft_source=b.DRAFT_Q4_SELF, draft=m7["qmodel"], max_len=max_len)
    r.prefill(prompt)
    r.reset(N_NEW)
    n0, ms = 0, []
    while n0 < N_NEW:
        r.step()
        st, got = r.read_state()
        assert st.m_last >= 1
        assert r.tcache.length() == P + st.n_committed
        ms.append(st.m_last)
        n0 = st.n_committed
    assert list(got[:N_NEW]) == ar[:N_NEW]
    assert r.ws.error_bits() == 0
    say(f"7B substitute draft (depth {D}): {len(ms)} rounds, accepted per round {ms}")


def _against_golden(gpu_row, rec, what):
    """Sampled columns within the logits tolerance; the full-vocabulary argmax equal to the
    oracle's unless the oracle's top-2 margin is below 0.1.  Returns True if exempt."""
    cols = np.asarray(rec["cols"])
    assert_logits_close(np.asarray(gpu_row, np.float64)[cols], np.asarray(rec["values"], np.float64), what)
    ga = int(np.argmax(gpu_row))
    if ga == rec["argmax"]:
        return False
    assert rec["margin"] < MARGIN, f"{what}: argmax gpu {ga} oracle {rec['argmax']} margin {rec['margin']:.4f}"
    return True


def test_7b_2k_values_against_oracle_goldens(m7):
    """Config 5 at its own context: saved_next after the 2048-token prefill, the 4-bit
    draft's first step on the target's cache, and the 8-row verify block over the oracle's
    greedy tokens g_1..g_8 (row i against the oracle's one-token step i)."""
    from block_verify_amd.synth import make_prompt
    with open(GOLDEN) as f:
        gold = json.load(f)
    b, S = m7["b"], m7["S"]
    assert gold["prompt_len"] == P and gold["shape"] == S.name
    prompt = make_prompt(S.vocab, P)
    cache = b.Cache(S, P + 64)
    ws = b.Workspace(S, P + 64)
    saved = torch.empty(S.vocab, dtype=torch.float32, device="cuda")
    b.prefill(m7["model"], cache, torch.from_numpy(prompt).cuda(), ws, logits=saved)
    exempt = int(_against_golden(to_np(saved), gold["saved_next"], "7B 2K saved_next"))
    g = np.asarray(gold["tokens"], np.int32)
    q4l = torch.empty((1, S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(m7["qmodel"], cache, torch.from_numpy(g[:1]).cuda(), ws, logits=q4l)
    exempt += int(_against_golden(to_np(q4l)[0], gold["q4_step"], "7B 2K 4-bit draft step"))
    cache.trim(P, ws)
    rows = torch.empty((len(g), S.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(m7["model"], cache, torch.from_numpy(g).cuda(), ws, logits=rows)
    r = to_np(rows)
    for i, rec in enumerate(gold["rows"]):
        exempt += int(_against_golden(r[i], rec, f"7B 2K verify row {i}"))
    assert cache.length() == P + len(g)
    assert ws.error_bits() == 0
    say(f"7B 2K goldens: {len(g) + 2} rows, {exempt} argmax differences where the oracle margin < {MARGIN}")
