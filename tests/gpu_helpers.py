"""Shared pieces of the GPU parity tests (imported by tests marked gpu only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# logits tolerance of the parity bar: |gpu - oracle| <= ATOL + RTOL * |oracle|
RTOL = 2e-2
ATOL = 5e-2
# tokens: exact, except where the oracle's top-2 margin is below this
MARGIN = 0.1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_logits_close(gpu: np.ndarray, ora: np.ndarray, what: str = "logits"):
    gpu = np.asarray(gpu, np.float64)
    ora = np.asarray(ora, np.float64)
    assert gpu.shape == ora.shape, (gpu.shape, ora.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ora)
    bound = ATOL + RTOL * np.abs(ora)
    worst = np.argmax(err - bound)
    ok = np.all(err <= bound)
    say(f"{what}: max|err| {err.max():.3e}  max rel-to-bound {(err / bound).max():.3f}  "
        f"oracle max|x| {np.abs(ora).max():.3f}")
    assert ok, f"{what}: element {np.unravel_index(worst, err.shape)} gpu {gpu.flat[worst]} oracle {ora.flat[worst]}"


def oracle_margin(logits: np.ndarray) -> float:
    a = np.partition(np.asarray(logits, np.float64), -2)[-2:]
    return float(a[1] - a[0])


def tokens_match_teacher_forced(gpu_tokens, oracle_logits_rows, margin=MARGIN):
    """Each GPU token equals the oracle argmax unless the oracle margin there is < margin.

    oracle_logits_rows[i] are the oracle's logits predicting token i given the
    prompt and the GPU's tokens before i.  Returns (n_exempt, first_mismatch).
    """
    exempt = 0
    for i, t in enumerate(gpu_tokens):
        row = oracle_logits_rows[i]
        a = int(np.argmax(row))
        if a == int(t):
            continue
        if oracle_margin(row) < margin:
            exempt += 1
            continue
        raise AssertionError(f"token {i}: gpu {t} oracle {a} margin {oracle_margin(row):.4f}")
    return exempt


def to_np(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b).astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# Stochastic rounds: the GPU's decisions against the oracle's rule on the GPU's
# own logits.  Probabilities on the GPU are float32 (expf of logit - lse), the
# oracle's float64, so a decision whose uniform lies within BOUNDARY of the
# threshold (accept test) or of a CDF step (inverse-CDF sample, relative to the
# total mass) may legitimately differ; such cases are counted, not failed.
BOUNDARY = 1e-6


def softmax64(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def near_cdf_step(weights, u, i):
    """True when u * total lies within BOUNDARY * total of the CDF steps around index i."""
    c = np.cumsum(np.asarray(weights, np.float64))
    t = u * c[-1]
    lo = c[i - 1] if i > 0 else 0.0
    return min(abs(t - lo), abs(t - c[min(i, len(c) - 1)])) < BOUNDARY * c[-1]


def near_truncation_boundary(weights, top_k, top_p, band=BOUNDARY):
    """True when the truncated set of `weights` could change under a relative change of
    `band`: the top_k-th and next weights nearly tie, or the running mass of the survivors
    passes top_p of their total within band."""
    w = np.asarray(weights, np.float64)
    order = np.lexsort((np.arange(w.shape[0]), -w))
    near = False
    if 0 < top_k < w.shape[0]:
        a, b2 = w[order[top_k - 1]], w[order[top_k]]
        near |= abs(a - b2) <= band * max(a, 1e-300)
    if top_p < 1.0:
        kept = order[:top_k] if 0 < top_k < w.shape[0] else order
        c = np.cumsum(w[kept])
        near |= bool(np.any(np.abs(c - top_p * c[-1]) <= band * c[-1]))
    return near


def check_stochastic_round(saved, rows, qz, drafts, m_gpu, com_gpu, seed, rnd, bonus=True, temperature=1.0,
                           top_k=0, top_p=1.0):
    """Replay one schedule-A round of modified rejection sampling in the oracle
    (oracle.spec.draft_sample and oracle.spec.stochastic_round) on the GPU's logits.

    saved: target logits before the round ([V]); rows: the k verify rows;
    qz: the k draft logit rows the GPU drew from; drafts: the GPU's k draft
    tokens; m_gpu / com_gpu: the GPU's accepted count and committed tokens.
    Returns the number of boundary exemptions (0 or more); raises on a
    decision that differs away from a boundary.
    """
    from oracle import accept as acc
    from oracle import philox
    from oracle.spec import draft_sample, stochastic_round
    k = len(drafts)
    drafts = [int(x) for x in drafts]
    exempt = 0
    for j in range(k):
        d = draft_sample(qz[j], seed, rnd, j, temperature)
        if d != drafts[j]:
            u = philox.uniform(seed, rnd, j, philox.STREAM_DRAFT)
            assert near_cdf_step(acc.softmax(qz[j], temperature), u, drafts[j]), \
                f"round {rnd} draft {j}: gpu {drafts[j]} oracle {d}"
            exempt += 1
    m, com, info = stochastic_round(saved, rows, qz, drafts, seed, rnd, bonus, temperature, top_k, top_p)
    if m == m_gpu and list(com) == [int(x) for x in com_gpu]:
        return exempt
    near_accept = any(abs(u - a) < BOUNDARY for u, a in zip(info["u_accept"], info["ratios"]))
    near_sample = (m == m_gpu and info["sample_weights"] is not None and
                   (near_cdf_step(info["sample_weights"], info["u_resample"], int(com_gpu[-1])) or
                    near_truncation_boundary(info["source_weights"], top_k, top_p)))
    assert near_accept or near_sample, f"round {rnd}: gpu m={m_gpu} {list(com_gpu)} oracle m={m} {com}"
    return exempt + 1


def q4_oracle_weights(shape, target_tensors, q4_tensors, cache=True):
    """Oracle view of the substitute draft: the target's tensors with every
    4-bit linear replaced by its (codes, scale, zero), dequantised on use."""
    from oracle.model import OracleWeights
    out = list(target_tensors)
    for i, t in enumerate(q4_tensors):
        if isinstance(t, tuple):
            out[i] = t
    return OracleWeights(shape, out, cache=cache)
