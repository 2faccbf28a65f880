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


def check_stochastic_round(saved, rows, qz, drafts, m_gpu, com_gpu, seed, rnd):
    """Replay one schedule-A round of modified rejection sampling in the oracle.

    saved: target logits before the round ([V]); rows: the k verify rows;
    qz: the k noisy draft logits the GPU drew from; drafts: the GPU's k draft
    tokens; m_gpu / com_gpu: the GPU's accepted count and committed tokens.
    Returns the number of boundary exemptions (0 or more); raises on a
    decision that differs away from a boundary.
    """
    from oracle import accept as acc
    from oracle import philox
    k = len(drafts)
    exempt = 0
    q_rows = [softmax64(qz[j]) for j in range(k)]
    for j in range(k):
        u = philox.uniform(seed, rnd, j, philox.STREAM_DRAFT)
        d = acc.sample_inverse_cdf(q_rows[j], u)
        if d != int(drafts[j]):
            assert near_cdf_step(q_rows[j], u, int(drafts[j])), f"round {rnd} draft {j}: gpu {drafts[j]} oracle {d}"
            exempt += 1
    p_rows = [softmax64(saved)] + [softmax64(r) for r in rows]
    ua = [philox.uniform(seed, rnd, j, philox.STREAM_ACCEPT) for j in range(k)]
    ur = philox.uniform(seed, rnd, 0, philox.STREAM_RESAMPLE)
    m, com, info = acc.stochastic_accept(p_rows, q_rows, [int(x) for x in drafts], ua, ur)
    if m == m_gpu and list(com) == [int(x) for x in com_gpu]:
        return exempt
    near_accept = any(abs(ua[j] - info["ratios"][j]) < BOUNDARY for j in range(len(info["ratios"])))
    if m == m_gpu:
        j = m
        src = acc.residual(p_rows[j], q_rows[j]) if j < k else p_rows[k]
        if j < k and src.sum() <= acc.RESIDUAL_EPS:
            src = p_rows[j]
        near_sample = near_cdf_step(src, ur, int(com_gpu[-1]))
    else:
        near_sample = False
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
