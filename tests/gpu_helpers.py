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
