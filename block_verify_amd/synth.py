"""Seeded synthetic inputs shared by the HIP path's harness and the oracle.

Everything here is input preparation: random-init bf16 weights, prompt ids,
the corrupted greedy-continuation draft table, Gaussian logit noise and the
4-bit group-64 min-max quantisation of the substitute draft's weights.  None
of it is a step of the verify forward or of the acceptance rule.

Determinism: every tensor is drawn in row blocks, each block from its own
numpy PCG64 stream seeded by (seed, tensor index, block index), so the bytes
do not depend on how many threads generate them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .shapes import (ModelShape, SEED_CORRUPT, SEED_NOISE, SEED_PROMPT)

WEIGHT_STD = 0.02
_BLOCK_ELEMS = 1 << 22


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _n_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gen_linear(seed: int, index: int, shape) -> np.ndarray:
    rows = shape[0]
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, cols), dtype=np.uint16)
    rows_per_block = max(1, _BLOCK_ELEMS // cols)
    blocks = [(b, r0, min(rows, r0 + rows_per_block))
              for b, r0 in enumerate(range(0, rows, rows_per_block))]

    def work(blk):
        b, r0, r1 = blk
        rng = np.random.default_rng([seed, index, b])
        v = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        v *= np.float32(WEIGHT_STD)
        out[r0:r1] = f32_to_bf16_bits(v)

    if len(blocks) == 1:
        work(blocks[0])
    else:
        with ThreadPoolExecutor(_n_threads()) as ex:
            list(ex.map(work, blocks))
    return out.reshape(shape)


def make_weights(shape: ModelShape, seed: int, only=None) -> list:
    """bf16 bit patterns (uint16) of every tensor, in canonical order.

    Linear and embedding weights ~ N(0, 0.02) rounded to bf16; norm gains 1.0.
    ``only`` optionally restricts generation to a set of tensor indices (the
    others are None), used by sampled checks that need a few tensors only.
    """
    specs = shape.tensor_specs()
    out = [None] * len(specs)
    one = np.uint16(0x3F80)  # 1.0 in bf16
    for i, (_, shp, kind) in enumerate(specs):
        if only is not None and i not in only:
            continue
        if kind == "norm":
            out[i] = np.full(shp, one, dtype=np.uint16)
        else:
            out[i] = _gen_linear(seed, i, shp)
    return out


def make_prompt(vocab: int, length: int, seed: int = SEED_PROMPT) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, vocab, length).astype(np.int32)


def make_draft_table(greedy: np.ndarray, vocab: int, corrupt_p: float,
                     seed: int = SEED_CORRUPT) -> np.ndarray:
    """Per-generated-position draft table.

    ``greedy[n]`` is the target's greedy token number n (0-based) of the
    continuation.  Each position is independently replaced, with probability
    ``corrupt_p``, by a uniformly drawn *different* token.
    """
    greedy = np.asarray(greedy, dtype=np.int64)
    n = greedy.shape[0]
    rng = np.random.default_rng(seed)
    u = rng.random(n)
    r = rng.integers(0, vocab - 1, n)
    repl = (greedy + 1 + r) % vocab
    return np.where(u < corrupt_p, repl, greedy).astype(np.int32)


def make_near_miss_table(greedy: np.ndarray, runner_up: np.ndarray, corrupt_p: float,
                         seed: int = SEED_CORRUPT) -> np.ndarray:
    """Draft table with the corruption mask of make_draft_table (same seed, same
    draws), but a corrupted position carries ``runner_up[n]``, the target's
    second-ranked token there, instead of a uniform random token: drafts that
    miss the top-1 by a small logit gap."""
    greedy = np.asarray(greedy, dtype=np.int64)
    n = greedy.shape[0]
    u = np.random.default_rng(seed).random(n)
    return np.where(u < corrupt_p, np.asarray(runner_up, dtype=np.int64)[:n], greedy).astype(np.int32)


def make_noise(n_pos: int, vocab: int, seed: int = SEED_NOISE) -> np.ndarray:
    """N(0,1) float32 logit noise, one row per generated position."""
    return np.random.default_rng(seed).standard_normal((n_pos, vocab), dtype=np.float32)


# ----------------------------------------------------------------------------
# 4-bit group-64 min-max quantisation (preparation of the substitute draft).
# ----------------------------------------------------------------------------
Q4_GROUP = 64


def quantize_q4g64(w_bf16: np.ndarray):
    """Asymmetric 4-bit, group 64 along the input dimension, fp16 scale/zero.

    Returns (packed uint8 [N, K/2] with the even input index in the low
    nibble, scale fp16 [N, K/64], zero fp16 [N, K/64]).  A group whose max
    equals its min gets scale 1, codes 0 and zero -min.
    """
    N, K = w_bf16.shape
    assert K % Q4_GROUP == 0
    w = bf16_bits_to_f32(w_bf16).reshape(N, K // Q4_GROUP, Q4_GROUP)
    mn = w.min(axis=2)
    mx = w.max(axis=2)
    flat = mx == mn
    s = np.where(flat, np.float32(1.0), (mx - mn) / np.float32(15.0)).astype(np.float32)
    s_h = s.astype(np.float16)
    z_h = np.where(flat, -mn, -mn / s_h.astype(np.float32)).astype(np.float16)
    q = np.rint(w / s_h.astype(np.float32)[..., None] + z_h.astype(np.float32)[..., None])
    q = np.clip(q, 0, 15)
    q = np.where(flat[..., None], 0, q).astype(np.uint8).reshape(N, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_h, z_h


def make_q4_draft(shape, tensors):
    """Substitute-draft tensors: every linear except the LM head quantised to
    4-bit group 64 (codes, scale, zero); norms kept; embedding, final norm
    and LM head None (shared with the target)."""
    specs = shape.tensor_specs()
    out = [None] * len(specs)
    lin = []
    for i, (name, _, kind) in enumerate(specs):
        if name in ("embed", "lm_head", "final_norm"):
            continue
        if kind == "linear":
            lin.append(i)
        else:
            out[i] = tensors[i]
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        for i, q in zip(lin, ex.map(lambda j: quantize_q4g64(tensors[j]), lin)):
            out[i] = q
    return out
