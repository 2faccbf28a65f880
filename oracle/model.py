"""Oracle decoder forward with an explicit KV cache (float64, numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed:
* "SpecDec-Context-Scaling 项目解读" (richardf123.github.io), section 2.2:
  a self-built forward that serves prefill, decode and block verification,
  with an independent KV-cache API that supports trim.
* Same page, section 3.2: the cache length equals the number of committed
  tokens that later steps may condition on; trim drops the tail.
* Same page, section 2.1: chunked prefill with chunk 2048.
* Causal attention (explainer on wmrh.cn, section 3.2): position i sees only
  positions <= i, so one block forward yields every row of a block.

* Same page, section 2.1 (the frozen configuration table): computation in
  BF16 and the target's KV cache executed in BF16.  The cache therefore
  stores every K and V entry rounded to bf16 (round to nearest even) when it
  is appended; everything else here stays float64.  ``kv_bf16=False`` keeps
  full-precision entries (the plain decoder, for cross-checks).

Decoder details the pages do not give (the plainest Qwen2-style reading):
pre-norm RMSNorm with eps 1e-6, rotate-half RoPE, grouped-query attention
(query head h reads kv head h // group), no biases, SwiGLU MLP, untied LM
head.  Parity of logit *values* is not pinned by the pages (they print
none); the tests pin this module by closed forms, invariants and brute force.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


class OracleWeights:
    """float64 view of one decoder's weights.

    ``tensors`` is the canonical list of bf16 bit arrays (see
    ``ModelShape.tensor_specs``); entries may also be float arrays already,
    or 4-bit group-64 (codes, scale, zero) tuples of the substitute draft,
    dequantised on use as in ``oracle.q4``.  With ``cache`` False each matrix
    is upcast on use and dropped, which keeps 7B-sized models inside host
    memory.
    """

    def __init__(self, shape, tensors, cache: bool = True):
        self.shape = shape
        self.tensors = tensors
        self.cache = cache
        self._f64 = {}
        self.index = {name: i for i, (name, _, _) in enumerate(shape.tensor_specs())}

    def __getitem__(self, name: str) -> np.ndarray:
        i = self.index[name]
        if i in self._f64:
            return self._f64[i]
        t = self.tensors[i]
        if isinstance(t, tuple):
            from oracle.q4 import dequantize
            a = dequantize(*t)
        elif t.dtype == np.uint16:
            a = bf16_to_f64(t)
        else:
            a = np.asarray(t, dtype=np.float64)
        if self.cache:
            self._f64[i] = a
        return a

    def embed_rows(self, tokens) -> np.ndarray:
        t = self.tensors[self.index["embed"]]
        rows = t[np.asarray(tokens, dtype=np.int64)]
        return bf16_to_f64(rows) if rows.dtype == np.uint16 else np.asarray(rows, np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even), as float64."""
    m, e = np.frexp(np.asarray(a, dtype=np.float64))   # a = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


class OracleCache:
    """Contiguous K/V per layer: [n_kv_heads, max_len, head_dim], entries bf16-valued
    (float64 arrays) unless kv_bf16 is False."""

    def __init__(self, shape, max_len: int, kv_bf16: bool = True):
        self.shape = shape
        self.max_len = max_len
        self.kv_bf16 = kv_bf16
        self.k = [np.zeros((shape.n_kv_heads, max_len, shape.head_dim)) for _ in range(shape.n_layers)]
        self.v = [np.zeros((shape.n_kv_heads, max_len, shape.head_dim)) for _ in range(shape.n_layers)]
        self.length = 0

    def trim(self, new_len: int) -> None:
        """Keep the first new_len positions (the rest is dead)."""
        if not 0 <= new_len <= self.length:
            raise ValueError(f"trim to {new_len} outside [0, {self.length}]")
        self.length = new_len

    def clone(self) -> "OracleCache":
        c = OracleCache.__new__(OracleCache)
        c.shape, c.max_len, c.length, c.kv_bf16 = self.shape, self.max_len, self.length, self.kv_bf16
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        return c


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, per row."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def rope_rotate_half(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing (i, i + d/2).

    x: [rows, heads, d]; pos: [rows] absolute positions.  Pair i turns by
    pos * theta^(-2i/d).
    """
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, pos: np.ndarray, group: int) -> np.ndarray:
    """Grouped-query causal attention for a block of rows.

    q: [rows, n_q, d] at absolute positions ``pos``; k, v: [n_kv, T, d] hold
    positions 0..T-1.  Row i attends keys 0..pos[i] with scale 1/sqrt(d).
    Returns [rows, n_q * d].
    """
    rows, n_q, d = q.shape
    T = k.shape[1]
    out = np.empty((rows, n_q, d))
    key_idx = np.arange(T)
    mask = key_idx[None, :] <= np.asarray(pos)[:, None]          # [rows, T]
    for h in range(n_q):
        kv = h // group
        s = q[:, h, :] @ k[kv].T / np.sqrt(d)                      # [rows, T]
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[kv]
    return out.reshape(rows, n_q * d)


def forward(w: OracleWeights, cache: OracleCache, tokens, last_only: bool = False) -> np.ndarray:
    """Run ``tokens`` at positions cache.length.. ; append their K/V; return logits.

    This single function is the prefill, the M=1 decode step and the M=k
    block verification: only the number of rows differs.
    """
    sh = w.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    M = tokens.shape[0]
    t = cache.length
    if t + M > cache.max_len:
        raise ValueError("KV cache capacity exceeded")
    pos = t + np.arange(M)
    x = w.embed_rows(tokens)
    for l in range(sh.n_layers):
        h = rms_norm(x, w[f"l{l}.attn_norm"], sh.rms_eps)
        q = (h @ w[f"l{l}.wq"].T).reshape(M, sh.n_q_heads, sh.head_dim)
        k = (h @ w[f"l{l}.wk"].T).reshape(M, sh.n_kv_heads, sh.head_dim)
        v = (h @ w[f"l{l}.wv"].T).reshape(M, sh.n_kv_heads, sh.head_dim)
        q = rope_rotate_half(q, pos, sh.rope_theta)
        k = rope_rotate_half(k, pos, sh.rope_theta)
        store = round_bf16 if cache.kv_bf16 else np.asarray
        cache.k[l][:, t:t + M, :] = store(k.transpose(1, 0, 2))
        cache.v[l][:, t:t + M, :] = store(v.transpose(1, 0, 2))
        o = causal_attention(q, cache.k[l][:, :t + M], cache.v[l][:, :t + M], pos, sh.group)
        x = x + o @ w[f"l{l}.wo"].T
        h2 = rms_norm(x, w[f"l{l}.mlp_norm"], sh.rms_eps)
        x = x + (silu(h2 @ w[f"l{l}.wgate"].T) * (h2 @ w[f"l{l}.wup"].T)) @ w[f"l{l}.wdown"].T
    cache.length = t + M
    if last_only:
        x = x[-1:]
    return rms_norm(x, w["final_norm"], sh.rms_eps) @ w["lm_head"].T


def prefill(w: OracleWeights, cache: OracleCache, tokens, chunk: int = 2048) -> np.ndarray:
    """Build the cache for ``tokens`` chunk by chunk; return the last row's logits."""
    tokens = np.asarray(tokens)
    last = None
    for c0 in range(0, tokens.shape[0], chunk):
        last = forward(w, cache, tokens[c0:c0 + chunk], last_only=True)[0]
    return last


def full_recompute_logits(w: OracleWeights, tokens, kv_bf16: bool = True) -> np.ndarray:
    """Logits of every position of ``tokens`` from a fresh cache (no reuse)."""
    tokens = np.asarray(tokens)
    c = OracleCache(w.shape, tokens.shape[0], kv_bf16)
    return forward(w, c, tokens)
