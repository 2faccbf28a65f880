"""Oracle draft tree: construction, tree-attention verify, longest-path acceptance.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"SubSpec" summary (jjl357.github.io), section 4.2 (the context-aware draft
tree): over D steps every current leaf is fed to the draft model; each
candidate next token scores its conditional draft probability times the
score of its parent's path; the k best candidates become the next leaves.
Before the cumulative scores are formed the draft distribution is sharpened
with temperature 0.2.  The tree holds k x D draft tokens besides its root.

The target verifies the whole tree in one forward: a node sees the cached
context and its own ancestors only (tree-causal attention), at position
t + depth.  Greedy acceptance walks from the root: the target's choice at a
node selects the child carrying that token, if there is one, and the walk
stops where there is none; the accepted path and the target's choice after
it are committed (the block verify of "SpecDec-Context-Scaling 项目解读",
section 3, is the special case of a single chain).

Block layout used here: row 0 is the root (the round's pending token, the
last committed token whose K/V is not yet cached), rows 1..n-1 the draft
nodes in construction order; parents[i] < i is the row of node i's parent,
parents[0] = -1.  Readings where the pages are silent: candidates tie-break
by (leaf row, token id), lower first; a node's children are searched in row
order and the first match is taken.
"""
from __future__ import annotations

import numpy as np

from . import accept as acc
from .model import OracleCache, OracleWeights, rms_norm, rope_rotate_half, round_bf16, silu

SHARPEN_T = 0.2


def depths(parents) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            if not p < i:
                raise ValueError("a parent precedes its child")
            d[i] = d[p] + 1
    return d


def ancestor_mask(parents) -> np.ndarray:
    """[n, n] bool: mask[i, j] iff row j is row i or one of its ancestors."""
    n = len(parents)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j >= 0:
            m[i, j] = True
            j = parents[j]
    return m


def tree_forward(w: OracleWeights, cache: OracleCache, tokens, parents) -> np.ndarray:
    """One forward of a token tree at the cache's current length t: row i sits at
    position t + depth(i), sees cache positions 0..t-1 and its ancestors-or-self in the
    block, and appends its K/V at slot t + i.  Returns the logits [n, V]."""
    sh = w.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    t = cache.length
    if t + n > cache.max_len:
        raise ValueError("KV cache capacity exceeded")
    pos = t + depths(parents)
    anc = ancestor_mask(parents)
    # key visibility: the whole cached prefix, then the block's ancestors-or-self
    vis = np.concatenate([np.ones((n, t), dtype=bool), anc], axis=1)
    x = w.embed_rows(tokens)
    for l in range(sh.n_layers):
        h = rms_norm(x, w[f"l{l}.attn_norm"], sh.rms_eps)
        q = rope_rotate_half((h @ w[f"l{l}.wq"].T).reshape(n, sh.n_q_heads, sh.head_dim), pos, sh.rope_theta)
        k = rope_rotate_half((h @ w[f"l{l}.wk"].T).reshape(n, sh.n_kv_heads, sh.head_dim), pos, sh.rope_theta)
        v = (h @ w[f"l{l}.wv"].T).reshape(n, sh.n_kv_heads, sh.head_dim)
        store = round_bf16 if cache.kv_bf16 else np.asarray
        cache.k[l][:, t:t + n, :] = store(k.transpose(1, 0, 2))
        cache.v[l][:, t:t + n, :] = store(v.transpose(1, 0, 2))
        K, Vv = cache.k[l][:, :t + n], cache.v[l][:, :t + n]
        o = np.empty((n, sh.n_q_heads, sh.head_dim))
        for hq in range(sh.n_q_heads):
            kv = hq // sh.group
            s = q[:, hq, :] @ K[kv].T / np.sqrt(sh.head_dim)
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o[:, hq, :] = p @ Vv[kv]
        x = x + o.reshape(n, -1) @ w[f"l{l}.wo"].T
        h2 = rms_norm(x, w[f"l{l}.mlp_norm"], sh.rms_eps)
        x = x + (silu(h2 @ w[f"l{l}.wgate"].T) * (h2 @ w[f"l{l}.wup"].T)) @ w[f"l{l}.wdown"].T
    cache.length = t + n
    return rms_norm(x, w["final_norm"], sh.rms_eps) @ w["lm_head"].T


def tree_accept_greedy(tokens, parents, row_argmax):
    """Longest accepted path.  row_argmax[i] is the target's choice after row i.  From the
    root (row 0) the walk moves to the first child (in row order) whose token equals the
    current choice.  Returns (path rows after the root, committed tokens): the path's
    tokens, then the target's choice at the path's end."""
    children = [[] for _ in tokens]
    for i, p in enumerate(parents):
        if p >= 0:
            children[p].append(i)
    node, path = 0, []
    while True:
        v = int(row_argmax[node])
        nxt = next((c for c in children[node] if int(tokens[c]) == v), None)
        if nxt is None:
            return path, [int(tokens[i]) for i in path] + [v]
        path.append(nxt)
        node = nxt


def compact(cache: OracleCache, t: int, path) -> None:
    """Keep the root (slot t) and move the accepted path's K/V to slots t+1..t+m; the
    cache then holds t + 1 + m positions."""
    rows = [t] + [t + i for i in path]
    for l in range(len(cache.k)):
        cache.k[l][:, t:t + len(rows)] = cache.k[l][:, rows].copy()
        cache.v[l][:, t:t + len(rows)] = cache.v[l][:, rows].copy()
    cache.length = t + len(rows)


def select_children(leaf_rows, leaf_logits, scores, k: int, temperature: float = SHARPEN_T):
    """One step of the construction ("SubSpec" summary, section 4.2): every (leaf,
    token) pair scores the leaf's cumulative probability times the leaf's sharpened
    draft probability of the token; returns the k best as (score, leaf row, token),
    best first (ties: the lower leaf row, then the lower token id).  ``scores`` maps a
    row to its cumulative probability."""
    cand = []
    for leaf, z in zip(leaf_rows, leaf_logits):
        s = scores[leaf] * acc.softmax(np.asarray(z, dtype=np.float64), temperature)
        top = np.argsort(-s, kind="stable")[:k]
        cand += [(float(s[j]), int(leaf), int(j)) for j in top]
    cand.sort(key=lambda x: (-x[0], x[1], x[2]))
    return cand[:k]


def build_draft_tree(draft_w: OracleWeights, cache: OracleCache, root: int, k: int, depth: int,
                     temperature: float = SHARPEN_T):
    """The context-aware draft tree ("SubSpec" summary, section 4.2) rooted at `root`
    (the pending token) over the cache's committed prefix: `depth` steps, each feeding
    every current leaf to the draft model and keeping the k best (leaf, token) candidates
    by cumulative sharpened probability.  The cache is left unchanged.  Returns (tokens,
    parents) in block layout (row 0 = root)."""
    tokens, parents, score = [int(root)], [-1], [1.0]
    leaves = [0]
    for _ in range(depth):
        c = cache.clone()
        logits = tree_forward(draft_w, c, tokens, parents)
        leaves_new = []
        for s_, leaf, tok in select_children(leaves, [logits[l] for l in leaves], score, k, temperature):
            tokens.append(tok)
            parents.append(leaf)
            score.append(s_)
            leaves_new.append(len(tokens) - 1)
        leaves = leaves_new
    return tokens, parents


def spec_tree_greedy(w: OracleWeights, draft_w: OracleWeights, prompt, n_new: int, k: int, depth: int,
                     temperature: float = SHARPEN_T, max_len: int | None = None):
    """Greedy speculative decoding with a draft tree (block layout with the pending root):
    build the tree from the draft, verify it in one tree forward, accept the longest
    path, keep root + path in the cache, the target's choice becomes the next pending
    token.  Returns (tokens, accepted per round, cache)."""
    from .model import prefill
    prompt = np.asarray(prompt)
    P = prompt.shape[0]
    cache = OracleCache(w.shape, max_len or (P + n_new + k * depth + 4))
    prefill(w, cache, prompt[:-1])
    pending = int(prompt[-1])
    committed, ms = [], []
    while len(committed) < n_new:
        t = cache.length
        toks, pars = build_draft_tree(draft_w, cache, pending, k, depth, temperature)
        rows = tree_forward(w, cache, toks, pars)
        path, com = tree_accept_greedy(toks, pars, [acc.argmax_lowest(r) for r in rows])
        compact(cache, t, path)
        committed += com
        ms.append(len(path))
        pending = com[-1]
        assert cache.length == P + len(committed) - 1
    return committed[:n_new], ms, cache
