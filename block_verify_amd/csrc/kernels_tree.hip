// gfx950 kernels of the draft tree ("SubSpec" summary, jjl357.github.io,
// section 4.2): the selection step of the context-aware tree construction
// and the greedy acceptance of a verified tree.
//
// Block layout: node 0 is the root (the round's pending token), nodes 1.. the
// draft nodes in construction order, each node's parent an earlier node; a
// tree forward at cache length t puts node i at slot t + i.
//
// Construction: each step feeds the current leaves to the draft model; every
// (leaf, token) pair scores log P_leaf + log softmax(z_leaf / T)[token] (the
// leaf's cumulative log probability plus the sharpened draft log
// probability); the k best pairs become the next leaves.  Order: higher score
// first, then the lower leaf node, then the lower token id.  A leaf
// contributes at most k pairs, so only its k largest logits (ties: lower
// token id) are candidates: one launch finds them per vocabulary slice with
// each slice's (max, sum of exp) at temperature T; a single workgroup merges
// the slices per leaf and ranks the leaves' candidates.
//
// Acceptance: from the root, the first child (in node order) carrying the
// target's argmax at the current node continues the path; the path's K/V
// move to slots t + 1 .. t + m, the root stays at slot t, and the path's
// tokens plus the target's choice after it are committed.
#include "internal.h"

#include <math.h>

namespace sd {

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256, kSelWaves = kSelThreads / 64;

// (value desc, index asc) ordering: a before b.
__device__ __forceinline__ bool ranks_before(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Workgroup-wide best (value desc, index asc); every thread gets it.
__device__ __forceinline__ void wg_best(float& v, int& idx, float* sv, int* si) {
  warp_argmax(v, idx);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();   // the previous call's readers are done with sv / si
  if (lane == 0) { sv[w] = v; si[w] = idx; }
  __syncthreads();
  v = sv[0];
  idx = si[0];
  for (int u = 1; u < (int)(blockDim.x >> 6); ++u)
    if (ranks_before(sv[u], si[u], v, idx)) { v = sv[u]; idx = si[u]; }
}

// One workgroup per (vocabulary slice b, leaf j): the slice's maximum logit,
// its sum of exp((z - max) / T), and its k largest logits (ties: lower
// token id) as (logit, token) pairs, found in k passes that each take the
// best entry ranking after the previous pick.
__global__ __launch_bounds__(kSelThreads) void tree_cand_kernel(const float* __restrict__ logits, int V, int slice,
                                                                int nblk, int k, float inv_t,
                                                                float* __restrict__ stats, float* __restrict__ cand) {
  __shared__ float sv[kSelWaves];
  __shared__ int si[kSelWaves];
  const int b = blockIdx.x, j = blockIdx.y;
  const float* z = logits + (size_t)j * V;
  const int v0 = b * slice, v1 = min(V, v0 + slice);
  float mx = -INFINITY;
  int mi = 0x7fffffff;
  for (int v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
    const float x = z[v];
    if (ranks_before(x, v, mx, mi)) { mx = x; mi = v; }
  }
  wg_best(mx, mi, sv, si);
  float se = 0.f;
  if (mx > -INFINITY)
    for (int v = v0 + threadIdx.x; v < v1; v += blockDim.x) se += __expf((z[v] - mx) * inv_t);
  se = warp_sum(se);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sv[threadIdx.x >> 6] = se;
  __syncthreads();
  float* out = cand + (size_t)(j * nblk + b) * k * 2;
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int u = 0; u < kSelWaves; ++u) tot += sv[u];
    stats[(size_t)(j * nblk + b) * 2] = mx;
    stats[(size_t)(j * nblk + b) * 2 + 1] = tot;
    out[0] = mx;
    out[1] = __int_as_float(mi);
  }
  // picks 1 .. k-1: the best entry ranking after the previous pick
  float pv = mx;
  int pi = mi;
  for (int r = 1; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
      const float x = z[v];
      if (ranks_before(pv, pi, x, v) && ranks_before(x, v, bv, bi)) { bv = x; bi = v; }
    }
    wg_best(bv, bi, sv, si);
    if (threadIdx.x == 0) {
      out[2 * r] = bv;
      out[2 * r + 1] = __int_as_float(bi);
    }
    pv = bv;
    pi = bi;
  }
}

// One workgroup: per leaf j the vocabulary's max and log-sum-exp at T (the
// slices' stats merged in slice order) and its k best candidates; then the k
// best (leaf, token) pairs by score become nodes n_new .. n_new + k - 1 with
// parent n0 + j.  Scores: scores[n0 + j] + (z - max) / T - log(sum).
constexpr int kSelMaxK = 16;
__global__ __launch_bounds__(kSelThreads) void tree_select_kernel(const float* __restrict__ stats,
                                                                  const float* __restrict__ cand, int nblk, int k,
                                                                  int r, int n0, int n_new, int V, float inv_t,
                                                                  int32_t* __restrict__ tokens,
                                                                  int32_t* __restrict__ parents,
                                                                  float* __restrict__ scores) {
  __shared__ float sv[kSelWaves];
  __shared__ int si[kSelWaves];
  __shared__ float pool_s[kSelMaxK * kSelMaxK];
  __shared__ int pool_t[kSelMaxK * kSelMaxK];
  const int nc = nblk * k;
  for (int j = 0; j < r; ++j) {
    const float* st = stats + (size_t)j * nblk * 2;
    const float* cj = cand + (size_t)j * nc * 2;
    // max over slices, then the sum of their exp terms in slice order
    float mx = -INFINITY;
    int dummy = 0;
    for (int b = threadIdx.x; b < nblk; b += blockDim.x) mx = fmaxf(mx, st[2 * b]);
    wg_best(mx, dummy, sv, si);
    float lse = 0.f;
    if (threadIdx.x == 0) {
      float tot = 0.f;
      for (int b = 0; b < nblk; ++b) {
        const float mb = st[2 * b];
        if (mb > -INFINITY) tot += st[2 * b + 1] * __expf((mb - mx) * inv_t);
      }
      sv[0] = logf(tot);
    }
    __syncthreads();
    lse = sv[0];
    const float base = scores[n0 + j];
    // the leaf's k best candidates over its slices' lists
    float pv = INFINITY;
    int pi = -1;
    for (int r2 = 0; r2 < k; ++r2) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = threadIdx.x; c < nc; c += blockDim.x) {
        const float x = cj[2 * c];
        const int v = __float_as_int(cj[2 * c + 1]);
        if (v >= 0 && v < V && ranks_before(pv, pi, x, v) && ranks_before(x, v, bv, bi)) { bv = x; bi = v; }
      }
      wg_best(bv, bi, sv, si);
      if (threadIdx.x == 0) {
        const bool ok = bi >= 0 && bi < V && bv > -INFINITY;
        pool_s[j * k + r2] = ok ? base + (bv - mx) * inv_t - lse : -INFINITY;
        pool_t[j * k + r2] = ok ? bi : 0;
      }
      pv = bv;
      pi = bi;
    }
  }
  __syncthreads();
  // rank the r * k pairs by (score desc, key asc) with key = leaf * 2^24 +
  // token, i.e. ties go to the lower leaf, then the lower token; a slot
  // without a finite candidate (only with non-finite logits) ranks last under
  // a key of its own
  const int np = r * k;
  const int e = threadIdx.x;
  const float my = e < np ? pool_s[e] : -INFINITY;
  const int mykey = e >= np ? 0x7fffffff : my > -INFINITY ? (e / k) * (1 << 24) + pool_t[e] : (1 << 28) + e;
  bool taken = e >= np;
  for (int i = 0; i < k; ++i) {
    float bv = taken ? -INFINITY : my;
    int bk = taken ? 0x7fffffff : mykey;
    wg_best(bv, bk, sv, si);
    if (!taken && bk == mykey) {
      taken = true;
      tokens[n_new + i] = pool_t[e];
      parents[n_new + i] = n0 + e / k;
      scores[n_new + i] = my;
    }
  }
}

hipError_t launch_tree_select(const float* logits, int r, int V, int k, float inv_t, int n0, int n_new,
                              float* scratch, int32_t* tokens, int32_t* parents, float* scores, hipStream_t s) {
  if (k > kSelMaxK || r > kSelMaxK || r < 1 || k < 1) return hipErrorInvalidValue;
  int nblk = (V + 2047) / 2048;
  if (nblk > 128) nblk = 128;
  const int slice = (V + nblk - 1) / nblk;
  float* stats = scratch;
  float* cand = scratch + (size_t)r * nblk * 2;
  tree_cand_kernel<<<dim3(nblk, r), kSelThreads, 0, s>>>(logits, V, slice, nblk, k, inv_t, stats, cand);
  tree_select_kernel<<<1, kSelThreads, 0, s>>>(stats, cand, nblk, k, r, n0, n_new, V, inv_t, tokens, parents,
                                               scores);
  return hipGetLastError();
}

size_t tree_select_scratch_bytes(int r, int V, int k) {
  int nblk = (V + 2047) / 2048;
  if (nblk > 128) nblk = 128;
  return ((size_t)r * nblk * 2 + (size_t)r * nblk * k * 2) * sizeof(float);
}

// The construction's first step: node 0 = the root, score 0, and the cache
// length saved for the restore at the end.
__global__ void tree_root_kernel(const int32_t* __restrict__ root, const int32_t* __restrict__ d_len,
                                 int32_t* __restrict__ saved, int32_t* __restrict__ tokens,
                                 int32_t* __restrict__ parents, float* __restrict__ scores) {
  if (threadIdx.x == 0) {
    tokens[0] = *root;
    parents[0] = -1;
    scores[0] = 0.f;
    *saved = *d_len;
  }
}

hipError_t launch_tree_root(const int32_t* root, const int32_t* d_len, int32_t* saved, int32_t* tokens,
                            int32_t* parents, float* scores, hipStream_t s) {
  tree_root_kernel<<<1, 64, 0, s>>>(root, d_len, saved, tokens, parents, scores);
  return hipGetLastError();
}

// The construction's last step: the length as it was before the first (the
// fed nodes' K/V stay in the slots past it, to be overwritten by the verify).
__global__ void tree_restore_kernel(int32_t* d_len, const int32_t* __restrict__ saved) {
  if (threadIdx.x == 0) *d_len = *saved;
}

hipError_t launch_tree_restore(int32_t* d_len, const int32_t* saved, hipStream_t s) {
  tree_restore_kernel<<<1, 64, 0, s>>>(d_len, saved);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Acceptance
// ---------------------------------------------------------------------------
constexpr int kAccThreads = 256;

struct PathLds {
  int tok[kMaxTreeNodes];
  int nxt[kMaxTreeNodes];
  int path[kMaxTreeNodes];
  int m;
};

// The accepted path into L.path[0 .. L.m): node i continues from its parent p
// when its token is p's argmax and no earlier child of p carries that token.
// Every thread of the workgroup calls it.
__device__ void tree_path(const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents, int n,
                          const int32_t* __restrict__ argmax, PathLds& L) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    L.tok[i] = tokens[i];
    L.nxt[i] = -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int p = parents[i];
    if (p < 0 || p >= i || L.tok[i] != argmax[p]) continue;
    bool first = true;
    for (int j = p + 1; j < i && first; ++j)
      if (parents[j] == p && L.tok[j] == L.tok[i]) first = false;
    if (first) L.nxt[p] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int node = 0, m = 0;
    while (L.nxt[node] > node && m < n - 1) {
      node = L.nxt[node];
      L.path[m++] = node;
    }
    L.m = m;
  }
  __syncthreads();
}

// One workgroup per (layer, kv head): the path's K rows and V^T columns move
// to slots t+1.. in runs of kMaxRows, each run read into LDS before it is
// written.  A later run's sources (slots >= t + path[i] > t + i) lie past an
// earlier run's destinations.
template <int HD>
__global__ __launch_bounds__(kAccThreads) void tree_compact_kernel(bf16_bits* __restrict__ kv,
                                                                   const int32_t* __restrict__ d_len, int lp, int nkv,
                                                                   const int32_t* __restrict__ tokens,
                                                                   const int32_t* __restrict__ parents, int n,
                                                                   const int32_t* __restrict__ argmax) {
  __shared__ PathLds L;
  __shared__ bf16_bits kbuf[kMaxRows][HD], vbuf[kMaxRows][HD];
  const int l = blockIdx.x, h = blockIdx.y;
  const int t = *d_len - n;
  tree_path(tokens, parents, n, argmax, L);
  const int m = L.m;
  if (t < 0 || m == 0) return;
  bf16_bits* K = kv + (size_t)l * 2 * nkv * lp * HD + (size_t)h * lp * HD;
  bf16_bits* Vt = kv + (size_t)l * 2 * nkv * lp * HD + (size_t)nkv * lp * HD + (size_t)h * HD * lp;
  for (int c0 = 0; c0 < m; c0 += kMaxRows) {
    const int cn = min(kMaxRows, m - c0);
    for (int idx = threadIdx.x; idx < cn * HD; idx += blockDim.x) {
      const int i = idx / HD, d = idx % HD, src = t + L.path[c0 + i];
      kbuf[i][d] = K[(size_t)src * HD + d];
      vbuf[i][d] = Vt[(size_t)d * lp + src];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < cn * HD; idx += blockDim.x) {
      const int i = idx / HD, d = idx % HD, dst = t + 1 + c0 + i;
      K[(size_t)dst * HD + d] = kbuf[i][d];
      Vt[(size_t)d * lp + dst] = vbuf[i][d];
    }
    __syncthreads();
  }
}

// The commit, after the compaction has read the length: the path's tokens
// and the target's choice after it, their count, the length t + 1 + m, the
// next root (optional) and the job log (optional: log[0] tokens so far, the
// tokens from log[1]).
__global__ __launch_bounds__(kAccThreads) void tree_commit_kernel(
    int32_t* __restrict__ d_len, const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents, int n,
    const int32_t* __restrict__ argmax, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_count,
    int32_t* __restrict__ root, int32_t* __restrict__ log, int log_cap, int32_t* __restrict__ err) {
  __shared__ PathLds L;
  const int t = *d_len - n;
  tree_path(tokens, parents, n, argmax, L);
  if (t < 0) {
    if (threadIdx.x == 0) raise_error(err, kErrTrim);
    return;
  }
  const int m = L.m;
  const int have = log ? log[0] : 0;
  for (int i = threadIdx.x; i <= m; i += blockDim.x) {
    const int v = i < m ? L.tok[L.path[i]] : argmax[m ? L.path[m - 1] : 0];
    out_tokens[i] = v;
    if (log && have + i < log_cap) log[1 + have + i] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int last = argmax[m ? L.path[m - 1] : 0];
    *out_count = m + 1;
    *d_len = t + 1 + m;
    if (root) *root = last;
    if (log) {
      if (have + m + 1 > log_cap) raise_error(err, kErrOutput);
      log[0] = min(log_cap, have + m + 1);
    }
  }
}

hipError_t launch_tree_accept(const specdec_cache* c, const int32_t* tokens, const int32_t* parents, int n,
                              const int32_t* argmax, int32_t* out_tokens, int32_t* out_count, int32_t* root,
                              int32_t* log, int log_cap, int32_t* err, hipStream_t s) {
  const Dims& d = c->d;
  dim3 grid(d.L, d.nkv);
  if (d.hd == 128)
    tree_compact_kernel<128><<<grid, kAccThreads, 0, s>>>(c->kv, c->d_len, c->lp, d.nkv, tokens, parents, n, argmax);
  else
    tree_compact_kernel<64><<<grid, kAccThreads, 0, s>>>(c->kv, c->d_len, c->lp, d.nkv, tokens, parents, n, argmax);
  tree_commit_kernel<<<1, kAccThreads, 0, s>>>(c->d_len, tokens, parents, n, argmax, out_tokens, out_count, root, log,
                                               log_cap, err);
  return hipGetLastError();
}

}  // namespace sd
