// gfx950 kernels of the draft tree's greedy acceptance ("SubSpec" summary,
// jjl357.github.io, section 4.2: a tree of draft tokens verified in one
// target forward).  After a tree forward of n rows at cache length t (rows
// 0..n-1 at slots t..t+n-1, row 0 the root), the target's argmax of a row
// selects which child continues the accepted path; the path's K/V move to
// slots t+1.., the root stays at slot t, and the path's tokens plus the
// target's choice at its end are committed.
#include "internal.h"

namespace sd {

// The accepted path (rows after the root) from the rows' argmax: from the
// root, the first child in row order whose token is the current row's argmax.
// Returns its length; path[] receives the rows.
__device__ int tree_path(const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents, int n,
                         const int32_t* __restrict__ argmax, int* path) {
  int node = 0, m = 0;
  while (m < n - 1) {
    const int v = argmax[node];
    int nxt = -1;
    for (int c = node + 1; c < n; ++c)
      if (parents[c] == node && tokens[c] == v) { nxt = c; break; }
    if (nxt < 0) break;
    path[m++] = nxt;
    node = nxt;
  }
  return m;
}

// One workgroup per (layer, kv head): K rows and V^T columns of the path's
// slots are read into LDS first, then written to slots t+1.. (a destination
// may be another path row's source).
template <int HD>
__global__ __launch_bounds__(256) void tree_compact_kernel(bf16_bits* __restrict__ kv, const int32_t* __restrict__ d_len,
                                                           int lp, int nkv, const int32_t* __restrict__ tokens,
                                                           const int32_t* __restrict__ parents, int n,
                                                           const int32_t* __restrict__ argmax) {
  __shared__ int path[kMaxRows];
  __shared__ int s_m;
  __shared__ bf16_bits kbuf[kMaxRows][HD], vbuf[kMaxRows][HD];
  const int l = blockIdx.x, h = blockIdx.y;
  const int t = *d_len - n;
  if (threadIdx.x == 0) s_m = tree_path(tokens, parents, n, argmax, path);
  __syncthreads();
  const int m = s_m;
  if (t < 0 || m == 0) return;
  bf16_bits* K = kv + (size_t)l * 2 * nkv * lp * HD + (size_t)h * lp * HD;
  bf16_bits* Vt = kv + (size_t)l * 2 * nkv * lp * HD + (size_t)nkv * lp * HD + (size_t)h * HD * lp;
  for (int idx = threadIdx.x; idx < m * HD; idx += blockDim.x) {
    const int i = idx / HD, d = idx % HD, src = t + path[i];
    kbuf[i][d] = K[(size_t)src * HD + d];
    vbuf[i][d] = Vt[(size_t)d * lp + src];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < m * HD; idx += blockDim.x) {
    const int i = idx / HD, d = idx % HD, dst = t + 1 + i;
    K[(size_t)dst * HD + d] = kbuf[i][d];
    Vt[(size_t)d * lp + dst] = vbuf[i][d];
  }
}

// The commit, after the compaction has read the length: tokens, count, and
// the length t + 1 + m.
__global__ void tree_commit_kernel(int32_t* __restrict__ d_len, const int32_t* __restrict__ tokens,
                                   const int32_t* __restrict__ parents, int n, const int32_t* __restrict__ argmax,
                                   int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_count,
                                   int32_t* __restrict__ err) {
  if (threadIdx.x != 0) return;
  int path[kMaxRows];
  const int t = *d_len - n;
  if (t < 0) { raise_error(err, kErrTrim); return; }
  const int m = tree_path(tokens, parents, n, argmax, path);
  for (int i = 0; i < m; ++i) out_tokens[i] = tokens[path[i]];
  out_tokens[m] = argmax[m ? path[m - 1] : 0];
  *out_count = m + 1;
  *d_len = t + 1 + m;
}

hipError_t launch_tree_accept(const specdec_cache* c, const int32_t* tokens, const int32_t* parents, int rows,
                              const int32_t* argmax, int32_t* out_tokens, int32_t* out_count, int32_t* err,
                              hipStream_t s) {
  const Dims& d = c->d;
  dim3 grid(d.L, d.nkv);
  if (d.hd == 128)
    tree_compact_kernel<128><<<grid, 256, 0, s>>>(c->kv, c->d_len, c->lp, d.nkv, tokens, parents, rows, argmax);
  else
    tree_compact_kernel<64><<<grid, 256, 0, s>>>(c->kv, c->d_len, c->lp, d.nkv, tokens, parents, rows, argmax);
  tree_commit_kernel<<<1, 64, 0, s>>>(c->d_len, tokens, parents, rows, argmax, out_tokens, out_count, err);
  return hipGetLastError();
}

}  // namespace sd
