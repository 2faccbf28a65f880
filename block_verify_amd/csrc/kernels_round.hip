// gfx950 kernels of the speculative round's control path: draft provision,
// acceptance (greedy longest prefix or modified rejection sampling), the
// length-pointer trim of every cache, and the reset to a post-prefill
// snapshot.  All decisions stay on the device; the host never reads a
// token inside a round.
//
// Greedy rule: "SpecDec-Context-Scaling 项目解读" (richardf123.github.io),
// section 3 and section 3.1 (saved_next verifies d_1, rows[j-1] verifies
// d_(j+1), rows[k-1] only for the bonus) and section 3.2 (trim to t+m before
// the repair forward).  Stochastic rule: the wmrh.cn explainer, section 2.2,
// and "mini-infer系统实战-13" (smarter.xin), modified rejection sampling
// section (ratio min(1, p/(q+1e-10)), strict u < ratio, residual
// norm(max(0, p-q)) with a fallback to p when its mass is <= 1e-10, bonus
// from the last row on full acceptance).
#include "round_dev.h"

#include <math.h>

namespace sd {

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon et al., SC'11): 4x64-bit counter, 2x64-bit key, ten
// rounds of two 64x64->128 multiplies, key bumped by the Weyl constants.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0; k1 += W1;
  }
}

// Uniform in [0,1) from the top 24 bits of output word 0 of counter
// (round, slot, stream, 0) under key (seed, 0).
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t rnd, uint64_t slot, uint64_t stream) {
  uint64_t c[4] = {rnd, slot, stream, 0ull};
  philox4x64_10(c, seed, 0ull);
  return (float)((c[0] >> 40) & 0xFFFFFFull) * (1.0f / 16777216.0f);
}

__global__ void philox_words_kernel(const uint64_t* __restrict__ ctr, const uint64_t* __restrict__ key, int n,
                                    uint64_t* __restrict__ out) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t c[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
  philox4x64_10(c, key[2 * i], key[2 * i + 1]);
  out[4 * i] = c[0]; out[4 * i + 1] = c[1]; out[4 * i + 2] = c[2]; out[4 * i + 3] = c[3];
}

hipError_t launch_philox_words(const uint64_t* ctr, const uint64_t* key, int n, uint64_t* out, hipStream_t s) {
  philox_words_kernel<<<(n + 255) / 256, 256, 0, s>>>(ctr, key, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Round start: decide whether the round runs, lay out the verify block's
// tokens ([pending] + drafts under schedule B) from the draft table.
// ---------------------------------------------------------------------------
__global__ void round_start_kernel(RoundDev r) {
  if (threadIdx.x != 0) return;
  specdec_round_state* st = r.state;
  int open = st->n_committed < st->n_target;
  r.flags[kFlagOpen] = open;
  r.flags[kFlagRepair] = open;
  r.flags[kFlagCopySaved] = 0;
  if (!open) return;
  const int base = r.schedule == SPECDEC_SCHEDULE_B ? 1 : 0;
  if (base) r.block[0] = st->last_tok;
  if (r.draft_source == SPECDEC_DRAFT_TABLE || r.draft_source == SPECDEC_DRAFT_MODEL) {
    const int n0 = st->n_committed;
    for (int j = 0; j < r.k; ++j) {
      int idx = n0 + j, t = 0;
      if (idx < r.table_len) t = r.table[idx];
      else raise_error(r.err, kErrTable);
      r.block[base + j] = t;
    }
  } else if (r.draft_source == SPECDEC_DRAFT_Q4_SELF) {
    r.block[0] = st->saved_argmax;   // d_1 = the target's own choice (always accepted)
  }
}

// ---------------------------------------------------------------------------
// Greedy acceptance + trim (exact, or relaxed by a logit gap).
// ---------------------------------------------------------------------------
__global__ void accept_greedy_kernel(RoundDev r) {
  if (threadIdx.x != 0) return;
  if (r.flags[kFlagOpen] == 0) return;
  specdec_round_state* st = r.state;
  const int k = r.k, V = r.V;
  const bool B = r.schedule == SPECDEC_SCHEDULE_B;
  const int32_t* d = r.block + (B ? 1 : 0);
  auto v = [&](int j) -> int32_t { return B ? r.rows_argmax[j] : (j == 0 ? st->saved_argmax : r.rows_argmax[j - 1]); };
  // target logits at draft j's position
  auto row = [&](int j) -> const float* {
    return B ? r.rows_logits + (size_t)j * V : (j == 0 ? r.saved_logits : r.rows_logits + (size_t)(j - 1) * V);
  };
  auto passes = [&](int j) -> bool {
    if (r.mode != SPECDEC_RELAXED) return d[j] == v(j);
    if (d[j] < 0 || d[j] >= V) return false;
    const float* z = row(j);
    const float gap = z[v(j)] - z[d[j]];   // in fp32, as the logits are stored
    return gap <= r.relax_delta;
  };
  int m = 0;
  while (m < k && passes(m)) ++m;
  const bool emit_c = (m < k) || r.bonus;
  int n = st->n_committed;
  int32_t* toks = reinterpret_cast<int32_t*>(st + 1);
  for (int j = 0; j < m; ++j) {
    if (n < st->cap) toks[n] = d[j]; else raise_error(r.err, kErrOutput);
    ++n;
  }
  int32_t c = -1;
  if (emit_c) {
    c = v(m);
    if (n < st->cap) toks[n] = c; else raise_error(r.err, kErrOutput);
    ++n;
    st->last_tok = c;
    // the verify appended k (A) or k+1 (B) rows; keep m (A) or 1+m (B)
    *r.t_len -= (k - m);
    if (r.d_len) *r.d_len -= (k - m);
  } else {
    st->last_tok = d[k - 1];
    st->saved_argmax = r.rows_argmax[k - 1];   // rows[k-1] becomes saved_next, no repair
    st->saved_lse = r.rows_lse[k - 1];
    r.flags[kFlagCopySaved] = 1;
  }
  st->n_committed = n;
  st->m_last = m;
  st->accepted_total += m;
  st->round += 1;
  r.flags[kFlagRepair] = emit_c ? 1 : 0;
  r.repair_tok[0] = c;
}

// Copy the repair forward's argmax / lse into the state (schedule A) and, in
// stochastic mode, keep its logits as the next round's saved_next (already
// written in place by the forward).
__global__ void repair_done_kernel(RoundDev r) {
  if (threadIdx.x != 0) return;
  if (r.flags[kFlagRepair] == 0) return;
  r.state->saved_argmax = r.repair_argmax[0];
  r.state->saved_lse = r.repair_lse[0];
}

// Rewind a cache by n positions (the shared-cache draft steps are rewritten
// by the verify block).
__global__ void rewind_kernel(RoundDev r, int32_t* len, int n) {
  if (threadIdx.x != 0) return;
  if (r.flags[kFlagOpen] == 0) return;
  if (*len - n < 0) { raise_error(r.err, kErrTrim); return; }
  *len -= n;
}

// ---------------------------------------------------------------------------
// Snapshot after prefill and reset to it.
// ---------------------------------------------------------------------------
__global__ void snapshot_kernel(RoundDev r, const int32_t* d_prompt_last) {
  const int V = r.V;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < V; i += gridDim.x * blockDim.x)
    r.snap_logits[i] = r.saved_logits[i];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    r.snap[kSnapTLen] = *r.t_len;
    r.snap[kSnapDLen] = r.d_len ? *r.d_len : 0;
    r.snap[kSnapArgmax] = r.repair_argmax[0];
    r.snap[kSnapLse] = __float_as_int(r.repair_lse[0]);
    r.snap[kSnapLast] = d_prompt_last ? *d_prompt_last : -1;
  }
}

__global__ void reset_kernel(RoundDev r, int32_t n_target) {
  const int V = r.V;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < V; i += gridDim.x * blockDim.x)
    r.saved_logits[i] = r.snap_logits[i];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    specdec_round_state* st = r.state;
    st->n_committed = 0;
    st->round = 0;
    st->m_last = 0;
    st->accepted_total = 0;
    st->n_target = n_target;
    st->cap = r.state_cap;
    st->saved_argmax = r.snap[kSnapArgmax];
    st->saved_lse = __int_as_float(r.snap[kSnapLse]);
    st->last_tok = r.snap[kSnapLast];
    *r.t_len = r.snap[kSnapTLen];
    if (r.d_len) *r.d_len = r.snap[kSnapDLen];
    r.flags[kFlagOpen] = 0;
    r.flags[kFlagRepair] = 0;
  }
}

// ---------------------------------------------------------------------------
// Inverse-CDF sampling over a whole row by one workgroup of NT threads (the
// rare fallback of the residual): each thread sums a contiguous segment in
// float64 (index order), thread 0 scans the segment sums in order for the
// segment whose running total first exceeds u * total, and that segment is
// walked in index order.  Weight of entry i is wfun(i) >= 0.
// ---------------------------------------------------------------------------
template <int NT, class WF>
__device__ int block_sample(WF wfun, int V, float u, double* sh, double* total_out) {
  const int tid = threadIdx.x;
  const int seg = (V + NT - 1) / NT;
  const int i0 = tid * seg, i1 = min(V, i0 + seg);
  double s = 0.0;
  for (int i = i0; i < i1; ++i) s += (double)wfun(i);
  sh[tid] = s;
  __syncthreads();
  __shared__ int pick_seg;
  __shared__ double pick_base;
  __shared__ int picked;
  if (tid == 0) {
    double run = 0.0;
    for (int t = 0; t < NT; ++t) run += sh[t];
    double total = run;
    double target = (double)u * total;
    run = 0.0;
    int ps = NT - 1;
    double base = 0.0;
    for (int t = 0; t < NT; ++t) {
      if (run + sh[t] > target) { ps = t; base = run; break; }
      run += sh[t];
    }
    pick_seg = ps;
    pick_base = base;
    picked = -1;
    *total_out = total;
  }
  __syncthreads();
  if (tid == pick_seg) {
    double target = (double)u * (*total_out);
    double run = pick_base;
    int pk = -1, last_pos = -1;
    for (int i = i0; i < i1; ++i) {
      double wi = (double)wfun(i);
      if (wi > 0.0) last_pos = i;
      run += wi;
      if (run > target) { pk = i; break; }
    }
    if (pk < 0) pk = last_pos >= 0 ? last_pos : max(0, i1 - 1);
    picked = pk;
  }
  __syncthreads();
  int res = picked;
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------------------
// Row sampling spread over the chip.  A row of V entries is cut into slices
// of kSliceElems; one 256-thread workgroup per slice.
//   stats:   slice max and sum of exp(x - slice max) (noisy draft rows only,
//            which also writes x = z + noise);
//   weights: log-sum-exp of the row from the slice stats (every workgroup
//            combines them in slice order), then the float64 sum of the
//            slice's sampling weights;
//   select:  one workgroup scans the slice sums in order for u * total,
//            then walks the chosen slice with a prefix sum.
// Orders are fixed by index, so the result does not depend on timing.
// ---------------------------------------------------------------------------
constexpr int kSliceThreads = 256;
constexpr int kPerThread = kSliceElems / kSliceThreads;

template <typename T>
__device__ __forceinline__ T block_reduce_256(T v, T* sh, bool is_max) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int s2 = kSliceThreads / 2; s2 > 0; s2 >>= 1) {
    if (t < s2) sh[t] = is_max ? (sh[t] > sh[t + s2] ? sh[t] : sh[t + s2]) : sh[t] + sh[t + s2];
    __syncthreads();
  }
  T r = sh[0];
  __syncthreads();
  return r;
}

// Weight modes of the sampler (kWNone: the round draws no last token).
enum { kWDraft = 0, kWResidual = 1, kWTarget = 2, kWNone = 3 };

// Noisy self-draft, step j: x = z + noise[n0 + j] into q_logits[j]; slice
// stats of x / T.
__global__ __launch_bounds__(kSliceThreads) void draft_stats_kernel(RoundDev r, const float* __restrict__ z, int j) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ float shf[kSliceThreads];
  const int V = r.V, sl = blockIdx.x;
  const int row = r.state->n_committed + j;
  const bool ok = row < r.noise_rows;
  if (!ok && sl == 0 && threadIdx.x == 0) raise_error(r.err, kErrTable);
  const float* nz = r.noise + (size_t)(ok ? row : 0) * V;
  float* qz = r.q_logits + (size_t)j * V;
  float xv[kPerThread];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = sl * kSliceElems + e * kSliceThreads + threadIdx.x;
    xv[e] = -INFINITY;
    if (i < V) {
      const float x = z[i] + nz[i];
      qz[i] = x;
      xv[e] = x * r.inv_t;
    }
    mx = fmaxf(mx, xv[e]);
  }
  mx = block_reduce_256(mx, shf, true);
  float se = 0.f;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) se += (xv[e] == -INFINITY) ? 0.f : expf(xv[e] - mx);
  se = block_reduce_256(se, shf, false);
  if (threadIdx.x == 0) { r.smax[sl] = mx; r.ssum[sl] = se; }
}

// log-sum-exp of a row from its S slice stats (slice order; same value in every workgroup).
__device__ float combine_lse(const float* smax, const float* ssum, int S, float* shf) {
  float mx = -INFINITY;
  for (int s2 = threadIdx.x; s2 < S; s2 += kSliceThreads) mx = fmaxf(mx, smax[s2]);
  mx = block_reduce_256(mx, shf, true);
  float l = 0.f;
  for (int s2 = threadIdx.x; s2 < S; s2 += kSliceThreads) l += ssum[s2] * expf(smax[s2] - mx);
  l = block_reduce_256(l, shf, false);
  return mx + logf(l);
}

// Tempered target rows (temperature != 1): slice stats of z / T for row 0
// (saved_next) and rows 1..k (the verify rows), then each row's log-sum-exp.
__global__ __launch_bounds__(kSliceThreads) void tempered_stats_kernel(RoundDev r) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ float shf[kSliceThreads];
  const int V = r.V, sl = blockIdx.x, row = blockIdx.y, S = gridDim.x;
  const float* z = row == 0 ? r.saved_logits : r.rows_logits + (size_t)(row - 1) * V;
  float xv[kPerThread];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = sl * kSliceElems + e * kSliceThreads + threadIdx.x;
    xv[e] = i < V ? z[i] * r.inv_t : -INFINITY;
    mx = fmaxf(mx, xv[e]);
  }
  mx = block_reduce_256(mx, shf, true);
  float se = 0.f;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) se += (xv[e] == -INFINITY) ? 0.f : expf(xv[e] - mx);
  se = block_reduce_256(se, shf, false);
  if (threadIdx.x == 0) { r.tsmax[row * S + sl] = mx; r.tssum[row * S + sl] = se; }
}

__global__ __launch_bounds__(kSliceThreads) void tempered_lse_kernel(RoundDev r, int S) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ float shf[kSliceThreads];
  const int row = blockIdx.x;
  const float l = combine_lse(r.tsmax + row * S, r.tssum + row * S, S, shf);
  if (threadIdx.x == 0) r.t_lse[row] = l;
}

// The sampling weight of entry i for the current mode, as an fp32 value
// (every kernel that needs it computes it the same way).
struct SampleRows {
  const float* lp; float lp_lse;   // target row (residual / bonus)
  const float* lq; float lq_lse;   // draft row (draft sample / residual)
  float inv_t;                     // 1 / temperature
  uint64_t thresh;                 // truncation: entries whose key is below are dropped (0: none)
  int mode;
};
__device__ __forceinline__ float raw_weight(const SampleRows& w, int i) {
  if (w.mode == kWDraft) return expf(w.lq[i] * w.inv_t - w.lq_lse);
  if (w.mode == kWTarget) return expf(w.lp[i] * w.inv_t - w.lp_lse);
  return fmaxf(0.f, expf(w.lp[i] * w.inv_t - w.lp_lse) - expf(w.lq[i] * w.inv_t - w.lq_lse));
}
__device__ __forceinline__ uint64_t trunc_key(float wv, int i) {
  return ((uint64_t)__float_as_uint(wv) << kKeyIndexBits) | (uint64_t)((1 << kKeyIndexBits) - 1 - i);
}
__device__ __forceinline__ double sample_weight(const SampleRows& w, int i) {
  const float v = raw_weight(w, i);
  if (w.thresh != 0 && trunc_key(v, i) < w.thresh) return 0.0;
  return (double)v;
}

// The accept step's sampling rows for accepted count m and weight mode:
// target row m (saved_next for m = 0), draft row m (residual only).
__device__ SampleRows accept_rows(const RoundDev& r, int m, int mode, uint64_t thresh) {
  const specdec_round_state* st = r.state;
  const bool tempered = r.inv_t != 1.0f;
  SampleRows w;
  w.lp = m == 0 ? r.saved_logits : r.rows_logits + (size_t)(m - 1) * r.V;
  w.lp_lse = tempered ? r.t_lse[m] : (m == 0 ? st->saved_lse : r.rows_lse[m - 1]);
  w.lq = r.q_logits + (size_t)(m < r.k ? m : 0) * r.V;
  w.lq_lse = r.q_lse[m < r.k ? m : 0];
  w.inv_t = r.inv_t;
  w.thresh = thresh;
  w.mode = mode;
  return w;
}

// Slice sums of the sampling weights.  j >= 0: draft step j (log-sum-exp of
// the noisy row first, stored in q_lse[j]); j < 0: the accept step's row and
// mode from sctl, truncated when `masked`.
__global__ __launch_bounds__(kSliceThreads) void slice_weights_kernel(RoundDev r, int j, int masked) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ float shf[kSliceThreads];
  __shared__ double shd[kSliceThreads];
  const int V = r.V, sl = blockIdx.x;
  SampleRows w;
  if (j >= 0) {
    const float lse = combine_lse(r.smax, r.ssum, gridDim.x, shf);
    if (sl == 0 && threadIdx.x == 0) r.q_lse[j] = lse;
    w.lq = r.q_logits + (size_t)j * V;
    w.lq_lse = lse;
    w.lp = nullptr; w.lp_lse = 0.f;
    w.inv_t = r.inv_t;
    w.thresh = 0;
    w.mode = kWDraft;
  } else {
    if (r.sctl[1] == kWNone) return;
    w = accept_rows(r, r.sctl[0], r.sctl[1], masked ? r.trunc->thresh : 0);
  }
  double acc = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = sl * kSliceElems + e * kSliceThreads + threadIdx.x;
    if (i < V) acc += sample_weight(w, i);
  }
  acc = block_reduce_256(acc, shd, false);
  if (threadIdx.x == 0) r.sw[sl] = acc;
}

// Inverse CDF over the slice sums: the smallest index whose running weight
// exceeds u * total.  Returns -1 when the total is not above `floor`.
__device__ int select_index(const RoundDev& r, const SampleRows& w, int S, float u, double floor_total,
                            double* shd, int* shi) {
  __shared__ int s_pick;
  __shared__ double s_base, s_target;
  const int t = threadIdx.x;
  if (t == 0) {
    double total = 0.0;
    for (int s2 = 0; s2 < S; ++s2) total += r.sw[s2];
    const double target = (double)u * total;
    double run = 0.0;
    int ps = -1;
    if (total > floor_total) {
      ps = S - 1;
      for (int s2 = 0; s2 < S; ++s2) {
        if (run + r.sw[s2] > target) { ps = s2; break; }
        run += r.sw[s2];
      }
    }
    s_pick = ps;
    s_base = run;
    s_target = target;
  }
  __syncthreads();
  const int ps = s_pick;
  if (ps < 0) return -1;
  // inclusive prefix sum of the chosen slice, element order
  double v[kPerThread];
  double own = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = ps * kSliceElems + t * kPerThread + e;
    v[e] = i < r.V ? sample_weight(w, i) : 0.0;
    own += v[e];
  }
  shd[t] = own;
  __syncthreads();
  for (int off = 1; off < kSliceThreads; off <<= 1) {   // Hillis-Steele scan of thread totals
    const double add = t >= off ? shd[t - off] : 0.0;
    __syncthreads();
    shd[t] += add;
    __syncthreads();
  }
  double run = s_base + (t > 0 ? shd[t - 1] : 0.0);
  int hit = 0x7fffffff, last = -1;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = ps * kSliceElems + t * kPerThread + e;
    if (v[e] > 0.0) last = i;
    run += v[e];
    if (hit == 0x7fffffff && run > s_target && v[e] > 0.0) hit = i;
  }
  shi[t] = hit;
  __syncthreads();
  for (int s2 = kSliceThreads / 2; s2 > 0; s2 >>= 1) {
    if (t < s2) shi[t] = min(shi[t], shi[t + s2]);
    __syncthreads();
  }
  int pick = shi[0];
  __syncthreads();
  if (pick == 0x7fffffff) {   // rounding left u * total past the walked slice: its last positive entry
    shi[t] = last;
    __syncthreads();
    for (int s2 = kSliceThreads / 2; s2 > 0; s2 >>= 1) {
      if (t < s2) shi[t] = max(shi[t], shi[t + s2]);
      __syncthreads();
    }
    pick = shi[0] >= 0 ? shi[0] : ps * kSliceElems;
    __syncthreads();
  }
  return pick;
}

// Draft step j: the sampled token goes into the verify block.
__global__ __launch_bounds__(kSliceThreads) void draft_select_kernel(RoundDev r, int j) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ double shd[kSliceThreads];
  __shared__ int shi[kSliceThreads];
  SampleRows w;
  w.lq = r.q_logits + (size_t)j * r.V;
  w.lq_lse = r.q_lse[j];
  w.lp = nullptr; w.lp_lse = 0.f;
  w.inv_t = r.inv_t;
  w.thresh = 0;
  w.mode = kWDraft;
  const float u = philox_uniform(r.seed, (uint64_t)r.state->round, (uint64_t)j, 0);
  const int tok = select_index(r, w, n_slices(r.V), u, -1.0, shd, shi);
  if (threadIdx.x == 0) r.block[j] = tok;
}

// Modified rejection sampling over the k drafts of the round (schedule A):
// p_1 = softmax(saved_next / T), p_(j+1) = softmax(rows[j] / T), q_j as drawn.
// Decides m (accept while u_j < min(1, p_j(d_j) / (q_j(d_j) + 1e-10))) and
// which row the last token is drawn from: the residual of row m, the bonus
// row, or none (full acceptance without the bonus).
__global__ void accept_decide_kernel(RoundDev r) {
  if (r.flags[kFlagOpen] == 0) return;
  if (threadIdx.x != 0) return;
  specdec_round_state* st = r.state;
  const int k = r.k, V = r.V;
  const bool tempered = r.inv_t != 1.0f;
  int m = 0;
  for (; m < k; ++m) {
    const float* lp = m == 0 ? r.saved_logits : r.rows_logits + (size_t)(m - 1) * V;
    const float lp_lse = tempered ? r.t_lse[m] : (m == 0 ? st->saved_lse : r.rows_lse[m - 1]);
    const float* lq = r.q_logits + (size_t)m * V;
    const int x = r.block[m];
    const float px = expf(lp[x] * r.inv_t - lp_lse), qx = expf(lq[x] * r.inv_t - r.q_lse[m]);
    const float ratio = fminf(1.0f, px / (qx + 1e-10f));
    const float ua = philox_uniform(r.seed, (uint64_t)st->round, (uint64_t)m, 1);
    if (r.dbg) { r.dbg[2 * m] = ratio; r.dbg[2 * m + 1] = ua; }
    if (!(ua < ratio)) break;
  }
  const int mode = m < k ? kWResidual : (r.bonus ? kWTarget : kWNone);
  r.sctl[0] = m;
  r.sctl[1] = mode;
  TruncState* ts = r.trunc;
  ts->prefix = 0;
  ts->need = 0;
  ts->target = 0;
  ts->kthresh = 0;
  ts->thresh = 0;
  ts->active = mode != kWNone;
}

// Truncation, first step: the untruncated total decides the residual's
// fallback to p (mass <= 1e-10) before anything is cut.
__global__ void trunc_begin_kernel(RoundDev r, int S) {
  if (r.flags[kFlagOpen] == 0) return;
  if (threadIdx.x != 0 || r.sctl[1] == kWNone) return;
  double total = 0.0;
  for (int s2 = 0; s2 < S; ++s2) total += r.sw[s2];
  if (r.sctl[1] == kWResidual && !(total > 1e-10)) r.sctl[1] = kWTarget;
}

// Radix-select pass `pass` of stage `stage` (0: top-k by count, 1: top-p by
// mass): per-slice histograms of the current key digit over the candidates
// (keys that match the resolved prefix; in the top-p stage also at or above
// the top-k threshold).  Counts and fixed-point masses are integer LDS
// atomics, exact in any order.
__device__ __forceinline__ uint64_t mass_fixed(float w) { return (uint64_t)((double)w * kMassScale); }

__global__ __launch_bounds__(kSliceThreads) void trunc_hist_kernel(RoundDev r, int pass, int stage) {
  if (r.flags[kFlagOpen] == 0 || r.trunc->active == 0 || (pass > 0 && r.trunc->done)) return;
  __shared__ int hc[kTruncBins];
  __shared__ unsigned long long hm[kTruncBins];
  const int V = r.V, sl = blockIdx.x, t = threadIdx.x;
  hc[t] = 0;
  hm[t] = 0ull;
  const TruncState& ts = *r.trunc;
  const SampleRows w = accept_rows(r, r.sctl[0], r.sctl[1], 0);
  const int shift = 8 * (kTruncPasses - 1 - pass), hi = shift + 8;
  const uint64_t prefix = ts.prefix, kth = stage == 1 ? ts.kthresh : 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = sl * kSliceElems + e * kSliceThreads + t;
    if (i < V) {
      const float v = raw_weight(w, i);
      const uint64_t key = trunc_key(v, i);
      if ((key >> hi) == (prefix >> hi) && key >= kth) {
        const int d = (int)((key >> shift) & 0xFF);
        atomicAdd(&hc[d], 1);
        if (stage == 1) atomicAdd(&hm[d], (unsigned long long)mass_fixed(v));
      }
    }
  }
  __syncthreads();
  r.hcnt[sl * kTruncBins + t] = hc[t];
  r.hmass[sl * kTruncBins + t] = hm[t];
}

// Radix-select resolve: bins summed over slices (integers: any order); the
// digit whose bin holds the top_k-th largest key (stage 0) or where the
// running mass from the top reaches top_p of the candidates' mass (stage 1).
constexpr int kResolveThreads = 1024, kResolveParts = kResolveThreads / kTruncBins;
__global__ __launch_bounds__(kResolveThreads) void trunc_resolve_kernel(RoundDev r, int pass, int stage, int S) {
  if (r.flags[kFlagOpen] == 0 || r.trunc->active == 0 || (pass > 0 && r.trunc->done)) return;
  __shared__ long long pc[kResolveParts][kTruncBins];
  __shared__ unsigned long long pm[kResolveParts][kTruncBins];
  const int b = threadIdx.x % kTruncBins, part = threadIdx.x / kTruncBins;
  long long c = 0;
  unsigned long long ms = 0;
  for (int s2 = part; s2 < S; s2 += kResolveParts) {
    c += r.hcnt[s2 * kTruncBins + b];
    ms += r.hmass[s2 * kTruncBins + b];
  }
  pc[part][b] = c;
  pm[part][b] = ms;
  __syncthreads();
  __shared__ long long bc[kTruncBins];
  __shared__ unsigned long long bm[kTruncBins];
  if (threadIdx.x < kTruncBins) {
    long long cc = 0;
    unsigned long long mm = 0;
    for (int q = 0; q < kResolveParts; ++q) { cc += pc[q][b]; mm += pm[q][b]; }
    bc[b] = cc;
    bm[b] = mm;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  TruncState& ts = *r.trunc;
  const int shift = 8 * (kTruncPasses - 1 - pass);
  if (pass == 0) {
    ts.prefix = 0;
    ts.done = 0;
    if (stage == 0) {
      ts.need = r.top_k;
    } else {
      unsigned long long total = 0;
      for (int i = 0; i < kTruncBins; ++i) total += bm[i];
      ts.target = (uint64_t)((double)r.top_p * (double)total);
    }
  }
  int digit = -1;
  if (stage == 0) {
    long long cum = 0;
    for (int i = kTruncBins - 1; i >= 0; --i) {
      if (cum + bc[i] >= ts.need) { digit = i; ts.need -= cum; break; }
      cum += bc[i];
    }
  } else {
    unsigned long long cum = 0;
    for (int i = kTruncBins - 1; i >= 0; --i) {
      if (bc[i] > 0 && cum + bm[i] >= ts.target) { digit = i; ts.target -= cum; break; }
      cum += bm[i];
    }
  }
  if (digit < 0) {   // the target lies in entries of zero mass: keep every candidate
    for (int i = 0; i < kTruncBins; ++i)
      if (bc[i] > 0) { digit = i; break; }
    if (stage == 1) ts.target = 0;
  }
  if (digit < 0) digit = 0;
  ts.prefix |= (uint64_t)digit << shift;
  // Settled early when every candidate left in the chosen bin is kept: the
  // lowest key with this prefix is then the threshold (top-k: the bin's count
  // is what is still needed; top-p: the bin holds one entry, the last one the
  // shortest run takes).
  const bool settled = stage == 0 ? bc[digit] == ts.need : bc[digit] == 1;
  if (settled || pass == kTruncPasses - 1) {
    ts.done = 1;
    ts.thresh = ts.prefix;
    if (stage == 0) ts.kthresh = ts.prefix;
  }
}

// The resample (or bonus) and the commit: tokens, lengths, repair token.
__global__ __launch_bounds__(kSliceThreads) void accept_select_kernel(RoundDev r, int truncated) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ double shd[kSliceThreads];
  __shared__ int shi[kSliceThreads];
  __shared__ double total;
  specdec_round_state* st = r.state;
  const int k = r.k, m = r.sctl[0], mode = r.sctl[1];
  const float ur = philox_uniform(r.seed, (uint64_t)st->round, 0, 2);
  int c = -1;
  if (mode != kWNone) {
    if (truncated) {
      c = select_index(r, accept_rows(r, m, mode, r.trunc->thresh), n_slices(r.V), ur, -1.0, shd, shi);
    } else {
      c = select_index(r, accept_rows(r, m, mode, 0), n_slices(r.V), ur, mode == kWResidual ? 1e-10 : -1.0, shd,
                       shi);
      if (c < 0) {   // residual mass <= 1e-10: sample p of that row (one workgroup, rare)
        const SampleRows wp = accept_rows(r, m, kWTarget, 0);
        c = block_sample<kSliceThreads>([&](int i) { return sample_weight(wp, i); }, r.V, ur, shd, &total);
      }
    }
  }
  if (threadIdx.x == 0) {
    int n = st->n_committed;
    int32_t* toks = reinterpret_cast<int32_t*>(st + 1);
    for (int j = 0; j < m; ++j) {
      if (n < st->cap) toks[n] = r.block[j]; else raise_error(r.err, kErrOutput);
      ++n;
    }
    if (mode != kWNone) {
      if (n < st->cap) toks[n] = c; else raise_error(r.err, kErrOutput);
      ++n;
      st->last_tok = c;
      *r.t_len -= (k - m);
      r.flags[kFlagRepair] = 1;
    } else {
      // all k drafts kept, no bonus: the cache keeps them, the last verify
      // row becomes saved_next and no repair forward runs
      st->last_tok = r.block[k - 1];
      st->saved_argmax = r.rows_argmax[k - 1];
      st->saved_lse = r.rows_lse[k - 1];
      r.flags[kFlagRepair] = 0;
      r.flags[kFlagCopySaved] = 1;
    }
    st->n_committed = n;
    st->m_last = m;
    st->accepted_total += m;
    st->round += 1;
    r.repair_tok[0] = c;
    if (r.dbg) { r.dbg[2 * kMaxK] = ur; r.dbg[2 * kMaxK + 1] = __int_as_float(m); }
  }
}

// saved_next = the last verify row (a fully accepted round without bonus).
__global__ void copy_saved_kernel(RoundDev r) {
  if (r.flags[kFlagOpen] == 0 || r.flags[kFlagCopySaved] == 0) return;
  const float* src = r.rows_logits + (size_t)(r.k - 1) * r.V;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < r.V; i += gridDim.x * blockDim.x) r.saved_logits[i] = src[i];
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
hipError_t launch_round_start(const RoundDev& r, hipStream_t s) { round_start_kernel<<<1, 64, 0, s>>>(r); return hipGetLastError(); }
hipError_t launch_accept_greedy(const RoundDev& r, hipStream_t s) { accept_greedy_kernel<<<1, 64, 0, s>>>(r); return hipGetLastError(); }
hipError_t launch_repair_done(const RoundDev& r, hipStream_t s) { repair_done_kernel<<<1, 64, 0, s>>>(r); return hipGetLastError(); }
hipError_t launch_rewind(const RoundDev& r, int32_t* len, int n, hipStream_t s) { rewind_kernel<<<1, 64, 0, s>>>(r, len, n); return hipGetLastError(); }
hipError_t launch_snapshot(const RoundDev& r, const int32_t* last, hipStream_t s) { snapshot_kernel<<<64, 256, 0, s>>>(r, last); return hipGetLastError(); }
hipError_t launch_reset(const RoundDev& r, int32_t n_target, hipStream_t s) { reset_kernel<<<64, 256, 0, s>>>(r, n_target); return hipGetLastError(); }
hipError_t launch_copy_saved(const RoundDev& r, hipStream_t s) { copy_saved_kernel<<<64, 256, 0, s>>>(r); return hipGetLastError(); }
hipError_t launch_draft_sample(const RoundDev& r, const float* z, int j, hipStream_t s) {
  const int S = n_slices(r.V);
  draft_stats_kernel<<<S, kSliceThreads, 0, s>>>(r, z, j);
  slice_weights_kernel<<<S, kSliceThreads, 0, s>>>(r, j, 0);
  draft_select_kernel<<<1, kSliceThreads, 0, s>>>(r, j);
  return hipGetLastError();
}
hipError_t launch_accept_stochastic(const RoundDev& r, hipStream_t s) {
  const int S = n_slices(r.V);
  if (r.inv_t != 1.0f) {
    tempered_stats_kernel<<<dim3(S, r.k + 1), kSliceThreads, 0, s>>>(r);
    tempered_lse_kernel<<<r.k + 1, kSliceThreads, 0, s>>>(r, S);
  }
  accept_decide_kernel<<<1, 64, 0, s>>>(r);
  slice_weights_kernel<<<S, kSliceThreads, 0, s>>>(r, -1, 0);
  const bool tk = r.top_k > 0 && r.top_k < r.V, tp = r.top_p < 1.0f;
  if (tk || tp) {
    trunc_begin_kernel<<<1, 64, 0, s>>>(r, S);
    for (int stage = tk ? 0 : 1; stage <= (tp ? 1 : 0); ++stage)
      for (int pass = 0; pass < kTruncPasses; ++pass) {
        trunc_hist_kernel<<<S, kSliceThreads, 0, s>>>(r, pass, stage);
        trunc_resolve_kernel<<<1, kResolveThreads, 0, s>>>(r, pass, stage, S);
      }
    slice_weights_kernel<<<S, kSliceThreads, 0, s>>>(r, -1, 1);
  }
  accept_select_kernel<<<1, kSliceThreads, 0, s>>>(r, (tk || tp) ? 1 : 0);
  return hipGetLastError();
}

}  // namespace sd
