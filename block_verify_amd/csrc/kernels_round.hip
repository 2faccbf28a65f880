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
// Greedy acceptance + trim.
// ---------------------------------------------------------------------------
__global__ void accept_greedy_kernel(RoundDev r) {
  if (threadIdx.x != 0) return;
  if (r.flags[kFlagOpen] == 0) return;
  specdec_round_state* st = r.state;
  const int k = r.k;
  const bool B = r.schedule == SPECDEC_SCHEDULE_B;
  const int32_t* d = r.block + (B ? 1 : 0);
  auto v = [&](int j) -> int32_t { return B ? r.rows_argmax[j] : (j == 0 ? st->saved_argmax : r.rows_argmax[j - 1]); };
  int m = 0;
  while (m < k && d[m] == v(m)) ++m;
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
// Inverse-CDF sampling over one vocabulary row with 1024 threads: each
// thread sums a contiguous segment in float64 (index order), a fixed-order
// scan of the segment sums locates the segment whose running total first
// exceeds u * total, and that segment is walked in index order.
// Weight of entry i is wfun(i) >= 0.
// ---------------------------------------------------------------------------
constexpr int kSampleThreads = 1024;

template <class WF>
__device__ int block_sample(WF wfun, int V, float u, double* sh, double* total_out) {
  const int tid = threadIdx.x;
  const int seg = (V + kSampleThreads - 1) / kSampleThreads;
  const int i0 = tid * seg, i1 = min(V, i0 + seg);
  double s = 0.0;
  for (int i = i0; i < i1; ++i) s += (double)wfun(i);
  sh[tid] = s;
  __syncthreads();
  // inclusive scan of segment sums, thread 0 walks them in order
  __shared__ int pick_seg;
  __shared__ double pick_base;
  __shared__ int picked;
  if (tid == 0) {
    double run = 0.0;
    for (int t = 0; t < kSampleThreads; ++t) run += sh[t];
    double total = run;
    double target = (double)u * total;
    run = 0.0;
    int ps = kSampleThreads - 1;
    double base = 0.0;
    for (int t = 0; t < kSampleThreads; ++t) {
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

// Block-wide max and sum-exp (fixed tree) of a row; returns lse.
__device__ float block_lse(const float* __restrict__ row, const float* __restrict__ add, int V, float* shf) {
  const int tid = threadIdx.x;
  float mx = -INFINITY;
  for (int i = tid; i < V; i += blockDim.x) mx = fmaxf(mx, row[i] + (add ? add[i] : 0.f));
  shf[tid] = mx;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if (tid < s) shf[tid] = fmaxf(shf[tid], shf[tid + s]);
    __syncthreads();
  }
  mx = shf[0];
  __syncthreads();
  float se = 0.f;
  for (int i = tid; i < V; i += blockDim.x) se += expf(row[i] + (add ? add[i] : 0.f) - mx);
  shf[tid] = se;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if (tid < s) shf[tid] += shf[tid + s];
    __syncthreads();
  }
  float lse = mx + logf(shf[0]);
  __syncthreads();
  return lse;
}

// Noisy self-draft, step j: q_j = softmax(z_j + noise[n0 + j]); stores the
// noisy logits and their lse, draws d_j with the draft stream of Philox and
// writes it into the verify block.
__global__ __launch_bounds__(kSampleThreads) void draft_sample_kernel(RoundDev r, const float* __restrict__ z, int j) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ double shd[kSampleThreads];
  __shared__ float shf[kSampleThreads];
  __shared__ double total;
  const int V = r.V;
  specdec_round_state* st = r.state;
  const int row = st->n_committed + j;
  const bool ok = row < r.noise_rows;
  if (!ok && threadIdx.x == 0) raise_error(r.err, kErrTable);
  const float* nz = r.noise + (size_t)(ok ? row : 0) * V;
  float* qz = r.q_logits + (size_t)j * V;
  for (int i = threadIdx.x; i < V; i += blockDim.x) qz[i] = z[i] + nz[i];
  __syncthreads();
  float lse = block_lse(qz, nullptr, V, shf);
  float u = philox_uniform(r.seed, (uint64_t)st->round, (uint64_t)j, 0);
  int tok = block_sample([&](int i) { return expf(qz[i] - lse); }, V, u, shd, &total);
  if (threadIdx.x == 0) {
    r.q_lse[j] = lse;
    r.block[j] = tok;
  }
}

// Modified rejection sampling over the k drafts of the round (schedule A):
// p_1 = softmax(saved_next), p_(j+1) = softmax(rows[j]), q_j as drawn.
__global__ __launch_bounds__(kSampleThreads) void accept_stochastic_kernel(RoundDev r) {
  if (r.flags[kFlagOpen] == 0) return;
  __shared__ double shd[kSampleThreads];
  __shared__ double total;
  specdec_round_state* st = r.state;
  const int k = r.k, V = r.V;
  const int32_t* d = r.block;
  auto prow = [&](int j) -> const float* { return j == 0 ? r.saved_logits : r.rows_logits + (size_t)(j - 1) * V; };
  auto plse = [&](int j) -> float { return j == 0 ? st->saved_lse : r.rows_lse[j - 1]; };
  const float ur = philox_uniform(r.seed, (uint64_t)st->round, 0, 2);
  int m = 0;
  int c = -1;
  for (; m < k; ++m) {
    const float* lp = prow(m);
    const float lp_lse = plse(m);
    const float* lq = r.q_logits + (size_t)m * V;
    const float lq_lse = r.q_lse[m];
    const int x = d[m];
    float px = expf(lp[x] - lp_lse), qx = expf(lq[x] - lq_lse);
    float ratio = fminf(1.0f, px / (qx + 1e-10f));
    float ua = philox_uniform(r.seed, (uint64_t)st->round, (uint64_t)m, 1);
    if (threadIdx.x == 0 && r.dbg) { r.dbg[2 * m] = ratio; r.dbg[2 * m + 1] = ua; }
    if (ua < ratio) continue;
    // first rejection: residual norm(max(0, p - q)), fallback to p
    auto wres = [&](int i) { return fmaxf(0.f, expf(lp[i] - lp_lse) - expf(lq[i] - lq_lse)); };
    c = block_sample(wres, V, ur, shd, &total);
    if (!(total > 1e-10)) c = block_sample([&](int i) { return expf(lp[i] - lp_lse); }, V, ur, shd, &total);
    break;
  }
  if (m == k) {
    const float* lp = prow(k);
    const float lp_lse = plse(k);
    c = block_sample([&](int i) { return expf(lp[i] - lp_lse); }, V, ur, shd, &total);
  }
  if (threadIdx.x == 0) {
    int n = st->n_committed;
    int32_t* toks = reinterpret_cast<int32_t*>(st + 1);
    for (int j = 0; j < m; ++j) {
      if (n < st->cap) toks[n] = d[j]; else raise_error(r.err, kErrOutput);
      ++n;
    }
    if (n < st->cap) toks[n] = c; else raise_error(r.err, kErrOutput);
    ++n;
    st->n_committed = n;
    st->m_last = m;
    st->accepted_total += m;
    st->last_tok = c;
    st->round += 1;
    *r.t_len -= (k - m);
    r.flags[kFlagRepair] = 1;
    r.repair_tok[0] = c;
    if (r.dbg) { r.dbg[2 * kMaxK] = ur; r.dbg[2 * kMaxK + 1] = __int_as_float(m); }
  }
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
hipError_t launch_draft_sample(const RoundDev& r, const float* z, int j, hipStream_t s) {
  draft_sample_kernel<<<1, kSampleThreads, 0, s>>>(r, z, j);
  return hipGetLastError();
}
hipError_t launch_accept_stochastic(const RoundDev& r, hipStream_t s) {
  accept_stochastic_kernel<<<1, kSampleThreads, 0, s>>>(r);
  return hipGetLastError();
}

}  // namespace sd
