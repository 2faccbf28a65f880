// Pieces shared by the skinny-product kernels (bf16 MFMA and 4-bit):
// parameters, query operand tiles, the RMSNorm scale and the epilogues.
#pragma once

#include "internal.h"

#include <math.h>

namespace sd {

enum class Epi { QKV, RESID, SWIGLU, LMHEAD, PARTIAL };

// Row order of the packed linears (see PackKind).
__device__ __forceinline__ void pack_row_slot(int kind, int r, int hd, int& g, int& i) {
  if (kind == PACK_PLAIN) {
    g = r >> 4; i = r & 15;
  } else if (kind == PACK_ROPE) {
    int head = r / hd, d = r % hd, half = hd >> 1;
    int per_head = hd >> 4;
    if (d < half) { g = head * per_head + (d >> 3); i = d & 7; }
    else { g = head * per_head + ((d - half) >> 3); i = 8 + ((d - half) & 7); }
  } else if (kind == PACK_GATE) {
    g = r >> 3; i = r & 7;
  } else {
    g = r >> 3; i = 8 + (r & 7);
  }
}

struct GemvParams {
  const bf16x8_t* A;     // weight tiles
  const bf16x8_t* B;     // activation tiles
  int KB;                // k-blocks of 32 inputs
  int n_groups;          // 16-row output groups
  int rows;              // activation rows M
  const int32_t* gate;
  int32_t* err;
  // norm (QKV, SWIGLU, LMHEAD): r from ss partials
  const float* ss_in;
  int H;
  float eps;
  // QKV
  bf16_bits* qb;         // query operand tiles per kv head
  bf16_bits* k_cache;
  bf16_bits* v_cache;
  const float2* rope;
  const int32_t* d_len;
  int max_len;           // cache capacity (positions)
  const int32_t* tree_depth;   // tree forward: per row, its RoPE position minus pos0 (a depth offset), else null
  int kv_stride;         // padded positions per head (K rows; V^T row length)
  int nq, nkv, hd;
  // RESID
  float* x;
  const float* gain_next;
  bf16_bits* xb_out;
  float* ss_out;
  // SWIGLU
  bf16_bits* hb_out;
  int F;
  // LMHEAD
  float* logits;
  int V;
  float* lm_part;        // [rows][gridDim.x][3]
  // PARTIAL (split-K): [nsplit][kMaxRows][H] (value, tag) pairs of the
  // splits' partial outputs and one launch sequence number per row group;
  // the last split sums the others' values and runs the RESID epilogue
  float* part;
  int nsplit;
  int32_t* cnt;
};

// Stores and loads that bypass the non-coherent per-XCD caches (agent
// scope), for values one workgroup hands to another inside one launch.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Reads of such values: buffer loads with the sc1 cache policy (the same
// coherence as agent-scope atomic loads, but ordinary loads the compiler
// may issue back to back).  The descriptor covers 2 GiB from `base`; its
// only user, the split-K partial buffer, is bounded below (byte offsets are
// 32-bit and must stay under the record count).
typedef __amdgpu_buffer_rsrc_t agent_rsrc_t;
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ agent_rsrc_t agent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ float load_agent(agent_rsrc_t r, size_t index) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)(index * 4), 0, kCpolSc1));
}
// 64-bit (value, tag) words: one store and one load each, so a reader sees
// both halves of one write (naturally aligned 8-byte accesses).
__device__ __forceinline__ void store_agent_pair(float* p, float v, uint32_t tag) {
  const uint64_t w = (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t load_agent_pair(agent_rsrc_t r, size_t index) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (uint32_t)(index * 8), 0, kCpolSc1);
}
constexpr int kHandoffSpins = 1 << 18;   // bound of a finisher's wait for one value
static_assert((long long)kMaxSplit * kMaxRows * kMaxHidden * 8 < 0x7FFFFFFFLL,
              "split-K partials must fit one 2 GiB buffer descriptor");

// Wait until this wave's outstanding vector memory operations completed.
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

// Epilogue operands that do not depend on the product: the residual rows
// and next-norm gains (RESID, PARTIAL) and the RoPE rotations and cache
// position of the query/key groups (QKV).  The epilogue wave requests them
// while its weight tiles are in flight, so the epilogue waits on no load of
// its own.  Lane l holds entry idx = l + 64 j of the epilogue's loops.
// Sized for the NC activation rows a launch shape covers (NC = 8 per
// operand tile), so a one-tile pass holds a few registers only.
template <int NC>
struct EpiPre {
  static constexpr int kX = (16 * NC + 63) / 64;   // residual values per lane
  static constexpr int kR = (8 * NC + 63) / 64;    // RoPE pairs per lane
  float xv[kX];
  float gain;
  float2 cs[kR];
  int pos0;
  uint32_t seq;   // PARTIAL: the row group's launch sequence number before this launch
};

// RESID / PARTIAL: x[m][16 g + i] for idx = 16 m + i, and gain_next[16 g + i]
// (i = lane % 16 for every j).  Row group g owns these x entries for the
// whole launch, so reading them before the product is safe.
template <Epi E, int NC>
__device__ __forceinline__ void epi_prefetch_x(const GemvParams& p, int lane, int g, int M, EpiPre<NC>& pre) {
  if constexpr (E == Epi::PARTIAL) {
    if (g < p.n_groups) pre.seq = (uint32_t)p.cnt[g];
  }
  if constexpr (E == Epi::RESID || E == Epi::PARTIAL) {
    if (g < p.n_groups) {
      pre.gain = p.gain_next[16 * g + (lane & 15)];
#pragma unroll
      for (int j = 0; j < EpiPre<NC>::kX; ++j) {
        const int idx = lane + 64 * j;
        if (idx < 16 * M) pre.xv[j] = p.x[(size_t)(idx >> 4) * p.H + 16 * g + (idx & 15)];
      }
    }
  }
}

// QKV: the rotation pairs of this query/key group at positions pos0 + m
// (idx = 8 m + i, i = lane % 8); pos0 is the cache length read at launch.
// A tree forward rotates row m at pos0 + tree_depth[m] (the tree's base
// slot plus the node's depth) instead; its K/V still go to slot pos0 + m.
template <Epi E, int NC>
__device__ __forceinline__ void epi_prefetch_rope(const GemvParams& p, int lane, int g, int M, EpiPre<NC>& pre) {
  if constexpr (E == Epi::QKV) {
    const int qg = p.nq * p.hd / 16, kg = p.nkv * p.hd / 16;
    if (g < qg + kg) {
      const int sub = (g >= qg ? g - qg : g) % (p.hd / 16), half = p.hd / 2;
#pragma unroll
      for (int j = 0; j < EpiPre<NC>::kR; ++j) {
        const int idx = lane + 64 * j, m = idx >> 3, slot = pre.pos0 + m;
        if (m < M && slot < p.max_len) {
          const int pos = p.tree_depth ? pre.pos0 + p.tree_depth[m] : slot;
          pre.cs[j] = p.rope[(size_t)pos * half + 8 * sub + (idx & 7)];
        }
      }
    }
  }
}

// Residual epilogue of 16 outputs (one row group g) x M rows: x += y,
// the next norm's operand tiles of x * gain and the group's sum of squares
// (the 16 lanes of a row sum in a fixed tree).  f[i][m] holds y; pre holds
// x and the gains.
template <int NC>
__device__ __forceinline__ void resid_epilogue(const GemvParams& p, float (*f)[NC + 1], const EpiPre<NC>& pre, int lane,
                                               int g, int M) {
  const int KBo = p.H >> 5, NP = p.H >> 4;
#pragma unroll
  for (int j = 0; j < EpiPre<NC>::kX; ++j) {
    const int idx = lane + 64 * j;
    const bool ok = idx < 16 * M;
    const int i = idx & 15, m = idx >> 4, n = 16 * g + i;
    float sq = 0.f;
    if (ok) {
      const float xn = pre.xv[j] + f[i][m];
      p.x[(size_t)m * p.H + n] = xn;
      btile_put(p.xb_out, KBo, m, n, xn * pre.gain);
      sq = xn * xn;
    }
    // lanes 16 m' .. 16 m' + 15 of this pass hold row m' + 4 j
    sq = row16_sum(sq);
    if (ok && i == 0) p.ss_out[(size_t)m * NP + g] = sq;
  }
}

// Query operand tiles: per kv head, query rows r = m * G + g (g = query head
// within the group), 16 rows per tile, the bf16 hi and lo parts of q / sqrt(d)
// in separate tiles: [tile][k-block over the head dim][hi|lo][64 lanes][8].
// Lane l of a tile holds row 16 * tile + (l % 16), dims 32 * kb + 8 * (l / 16) .. +7.
constexpr int kQTiles = kMaxRows * 8 / 16;   // up to 8 * kMaxRows query rows
__device__ __forceinline__ size_t qtile_head(int h, int hd) { return (size_t)h * kQTiles * (hd / 32) * 2 * kTileU16; }
__device__ __forceinline__ void qtile_put(bf16_bits* qh, int KBH, int row, int dim, float v) {
  const int tq = row >> 4, j = row & 15, kb = dim >> 5, sg = (dim >> 3) & 3, e = dim & 7;
  const size_t base = ((size_t)(tq * KBH + kb) * 2) * kTileU16 + (size_t)((sg * 16 + j) * 8 + e);
  const bf16_bits hi = f2bf(v);
  qh[base] = hi;
  qh[base + kTileU16] = f2bf(v - bf2f(hi));
}

// Sums of squares of the normalised input (per-16-feature partials), loaded
// before the weight stream so their latency hides under it.
template <int RPW, int NW>
__device__ __forceinline__ void norm_prefetch(const GemvParams& p, int w, int lane, int M, float (&ssv)[RPW][4]) {
  const int NP = p.H >> 4;
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int m = w + j * NW;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gg = lane + 64 * u;
      ssv[j][u] = (m < M && gg < NP) ? p.ss_in[(size_t)m * NP + gg] : 0.f;
    }
  }
}

// r_m = 1 / sqrt(mean(x_m^2) + eps) with a fixed reduction order per row.
template <int RPW, int NW>
__device__ __forceinline__ void norm_finish(const GemvParams& p, int w, int lane, int M, const float (&ssv)[RPW][4],
                                            float* rsc) {
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int m = w + j * NW;
    if (m < M) {
      float sq = ((ssv[j][0] + ssv[j][1]) + ssv[j][2]) + ssv[j][3];
      sq = warp_sum(sq);
      if (lane == 0) rsc[m] = 1.0f / sqrtf(sq / (float)p.H + p.eps);
    }
  }
}

// Epilogue of one skinny product, shared by the bf16 MFMA and the 4-bit
// kernels.  fin[rg][i][m] holds the finished dot product of output row i of
// row group g (rows in the packed order of the weight) with activation row
// m; rsc[m] the RMSNorm scale of row m (norm epilogues).  LMHEAD runs on the
// whole workgroup; the others on wave (rg, ks == 0) of each row group.
template <int WG_ROWS, int NC, Epi E>
__device__ __forceinline__ void gemv_epilogue(const GemvParams& p, float (*fin)[16][NC + 1], const float* rsc,
                                              const EpiPre<NC>& pre, int w, int lane, int rg, int ks, int g, int sidx,
                                              int M) {
  (void)w;
  if constexpr (E == Epi::LMHEAD) {
    // logits and this workgroup's (max, argmax, sum exp) per row
    for (int idx = threadIdx.x; idx < WG_ROWS * 16 * M; idx += blockDim.x) {
      int rr = idx / (16 * M), rem = idx % (16 * M), m = rem / 16, i = rem % 16;
      int gg = blockIdx.x * WG_ROWS + rr;
      float v = fin[rr][i][m] * rsc[m];
      fin[rr][i][m] = v;
      if (gg < p.n_groups) p.logits[(size_t)m * p.V + 16 * gg + i] = v;
    }
    __syncthreads();
    {
      // rows spread over the waves; each row's order is fixed by its lanes
      for (int m = w; m < M; m += (int)(blockDim.x >> 6)) {
        // lane owns entries lane and lane + 64 of the workgroup's 16 * WG_ROWS
        float best = -INFINITY;
        int bidx = 0x7fffffff;
        for (int e = lane; e < 16 * WG_ROWS; e += 64) {
          int rr = e >> 4, i = e & 15, gg = blockIdx.x * WG_ROWS + rr;
          if (gg < p.n_groups) {
            float v = fin[rr][i][m];
            int idx = 16 * gg + i;
            if (v > best || (v == best && idx < bidx)) { best = v; bidx = idx; }
          }
        }
        warp_argmax(best, bidx);
        float se = 0.f;
        for (int e = lane; e < 16 * WG_ROWS; e += 64) {
          int rr = e >> 4, i = e & 15, gg = blockIdx.x * WG_ROWS + rr;
          if (gg < p.n_groups) se += expf(fin[rr][i][m] - best);
        }
        se = warp_sum(se);
        if (lane == 0) {
          float* pp = p.lm_part + ((size_t)m * gridDim.x + blockIdx.x) * 3;
          pp[0] = best;
          pp[1] = __int_as_float(bidx);
          pp[2] = se;
        }
      }
    }
    return;
  }

  if (ks != 0 || g >= p.n_groups) return;
  // one wave per row group runs the epilogue
  float (*f)[NC + 1] = fin[rg];
  if constexpr (E == Epi::QKV) {
    const int pos0 = pre.pos0;
    const int qg = p.nq * p.hd / 16, kg = p.nkv * p.hd / 16;
    const int per_head = p.hd / 16, half = p.hd / 2;
    if (g < qg + kg) {
      const bool is_k = g >= qg;
      const int gg = is_k ? g - qg : g;
      const int head = gg / per_head, sub = gg % per_head;
#pragma unroll
      for (int j = 0; j < EpiPre<NC>::kR; ++j) {
        const int idx = lane + 64 * j, i = idx & 7, m = idx >> 3;
        const int pos = pos0 + m;
        if (m >= M || pos >= p.max_len) continue;
        float r = rsc[m];
        float y1 = f[i][m] * r, y2 = f[i + 8][m] * r;
        int d1 = 8 * sub + i;
        const float2 cs = pre.cs[j];
        // explicit fused forms: the rounding must not depend on how the
        // compiler contracts this loop in each launch shape
        const float o1 = fmaf(y1, cs.x, -(y2 * cs.y));
        const float o2 = fmaf(y2, cs.x, y1 * cs.y);
        if (!is_k) {
          const int G = p.nq / p.nkv;
          const float qs = 1.0f / sqrtf((float)p.hd);
          bf16_bits* qh = p.qb + qtile_head(head / G, p.hd);
          const int rq = m * G + head % G;
          qtile_put(qh, p.hd >> 5, rq, d1, o1 * qs);
          qtile_put(qh, p.hd >> 5, rq, d1 + half, o2 * qs);
        } else {
          bf16_bits* kc = p.k_cache + ((size_t)head * p.kv_stride + pos) * p.hd;
          kc[d1] = f2bf(o1);
          kc[d1 + half] = f2bf(o2);
        }
      }
    } else {
      const int r0 = 16 * (g - qg - kg);
      const int head = r0 / p.hd, d0 = r0 % p.hd;
      for (int idx = lane; idx < 16 * M; idx += 64) {
        int i = idx & 15, m = idx >> 4;
        int pos = pos0 + m;
        if (pos >= p.max_len) continue;
        p.v_cache[((size_t)head * p.hd + d0 + i) * p.kv_stride + pos] = f2bf(f[i][m] * rsc[m]);
      }
    }
  } else if constexpr (E == Epi::SWIGLU) {
    const int KBo = p.F >> 5;
    for (int idx = lane; idx < 8 * M; idx += 64) {
      int i = idx & 7, m = idx >> 3;
      float r = rsc[m];
      float gt = f[i][m] * r, up = f[i + 8][m] * r;
      float h = gt / (1.0f + __expf(-gt)) * up;
      btile_put(p.hb_out, KBo, m, 8 * g + i, h);
    }
  } else if constexpr (E == Epi::PARTIAL) {
    // Split-K hand-off.  Splits 0 .. nsplit-2 store their 16 outputs x M rows
    // as (value, tag) pairs and are done; split nsplit-1 finishes the row
    // group.  The tag is the row group's launch sequence number (seq + 1,
    // seq read from the workspace at launch), so the finisher's loads are
    // their own readiness test: it takes a value once its tag matches (a
    // bounded wait; the producers of a row group come first in launch order
    // and wait on nothing).  The splits are summed in split order and the
    // finisher stores the new sequence number for the next launch.
    const uint32_t tag = pre.seq + 1u;
    const int last = p.nsplit - 1;
    if (sidx != last) {
      float* dst = p.part + (size_t)sidx * kMaxRows * p.H * 2;
      for (int idx = lane; idx < 16 * M; idx += 64) {
        const int i = idx & 15, m = idx >> 4;
        store_agent_pair(dst + ((size_t)m * p.H + 16 * g + i) * 2, f[i][m], tag);
      }
      return;
    }
    const agent_rsrc_t pr = agent_rsrc(p.part);
    bool late = false;
    // a value once its tag matches (reloading while it does not)
    auto take = [&](u32x2_t w, size_t at) -> float {
      for (int spin = 0; w.y != tag; ++spin) {
        if (spin == kHandoffSpins) { late = true; break; }
        __builtin_amdgcn_s_sleep(1);
        w = load_agent_pair(pr, at);
      }
      return __uint_as_float(w.x);
    };
    // two lane-strided entries at a time (all of them when M <= 8), each
    // split's pair of loads in flight together
    for (int idxa = lane; idxa < 16 * M; idxa += 128) {
      const int idxb = idxa + 64;
      const bool vb = idxb < 16 * M;
      const int ib = vb ? idxb : idxa;
      float ya = 0.f, yb = 0.f;
      for (int s2 = 0; s2 < last; ++s2) {
        const size_t base = (size_t)s2 * kMaxRows * p.H + 16 * g;
        const size_t ata = base + (size_t)(idxa >> 4) * p.H + (idxa & 15);
        const size_t atb = base + (size_t)(ib >> 4) * p.H + (ib & 15);
        const u32x2_t wa = load_agent_pair(pr, ata), wb = load_agent_pair(pr, atb);
        ya += take(wa, ata);
        yb += take(wb, atb);
      }
      f[idxa & 15][idxa >> 4] = ya + f[idxa & 15][idxa >> 4];
      if (vb) f[idxb & 15][idxb >> 4] = yb + f[idxb & 15][idxb >> 4];
    }
    if (late) raise_error(p.err, kErrSync);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    resid_epilogue<NC>(p, f, pre, lane, g, M);
    if (lane == 0) p.cnt[g] = (int32_t)tag;
  } else {  // RESID
    resid_epilogue<NC>(p, f, pre, lane, g, M);
  }
}

// After the product of a skinny GEMV: red holds NW = WG_ROWS * WK wave slots
// of 16 output rows x NT * 8 activation rows; fin (LM head only) one slot per
// row group.
// The waves' partials in LDS (written by the product, see below), the
// reduction over the k-split waves in a fixed order and the epilogue.
template <int NT, int WG_ROWS, int WK, Epi E>
__device__ __forceinline__ void gemv_reduce_epilogue(const GemvParams& p, float (*red)[16][NT * 8 + 1],
                                                     float (*fin)[16][NT * 8 + 1], const float* rsc,
                                                     const EpiPre<NT * 8>& pre, int w, int lane, int rg, int ks,
                                                     int g, int sidx, int M, int n_groups) {
  constexpr int NC = NT * 8;
  __syncthreads();
  if constexpr (E == Epi::SWIGLU) {
    // the epilogue wave sums the k-split partials of its own entries, in the
    // order of the reduction below, and needs no second pass through LDS
    if (ks != 0 || g >= n_groups) return;
    const int KBo = p.F >> 5;
    for (int idx = lane; idx < 8 * M; idx += 64) {
      const int i = idx & 7, m = idx >> 3;
      float gt = 0.f, up = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < WK; ++s2) {
        gt += red[rg * WK + s2][i][m];
        up += red[rg * WK + s2][i + 8][m];
      }
      const float r = rsc[m];
      gt *= r;
      up *= r;
      btile_put(p.hb_out, KBo, m, 8 * g + i, gt / (1.0f + __expf(-gt)) * up);
    }
    return;
  } else if constexpr (E != Epi::LMHEAD) {
    // one wave per row group: it sums the k-split partials of the group (in
    // the order of the reduction below) into its first wave's slot, which
    // then serves as the group's finished products
    if (ks != 0 || g >= n_groups) return;
    constexpr int kE = (16 * NC + 63) / 64;
    float v[kE];
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const int idx = lane + 64 * j;
      if (idx < 16 * NC) {
        const int i = idx / NC, m = idx % NC;
        v[j] = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < WK; ++s2) v[j] += red[rg * WK + s2][i][m];
      }
    }
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const int idx = lane + 64 * j;
      if (idx < 16 * NC) red[rg * WK][idx / NC][idx % NC] = v[j];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    gemv_epilogue<WG_ROWS, NC, E>(p, red + rg * (WK - 1), rsc, pre, w, lane, rg, 0, g, sidx, M);
    return;
  }
  // fixed-order reduction over the k-split waves (whole-workgroup epilogue)
  for (int idx = threadIdx.x; idx < WG_ROWS * 16 * NC; idx += blockDim.x) {
    int rr = idx / (16 * NC), rem = idx % (16 * NC), i = rem / NC, m = rem % NC;
    float v = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < WK; ++s2) v += red[rr * WK + s2][i][m];
    fin[rr][i][m] = v;
  }
  __syncthreads();

  gemv_epilogue<WG_ROWS, NC, E>(p, fin, rsc, pre, w, lane, rg, ks, g, sidx, M);
}

// gemv_reduce_epilogue after an MFMA product: the hi and lo columns of
// each accumulator are added in registers and stored as the wave's partials.
template <int NT, int WG_ROWS, int WK, Epi E>
__device__ __forceinline__ void gemv_finish(const GemvParams& p, const f32x4_t (&acc)[NT], float (*red)[16][NT * 8 + 1],
                                            float (*fin)[16][NT * 8 + 1], const float* rsc,
                                            const EpiPre<NT * 8>& pre, int w, int lane, int rg, int ks, int g,
                                            int sidx, int M, int n_groups) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[t][r] + swap1(acc[t][r]);
      if ((lane & 1) == 0) red[w][4 * (lane >> 4) + r][t * 8 + ((lane & 15) >> 1)] = v;
    }
  gemv_reduce_epilogue<NT, WG_ROWS, WK, E>(p, red, fin, rsc, pre, w, lane, rg, ks, g, sidx, M, n_groups);
}

}  // namespace sd
