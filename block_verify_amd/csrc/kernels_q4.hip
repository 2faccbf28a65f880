// gfx950 kernels of the 4-bit group-64 substitute weights.
//
// Definition: "SubSpec" summary (jjl357.github.io), section 4.1.1 -- every
// linear weight of the draft is an affine 4-bit code per group of 64
// consecutive inputs of one output row, weight = (code - zero) * scale with
// half-precision scale and zero; the embedding and LM head stay bf16 and are
// shared with the target.
//
// The product is HBM-bound (0.5625 bytes per weight), so no matrix cores:
// each lane decodes 32 codes per 16-byte load into exact fp16 integers with
// one and-or per code pair (the codes are or-ed into the mantissa of 1024.0
// and 1024.0 is subtracted), and accumulates code * x pairs with the fp32
// two-way dot product.  The zero point is applied once per half group:
//   sum_i (q_i - z) * s * x_i = s * (sum_i q_i * x_i - z * sum_i x_i),
// with sum_i x_i taken per 32 inputs from sums of 8 made while the
// activation rows (at most four) are staged in LDS as fp16; each wave
// requests its first batch of codes before that staging.  Reductions run in a fixed order, so a
// row's result does not depend on how many rows share the pass.
#include "gemv_common.h"

namespace sd {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Packing (setup).  Source: codes uint8 [N][K/2] (even input in the low
// nibble), then fp16 scale [N][K/64], then fp16 zero [N][K/64].
// Destination, per 16-row group g and 128-input block b:
//   codes  [g][b][lane][4 words]: lane l holds row l % 16, inputs
//          128 b + 32 (l / 16) .. +31; word j covers 8 of them with input
//          2c in nibble c and input 2c + 1 in nibble c + 4 (c = 0..3), so an
//          and-or with 0x000F000F after a shift by 4c yields the fp16 pair.
//   scales [g][b][half][16 rows] of (scale, zero) fp16 pairs.
// A block past K (K % 128 == 64) holds zero codes and zero scale / zero.
// ---------------------------------------------------------------------------
__global__ void pack_q4_kernel(const uint8_t* __restrict__ src, int rows, int K, int kind, int hd, int group_base,
                               int NB, uint32_t* __restrict__ codes, uint32_t* __restrict__ scales) {
  const size_t total = (size_t)rows * NB * 4;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(src + (size_t)rows * (K / 2));
  const uint16_t* zc = sc + (size_t)rows * (K / 64);
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(idx / ((size_t)NB * 4));
    const int rem = (int)(idx % ((size_t)NB * 4));
    const int b = rem >> 2, qq = rem & 3;
    int g, i;
    pack_row_slot(kind, r, hd, g, i);
    g += group_base;
    const int lane = qq * 16 + i;
    const int k0 = b * 128 + 32 * qq;
    uint32_t* dst = codes + (((size_t)g * NB + b) * 64 + lane) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
      const int kk = k0 + 8 * j;
      if (kk < K) {
        const uint8_t* sb = src + (size_t)r * (K / 2) + kk / 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t byte = sb[c];
          word |= (byte & 0xFu) << (4 * c);
          word |= (byte >> 4) << (16 + 4 * c);
        }
      }
      dst[j] = word;
    }
    if ((qq & 1) == 0) {
      const int gi = 2 * b + (qq >> 1);
      uint32_t sz = 0;
      if (gi * 64 < K) {
        const size_t si = (size_t)r * (K / 64) + gi;
        sz = (uint32_t)sc[si] | ((uint32_t)zc[si] << 16);
      }
      scales[(((size_t)g * NB + b) * 2 + (qq >> 1)) * 16 + i] = sz;
    }
  }
}

hipError_t launch_pack_q4(const void* src, int rows, int K, int kind, int hd, int group_base, uint8_t* codes,
                          uint8_t* scales, hipStream_t s) {
  const int NB = (K + 127) / 128;
  size_t total = (size_t)rows * NB * 4;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 65535 * 4) blocks = 65535 * 4;
  pack_q4_kernel<<<blocks, 256, 0, s>>>(static_cast<const uint8_t*>(src), rows, K, kind, hd, group_base, NB,
                                        reinterpret_cast<uint32_t*>(codes), reinterpret_cast<uint32_t*>(scales));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 4-bit skinny product.  Workgroup = WG_ROWS row groups x WK k-split waves
// (PARTIAL: one row group, split nsplit ways over the workgroups).
// ---------------------------------------------------------------------------
struct Q4Params {
  const u32x4_t* codes;
  const uint32_t* scales;
  int K;    // inputs
  int NB;   // 128-input blocks
};

template <int WG_ROWS, int WK, int U, Epi E>
__global__ __launch_bounds__(64 * WG_ROWS * WK) void q4_gemv_kernel(GemvParams p, Q4Params q) {
  EpiPre<8> pre;
  // the gate word (the length stands in for a null gate) and the cache
  // position are requested together, before any branch
  const int gv = *(p.gate ? p.gate : p.d_len);
  if constexpr (E == Epi::QKV) pre.pos0 = *p.d_len;
  if (p.gate && gv == 0) return;
  constexpr int NW = WG_ROWS * WK;
  constexpr int NC = 8;
  constexpr int RPW = (kQ4MaxRows + NW - 1) / NW;
  constexpr int NT = 64 * NW;
  extern __shared__ __align__(16) unsigned char q4_lds[];
  __shared__ float red[NW][16][NC + 1];
  __shared__ float rsc[kMaxRows];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = w / WK, ks = w % WK;
  const int nsplit = (E == Epi::PARTIAL) ? p.nsplit : 1;
  const int sidx = (E == Epi::PARTIAL) ? (int)(blockIdx.x % nsplit) : 0;
  const int g = (E == Epi::PARTIAL) ? (int)(blockIdx.x / nsplit) : (int)(blockIdx.x * WG_ROWS + rg);
  const int M = p.rows;
  // 32-bit unsigned arithmetic (small terms; a 64-bit division is long)
  const int b0s = (int)((unsigned)sidx * (unsigned)q.NB / (unsigned)nsplit);
  const int b1s = (int)((unsigned)(sidx + 1) * (unsigned)q.NB / (unsigned)nsplit);
  const int KR = (b1s - b0s) * 128;
  _Float16* xs = reinterpret_cast<_Float16*>(q4_lds);                       // [M][KR]
  float* x8 = reinterpret_cast<float*>(q4_lds + (size_t)M * KR * 2);       // [M][KR / 8] sums of 8

  // The activation rows of this split are staged in LDS as fp16 (x = hi + lo
  // of the tiles) with the float sum of every 8 staged values.  Their loads
  // (L2-resident) go out first, SP per thread, then the wave's first batch of
  // codes (HBM): loads complete in issue order, so writing the activations to
  // LDS then waits for them only.  The loads are unconditional (an index past
  // the rows re-reads entry 0): guarded loads into registers are each waited on.
  const bf16_bits* bt = reinterpret_cast<const bf16_bits*>(p.B);
  const int k8n = KR >> 3, nstage = M * k8n;
  // staging pairs in flight per thread: enough for one activation row of
  // the 7B-shape splits in one pass (the down projection's split is longest)
  constexpr int SP = (E == Epi::PARTIAL) ? 3 : 1;
  uint4 hv[SP], lv[SP];
  auto stage_load = [&](int base) {
#pragma unroll
    for (int j = 0; j < SP; ++j) {
      int idx = base + (int)threadIdx.x + NT * j;
      if (idx >= nstage) idx = 0;
      const int m = idx / k8n;
      int k = b0s * 128 + (idx % k8n) * 8;
      if (k >= q.K) k = 0;   // the block past K reads a valid tile and stores zeros
      const size_t bi = btile_index(p.KB, m, k);
      hv[j] = *reinterpret_cast<const uint4*>(bt + bi);
      lv[j] = *reinterpret_cast<const uint4*>(bt + bi + kBtileLo);
    }
  };
  auto stage_store = [&](int base) {
#pragma unroll
    for (int j = 0; j < SP; ++j) {
      const int idx = base + (int)threadIdx.x + NT * j;
      if (idx < nstage) {
        const int m = idx / k8n, k = b0s * 128 + (idx % k8n) * 8;
        half8_t o;
        if (k < q.K) {
          const uint32_t hw[4] = {hv[j].x, hv[j].y, hv[j].z, hv[j].w}, lw[4] = {lv[j].x, lv[j].y, lv[j].z, lv[j].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[2 * e] = (_Float16)(__uint_as_float(hw[e] << 16) + __uint_as_float(lw[e] << 16));
            o[2 * e + 1] = (_Float16)(__uint_as_float(hw[e] & 0xFFFF0000u) + __uint_as_float(lw[e] & 0xFFFF0000u));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (_Float16)0.0f;
        }
        *reinterpret_cast<half8_t*>(xs + (size_t)m * KR + (k - b0s * 128)) = o;
        float s8 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s8 += (float)o[e];
        x8[idx] = s8;
      }
    }
  };

  constexpr bool kNorm = (E == Epi::QKV || E == Epi::SWIGLU);
  float ssv[RPW][4];
  const bool active = g < p.n_groups;
  const int nb = b1s - b0s;
  const int kb0 = b0s + (int)((unsigned)ks * (unsigned)nb / WK), kb1 = b0s + (int)((unsigned)(ks + 1) * (unsigned)nb / WK);
  const int n = active ? kb1 - kb0 : 0;
  const u32x4_t* cp = q.codes + (size_t)(active ? g : 0) * q.NB * 64 + lane;
  const uint32_t* sp = q.scales + (size_t)(active ? g : 0) * q.NB * 32 + (lane >> 5) * 16 + (lane & 15);

  // Runs once per wave after its first code requests: the small prefetches,
  // the staging writes (and any further staging) and the workgroup barrier.
  auto after_first = [&] {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kNorm) norm_prefetch<RPW, NW>(p, w, lane, M, ssv);
    if (ks == 0) {
      epi_prefetch_x<E, NC>(p, lane, g, M, pre);
      epi_prefetch_rope<E, NC>(p, lane, g, M, pre);
    }
    stage_store(0);
    for (int base = SP * NT; base < nstage; base += SP * NT) {
      stage_load(base);
      stage_store(base);
    }
    __syncthreads();
  };

  float y[kQ4MaxRows];
#pragma unroll
  for (int m = 0; m < kQ4MaxRows; ++m) y[m] = 0.f;
  const int qq = lane >> 4;
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  // One batch of U code blocks from block b: straight-line loads (slots past
  // the wave's last block re-read it and are skipped), then the blocks in order.
  auto batch = [&](int b, bool first) {
    u32x4_t cv[U];
    uint32_t sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bb = b + u < kb1 ? b + u : kb1 - 1;
      cv[u] = __builtin_nontemporal_load(cp + (size_t)bb * 64);
      sv[u] = __builtin_nontemporal_load(sp + (size_t)bb * 32);
    }
    if (first) after_first();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b + u >= kb1) break;
      half2_t qv[16];
      const uint32_t cw[4] = {cv[u][0], cv[u][1], cv[u][2], cv[u][3]};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t t = ((cw[j] >> (4 * c)) & 0x000F000Fu) | 0x64006400u;
          qv[4 * j + c] = __builtin_bit_cast(half2_t, t) - k1024;
        }
      const half2_t szh = __builtin_bit_cast(half2_t, sv[u]);
      const float s = (float)szh[0], z = (float)szh[1];
      const int xoff = (b + u - b0s) * 128 + 32 * qq;
#pragma unroll
      for (int m = 0; m < kQ4MaxRows; ++m) {
        if (m < M) {
          const half8_t* xp = reinterpret_cast<const half8_t*>(xs + (size_t)m * KR + xoff);
          const float4 xq = *reinterpret_cast<const float4*>(x8 + (size_t)m * k8n + (xoff >> 3));
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const half8_t xv = xp[v];
            a0 = __builtin_amdgcn_fdot2(qv[4 * v], half2_t{xv[0], xv[1]}, a0, false);
            a1 = __builtin_amdgcn_fdot2(qv[4 * v + 1], half2_t{xv[2], xv[3]}, a1, false);
            a0 = __builtin_amdgcn_fdot2(qv[4 * v + 2], half2_t{xv[4], xv[5]}, a0, false);
            a1 = __builtin_amdgcn_fdot2(qv[4 * v + 3], half2_t{xv[6], xv[7]}, a1, false);
          }
          const float xsum = ((xq.x + xq.y) + xq.z) + xq.w;
          y[m] = fmaf(s, (a0 + a1) - z * xsum, y[m]);
        }
      }
    }
  };

  stage_load(0);
  if (n <= 0) {
    after_first();
  } else {
    // the first batch is peeled: the staging registers are dead after it
    batch(kb0, true);
    for (int b = kb0 + U; b < kb1; b += U) batch(b, false);
  }
  if constexpr (kNorm) norm_finish<RPW, NW>(p, w, lane, M, ssv, rsc);
  // the four quarters of a row (lanes i, i+16, i+32, i+48), then the waves
#pragma unroll
  for (int m = 0; m < kQ4MaxRows; ++m) {
    float v = y[m];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (lane < 16 && m < M) red[w][lane][m] = v;
  }
  __syncthreads();
  // one wave per row group sums the group's k-split partials (in wave
  // order) into its first wave's slot and runs the epilogue from there
  if (ks != 0 || g >= p.n_groups) return;
  constexpr int kE = (16 * kQ4MaxRows + 63) / 64;
  float v[kE];
#pragma unroll
  for (int j = 0; j < kE; ++j) {
    const int idx = lane + 64 * j;
    if (idx < 16 * M) {
      const int i = idx / M, m = idx % M;
      v[j] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < WK; ++s2) v[j] += red[rg * WK + s2][i][m];
    }
  }
#pragma unroll
  for (int j = 0; j < kE; ++j) {
    const int idx = lane + 64 * j;
    if (idx < 16 * M) red[rg * WK][idx / M][idx % M] = v[j];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  gemv_epilogue<WG_ROWS, NC, E>(p, red + rg * (WK - 1), rsc, pre, w, lane, rg, 0, g, sidx, M);
}

// Launch shapes (row groups per workgroup, k-split waves, code blocks in
// flight per wave); the down projection takes one row group per workgroup.
#ifndef SD_Q4_QKV
#define SD_Q4_QKV 1, 8, 4
#endif
#ifndef SD_Q4_O
#define SD_Q4_O 1, 8, 4
#endif
#ifndef SD_Q4_GU
#define SD_Q4_GU 2, 4, 8
#endif
#ifndef SD_Q4_DOWN
#define SD_Q4_DOWN 4, 10
#endif
template <int R, int W, int T>
constexpr int Q4Rows() { return R; }

size_t q4_lds_bytes(int rows, int K, int nsplit) {
  const int NB = (K + 127) / 128;
  const int per = (NB + nsplit - 1) / nsplit + 1;
  const size_t KR = (size_t)per * 128;
  return (size_t)rows * KR * 2 + (size_t)rows * (KR / 8) * 4;
}

template <int WG_ROWS, int WK, int U, Epi E>
static hipError_t launch_q4(const GemvParams& p, const Q4Params& q, int grid, hipStream_t s) {
  const int nsplit = (E == Epi::PARTIAL) ? p.nsplit : 1;
  const int b0 = 0;
  (void)b0;
  // largest split of this launch
  int most = 0;
  for (int si = 0; si < nsplit; ++si) {
    int a = (int)(((long)si * q.NB) / nsplit), b = (int)(((long)(si + 1) * q.NB) / nsplit);
    if (b - a > most) most = b - a;
  }
  const size_t lds = (size_t)p.rows * most * 128 * 2 + (size_t)p.rows * most * 16 * 4;
  q4_gemv_kernel<WG_ROWS, WK, U, E><<<grid, 64 * WG_ROWS * WK, lds, s>>>(p, q);
  return hipGetLastError();
}

hipError_t launch_q4_linear(Q4Linear which, const GemvParams& p, const uint8_t* codes, const uint8_t* scales, int K,
                            hipStream_t s) {
  Q4Params q;
  q.codes = reinterpret_cast<const u32x4_t*>(codes);
  q.scales = reinterpret_cast<const uint32_t*>(scales);
  q.K = K;
  q.NB = (K + 127) / 128;
  switch (which) {
    case Q4Linear::QKV:
      return launch_q4<SD_Q4_QKV, Epi::QKV>(p, q, (p.n_groups + Q4Rows<SD_Q4_QKV>() - 1) / Q4Rows<SD_Q4_QKV>(), s);
    case Q4Linear::O:
      return launch_q4<SD_Q4_O, Epi::RESID>(p, q, (p.n_groups + Q4Rows<SD_Q4_O>() - 1) / Q4Rows<SD_Q4_O>(), s);
    case Q4Linear::GATE_UP:
      return launch_q4<SD_Q4_GU, Epi::SWIGLU>(p, q, (p.n_groups + Q4Rows<SD_Q4_GU>() - 1) / Q4Rows<SD_Q4_GU>(), s);
    case Q4Linear::DOWN: return launch_q4<1, SD_Q4_DOWN, Epi::PARTIAL>(p, q, p.n_groups * p.nsplit, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sd
