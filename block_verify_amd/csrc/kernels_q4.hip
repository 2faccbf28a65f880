// gfx950 kernels of the 4-bit group-64 substitute weights.
//
// Definition: "SubSpec" summary (jjl357.github.io), section 4.1.1 -- every
// linear weight of the draft is an affine 4-bit code per group of 64
// consecutive inputs of one output row, weight = (code - zero) * scale with
// half-precision scale and zero; the embedding and LM head stay bf16 and are
// shared with the target.
//
// The product runs on the matrix cores like the bf16 one, against the same
// hi/lo activation tiles read straight from L2.  A code c becomes the exact
// bf16 value 128 + c with one and-or per code pair (c fills the low mantissa
// bits of 128.0), so an MFMA of the codes' tile accumulates
//   sum_i (128 + c_i) x_i,
// and a second MFMA with a tile of ones the group's sum_i x_i.  Per row and
// group of 64 inputs the weight sum is then
//   sum_i (c_i - z) s x_i = s * (sum_i (128 + c_i) x_i - (128 + z) * sum_i x_i),
// applied to the two accumulators in fp32 after each group.  Every product is
// exact and each column (activation row) is independent, so a row's result
// does not depend on how many rows share the pass.
#include "gemv_common.h"

namespace sd {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4q_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Packing (setup).  Source: codes uint8 [N][K/2] (even input in the low
// nibble), then fp16 scale [N][K/64], then fp16 zero [N][K/64].
// Destination, per 16-row group g and 128-input block b:
//   codes  [g][b][lane][4 words]: lane l holds row l % 16; word j covers
//          inputs 128 b + 32 j + 8 (l / 16) .. +7 (the MFMA operand A
//          slice of k-block j), input 2c of the eight in nibble c and input
//          2c + 1 in nibble c + 4, so that ((word >> 4c) & 0x000F000F)
//          holds operand pair c;
//   scales [g][b][half][16 rows] of (scale, zero) fp16 pairs, rows in the
//          order of the MFMA result (lane l reads rows 4 (l / 16) .. +3).
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
    const int b = rem >> 2, j = rem & 3;   // block, k-block within it
    int g, i;
    pack_row_slot(kind, r, hd, g, i);
    g += group_base;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
      const int kk = b * 128 + 32 * j + 8 * q;
      if (kk < K) {
        const uint8_t* sb = src + (size_t)r * (K / 2) + kk / 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t byte = sb[c];
          word |= (byte & 0xFu) << (4 * c);
          word |= (byte >> 4) << (16 + 4 * c);
        }
      }
      codes[(((size_t)g * NB + b) * 64 + (q * 16 + i)) * 4 + j] = word;
    }
    if (j < 2) {
      const int gi = 2 * b + j;
      uint32_t sz = 0;
      if (gi * 64 < K) {
        const size_t si = (size_t)r * (K / 64) + gi;
        sz = (uint32_t)sc[si] | ((uint32_t)zc[si] << 16);
      }
      scales[(((size_t)g * NB + b) * 2 + j) * 16 + i] = sz;
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
// 4-bit skinny product.
// ---------------------------------------------------------------------------
constexpr uint32_t kQ4Magic = 0x43004300u;   // bf16 128.0 in both halves
constexpr int32_t kBf16OnePair = 0x3F803F80;

// Operand A of one k-block: eight codes -> eight bf16 values 128 + code.
__device__ __forceinline__ i32x4q_t q4_decode(uint32_t w) {
  i32x4q_t a;
  a[0] = (int32_t)((w & 0x000F000Fu) | kQ4Magic);
  a[1] = (int32_t)(((w >> 4) & 0x000F000Fu) | kQ4Magic);
  a[2] = (int32_t)(((w >> 8) & 0x000F000Fu) | kQ4Magic);
  a[3] = (int32_t)(((w >> 12) & 0x000F000Fu) | kQ4Magic);
  return a;
}

__device__ __forceinline__ f32x4_t mfma_q(const i32x4q_t& a, const i32x4q_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// ---------------------------------------------------------------------------
// 4-bit skinny product.  A workgroup of kQ4RWaves waves takes up to `rg`
// row groups over one k-range (a split of the K range for the down
// projection; one split holds at most kQ4RWaves * kQ4RBlocks blocks of 128
// inputs).  Wave w keeps the activation tiles of its <= kQ4RBlocks blocks in
// registers, with their per-group sums, and streams the code tiles of the
// workgroup's row groups through them, the next row group's codes requested
// before the current one is computed.  The activations are the MFMA's
// operand A and the codes operand B, so the result C[m'][n] holds
// activation column m' (the hi or lo part of a row) against output row
// n = lane % 16: each lane applies one row's scale per group.  A pass of more
// than 8 rows repeats this per column tile of 8 rows (the codes streamed once
// per tile), so each row's arithmetic -- the k-range of every wave, the
// order of its blocks and the wave order of the sum -- does not depend on the
// pass.  The waves' partials meet in LDS; wave w runs the epilogues of row
// groups w, w + kQ4RWaves, ...
// ---------------------------------------------------------------------------
#ifndef SD_Q4_AHEAD
#define SD_Q4_AHEAD 3
#endif
#ifndef SD_Q4_WAVES
#define SD_Q4_WAVES 8
#endif
constexpr int kQ4RWaves = SD_Q4_WAVES, kQ4RBlocks = kQ4MaxBlocks / kQ4RWaves;
static_assert(kQ4RWaves * kQ4RBlocks == kQ4MaxBlocks, "one split's blocks");
// row groups of codes in flight per wave (fewer for wide passes: registers)
template <int NT>
struct Q4Ahead {
  static constexpr int value = NT == 1 ? SD_Q4_AHEAD : 2;
};
template <int NT>
struct Q4RGroups {
  // LDS: the partials of RG row groups from every wave, <= ~110 KB
  static constexpr int value = (NT == 1 ? 12 : NT == 2 ? 6 : NT == 3 ? 4 : 3) * 8 / kQ4RWaves;
};

template <int NT, Epi E>
__global__ __launch_bounds__(64 * kQ4RWaves) void q4_gemv_kernel(const int32_t* gate, const int32_t* d_len,
                                                                 const u32x4_t* __restrict__ codes,
                                                                 const uint32_t* __restrict__ scales,
                                                                 const bf16x8_t* __restrict__ B, int KB, int NB,
                                                                 int n_groups, int rows, int nsplit_arg, int rg_per_wg,
                                                                 GemvParams p) {
  constexpr int NW = kQ4RWaves, NC = 8 * NT, BLK = kQ4RBlocks, RG = Q4RGroups<NT>::value;
  constexpr int kQ4Ahead = Q4Ahead<NT>::value;
  constexpr int RPW = (NC + NW - 1) / NW;
  EpiPre<NC> pre;
  if constexpr (E == Epi::QKV) pre.pos0 = *d_len;
  if (gate) {
    if (*gate == 0) return;
  }
  __shared__ float red[RG][NW][16][NC + 1];
  __shared__ float rsc[kMaxRows];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsplit = (E == Epi::PARTIAL) ? nsplit_arg : 1;
  const unsigned slot = blockIdx.x >> 3;
  const int sidx = (E == Epi::PARTIAL) ? (int)(slot % (unsigned)nsplit) : 0;
  const int unit = (E == Epi::PARTIAL) ? (int)((slot / (unsigned)nsplit) * 8 + (blockIdx.x & 7)) : (int)blockIdx.x;
  const int g0 = unit * rg_per_wg;
  int nrg = n_groups - g0;
  if (nrg > rg_per_wg) nrg = rg_per_wg;
  const int M = rows;
  // this wave's blocks of this split
  const unsigned un = (unsigned)nsplit, ub = (unsigned)NB;
  const int s0 = (int)((unsigned)sidx * ub / un), s1 = (int)((unsigned)(sidx + 1) * ub / un);
  const unsigned span = (unsigned)(s1 - s0);
  const int b0 = s0 + (int)((unsigned)w * span / NW), b1 = s0 + (int)((unsigned)(w + 1) * span / NW);
  const int nb = b1 - b0;   // <= BLK (the launch sizes the splits so)

  constexpr bool kNorm = (E == Epi::QKV || E == Epi::SWIGLU);
  float ssv[RPW][4];
  if constexpr (kNorm) norm_prefetch<RPW, NW>(p, w, lane, M, ssv);

  const int col = lane & 15, q = lane >> 4;
  const u32x4_t* cbase = codes + (size_t)b0 * 64 + lane;
  const uint32_t* sbase = scales + (size_t)b0 * 32 + col;
  auto load_rg = [&](int g, u32x4_t (&c)[BLK], uint32_t (&sc)[BLK][2]) {
#pragma unroll
    for (int jb = 0; jb < BLK; ++jb) {
      const int b = jb < nb ? jb : 0;
      c[jb] = __builtin_nontemporal_load(cbase + ((size_t)g * NB + b) * 64);
      sc[jb][0] = __builtin_nontemporal_load(sbase + ((size_t)g * NB + b) * 32);
      sc[jb][1] = __builtin_nontemporal_load(sbase + ((size_t)g * NB + b) * 32 + 16);
    }
  };
  const i32x4q_t ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
#pragma unroll 1
  for (int t = 0; t < NT; ++t) {
    // activation tiles of column tile t for the wave's blocks (operand A):
    // unconditional loads of clamped indices; operand columns past the rows
    // read row 0's slot (their products are never used)
    const int aslot = btile_slot((col >> 1) < M - 8 * t ? col : (col & 1), q);
    const i32x4q_t* bt = reinterpret_cast<const i32x4q_t*>(B) + (size_t)t * KB * 64 + aslot;
    i32x4q_t act[BLK][4];
#pragma unroll
    for (int jb = 0; jb < BLK; ++jb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int kb = 4 * (b0 + jb) + j;
        if (jb >= nb || kb >= KB) kb = 0;   // a valid tile, never used
        act[jb][j] = bt[(size_t)kb * 64];
      }
    // the codes of the first kQ4Ahead - 1 row groups go out with the activation
    // loads; row group r + kQ4Ahead - 1 is requested before r is computed
    u32x4_t cv[kQ4Ahead][BLK];
    uint32_t sw[kQ4Ahead][BLK][2];
#pragma unroll
    for (int k = 0; k < kQ4Ahead - 1; ++k)
      if (k < nrg) load_rg(g0 + k, cv[k], sw[k]);
    if (t == 0 && w < nrg) {
      // the epilogue operands of this wave's row group (wave r ends row group r)
      epi_prefetch_x<E, NC>(p, lane, g0 + w, M, pre);
      epi_prefetch_rope<E, NC>(p, lane, g0 + w, M, pre);
    }
    f32x4_t sgs[BLK][2];
#pragma unroll
    for (int jb = 0; jb < BLK; ++jb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sgs[jb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (jb < nb && 4 * (b0 + jb) + 2 * h < KB) {
          sgs[jb][h] = mfma_q(act[jb][2 * h], ones, sgs[jb][h]);
          sgs[jb][h] = mfma_q(act[jb][2 * h + 1], ones, sgs[jb][h]);
        }
      }
    for (int r0 = 0; r0 < nrg; r0 += kQ4Ahead) {
#pragma unroll
      for (int k = 0; k < kQ4Ahead; ++k) {
        const int r = r0 + k;
        if (r >= nrg) break;
        // stage k holds row group r; stage (k + kQ4Ahead - 1) % kQ4Ahead takes r + kQ4Ahead - 1
        constexpr int kA = Q4Ahead<NT>::value;
        if (r + kA - 1 < nrg) load_rg(g0 + r + kA - 1, cv[(k + kA - 1) % kA], sw[(k + kA - 1) % kA]);
        f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < BLK; ++jb) {
          if (jb >= nb) break;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (4 * (b0 + jb) + 2 * h >= KB) break;
            f32x4_t ag = {0.f, 0.f, 0.f, 0.f};
            ag = mfma_q(act[jb][2 * h], q4_decode(cv[k][jb][2 * h]), ag);
            ag = mfma_q(act[jb][2 * h + 1], q4_decode(cv[k][jb][2 * h + 1]), ag);
            // output row n = lane % 16: y += s * (ag - (128 + z) * sg)
            const half2_t sz = __builtin_bit_cast(half2_t, sw[k][jb][h]);
            const float sc = (float)sz[0], tz = sc * (128.0f + (float)sz[1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = fmaf(-tz, sgs[jb][h][e], fmaf(sc, ag[e], y[e]));
          }
        }
        // C[m'][n], m' = 4 q + e: the hi and lo parts of activation row m' / 2
        red[r][w][col][8 * t + 2 * q] = y[0] + y[1];
        red[r][w][col][8 * t + 2 * q + 1] = y[2] + y[3];
      }
    }
  }
  if constexpr (kNorm) norm_finish<RPW, NW>(p, w, lane, M, ssv, rsc);
  __syncthreads();
  // wave w ends row groups w, w + NW, ...: the k-range partials of the row
  // group in wave order, then its epilogue (operands of the first prefetched
  // under the stream)
  for (int rr = w; rr < nrg; rr += NW) {
    if (rr != w) {
      epi_prefetch_x<E, NC>(p, lane, g0 + rr, M, pre);
      epi_prefetch_rope<E, NC>(p, lane, g0 + rr, M, pre);
    }
    float (*rw)[16][NC + 1] = red[rr];
    for (int idx = lane; idx < 16 * M; idx += 64) {
      const int i = idx & 15, m = idx >> 4;
      float v = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NW; ++s2) v += rw[s2][i][m];
      rw[0][i][m] = v;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    gemv_epilogue<RG, NC, E>(p, reinterpret_cast<float(*)[16][NC + 1]>(&red[0][0]) + rr * (NW - 1), rsc, pre, w,
                             lane, rr, 0, g0 + rr, sidx, M);
  }
}

template <int NT, Epi E>
static hipError_t launch_q4(const GemvParams& p, const uint8_t* codes, const uint8_t* scales, int NB, int nsplit,
                            hipStream_t s) {
  // row groups per workgroup: about one workgroup per CU
  int rg = (p.n_groups * nsplit + 255) / 256;
  if (rg < 1) rg = 1;
  if (rg > Q4RGroups<NT>::value) rg = Q4RGroups<NT>::value;
  const int units = (p.n_groups + rg - 1) / rg;
  const int grid = E == Epi::PARTIAL ? (units + 7) / 8 * 8 * nsplit : units;
  GemvParams q = p;
  q.nsplit = nsplit;
  q4_gemv_kernel<NT, E><<<grid, 64 * kQ4RWaves, 0, s>>>(p.gate, p.d_len, reinterpret_cast<const u32x4_t*>(codes),
                                                         reinterpret_cast<const uint32_t*>(scales), p.B, p.KB, NB,
                                                         p.n_groups, p.rows, nsplit, rg, q);
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_q4_nt(Q4Linear which, const GemvParams& p, const uint8_t* codes, const uint8_t* scales,
                               int NB, hipStream_t s) {
  constexpr int reach = kQ4RWaves * kQ4RBlocks;
  switch (which) {
    case Q4Linear::QKV: return launch_q4<NT, Epi::QKV>(p, codes, scales, NB, 1, s);
    case Q4Linear::O: return launch_q4<NT, Epi::RESID>(p, codes, scales, NB, 1, s);
    case Q4Linear::GATE_UP: return launch_q4<NT, Epi::SWIGLU>(p, codes, scales, NB, 1, s);
    case Q4Linear::DOWN: return launch_q4<NT, Epi::PARTIAL>(p, codes, scales, NB, (NB + reach - 1) / reach, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_q4_linear(Q4Linear which, const GemvParams& p, const uint8_t* codes, const uint8_t* scales, int K,
                            hipStream_t s) {
  const int NB = (K + 127) / 128;
  // one split covers kQ4MaxBlocks blocks: the K of QKV, O and gate/up, and
  // kMaxSplit splits of the down projection's K (checked with the shape)
  if ((which != Q4Linear::DOWN && NB > kQ4MaxBlocks) || NB > kMaxSplit * kQ4MaxBlocks) return hipErrorInvalidValue;
  switch ((p.rows + 7) / 8) {
    case 1: return launch_q4_nt<1>(which, p, codes, scales, NB, s);
    case 2: return launch_q4_nt<2>(which, p, codes, scales, NB, s);
    case 3: return launch_q4_nt<3>(which, p, codes, scales, NB, s);
    case 4: return launch_q4_nt<4>(which, p, codes, scales, NB, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sd
