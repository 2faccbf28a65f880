// gfx950 kernels of one decoder forward pass (prefill chunk, decode step or
// block verify; only the row count differs).
//
// Definitions: "SpecDec-Context-Scaling 项目解读" (richardf123.github.io),
// section 2.2 (one self-built forward for prefill, decode and block
// verification, appending K/V to a cache whose length the caller trims) and
// section 8 (the same target logits must come out of the M=1 and M=k
// shapes).  The decoder is the pre-norm RMSNorm / rotate-half RoPE /
// grouped-query attention / SwiGLU stack.
//
// Every matrix product here is a weight-streaming skinny product: M <= 32
// activation rows against a bf16 weight that is read once from HBM.  The
// weights are pre-packed into MFMA operand tiles so each wave-wide 16-byte
// load is a contiguous 1 KiB; activations are split into bf16 hi + lo parts
// in the second operand, so the fp32-accumulating bf16 MFMA keeps ~16 bits
// of the fp32 activations.  Row results never depend on which other rows
// share the pass: every reduction runs in an order fixed by the row's own
// data layout, never by the row count.
#include "gemv_common.h"

#include <math.h>

namespace sd {

// Launch shapes of the skinny products: (row groups per workgroup, k-split
// waves per row group, weight tiles in flight per wave), and the K splits of
// the down projection (kDownSplit).  All are fixed per matrix, never by the row count, so
// a row's summation order does not depend on how many rows share the pass.
#ifndef SD_CFG_QKV
#define SD_CFG_QKV 1, 8, 6
#endif
#ifndef SD_CFG_O
#define SD_CFG_O 1, 4, 12
#endif
#ifndef SD_CFG_GU
#define SD_CFG_GU 1, 8, 6
#endif
#ifndef SD_CFG_DOWN
#define SD_CFG_DOWN 1, 8, 19
#endif
#ifndef SD_CFG_LM
#define SD_CFG_LM 2, 2, 12
#endif
// U only sets how many tiles a wave keeps in flight (its k-blocks are
// accumulated in order either way), so multi-tile passes cap it by the
// registers a wave of this workgroup size may hold: (1 + NT) 4-register
// tiles per k-block in flight, ~40 registers for the rest.
// Passes of three or four column tiles keep at most 128 registers for tiles
// in flight (two waves per SIMD or more; 29-row forwards 2418 -> 2285 us).
#ifndef SD_WIDE_VGPRS
#define SD_WIDE_VGPRS 128
#endif
template <int R, int W, int T>
struct LaunchCfg {
  static constexpr int WG_ROWS = R, WK = W, THREADS = 64 * R * W;
  static constexpr int kVgprsFit = (512 / (THREADS / 256 > 1 ? THREADS / 256 : 1)) < 256
                                       ? 512 / (THREADS / 256 > 1 ? THREADS / 256 : 1) : 256;
  template <int NT>
  static constexpr int kVgprs = NT >= 3 && kVgprsFit > SD_WIDE_VGPRS ? SD_WIDE_VGPRS : kVgprsFit;
  template <int NT>
  static constexpr int U = NT == 1 ? T
                                   : ((kVgprs<NT> - 40) / ((1 + NT) * 4) < T
                                          ? ((kVgprs<NT> - 40) / ((1 + NT) * 4) > 1 ? (kVgprs<NT> - 40) / ((1 + NT) * 4)
                                                                                     : 1)
                                          : T);
};
using CfgQKV = LaunchCfg<SD_CFG_QKV>;
using CfgO = LaunchCfg<SD_CFG_O>;
using CfgGU = LaunchCfg<SD_CFG_GU>;
using CfgDown = LaunchCfg<SD_CFG_DOWN>;
using CfgLM = LaunchCfg<SD_CFG_LM>;
static_assert(CfgDown::WG_ROWS == 1, "the split-K launch maps one row group per workgroup");
static_assert(kDownSplit <= kMaxSplit, "partial buffer holds kMaxSplit splits");
#ifndef SD_O_SPLIT
#define SD_O_SPLIT 1
#endif
constexpr int kOSplit = SD_O_SPLIT;   // K splits of the O projection (1: one workgroup per row group)
static_assert(kOSplit <= kMaxSplit && (kOSplit == 1 || CfgO::WG_ROWS == 1), "O split-K shape");


hipError_t launch_advance(int32_t* d_len, int rows, int max_len, const int32_t* gate, hipStream_t s);

// ---------------------------------------------------------------------------
// Packing (setup): row-major bf16 -> MFMA weight tiles.
// ---------------------------------------------------------------------------
__global__ void pack_linear_kernel(const bf16_bits* __restrict__ src, int rows, int K, int kind, int hd,
                                   int group_base, bf16_bits* __restrict__ dst) {
  const int kc_per_row = K >> 3;
  const size_t total = (size_t)rows * kc_per_row;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    int r = (int)(idx / kc_per_row);
    int k = (int)(idx % kc_per_row) * 8;
    int g, i;
    pack_row_slot(kind, r, hd, g, i);
    const int KB = K >> 5;
    const int kb = k >> 5, s = (k >> 3) & 3;
    size_t d = (((size_t)(group_base + g) * KB + kb) * 64 + (s * 16 + i)) * 8;
    const uint4* sp = reinterpret_cast<const uint4*>(src + (size_t)r * K + k);
    *reinterpret_cast<uint4*>(dst + d) = *sp;
  }
}

__global__ void pack_norm_kernel(const bf16_bits* __restrict__ src, int n, float* __restrict__ dst) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf2f(src[i]);
}

__global__ void copy_u16_kernel(const bf16_bits* __restrict__ src, size_t n, bf16_bits* __restrict__ dst) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_pack(const Dims& d, int index, const void* srcv, void* blobv, const BlobLayout& lay,
                       hipStream_t s) {
  const bf16_bits* src = static_cast<const bf16_bits*>(srcv);
  char* blob = static_cast<char*>(blobv);
  auto lin = [&](size_t off, int rows, int K, int kind, int gbase) {
    size_t total = (size_t)rows * (K / 8);
    int blocks = (int)((total + 255) / 256);
    if (blocks > 65535 * 4) blocks = 65535 * 4;
    pack_linear_kernel<<<blocks, 256, 0, s>>>(src, rows, K, kind, d.hd, gbase,
                                               reinterpret_cast<bf16_bits*>(blob + off));
  };
  auto norm = [&](size_t off) {
    pack_norm_kernel<<<(d.H + 255) / 256, 256, 0, s>>>(src, d.H, reinterpret_cast<float*>(blob + off));
  };
  const int n_tensors = 3 + 9 * d.L;
  if (index == 0) {
    size_t n = (size_t)d.V * d.H;
    copy_u16_kernel<<<4096, 256, 0, s>>>(src, n, reinterpret_cast<bf16_bits*>(blob + lay.embed));
  } else if (index == n_tensors - 2) {
    norm(lay.final_norm);
  } else if (index == n_tensors - 1) {
    lin(lay.lm_head, d.V, d.H, PACK_PLAIN, 0);
  } else {
    int l = (index - 1) / 9, which = (index - 1) % 9;
    const LayerOffsets& o = lay.layer[l];
    const int qg = d.qdim() / 16, kg = d.kvdim() / 16;
    switch (which) {
      case 0: norm(o.attn_norm); break;
      case 1: lin(o.wqkv, d.qdim(), d.H, PACK_ROPE, 0); break;
      case 2: lin(o.wqkv, d.kvdim(), d.H, PACK_ROPE, qg); break;
      case 3: lin(o.wqkv, d.kvdim(), d.H, PACK_PLAIN, qg + kg); break;
      case 4: lin(o.wo, d.H, d.qdim(), PACK_PLAIN, 0); break;
      case 5: norm(o.mlp_norm); break;
      case 6: lin(o.wgu, d.F, d.H, PACK_GATE, 0); break;
      case 7: lin(o.wgu, d.F, d.H, PACK_UP, 0); break;
      case 8: lin(o.wdown, d.H, d.F, PACK_PLAIN, 0); break;
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Embedding gather: x = E[token]; writes x, the activation tiles of
// x * gain (first attention norm) and the per-16-feature sums of squares.
// ---------------------------------------------------------------------------
// Tree forwards (parents non-null): row m is node n0 + m of a tree whose
// nodes 0 .. n0 - 1 already sit in the cache (node i at slot base + i, base =
// length - n0).  Its workgroup stores depth - n0 (so that the row's RoPE
// position is length + that = base + depth) and the node's ancestors-or-self
// as a kMaxTreeNodes-bit mask over the tree's nodes; thread w < kTreeWords
// walks the parent chain for word w.  A parent must be an earlier node:
// otherwise the row is flagged and taken as a root.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens, const bf16_bits* __restrict__ E,
                                                    const float* __restrict__ gain, int H, int V, int rows,
                                                    float* __restrict__ x, bf16_bits* __restrict__ xb,
                                                    float* __restrict__ ss, const int32_t* __restrict__ d_len,
                                                    int max_len, int32_t* err, const int32_t* gate,
                                                    const int32_t* __restrict__ parents, int n0,
                                                    int32_t* __restrict__ tree) {
  if (gate && *gate == 0) return;
  const int m = blockIdx.x;
  if (parents && (int)threadIdx.x < kTreeWords) {
    const int wd = threadIdx.x, self = n0 + m;
    int depth = 0, node = self;
    bool bad = false;
    uint32_t word = (self >> 5) == wd ? 1u << (self & 31) : 0u;
    for (int step = 0; step < kMaxTreeNodes; ++step) {
      const int par = parents[node];
      if (par < 0) break;
      if (par >= node) { bad = true; break; }
      if ((par >> 5) == wd) word |= 1u << (par & 31);
      ++depth;
      node = par;
    }
    if (bad) {
      if (wd == 0) raise_error(err, kErrTree);
      depth = 0;
      word = (self >> 5) == wd ? 1u << (self & 31) : 0u;
    }
    if (wd == 0) tree[m] = depth - n0;
    tree[kMaxRows + m * kTreeWords + wd] = (int32_t)word;
  }
  int tok = tokens[m];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) raise_error(err, kErrTable);
    tok = 0;
  }
  if (m == 0 && threadIdx.x == 0 && *d_len + rows > max_len) raise_error(err, kErrCapacity);
  const bf16_bits* e = E + (size_t)tok * H;
  const int KB = H >> 5;
  for (int k = threadIdx.x; k < H; k += blockDim.x) {
    float v = bf2f(e[k]);
    x[(size_t)m * H + k] = v;
    btile_put(xb, KB, m, k, v * gain[k]);
  }
  const int NP = H >> 4;
  for (int g = threadIdx.x; g < NP; g += blockDim.x) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = bf2f(e[16 * g + i]);
      s = fmaf(v, v, s);
    }
    ss[(size_t)m * NP + g] = s;
  }
}

// ---------------------------------------------------------------------------
// Weight-streaming MFMA GEMV.
// ---------------------------------------------------------------------------
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// One batch of exactly R tiles: straight-line loads (a guarded load into a
// register array makes the compiler wait on it), then `issued` once when it
// is the wave's first batch, then the products in k order.  The activation
// tiles (cache hits) are requested before the weight tiles: the load
// counter completes in request order, so the product of tile u then waits
// for weight tiles 0..u only, not for the whole batch.
template <int NT, int R, typename Issued>
__device__ __forceinline__ void mfma_batch(const i32x4_t* a, const i32x4_t* const (&b)[NT], int i,
                                           f32x4_t (&acc)[NT], bool first, Issued& issued) {
  i32x4_t av[R];
  i32x4_t bv[R][NT];
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) bv[u][t] = b[t][(size_t)(i + u) * 64];
#pragma unroll
  for (int u = 0; u < R; ++u) av[u] = __builtin_nontemporal_load(a + (size_t)(i + u) * 64);
  if (first) {
    // the scheduling barriers keep the weight requests ahead of whatever
    // `issued` requests (the compiler would otherwise hoist those small
    // loads, and the waits they carry, above the weight stream)
    __builtin_amdgcn_sched_barrier(0);
    issued();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                      __builtin_bit_cast(bf16x8_t, bv[u][t]), acc[t], 0, 0, 0);
}

// The last r < U tiles of a wave's range, as a batch of exactly r.
template <int NT, int U, typename Issued>
__device__ __forceinline__ void mfma_tail(const i32x4_t* a, const i32x4_t* const (&b)[NT], int i, int r,
                                          f32x4_t (&acc)[NT], bool first, Issued& issued) {
  if constexpr (U > 1) {
    if (r == U - 1) mfma_batch<NT, (U > 1 ? U - 1 : 1)>(a, b, i, acc, first, issued);
    else mfma_tail<NT, (U > 1 ? U - 1 : 1)>(a, b, i, r, acc, first, issued);
  }
}

// Streams the weight tiles of one row group over k-blocks [kb0, kb1) through
// MFMA, up to U tiles in flight per wave (the activation tiles are
// L2-resident).  Tiles travel as 32-bit integer vectors (bit-cast to bf16
// only at the MFMA).  kb0/kb1 are wave-uniform, so every branch here is a
// scalar one.  `issued` runs once, right after the first batch of loads has
// been requested (also when the wave has no k-blocks).  bslot[t] is the
// lane's 16-byte slot in the activation tiles of column tile t.
template <int NT, int U, typename Issued>
__device__ __forceinline__ void mfma_stream(const bf16x8_t* __restrict__ A, const bf16x8_t* __restrict__ B, int KB,
                                            int kb0, int kb1, int lane, const int (&bslot)[NT], f32x4_t (&acc)[NT],
                                            Issued&& issued) {
  const i32x4_t* a = reinterpret_cast<const i32x4_t*>(A) + (size_t)kb0 * 64 + lane;
  const i32x4_t* b[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    b[t] = reinterpret_cast<const i32x4_t*>(B) + (size_t)(t * KB + kb0) * 64 + bslot[t];
  const int n = kb1 - kb0;
  if (n <= 0) {
    issued();
    return;
  }
  int i = 0;
  for (; i + U <= n; i += U) mfma_batch<NT, U>(a, b, i, acc, i == 0, issued);
  if (i < n) mfma_tail<NT, U>(a, b, i, n - i, acc, i == 0, issued);
}

// The same stream for a workgroup of R row groups that share the k-split:
// the R waves on one k-range load the batch's activation tiles once between
// them (wave rg takes tiles rg, rg + R, ...) and exchange them through LDS,
// so each wave requests U / R activation tiles per batch instead of U.  The
// products and their order are those of mfma_stream.  Every wave of the
// workgroup runs the same number of batches (nmax is the longest k-range),
// also when its row group is past the matrix (active == false: it still
// loads its share of the activation tiles).
template <int NT, int U, int R, typename Issued>
__device__ __forceinline__ void mfma_stream_shared(const bf16x8_t* __restrict__ A, bool active,
                                                   const bf16x8_t* __restrict__ B, int KB, int kb0, int kb1, int nmax,
                                                   int rg, int lane, const int (&bslot)[NT], f32x4_t (&acc)[NT],
                                                   i32x4_t (*bsh)[NT][64], Issued&& issued) {
  static_assert(U % R == 0, "each wave loads an equal share of a batch");
  constexpr int US = U / R;
  const i32x4_t* a = reinterpret_cast<const i32x4_t*>(A) + (size_t)kb0 * 64 + lane;
  const i32x4_t* b[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    b[t] = reinterpret_cast<const i32x4_t*>(B) + (size_t)(t * KB + kb0) * 64 + bslot[t];
  const int n = kb1 - kb0;   // equal for the R waves of this k-range
  for (int i = 0; i < nmax; i += U) {
    if (i > 0) __syncthreads();   // the previous batch's tiles have been read
    // this wave's share of the activation tiles first, then its weight tiles
    i32x4_t bs[US][NT];
    if (n > 0)
#pragma unroll
      for (int j = 0; j < US; ++j) {
        const int u = rg + R * j, kb = i + u < n ? i + u : n - 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) bs[j][t] = b[t][(size_t)kb * 64];
      }
    i32x4_t av[U];
    if (active && n > 0)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kb = i + u < n ? i + u : n - 1;
        av[u] = __builtin_nontemporal_load(a + (size_t)kb * 64);
      }
    if (i == 0) {
      __builtin_amdgcn_sched_barrier(0);
      issued();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (n > 0)
#pragma unroll
      for (int j = 0; j < US; ++j)
#pragma unroll
        for (int t = 0; t < NT; ++t) bsh[rg + R * j][t][lane] = bs[j][t];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (active)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i + u < n)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                            __builtin_bit_cast(bf16x8_t, bsh[u][t][lane]), acc[t], 0,
                                                            0, 0);
  }
  if (nmax <= 0) issued();
}

// ---------------------------------------------------------------------------
// Vector alternative to the MFMA product, built with SD_VECTOR_GEMV=1 to
// measure the MFMA choice against: each lane keeps the weight tile's eight
// inputs of its row, takes each activation row's hi and lo values of those
// inputs from the operand tile by a row broadcast (DPP), and accumulates with
// the bf16 two-way dot product in fp32; the four input quarters of a row are
// added at the end.  Its summation order differs from the MFMA's, so the two
// agree within rounding, not bit for bit.
// ---------------------------------------------------------------------------
#ifndef SD_VECTOR_GEMV
#define SD_VECTOR_GEMV 0
#endif
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int C>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + C, 0xF, 0xF, false);
}
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
// activation rows Mi.. of one tile (operand columns 2m and 2m + 1) against
// the lane's eight weights
template <int Mi>
__device__ __forceinline__ void vec_rows(const i32x4_t& a, const i32x4_t& b, float (&acc)[8], int mmax) {
  if constexpr (Mi < 8) {
    if (Mi < mmax) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t ad = (uint32_t)a[d], bd = (uint32_t)b[d];
        acc[Mi] = dot2bf(ad, row_bcast<2 * Mi>(bd), acc[Mi]);
        acc[Mi] = dot2bf(ad, row_bcast<2 * Mi + 1>(bd), acc[Mi]);
      }
      vec_rows<Mi + 1>(a, b, acc, mmax);
    }
  }
}

template <int NT, int R, typename Issued>
__device__ __forceinline__ void vec_batch(const i32x4_t* a, const i32x4_t* const (&b)[NT], int i, float (&vacc)[NT][8],
                                          int M, bool first, Issued& issued) {
  i32x4_t av[R];
  i32x4_t bv[R][NT];
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) bv[u][t] = b[t][(size_t)(i + u) * 64];
#pragma unroll
  for (int u = 0; u < R; ++u) av[u] = __builtin_nontemporal_load(a + (size_t)(i + u) * 64);
  if (first) {
    __builtin_amdgcn_sched_barrier(0);
    issued();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) vec_rows<0>(av[u], bv[u][t], vacc[t], M - 8 * t);
}

template <int NT, int U, typename Issued>
__device__ __forceinline__ void vec_tail(const i32x4_t* a, const i32x4_t* const (&b)[NT], int i, int r,
                                         float (&vacc)[NT][8], int M, bool first, Issued& issued) {
  if constexpr (U > 1) {
    if (r == U - 1) vec_batch<NT, (U > 1 ? U - 1 : 1)>(a, b, i, vacc, M, first, issued);
    else vec_tail<NT, (U > 1 ? U - 1 : 1)>(a, b, i, r, vacc, M, first, issued);
  }
}

template <int NT, int U, typename Issued>
__device__ __forceinline__ void vec_stream(const bf16x8_t* __restrict__ A, const bf16x8_t* __restrict__ B, int KB,
                                           int kb0, int kb1, int lane, const int (&bslot)[NT], float (&vacc)[NT][8],
                                           int M, Issued&& issued) {
  const i32x4_t* a = reinterpret_cast<const i32x4_t*>(A) + (size_t)kb0 * 64 + lane;
  const i32x4_t* b[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    b[t] = reinterpret_cast<const i32x4_t*>(B) + (size_t)(t * KB + kb0) * 64 + bslot[t];
  const int n = kb1 - kb0;
  if (n <= 0) {
    issued();
    return;
  }
  int i = 0;
  for (; i + U <= n; i += U) vec_batch<NT, U>(a, b, i, vacc, M, i == 0, issued);
  if (i < n) vec_tail<NT, U>(a, b, i, n - i, vacc, M, i == 0, issued);
}

// The fields the weight stream needs come first as plain arguments, which
// the launch preloads into scalar registers; the rest of GemvParams is read
// from the argument block where it is used.
template <int NT, int WG_ROWS, int WK, int U, Epi E>
__global__ __launch_bounds__(64 * WG_ROWS * WK) void gemv_kernel(const int32_t* gate, const int32_t* d_len,
                                                                 const bf16x8_t* __restrict__ A,
                                                                 const bf16x8_t* __restrict__ B, int KB, int n_groups,
                                                                 int rows, int nsplit_arg, GemvParams p) {
  EpiPre<NT * 8> pre;
  // the cache position is waited on only in the epilogue prefetch; without
  // a gate the weight stream starts without waiting on any load
  if constexpr (E == Epi::QKV) pre.pos0 = *d_len;
  if (gate) {
    if (*gate == 0) return;
  }
  constexpr int NW = WG_ROWS * WK;
  constexpr int NC = NT * 8;        // activation rows covered
  constexpr int RPW = (NC + NW - 1) / NW;   // norm rows per wave (NC covers every row)
  // row groups of a workgroup share their activation tiles through LDS when
  // the batch fits (the arithmetic is the same either way)
  constexpr bool kShareB = !SD_VECTOR_GEMV && WG_ROWS > 1 && U % WG_ROWS == 0 && WK * U * NT * 1024 <= 48 * 1024;
  __shared__ i32x4_t bsh[kShareB ? WK : 1][kShareB ? U : 1][NT][64];
  __shared__ float red[NW][16][NC + 1];
  __shared__ float fin[E == Epi::LMHEAD ? WG_ROWS : 1][16][NC + 1];   // whole-workgroup epilogue only
  __shared__ float rsc[kMaxRows];

  const int lane = threadIdx.x & 63;
  // wave index as a provably uniform value: the k-range guards below become
  // scalar branches instead of EXEC-masked regions around MFMA operands
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = w / WK, ks = w % WK;
  const int nsplit = (E == Epi::PARTIAL) ? nsplit_arg : 1;
  // split-K: the splits of row group g are workgroups 8 (nsplit (g / 8) + s)
  // + g % 8, eight apart, so round-robin dispatch over the eight XCDs puts
  // a row group's producers and finisher on one XCD (and the producers
  // first); the launch rounds the row groups up to a multiple of 8
  const unsigned slot = blockIdx.x >> 3;
  const int sidx = (E == Epi::PARTIAL) ? (int)(slot % (unsigned)nsplit) : 0;
  const int g = (E == Epi::PARTIAL) ? (int)((slot / (unsigned)nsplit) * 8 + (blockIdx.x & 7))
                                    : (int)(blockIdx.x * WG_ROWS + rg);
  const int M = rows;

  // Right after the first weight requests (which need only the preloaded
  // arguments): the sums of squares of the normalised input, the epilogue
  // wave's residual operands and RoPE rotations.  They are used only after
  // the product, so their latency hides under the weight stream.
  constexpr bool kNorm = (E == Epi::QKV || E == Epi::SWIGLU || E == Epi::LMHEAD);
  float ssv[RPW][4];
  auto prefetch = [&] {
    if constexpr (kNorm) norm_prefetch<RPW, NW>(p, w, lane, M, ssv);
    if (ks == 0) {
      epi_prefetch_x<E, NC>(p, lane, g, M, pre);
      epi_prefetch_rope<E, NC>(p, lane, g, M, pre);
    }
  };

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // 32-bit unsigned arithmetic: every term is small (split index < 8,
  // k-blocks < 2^16), and a 64-bit division costs hundreds of instructions
  const unsigned uk = (unsigned)KB, un = (unsigned)nsplit;
  int s0 = (int)((unsigned)sidx * uk / un), s1 = (int)((unsigned)(sidx + 1) * uk / un);
  if (E == Epi::PARTIAL && nsplit == 2) {
    // the producer's smaller share is in memory by the time the finisher
    // has streamed its larger one (when that still fits one batch per wave
    // of the one-tile launch shape: the cut depends on the matrix only, never
    // on the row count)
    const unsigned sa = uk * kSplit0Share / 64u;
    const unsigned cut = (uk - sa + WK - 1) / WK <= (unsigned)CfgDown::template U<1> ? sa : uk / 2u;
    s0 = sidx == 0 ? 0 : (int)cut;
    s1 = sidx == 0 ? (int)cut : (int)uk;
  }
  const unsigned span = (unsigned)(s1 - s0);
  const int kb0 = s0 + (int)((unsigned)ks * span / WK), kb1 = s0 + (int)((unsigned)(ks + 1) * span / WK);
  // the lane's activation slot per column tile: operand columns past the
  // tile's rows read row 0's slot of the same part (their products are never
  // used), so a pass of M rows fetches 256 ceil(M / 2) bytes of each tile
  int bslot[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = lane & 15;
    bslot[t] = btile_slot((col >> 1) < M - 8 * t ? col : (col & 1), lane >> 4);
  }
#if SD_VECTOR_GEMV
  float vacc[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int m = 0; m < 8; ++m) vacc[t][m] = 0.f;
  if (g < n_groups) vec_stream<NT, U>(A + (size_t)g * KB * 64, B, KB, kb0, kb1, lane, bslot, vacc, M, prefetch);
  else prefetch();
  if constexpr (kNorm) norm_finish<RPW, NW>(p, w, lane, M, ssv, rsc);
  // the four input quarters of each row, then the wave's partials
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float v = vacc[t][m];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (lane < 16) red[w][lane][t * 8 + m] = v;
    }
  gemv_reduce_epilogue<NT, WG_ROWS, WK, E>(p, red, fin, rsc, pre, w, lane, rg, ks, g, sidx, M, n_groups);
  return;
#endif
  if constexpr (kShareB) {
    const int nmax = (int)((span + WK - 1) / WK);
    const int gg = g < n_groups ? g : 0;
    mfma_stream_shared<NT, U, WG_ROWS>(A + (size_t)gg * KB * 64, g < n_groups, B, KB, kb0, kb1, nmax, rg, lane, bslot,
                                       acc, bsh[ks], prefetch);
  } else if (g < n_groups) {
    mfma_stream<NT, U>(A + (size_t)g * KB * 64, B, KB, kb0, kb1, lane, bslot, acc, prefetch);
  } else {
    prefetch();
  }
  if constexpr (kNorm) norm_finish<RPW, NW>(p, w, lane, M, ssv, rsc);
  gemv_finish<NT, WG_ROWS, WK, E>(p, acc, red, fin, rsc, pre, w, lane, rg, ks, g, sidx, M, n_groups);
}

// Gate/up with several row groups per workgroup: wave w keeps the activation
// tiles of its k-range in registers while the workgroup's row groups stream
// past, and requests the next group's weight tiles before the current
// group's products.  The k-split, the product order and the epilogue's sums
// are those of gemv_kernel, so the results are the same bits.  KBW bounds
// the k-blocks of a wave's range (shorter ranges re-read their last tile and
// skip its product).
template <int NT, int WK, int KBW, int RGMAX>
__global__ __launch_bounds__(64 * WK) void gemv_rg_kernel(const int32_t* gate, const bf16x8_t* __restrict__ A,
                                                          const bf16x8_t* __restrict__ B, int KB, int n_groups,
                                                          int rows, int rg, GemvParams p) {
  if (gate) {
    if (*gate == 0) return;
  }
  constexpr int NC = NT * 8;
  constexpr int RPW = (NC + WK - 1) / WK;   // norm rows per wave
  __shared__ float red[RGMAX * WK][16][NC + 1];
  __shared__ float rsc[kMaxRows];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = rows;
  const int g0 = blockIdx.x * rg;
  int nrg = n_groups - g0;
  if (nrg > rg) nrg = rg;   // rg <= RGMAX (checked by the launch)
  const unsigned uk = (unsigned)KB;
  const int kb0 = (int)((unsigned)w * uk / WK), kb1 = (int)((unsigned)(w + 1) * uk / WK);
  const int n = kb1 - kb0;   // 1 .. KBW (checked by the launch)
  int bslot[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = lane & 15;
    bslot[t] = btile_slot((col >> 1) < M - 8 * t ? col : (col & 1), lane >> 4);
  }
  // the wave's activation tiles, once
  i32x4_t bv[KBW][NT];
#pragma unroll
  for (int j = 0; j < KBW; ++j) {
    const int kb = kb0 + (j < n ? j : n - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bv[j][t] = reinterpret_cast<const i32x4_t*>(B)[(size_t)(t * KB + kb) * 64 + bslot[t]];
  }
  const i32x4_t* a0 = reinterpret_cast<const i32x4_t*>(A) + (size_t)kb0 * 64 + lane;
  i32x4_t av[2][KBW];
  auto load_a = [&](int gg, i32x4_t(&dst)[KBW]) {
    const i32x4_t* a = a0 + (size_t)gg * KB * 64;
#pragma unroll
    for (int j = 0; j < KBW; ++j) dst[j] = __builtin_nontemporal_load(a + (size_t)(j < n ? j : n - 1) * 64);
  };
  load_a(g0, av[0]);
  float ssv[RPW][4];
  __builtin_amdgcn_sched_barrier(0);
  norm_prefetch<RPW, WK>(p, w, lane, M, ssv);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int rr = 0; rr < RGMAX; ++rr) {
    if (rr >= nrg) break;
    if (rr + 1 < nrg) load_a(g0 + rr + 1, av[(rr + 1) & 1]);
    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KBW; ++j)
      if (j < n)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[rr & 1][j]),
                                                          __builtin_bit_cast(bf16x8_t, bv[j][t]), acc[t], 0, 0, 0);
    // hi and lo columns added in registers: the wave's partials of this group
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[t][r] + swap1(acc[t][r]);
        if ((lane & 1) == 0) red[rr * WK + w][4 * (lane >> 4) + r][t * 8 + ((lane & 15) >> 1)] = v;
      }
  }
  norm_finish<RPW, WK>(p, w, lane, M, ssv, rsc);
  __syncthreads();
  // SwiGLU epilogue: wave w takes row groups w, w + WK, ...; it sums the
  // k-split partials of each entry in wave order
  const int KBo = p.F >> 5;
  for (int rr = w; rr < nrg; rr += WK) {
    const int g = g0 + rr;
    for (int idx = lane; idx < 8 * M; idx += 64) {
      const int i = idx & 7, m = idx >> 3;
      float gt = 0.f, up = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < WK; ++s2) {
        gt += red[rr * WK + s2][i][m];
        up += red[rr * WK + s2][i + 8][m];
      }
      const float r = rsc[m];
      gt *= r;
      up *= r;
      btile_put(p.hb_out, KBo, m, 8 * g + i, gt / (1.0f + __expf(-gt)) * up);
    }
  }
}

// The same for passes of two or more column tiles, whose partials of every
// row group would not fit LDS at once: the waves' partials of a row group go
// to one of two LDS slots, one barrier per row group, and wave rr % WK runs
// row group rr's epilogue while the others stream the next group (the next
// barrier keeps a slot from being rewritten before its epilogue has read
// it).  Same k-split, product order and sums as gemv_kernel.
template <int NT, int WK, int KBW>
__global__ __launch_bounds__(64 * WK) void gemv_rg2_kernel(const int32_t* gate, const bf16x8_t* __restrict__ A,
                                                           const bf16x8_t* __restrict__ B, int KB, int n_groups,
                                                           int rows, int rg, GemvParams p) {
  if (gate) {
    if (*gate == 0) return;
  }
  constexpr int NC = NT * 8;
  constexpr int RPW = (NC + WK - 1) / WK;   // norm rows per wave
  __shared__ float red[2][WK][16][NC + 1];
  __shared__ float rsc[kMaxRows];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = rows;
  const int g0 = blockIdx.x * rg;
  int nrg = n_groups - g0;
  if (nrg > rg) nrg = rg;
  const unsigned uk = (unsigned)KB;
  const int kb0 = (int)((unsigned)w * uk / WK), kb1 = (int)((unsigned)(w + 1) * uk / WK);
  const int n = kb1 - kb0;   // 1 .. KBW (checked by the launch)
  int bslot[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = lane & 15;
    bslot[t] = btile_slot((col >> 1) < M - 8 * t ? col : (col & 1), lane >> 4);
  }
  i32x4_t bv[KBW][NT];
#pragma unroll
  for (int j = 0; j < KBW; ++j) {
    const int kb = kb0 + (j < n ? j : n - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bv[j][t] = reinterpret_cast<const i32x4_t*>(B)[(size_t)(t * KB + kb) * 64 + bslot[t]];
  }
  const i32x4_t* a0 = reinterpret_cast<const i32x4_t*>(A) + (size_t)kb0 * 64 + lane;
  auto load_a = [&](int gg, i32x4_t(&dst)[KBW]) {
    const i32x4_t* a = a0 + (size_t)gg * KB * 64;
#pragma unroll
    for (int j = 0; j < KBW; ++j) dst[j] = __builtin_nontemporal_load(a + (size_t)(j < n ? j : n - 1) * 64);
  };
  i32x4_t av0[KBW], av1[KBW];
  load_a(g0, av0);
  float ssv[RPW][4];
  __builtin_amdgcn_sched_barrier(0);
  norm_prefetch<RPW, WK>(p, w, lane, M, ssv);
  __builtin_amdgcn_sched_barrier(0);
  const int KBo = p.F >> 5;
  auto step = [&](int rr, i32x4_t(&cur)[KBW], i32x4_t(&nxt)[KBW]) {
    if (rr + 1 < nrg) load_a(g0 + rr + 1, nxt);
    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KBW; ++j)
      if (j < n)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur[j]),
                                                          __builtin_bit_cast(bf16x8_t, bv[j][t]), acc[t], 0, 0, 0);
    float(*slot)[16][NC + 1] = red[rr & 1];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[t][r] + swap1(acc[t][r]);
        if ((lane & 1) == 0) slot[w][4 * (lane >> 4) + r][t * 8 + ((lane & 15) >> 1)] = v;
      }
    if (rr == 0) norm_finish<RPW, WK>(p, w, lane, M, ssv, rsc);
    __syncthreads();
    if (w == rr % WK) {
      const int g = g0 + rr;
      for (int idx = lane; idx < 8 * M; idx += 64) {
        const int i = idx & 7, m = idx >> 3;
        float gt = 0.f, up = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < WK; ++s2) {
          gt += slot[s2][i][m];
          up += slot[s2][i + 8][m];
        }
        const float r = rsc[m];
        gt *= r;
        up *= r;
        btile_put(p.hb_out, KBo, m, 8 * g + i, gt / (1.0f + __expf(-gt)) * up);
      }
    }
  };
  for (int rr = 0; rr < nrg; rr += 2) {
    step(rr, av0, av1);
    if (rr + 1 < nrg) step(rr + 1, av1, av0);
  }
}

// The row-group forms of gate/up: about one workgroup per CU, each taking
// rg = ceil(row groups / 256) of them, for a k-split of at most 8 k-blocks a
// wave; gemv_rg_kernel for passes of 3 to 8 rows, gemv_rg2_kernel for 17 to
// 32 (where the activation tiles outweigh the weights).  Passes of 1, 2 and
// 9 to 16 rows keep one row group per workgroup (faster there).  Returns
// false when no row-group form applies; every form gives the same bits, so
// the choice never shows in the results.
constexpr int kGuRgMinRows = 3;

template <int NT>
static bool launch_gu_rg(hipStream_t s, const GemvParams& p) {
  constexpr int WK = CfgGU::WK;
  constexpr int RGMAX = 8;
  // the vector comparison build keeps every product on gemv_kernel
  if (SD_VECTOR_GEMV || p.rows < kGuRgMinRows || p.KB < WK) return false;
  const int kbw = (p.KB + WK - 1) / WK;
  const int rg = (p.n_groups + 255) / 256;
  if (kbw > 8) return false;
  const int grid = (p.n_groups + rg - 1) / rg;
  if constexpr (NT == 1) {
    if (rg > RGMAX) return false;
    if (kbw <= 2)
      gemv_rg_kernel<NT, WK, 2, RGMAX><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    else if (kbw <= 4)
      gemv_rg_kernel<NT, WK, 4, RGMAX><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    else if (kbw <= 6)
      gemv_rg_kernel<NT, WK, 6, RGMAX><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    else
      gemv_rg_kernel<NT, WK, 8, RGMAX><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    return true;
  } else if constexpr (NT >= 3) {
    if (kbw <= 2)
      gemv_rg2_kernel<NT, WK, 2><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    else if (kbw <= 4)
      gemv_rg2_kernel<NT, WK, 4><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    else if (kbw <= 6)
      gemv_rg2_kernel<NT, WK, 6><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    else
      gemv_rg2_kernel<NT, WK, 8><<<grid, 64 * WK, 0, s>>>(p.gate, p.A, p.B, p.KB, p.n_groups, p.rows, rg, p);
    return true;
  } else {
    return false;
  }
}

// ---------------------------------------------------------------------------
// Causal grouped-query attention over the cache, split by 64-key chunks whose
// boundaries are fixed by absolute key index, then a fixed-order merge of the
// chunk partials per output.
//
// Chunk partial: one workgroup per (kv head, chunk, query-tile slice) with
// one wave per 16 keys.  Wave w loads the K rows of keys 16w..16w+15
// (operand A of S^T = K Q^T; 8 consecutive head dims per lane) and the V^T
// rows of its share of the head dims (operand A of O^T = V^T P^T over all
// keys of the chunk; the cache
// keeps V transposed so 8 consecutive keys of one head dim are 16 contiguous
// bytes), so each wave keeps a small, fixed set of loads in flight.  Per
// 16-row query tile: each wave's 16 x 16 score tile goes to LDS with the
// causal mask applied; every wave then reads the chunk's scores of its lanes' query
// rows, forms the row max and sum of exp over the chunk in one fixed order
// (so all waves hold identical values) and P^T for its own output dims.  The
// bf16 hi/lo split of q and of P runs along the MFMA k dimension (two MFMAs
// into one accumulator).  Keys past the current length are masked in the
// scores and zeroed in V^T.
// ---------------------------------------------------------------------------
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void pack_hilo8(const float (&v)[8], i32x4_t& hi_out, i32x4_t& lo_out) {
  u16x8_t h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16_bits hb = f2bf(v[e]);
    h[e] = hb;
    l[e] = f2bf(v[e] - bf2f(hb));
  }
  hi_out = __builtin_bit_cast(i32x4_t, h);
  lo_out = __builtin_bit_cast(i32x4_t, l);
}

__device__ __forceinline__ f32x4_t mfma_i(const i32x4_t& a, const i32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
                                                 0, 0);
}

constexpr int kAttnWaves = kAttnChunk / 16;   // waves per chunk workgroup: 16 keys each
#ifndef SD_ATTN_TILE_SPLIT
#define SD_ATTN_TILE_SPLIT 4
#endif
constexpr int kAttnTileSplit = SD_ATTN_TILE_SPLIT;   // workgroups sharing one chunk's query tiles
constexpr int kAttnMaxWgTiles = (kQTiles + kAttnTileSplit - 1) / kAttnTileSplit;   // query tiles per workgroup

// MAXT: query tiles a workgroup may hold (sizes the query staging in
// registers and LDS); the launch picks the smallest that covers its tiles.
template <int HD, int MAXT>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_chunk_kernel(
    const int32_t* gate, const int32_t* __restrict__ d_len, const bf16_bits* __restrict__ qb,
    const bf16_bits* __restrict__ Kc, const bf16_bits* __restrict__ Vt, int rows, int max_len, int lp, int G,
    float* __restrict__ o_part, float* __restrict__ ml_part, int max_chunks, const uint32_t* __restrict__ tree_anc,
    int tree_n0) {
  // the gate word (the length stands in for a null gate) and the length are
  // requested together, before any branch
  const int gv = *(gate ? gate : d_len);
  const int len = *d_len;
  constexpr int C = kAttnChunk;                 // keys per chunk
  constexpr int NW = kAttnWaves;
  constexpr int KBH = HD / 32;                  // k-blocks over the head dimension
  constexpr int DT = HD / 16;                   // 16-dim output tiles
  constexpr int DTW = (DT + NW - 1) / NW;       // output tiles per wave
  constexpr int KB2 = C / 32;                   // 32-key blocks of P^T
  __shared__ __attribute__((aligned(16))) float Pl[16][C + 4];
  static_assert(MAXT >= 1 && MAXT <= kAttnMaxWgTiles, "query tiles per workgroup");
  __shared__ i32x4_t qs[MAXT][KBH * 2][64];
  __shared__ uint32_t sanc[kMaxRows][kTreeWords];   // tree forwards: each row's ancestors-or-self
  const int c = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int T = len + rows;
  if (T > max_len) T = max_len;
  const int key0 = c * C;
  // one branch on both words, so neither load waits for the other
  if (((gate != nullptr) & (gv == 0)) | (key0 >= T)) return;
  const int R = rows * G, NTq = (R + 15) / 16;
  const int col = lane & 15, grp = lane >> 4;
  const size_t rstride = (size_t)kMaxRows * 8;

  // query tiles t0, t0 + TS, ... of this head (TS = gridDim.z workgroups per
  // chunk), staged once per workgroup in LDS: each wave loads a share
  const int t0 = blockIdx.z, TS = gridDim.z;
  if (t0 >= NTq) return;
  const int ntw = (NTq - t0 + TS - 1) / TS;   // tiles of this workgroup (<= MAXT)
  const i32x4_t* qh = reinterpret_cast<const i32x4_t*>(qb + qtile_head(h, HD));
  // this wave's share of the query tile parts, requested before the K/V rows
  // and written to LDS once every load of the wave is in flight
  // (unconditional loads, parts past the workgroup's tiles re-read part 0:
  // guarded loads into a register array would each be waited on)
  constexpr int QPW = (MAXT * KBH * 2 + NW - 1) / NW;
  i32x4_t qreg[QPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    int idx = w + NW * j;
    if (idx >= ntw * KBH * 2) idx = 0;
    const int pt = idx / (KBH * 2), part = idx % (KBH * 2);
    qreg[j] = qh[((size_t)(t0 + pt * TS) * KBH * 2 + part) * 64 + lane];
  }

  // this wave's 16 key rows
  const bf16_bits* kbase = Kc + (size_t)h * lp * HD;
  i32x4_t ka[KBH];
  {
    int krow = key0 + 16 * w + col;
    if (krow > T - 1) krow = T - 1;
#pragma unroll
    for (int kb = 0; kb < KBH; ++kb)
      ka[kb] = *reinterpret_cast<const i32x4_t*>(kbase + (size_t)krow * HD + kb * 32 + 8 * grp);
  }
  // this wave's V^T rows (head dims 16 * (DTW * w + j) + col), all keys of the chunk
  const bf16_bits* vbase = Vt + (size_t)h * HD * lp;
  i32x4_t va[DTW][KB2];
#pragma unroll
  for (int j = 0; j < DTW; ++j)
    if (DTW * w + j < DT)
#pragma unroll
      for (int kb2 = 0; kb2 < KB2; ++kb2)
        va[j][kb2] = *reinterpret_cast<const i32x4_t*>(vbase + (size_t)(16 * (DTW * w + j) + col) * lp + key0 +
                                                        32 * kb2 + 8 * grp);
#pragma unroll
  for (int kb2 = 0; kb2 < KB2; ++kb2) {
    const int nvalid = T - (key0 + 32 * kb2 + 8 * grp);
    if (nvalid < 8) {
      i32x4_t mask;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mask[j] = (2 * j < nvalid ? 0x0000FFFF : 0) | (2 * j + 1 < nvalid ? (int32_t)0xFFFF0000u : 0);
#pragma unroll
      for (int j = 0; j < DTW; ++j) va[j][kb2] &= mask;
    }
  }

#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int idx = w + NW * j;
    if (idx < ntw * KBH * 2) qs[idx / (KBH * 2)][idx % (KBH * 2)][lane] = qreg[j];
  }
  if (tree_anc)
    for (int i = threadIdx.x; i < rows * kTreeWords; i += blockDim.x) sanc[i / kTreeWords][i % kTreeWords] = tree_anc[i];
  const int tbase = len - tree_n0;   // tree forwards: the slot of node 0
  float* ob = o_part + ((size_t)h * max_chunks + c) * rstride * HD;
  float* mb = ml_part + ((size_t)h * max_chunks + c) * rstride * 2;
  // the staged query tiles are complete
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  for (int t = t0, pt = 0; t < NTq; t += TS, ++pt) {
    i32x4_t qt[KBH][2];
#pragma unroll
    for (int kb = 0; kb < KBH; ++kb) {
      qt[kb][0] = qs[pt][2 * kb][lane];
      qt[kb][1] = qs[pt][2 * kb + 1][lane];
    }
    const int row = 16 * t + col;
    const int m = row / G;
    const bool rvalid = row < R;
    // S^T tile of this wave's keys: lane (col = query row, grp) holds keys 16 w + 4 grp + r
    {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KBH; ++kb) {
        acc = mfma_i(ka[kb], qt[kb][0], acc);
        acc = mfma_i(ka[kb], qt[kb][1], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kidx = key0 + 16 * w + 4 * grp + r;
        // in a tree forward a key of the tree (slot tbase + node) is visible to
        // the node's descendants-or-self only
        const int bit = (kidx - tbase) & (kMaxTreeNodes - 1);
        const bool vis = !tree_anc || kidx < tbase || ((sanc[rvalid ? m : 0][bit >> 5] >> (bit & 31)) & 1u);
        const bool ok = rvalid && kidx < T && kidx <= len + m && vis;
        Pl[col][16 * w + 4 * grp + r] = ok ? acc[r] : -INFINITY;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // the row's C scores: lane (col, grp) holds keys 32 kb2 + 8 grp + e
    float sv[KB2][8];
#pragma unroll
    for (int kb2 = 0; kb2 < KB2; ++kb2) {
      const float4* src = reinterpret_cast<const float4*>(&Pl[col][32 * kb2 + 8 * grp]);
      const float4 p0 = src[0], p1 = src[1];
      sv[kb2][0] = p0.x; sv[kb2][1] = p0.y; sv[kb2][2] = p0.z; sv[kb2][3] = p0.w;
      sv[kb2][4] = p1.x; sv[kb2][5] = p1.y; sv[kb2][6] = p1.z; sv[kb2][7] = p1.w;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < KB2; ++kb2)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[kb2][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < KB2; ++kb2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = (mx == -INFINITY) ? 0.f : __expf(sv[kb2][e] - mx);
        sv[kb2][e] = pv;
        sum += pv;
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    if (w == 0 && grp == 0 && rvalid) { mb[row * 2] = mx; mb[row * 2 + 1] = sum; }
    // operand B: P^T (keys x query rows), hi and lo parts along k
    i32x4_t pb[KB2][2];
#pragma unroll
    for (int kb2 = 0; kb2 < KB2; ++kb2) pack_hilo8(sv[kb2], pb[kb2][0], pb[kb2][1]);
#pragma unroll
    for (int j = 0; j < DTW; ++j) {
      if (DTW * w + j >= DT) break;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb2 = 0; kb2 < KB2; ++kb2) {
        acc = mfma_i(va[j][kb2], pb[kb2][0], acc);
        acc = mfma_i(va[j][kb2], pb[kb2][1], acc);
      }
      // lane (col = query row, grp) holds O[row][16 (DTW w + j) + 4 grp + r]
      if (rvalid)
        *reinterpret_cast<float4*>(ob + (size_t)row * HD + 16 * (DTW * w + j) + 4 * grp) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    // the next tile rewrites the score tile
    __builtin_amdgcn_s_barrier();
  }
}

// Merge of the chunk partials of one (row, query head, 64 head dims); lane l
// owns head dim 64 * blockIdx.y + l.  Chunk c's weight is exp(m_c - max),
// with max the row maximum over the row's chunks (exact in any order).  The
// output and its normaliser accumulate in eight interleaved sums, s over
// the chunks c = s, s + 8, ... in increasing order, added as a pairwise tree
// and divided.  Every order depends only on the row's own position, and the
// two launch forms below give the same bits.
//
// Eight-wave form (caches of more than kMerge1Chunks chunks): wave w takes
// the chunks c = w, w + 8, ...  The partial loads of the first batch of
// chunks and the first statistics are issued before the cache length
// arrives (entries past the row's chunk count are read but never used).
// Thread t owns chunks t, t + 512, ...: it stores their statistics in LDS,
// and forms their weights once the workgroup maximum is known.
constexpr int kMaxMergeChunks = 1024;
constexpr int kMergeWaves = 8;   // residue classes of chunks, one wave each in the multi-wave form

// Pairwise sum of N values: ((v0 + v1) + (v2 + v3)) + ((v4 + v5) + (v6 + v7))
// for N = 8.
template <int N>
__device__ __forceinline__ float pair_tree(const float* v) {
  if constexpr (N == 1)
    return v[0];
  else
    return pair_tree<N / 2>(v) + pair_tree<N / 2>(v + N / 2);
}

template <int HD>
__global__ __launch_bounds__(64 * kMergeWaves) void attn_merge_kernel(
    const int32_t* gate, const int32_t* __restrict__ d_len, const float* __restrict__ o_part,
    const float* __restrict__ ml_part, int rows, int max_len, int nq, int nkv, int max_chunks,
    bf16_bits* __restrict__ ob) {
  __shared__ float sm[kMaxMergeChunks], sw[kMaxMergeChunks], sl[kMaxMergeChunks];
  __shared__ float wsum[kMergeWaves][64];
  __shared__ float wred[kMergeWaves], wl[kMergeWaves];
  const int gv = *(gate ? gate : d_len);   // requested with the length, before any branch
  const int len = *d_len;
  const int m = blockIdx.x / nq, hq = blockIdx.x % nq;
  const int G = nq / nkv, h = hq / G, r = m * G + hq % G;
  const size_t rstride = (size_t)kMaxRows * 8;
  const float* ml = ml_part + ((size_t)h * max_chunks * rstride + r) * 2;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d = 64 * blockIdx.y + lane;
  const float* op = o_part + ((size_t)h * max_chunks * rstride + r) * HD + d;
  const size_t cst = rstride * HD;
  constexpr int BATCH = 36;   // chunks per wave per pass
  constexpr int NT = 64 * kMergeWaves;
  float ov[BATCH];
#pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    const int c = w + kMergeWaves * u;
    ov[u] = (c < max_chunks) ? op[(size_t)c * cst] : 0.f;
  }
  float m0 = 0.f, l0 = 0.f;
  if ((int)threadIdx.x < max_chunks) {
    m0 = ml[(size_t)threadIdx.x * rstride * 2];
    l0 = ml[(size_t)threadIdx.x * rstride * 2 + 1];
  }
  if (gate && gv == 0) return;
  int pos = len + m;
  if (pos >= max_len) pos = max_len - 1;
  const int nch = pos / kAttnChunk + 1;
  // thread t owns chunks t, t + NT, ...: their statistics go to LDS and its
  // running max to a wave maximum (a maximum is exact in any order)
  float mloc = -INFINITY;
  if ((int)threadIdx.x < nch) { sm[threadIdx.x] = m0; sl[threadIdx.x] = l0; mloc = m0; }
  for (int c = threadIdx.x + NT; c < nch; c += NT) {
    const float mc = ml[(size_t)c * rstride * 2];
    sm[c] = mc;
    sl[c] = ml[(size_t)c * rstride * 2 + 1];
    mloc = fmaxf(mloc, mc);
  }
  mloc = warp_max(mloc);
  if (lane == 0) wred[w] = mloc;
  __syncthreads();
  float mx = wred[0];
#pragma unroll
  for (int v = 1; v < kMergeWaves; ++v) mx = fmaxf(mx, wred[v]);
  // chunk weights
  for (int c = threadIdx.x; c < nch; c += NT) sw[c] = (sm[c] == -INFINITY) ? 0.f : __expf(sm[c] - mx);
  __syncthreads();
  // the wave's residue class: weighted partials and normaliser terms
  float acc = 0.f, lac = 0.f;
#pragma unroll
  for (int u = 0; u < BATCH; ++u) {
    const int c = w + kMergeWaves * u;
    if (c < nch) {
      acc = fmaf(sw[c], ov[u], acc);
      lac = fmaf(sw[c], sl[c], lac);
    }
  }
  for (int c0 = kMergeWaves * BATCH; c0 < nch; c0 += kMergeWaves * BATCH) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = c0 + w + kMergeWaves * u;
      ov[u] = (c < nch) ? op[(size_t)c * cst] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = c0 + w + kMergeWaves * u;
      if (c < nch) {
        acc = fmaf(sw[c], ov[u], acc);
        lac = fmaf(sw[c], sl[c], lac);
      }
    }
  }
  wsum[w][lane] = acc;
  if (lane == 0) wl[w] = lac;
  __syncthreads();
  if (w == 0) {
    float ov4[kMergeWaves], lv4[kMergeWaves];
#pragma unroll
    for (int v = 0; v < kMergeWaves; ++v) {
      ov4[v] = wsum[v][lane];
      lv4[v] = wl[v];
    }
    const float o = pair_tree<kMergeWaves>(ov4);
    const float L = pair_tree<kMergeWaves>(lv4);
    btile_put(ob, (nq * HD) >> 5, m, hq * HD + d, o / L);
  }
}

// One-wave form (caches of at most kMerge1Chunks chunks): every partial of
// a lane and every chunk's statistics are requested at once, before the
// cache length arrives; lane c forms chunk c's weight and leaves it in LDS
// for the other lanes, which keep the eight residue-class sums side by side.
// Without barriers or cross-wave sums it is the faster form for short
// caches; one wave cannot keep the partials of a long cache in flight.
constexpr int kMerge1Chunks = 48;
static_assert(kMerge1Chunks % kMergeWaves == 0 && kMerge1Chunks <= 64, "one chunk per lane, whole residue classes");

template <int HD>
__global__ __launch_bounds__(64) void attn_merge1_kernel(const int32_t* gate, const int32_t* __restrict__ d_len,
                                                         const float* __restrict__ o_part,
                                                         const float* __restrict__ ml_part, int rows, int max_len,
                                                         int nq, int nkv, int max_chunks, bf16_bits* __restrict__ ob) {
  constexpr int B = kMerge1Chunks;
  __shared__ float sw[B], sl[B];
  const int gv = *(gate ? gate : d_len);   // requested with the length, before any branch
  const int len = *d_len;
  const int m = blockIdx.x / nq, hq = blockIdx.x % nq;
  const int G = nq / nkv, h = hq / G, r = m * G + hq % G;
  const size_t rstride = (size_t)kMaxRows * 8;
  const size_t cst = rstride * HD, mst = rstride * 2;
  const int lane = threadIdx.x;
  const float* ml = ml_part + ((size_t)h * max_chunks * rstride + r) * 2;
  const float* op = o_part + ((size_t)h * max_chunks * rstride + r) * HD + 64 * blockIdx.y + lane;
  // indices clamped to the launch's chunks (max_chunks <= B); entries past
  // the row's chunk count are read but never used
  float ov[B];
#pragma unroll
  for (int u = 0; u < B; ++u) ov[u] = op[(size_t)(u < max_chunks ? u : max_chunks - 1) * cst];
  const int c0 = lane < max_chunks ? lane : max_chunks - 1;
  const float m0 = ml[(size_t)c0 * mst], l0 = ml[(size_t)c0 * mst + 1];
  if (gate && gv == 0) return;
  int pos = len + m;
  if (pos >= max_len) pos = max_len - 1;
  const int nch = pos / kAttnChunk + 1;   // <= max_chunks
  const float mx = warp_max(lane < nch ? m0 : -INFINITY);
  if (lane < nch) {
    sw[lane] = (m0 == -INFINITY) ? 0.f : __expf(m0 - mx);
    sl[lane] = l0;
  }
  __syncthreads();
  constexpr int NR = kMergeWaves;
  float acc[NR], lac[NR];
#pragma unroll
  for (int v = 0; v < NR; ++v) acc[v] = lac[v] = 0.f;
#pragma unroll
  for (int c = 0; c < B; ++c) {
    if (c < nch) {
      const float wc = sw[c];
      acc[c % NR] = fmaf(wc, ov[c], acc[c % NR]);
      lac[c % NR] = fmaf(wc, sl[c], lac[c % NR]);
    }
  }
  const float o = pair_tree<NR>(acc);
  const float L = pair_tree<NR>(lac);
  btile_put(ob, (nq * HD) >> 5, m, hq * HD + 64 * blockIdx.y + lane, o / L);
}

// The merge form follows the cache capacity only (never the row count), and
// both forms give the same bits.
template <int HD>
static void launch_merge(hipStream_t s, int row_heads, const int32_t* gate, const int32_t* d_len, const float* o_part,
                         const float* ml_part, int rows, int max_len, int nq, int nkv, int max_chunks, bf16_bits* ob) {
  const dim3 grid(row_heads, HD / 64);
  if (max_chunks <= kMerge1Chunks)
    attn_merge1_kernel<HD><<<grid, 64, 0, s>>>(gate, d_len, o_part, ml_part, rows, max_len, nq, nkv, max_chunks, ob);
  else
    attn_merge_kernel<HD><<<grid, 64 * kMergeWaves, 0, s>>>(gate, d_len, o_part, ml_part, rows, max_len, nq, nkv,
                                                            max_chunks, ob);
}

// ---------------------------------------------------------------------------
// Final reduction of the LM-head partials: argmax (lowest index on ties) and
// log-sum-exp per row; then the cache length advances by the row count.  One
// 1024-thread workgroup per row: thread t takes partials t + 1024 j (all of
// them requested before any is used), then a wave reduction and the waves in
// order.
// ---------------------------------------------------------------------------
constexpr int kLmrThreads = 1024, kLmrWaves = kLmrThreads / 64, kLmrPer = 5;   // 5120 partials: a 151936- or 152064-entry vocabulary in two-row-group workgroups stays in registers

__global__ __launch_bounds__(kLmrThreads) void lm_reduce_kernel(const float* __restrict__ part, int n_wg, int rows,
                                                                int32_t* __restrict__ argmax_out,
                                                                float* __restrict__ lse_out,
                                                                int32_t* __restrict__ d_len, int max_len,
                                                                int32_t* err, const int32_t* gate) {
  if (gate && *gate == 0) return;
  const int m = blockIdx.x;
  const float* pp = part + (size_t)m * n_wg * 3;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ float sb[kLmrWaves], ss[kLmrWaves];
  __shared__ int si[kLmrWaves];
  float best = -INFINITY, se = 0.f;
  int bidx = 0x7fffffff;
  bool bad = false;
  float mv[kLmrPer], sv[kLmrPer];
  int iv[kLmrPer];
  // pass 1: this thread's partials (a batch of kLmrPer at a time)
  for (int i0 = 0; i0 < n_wg; i0 += kLmrThreads * kLmrPer) {
#pragma unroll
    for (int j = 0; j < kLmrPer; ++j) {
      int i = i0 + (int)threadIdx.x + kLmrThreads * j;
      const bool ok = i < n_wg;
      if (!ok) i = 0;   // a valid slot, not used
      mv[j] = pp[i * 3];
      iv[j] = __float_as_int(pp[i * 3 + 1]);
      sv[j] = pp[i * 3 + 2];
      if (!ok) { mv[j] = -INFINITY; iv[j] = 0x7fffffff; sv[j] = 0.f; }
    }
#pragma unroll
    for (int j = 0; j < kLmrPer; ++j) {
      if (i0 + (int)threadIdx.x + kLmrThreads * j < n_wg && !(fabsf(mv[j]) <= 3.0e38f)) bad = true;
      if (mv[j] > best || (mv[j] == best && iv[j] < bidx)) { best = mv[j]; bidx = iv[j]; }
    }
  }
  warp_argmax(best, bidx);
  if (lane == 0) { sb[w] = best; si[w] = bidx; }
  __syncthreads();
  float gmax = sb[0];
  int gidx = si[0];
  for (int v = 1; v < kLmrWaves; ++v)
    if (sb[v] > gmax || (sb[v] == gmax && si[v] < gidx)) { gmax = sb[v]; gidx = si[v]; }
  // pass 2: sum of exp relative to the row max (in registers when n_wg fits one batch)
  if (n_wg <= kLmrThreads * kLmrPer) {
#pragma unroll
    for (int j = 0; j < kLmrPer; ++j) se += sv[j] * expf(mv[j] - gmax);
  } else {
    for (int i = threadIdx.x; i < n_wg; i += kLmrThreads) se += pp[i * 3 + 2] * expf(pp[i * 3] - gmax);
  }
  se = warp_sum(se);
  if (lane == 0) ss[w] = se;
  __syncthreads();
  if (bad) raise_error(err, kErrNonFinite);
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int v = 0; v < kLmrWaves; ++v) tot += ss[v];
    if (argmax_out) argmax_out[m] = gidx;
    if (lse_out) lse_out[m] = gmax + logf(tot);
    // a forward past the capacity (flagged by the embedding) leaves the length as it was
    if (m == 0 && *d_len + rows <= max_len) *d_len += rows;
  }
}

// ---------------------------------------------------------------------------
// Host launcher of one forward pass.
// ---------------------------------------------------------------------------
template <int NT, int WG_ROWS, int WK, int U, Epi E>
static void launch_gemv(int wgs, hipStream_t s, const GemvParams& p) {
  gemv_kernel<NT, WG_ROWS, WK, U, E><<<wgs, 64 * WG_ROWS * WK, 0, s>>>(p.gate, p.d_len, p.A, p.B, p.KB, p.n_groups,
                                                                      p.rows, p.nsplit, p);
}

// The chunk kernel instantiated for the smallest tile capacity (1, 2 or 4)
// that holds the workgroup's wt query tiles.
template <int HD>
static void launch_attn(int wt, dim3 grid, hipStream_t s, const int32_t* gate, const int32_t* d_len,
                        const bf16_bits* qb, const bf16_bits* Kc, const bf16_bits* Vt, int rows, int max_len, int lp,
                        int G, float* o_part, float* ml_part, int max_chunks, const uint32_t* tree_anc, int tree_n0) {
  if (wt <= 1)
    attn_chunk_kernel<HD, 1><<<grid, 64 * kAttnWaves, 0, s>>>(gate, d_len, qb, Kc, Vt, rows, max_len, lp, G, o_part,
                                                              ml_part, max_chunks, tree_anc, tree_n0);
  else if (wt <= 2)
    attn_chunk_kernel<HD, 2><<<grid, 64 * kAttnWaves, 0, s>>>(gate, d_len, qb, Kc, Vt, rows, max_len, lp, G, o_part,
                                                              ml_part, max_chunks, tree_anc, tree_n0);
  else
    attn_chunk_kernel<HD, kAttnMaxWgTiles><<<grid, 64 * kAttnWaves, 0, s>>>(gate, d_len, qb, Kc, Vt, rows, max_len,
                                                                            lp, G, o_part, ml_part, max_chunks, tree_anc, tree_n0);
}

template <int NT>
static void launch_gemvs_layer(const FwdArgs& a, int l, GemvParams base) {
  const Dims& d = a.m->d;
  const LayerPtrs& L = a.m->layers[l];
  const WsPlan& pl = *a.plan;
  char* ws = a.ws;
  float* x = reinterpret_cast<float*>(ws + pl.x);
  bf16_bits* xb = reinterpret_cast<bf16_bits*>(ws + pl.xb);
  float* ss = reinterpret_cast<float*>(ws + pl.ss);
  bf16_bits* qb = reinterpret_cast<bf16_bits*>(ws + pl.qb);
  bf16_bits* ob = reinterpret_cast<bf16_bits*>(ws + pl.ob);
  bf16_bits* hb = reinterpret_cast<bf16_bits*>(ws + pl.hb);
  float* att_o = reinterpret_cast<float*>(ws + pl.att_o);
  float* att_ml = reinterpret_cast<float*>(ws + pl.att_ml);
  const uint32_t* tree_anc = a.parents ? reinterpret_cast<const uint32_t*>(ws + pl.tree) + kMaxRows : nullptr;
  hipStream_t s = a.stream;
  const bool q4 = d.wfmt == SPECDEC_W_Q4G64;

  // fused RMSNorm -> QKV -> RoPE -> K/V append (query rows into operand tiles)
  GemvParams p = base;
  p.A = L.wqkv; p.B = reinterpret_cast<const bf16x8_t*>(xb); p.KB = d.H / 32; p.n_groups = d.qkv_rows() / 16;
  p.ss_in = ss; p.qb = qb; p.k_cache = a.c->k_layer(l); p.v_cache = a.c->v_layer(l);
  if (q4) launch_q4_linear(Q4Linear::QKV, p, L.q_wqkv, L.s_wqkv, d.H, s);
  else
    launch_gemv<NT, CfgQKV::WG_ROWS, CfgQKV::WK, CfgQKV::template U<NT>, Epi::QKV>(
        (p.n_groups + CfgQKV::WG_ROWS - 1) / CfgQKV::WG_ROWS, s, p);

  // attention: chunk partials, then the merge into the O-projection operand tiles
  // query tiles of 16 rows per kv head, spread over up to kAttnTileSplit
  // workgroups per chunk (each tile's arithmetic is the same either way)
  const int ntq = (a.rows * d.group() + 15) / 16;
  const int ts_min = (ntq + kAttnMaxWgTiles - 1) / kAttnMaxWgTiles;
  int ts = ntq < kAttnTileSplit ? ntq : kAttnTileSplit;
  if (ts < ts_min) ts = ts_min;
  // A chunk's tile workgroups sit gx * nkv apart in dispatch order; with that
  // a multiple of eight, round-robin dispatch puts them on one XCD, whose L2
  // then serves the chunk's K and V to every reader after the first.  The
  // padding workgroups start past every cache and return at once.
  int gx = pl.max_chunks;
  if (ts > 1)
    while ((gx * d.nkv) % 8) ++gx;
  dim3 ag(gx, d.nkv, ts);
  const int wt = (ntq + ts - 1) / ts;   // query tiles per workgroup
  if (d.hd == 128) {
    launch_attn<128>(wt, ag, s, a.gate, a.c->d_len, qb, a.c->k_layer(l), a.c->v_layer(l), a.rows, a.c->max_len,
                     a.c->lp, d.group(), att_o, att_ml, pl.max_chunks, tree_anc, a.tree_n0);
    launch_merge<128>(s, a.rows * d.nq, a.gate, a.c->d_len, att_o, att_ml, a.rows, a.c->max_len, d.nq, d.nkv,
                      pl.max_chunks, ob);
  } else {
    launch_attn<64>(wt, ag, s, a.gate, a.c->d_len, qb, a.c->k_layer(l), a.c->v_layer(l), a.rows, a.c->max_len,
                    a.c->lp, d.group(), att_o, att_ml, pl.max_chunks, tree_anc, a.tree_n0);
    launch_merge<64>(s, a.rows * d.nq, a.gate, a.c->d_len, att_o, att_ml, a.rows, a.c->max_len, d.nq, d.nkv,
                     pl.max_chunks, ob);
  }

  // O projection + residual; next input is the MLP norm
  p = base;
  p.A = L.wo; p.B = reinterpret_cast<const bf16x8_t*>(ob); p.KB = d.qdim() / 32; p.n_groups = d.H / 16;
  p.x = x; p.gain_next = L.mlp_norm; p.xb_out = xb; p.ss_out = ss;
  if (q4) launch_q4_linear(Q4Linear::O, p, L.q_wo, L.s_wo, d.qdim(), s);
  else if (kOSplit > 1) {
    p.part = reinterpret_cast<float*>(ws + pl.part);
    p.nsplit = kOSplit;
    p.cnt = reinterpret_cast<int32_t*>(ws + pl.cnt);
    launch_gemv<NT, 1, CfgO::WK, CfgO::template U<NT>, Epi::PARTIAL>((p.n_groups + 7) / 8 * 8 * kOSplit, s, p);
  } else
    launch_gemv<NT, CfgO::WG_ROWS, CfgO::WK, CfgO::template U<NT>, Epi::RESID>(
        (p.n_groups + CfgO::WG_ROWS - 1) / CfgO::WG_ROWS, s, p);

  // RMSNorm -> gate/up -> SwiGLU
  p = base;
  p.A = L.wgu; p.B = reinterpret_cast<const bf16x8_t*>(xb); p.KB = d.H / 32; p.n_groups = d.F / 8;
  p.ss_in = ss; p.hb_out = hb;
  if (q4) launch_q4_linear(Q4Linear::GATE_UP, p, L.q_wgu, L.s_wgu, d.H, s);
  else if (!launch_gu_rg<NT>(s, p))
    launch_gemv<NT, CfgGU::WG_ROWS, CfgGU::WK, CfgGU::template U<NT>, Epi::SWIGLU>(
        (p.n_groups + CfgGU::WG_ROWS - 1) / CfgGU::WG_ROWS, s, p);

  // down projection + residual; next input is the next layer's (or final) norm
  p = base;
  p.A = L.wdown; p.B = reinterpret_cast<const bf16x8_t*>(hb); p.KB = d.F / 32; p.n_groups = d.H / 16;
  p.x = x; p.gain_next = (l + 1 < d.L) ? a.m->layers[l + 1].attn_norm : a.m->final_norm; p.xb_out = xb; p.ss_out = ss;
  p.part = reinterpret_cast<float*>(ws + pl.part);
  p.nsplit = kDownSplit;   // 4-bit launches size their own splits
  p.cnt = reinterpret_cast<int32_t*>(ws + pl.cnt);   // the last split finishes the residual
  if (q4) launch_q4_linear(Q4Linear::DOWN, p, L.q_wdown, L.s_wdown, d.F, s);
  else
    launch_gemv<NT, 1, CfgDown::WK, CfgDown::template U<NT>, Epi::PARTIAL>((p.n_groups + 7) / 8 * 8 * kDownSplit, s, p);
}

template <int NT>
static hipError_t launch_forward_nt(const FwdArgs& a) {
  const Dims& d = a.m->d;
  const WsPlan& pl = *a.plan;
  char* ws = a.ws;
  int32_t* err = a.err ? a.err : reinterpret_cast<int32_t*>(ws + pl.err);
  float* x = reinterpret_cast<float*>(ws + pl.x);
  bf16_bits* xb = reinterpret_cast<bf16_bits*>(ws + pl.xb);
  float* ss = reinterpret_cast<float*>(ws + pl.ss);
  hipStream_t s = a.stream;

  int32_t* tree = reinterpret_cast<int32_t*>(ws + pl.tree);
  embed_kernel<<<a.rows, 256, 0, s>>>(a.tokens, a.m->embed, a.m->layers[0].attn_norm, d.H, d.V, a.rows, x, xb, ss,
                                      a.c->d_len, a.c->max_len, err, a.gate, a.parents, a.tree_n0, tree);
  GemvParams base = {};
  base.tree_depth = a.parents ? tree : nullptr;
  base.rows = a.rows; base.gate = a.gate; base.err = err; base.H = d.H; base.eps = d.eps;
  base.rope = a.c->rope; base.d_len = a.c->d_len; base.max_len = a.c->max_len; base.kv_stride = a.c->lp;
  base.nq = d.nq; base.nkv = d.nkv; base.hd = d.hd; base.F = d.F; base.V = d.V;
  for (int l = 0; l < d.L; ++l) launch_gemvs_layer<NT>(a, l, base);

  if (a.skip_head) return launch_advance(a.c->d_len, a.rows, a.c->max_len, a.gate, s);
  GemvParams p = base;
  p.A = a.m->lm_head; p.B = reinterpret_cast<const bf16x8_t*>(xb); p.KB = d.H / 32; p.n_groups = d.V / 16;
  p.ss_in = ss; p.logits = a.logits;
  float* lm_part = reinterpret_cast<float*>(ws + pl.lm_part);
  p.lm_part = lm_part;
  int wgs = (p.n_groups + CfgLM::WG_ROWS - 1) / CfgLM::WG_ROWS;
  launch_gemv<NT, CfgLM::WG_ROWS, CfgLM::WK, CfgLM::template U<NT>, Epi::LMHEAD>(wgs, s, p);
  lm_reduce_kernel<<<a.rows, kLmrThreads, 0, s>>>(lm_part, wgs, a.rows, a.argmax, a.lse, a.c->d_len, a.c->max_len,
                                                  err, a.gate);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a) {
  int nt = (a.rows + 7) / 8;
  switch (nt) {
    case 1: return launch_forward_nt<1>(a);
    case 2: return launch_forward_nt<2>(a);
    case 3: return launch_forward_nt<3>(a);
    case 4: return launch_forward_nt<4>(a);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Trim: length = new_len if new_len <= length (else the error bit is set).
// With d_base the new length is *d_base + new_len (used by the round reset).
// ---------------------------------------------------------------------------
__global__ void trim_kernel(int32_t* d_len, int32_t new_len, const int32_t* d_base, int32_t* err) {
  if (threadIdx.x != 0) return;
  int32_t nl = d_base ? *d_base + new_len : new_len;
  if (nl < 0 || nl > *d_len) { raise_error(err, kErrTrim); return; }
  *d_len = nl;
}

hipError_t launch_trim(int32_t* d_len, int32_t new_len, const int32_t* d_base, int32_t* err, hipStream_t s) {
  trim_kernel<<<1, 64, 0, s>>>(d_len, new_len, d_base, err);
  return hipGetLastError();
}

__global__ void advance_kernel(int32_t* d_len, int rows, int max_len, const int32_t* gate) {
  if (gate && *gate == 0) return;
  if (threadIdx.x == 0 && *d_len + rows <= max_len) *d_len += rows;
}

hipError_t launch_advance(int32_t* d_len, int rows, int max_len, const int32_t* gate, hipStream_t s) {
  advance_kernel<<<1, 64, 0, s>>>(d_len, rows, max_len, gate);
  return hipGetLastError();
}

// Read-bandwidth probe: every 16-byte word of a buffer read once with the
// non-temporal loads of the weight stream, eight in flight per lane, folded
// into one word per lane that is stored only if it hits a constant (so the
// loads stay live without a write stream).
__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4_t* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  i32x4_t acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    i32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  const uint32_t x = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (x == 0x9E3779B9u) sink[0] = x;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, hipStream_t s) {
  stream_read_kernel<<<workgroups, 256, 0, s>>>(static_cast<const i32x4_t*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

// Copy the last row of a forward's outputs (prefill) to the caller's buffers.
__global__ void copy_last_kernel(const float* __restrict__ logits, const int32_t* __restrict__ argmax,
                                 const float* __restrict__ lse, int rows, int V, float* __restrict__ ldst,
                                 int32_t* __restrict__ adst, float* __restrict__ sdst) {
  const float* src = logits + (size_t)(rows - 1) * V;
  if (ldst)
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < V; i += gridDim.x * blockDim.x) ldst[i] = src[i];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (adst) *adst = argmax[rows - 1];
    if (sdst) *sdst = lse[rows - 1];
  }
}

hipError_t launch_copy_last(const FwdArgs& a, float* ldst, int32_t* adst, float* sdst) {
  copy_last_kernel<<<64, 256, 0, a.stream>>>(a.logits, a.argmax, a.lse, a.rows, a.m->d.V, ldst, adst, sdst);
  return hipGetLastError();
}

}  // namespace sd
