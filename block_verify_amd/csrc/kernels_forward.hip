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
#include "internal.h"

#include <math.h>

namespace sd {

enum class Epi { QKV, RESID, SWIGLU, LMHEAD };

hipError_t launch_advance(int32_t* d_len, int rows, const int32_t* gate, hipStream_t s);

// ---------------------------------------------------------------------------
// Packing (setup): row-major bf16 -> MFMA weight tiles.
// ---------------------------------------------------------------------------
enum PackKind { PACK_PLAIN = 0, PACK_ROPE = 1, PACK_GATE = 2, PACK_UP = 3 };

__global__ void pack_linear_kernel(const bf16_bits* __restrict__ src, int rows, int K, int kind, int hd,
                                   int group_base, bf16_bits* __restrict__ dst) {
  const int kc_per_row = K >> 3;
  const size_t total = (size_t)rows * kc_per_row;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    int r = (int)(idx / kc_per_row);
    int k = (int)(idx % kc_per_row) * 8;
    int g, i;
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
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens, const bf16_bits* __restrict__ E,
                                                    const float* __restrict__ gain, int H, int V, int rows,
                                                    float* __restrict__ x, bf16_bits* __restrict__ xb,
                                                    float* __restrict__ ss, const int32_t* __restrict__ d_len,
                                                    int max_len, int32_t* err, const int32_t* gate) {
  if (gate && *gate == 0) return;
  const int m = blockIdx.x;
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
template <int NT>
__device__ __forceinline__ void mfma_stream(const bf16x8_t* __restrict__ A, const bf16x8_t* __restrict__ B, int KB,
                                            int kb0, int kb1, int lane, f32x4_t (&acc)[NT]) {
  const bf16x8_t* a = A + (size_t)kb0 * 64 + lane;
  const bf16x8_t* b = B + (size_t)kb0 * 64 + lane;
  const size_t tstride = (size_t)KB * 64;
  const int n = kb1 - kb0;
  constexpr int U = (NT <= 2) ? 8 : 4;
  int i = 0;
  for (; i + U <= n; i += U) {
    bf16x8_t av[U];
    bf16x8_t bv[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) av[u] = __builtin_nontemporal_load(a + (size_t)(i + u) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t) bv[u][t] = b[t * tstride + (size_t)(i + u) * 64];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][t], acc[t], 0, 0, 0);
  }
  for (; i < n; ++i) {
    bf16x8_t av = __builtin_nontemporal_load(a + (size_t)i * 64);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bf16x8_t bv = b[t * tstride + (size_t)i * 64];
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[t], 0, 0, 0);
    }
  }
}

// r_m = 1 / sqrt(mean(x_m^2) + eps) from the per-16-feature partial sums.
// One wave per row; the reduction tree is fixed by the feature layout.
__device__ __forceinline__ float rms_scale_wave(const float* __restrict__ ss, int m, int NP, int H, float eps, int lane) {
  float s = 0.f;
  for (int g = lane; g < NP; g += 64) s += ss[(size_t)m * NP + g];
  s = warp_sum(s);
  return 1.0f / sqrtf(s / (float)H + eps);
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
  float* q_out;
  bf16_bits* k_cache;
  bf16_bits* v_cache;
  const float2* rope;
  const int32_t* d_len;
  int max_len;
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
};

template <int NT, int WG_ROWS, int WK, Epi E>
__global__ __launch_bounds__(64 * WG_ROWS * WK) void gemv_kernel(GemvParams p) {
  if (p.gate && *p.gate == 0) return;
  constexpr int NW = WG_ROWS * WK;
  constexpr int NC = NT * 8;        // activation rows covered
  __shared__ float red[NW][16][NT * 16 + 1];
  __shared__ float fin[WG_ROWS][16][NC + 1];
  __shared__ float rsc[kMaxRows];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rg = w / WK, ks = w % WK;
  const int g = blockIdx.x * WG_ROWS + rg;
  const int M = p.rows;

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (g < p.n_groups) {
    const int kb0 = (int)(((long)ks * p.KB) / WK), kb1 = (int)(((long)(ks + 1) * p.KB) / WK);
    mfma_stream<NT>(p.A + (size_t)g * p.KB * 64, p.B, p.KB, kb0, kb1, lane, acc);
  }
  // row scales for normalised inputs (overlaps other waves' streaming)
  if constexpr (E != Epi::RESID) {
    for (int m = w; m < M; m += NW) {
      float r = rms_scale_wave(p.ss_in, m, p.H >> 4, p.H, p.eps, lane);
      if (lane == 0) rsc[m] = r;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][4 * (lane >> 4) + r][t * 16 + (lane & 15)] = acc[t][r];
  __syncthreads();
  // fixed-order reduction over the k-split waves, then hi + lo
  for (int idx = threadIdx.x; idx < WG_ROWS * 16 * NC; idx += blockDim.x) {
    int rr = idx / (16 * NC), rem = idx % (16 * NC), i = rem / NC, m = rem % NC;
    int t = m >> 3, c = m & 7;
    float hi = 0.f, lo = 0.f;
#pragma unroll
    for (int s = 0; s < WK; ++s) {
      hi += red[rr * WK + s][i][t * 16 + c];
      lo += red[rr * WK + s][i][t * 16 + 8 + c];
    }
    fin[rr][i][m] = hi + lo;
  }
  __syncthreads();

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
    if (w == 0) {
      for (int m = 0; m < M; ++m) {
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
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          float ob = __shfl_xor(best, o, 64);
          int oi = __shfl_xor(bidx, o, 64);
          if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
        }
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
    const int pos0 = *p.d_len;
    const int qg = p.nq * p.hd / 16, kg = p.nkv * p.hd / 16;
    const int per_head = p.hd / 16, half = p.hd / 2;
    if (g < qg + kg) {
      const bool is_k = g >= qg;
      const int gg = is_k ? g - qg : g;
      const int head = gg / per_head, sub = gg % per_head;
      for (int idx = lane; idx < 8 * M; idx += 64) {
        int i = idx & 7, m = idx >> 3;
        int pos = pos0 + m;
        if (pos >= p.max_len) continue;
        float r = rsc[m];
        float y1 = f[i][m] * r, y2 = f[i + 8][m] * r;
        int d1 = 8 * sub + i;
        float2 cs = p.rope[(size_t)pos * half + d1];
        float o1 = y1 * cs.x - y2 * cs.y;
        float o2 = y2 * cs.x + y1 * cs.y;
        if (!is_k) {
          float* q = p.q_out + (size_t)m * p.nq * p.hd + head * p.hd;
          q[d1] = o1;
          q[d1 + half] = o2;
        } else {
          bf16_bits* kc = p.k_cache + ((size_t)head * p.max_len + pos) * p.hd;
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
        p.v_cache[((size_t)head * p.max_len + pos) * p.hd + d0 + i] = f2bf(f[i][m] * rsc[m]);
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
  } else {  // RESID
    const int KBo = p.H >> 5, NP = p.H >> 4;
    for (int idx = lane; idx < 16 * M; idx += 64) {
      int i = idx & 15, m = idx >> 4;
      int n = 16 * g + i;
      float xn = p.x[(size_t)m * p.H + n] + f[i][m];
      p.x[(size_t)m * p.H + n] = xn;
      f[i][m] = xn;
      btile_put(p.xb_out, KBo, m, n, xn * p.gain_next[n]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    for (int m = lane; m < M; m += 64) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s = fmaf(f[i][m], f[i][m], s);
      p.ss_out[(size_t)m * NP + g] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K causal attention over the cache (one workgroup per kv head and
// 64-key chunk) and the fixed-order merge of the chunk partials.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void attn_partial_kernel(const float* __restrict__ q, const bf16_bits* __restrict__ Kc,
                                                           const bf16_bits* __restrict__ Vc, const int32_t* __restrict__ d_len,
                                                           int rows, int max_len, int nq, int nkv,
                                                           float* __restrict__ o_part, float* __restrict__ ml_part,
                                                           int max_chunks, const int32_t* gate) {
  if (gate && *gate == 0) return;
  constexpr int C = kAttnChunk;
  constexpr int DL = HD / 64;   // head dims per lane
  __shared__ float Kt[HD][C + 1];
  __shared__ float Vs[C][HD + 1];
  __shared__ float qs[4][HD];
  const int c = blockIdx.x, h = blockIdx.y;
  const int len = *d_len;
  int T = len + rows;
  if (T > max_len) T = max_len;
  const int key0 = c * C;
  if (key0 >= T) return;
  const int nkeys = min(C, T - key0);
  const int G = nq / nkv;
  const bf16_bits* kb = Kc + ((size_t)h * max_len + key0) * HD;
  const bf16_bits* vb = Vc + ((size_t)h * max_len + key0) * HD;
  for (int e = threadIdx.x; e < C * (HD / 8); e += blockDim.x) {
    int j = e / (HD / 8), d8 = (e % (HD / 8)) * 8;
    uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
    if (j < nkeys) {
      kv4 = *reinterpret_cast<const uint4*>(kb + (size_t)j * HD + d8);
      vv4 = *reinterpret_cast<const uint4*>(vb + (size_t)j * HD + d8);
    }
    const bf16_bits* k16 = reinterpret_cast<const bf16_bits*>(&kv4);
    const bf16_bits* v16 = reinterpret_cast<const bf16_bits*>(&vv4);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      Kt[d8 + u][j] = bf2f(k16[u]);
      Vs[j][d8 + u] = bf2f(v16[u]);
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float scale = 1.0f / sqrtf((float)HD);
  const int R = rows * G;
  for (int r = w; r < R; r += 4) {
    const int m = r / G, hq = h * G + r % G;
    const float* qr = q + (size_t)m * nq * HD + (size_t)hq * HD;
#pragma unroll
    for (int u = 0; u < DL; ++u) qs[w][lane + 64 * u] = qr[lane + 64 * u];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    float s = 0.f;
#pragma unroll 16
    for (int d = 0; d < HD; ++d) s = fmaf(qs[w][d], Kt[d][lane], s);
    s *= scale;
    const bool valid = (lane < nkeys) && (key0 + lane <= len + m);
    s = valid ? s : -INFINITY;
    const float mx = warp_max(s);
    float* op = o_part + (((size_t)h * max_chunks + c) * (kMaxRows * 8) + r) * HD;
    float* mlp = ml_part + (((size_t)h * max_chunks + c) * (kMaxRows * 8) + r) * 2;
    if (mx == -INFINITY) {
      if (lane == 0) { mlp[0] = -INFINITY; mlp[1] = 0.f; }
      continue;
    }
    const float pj = valid ? __expf(s - mx) : 0.f;
    const float l = warp_sum(pj);
    float o[DL];
#pragma unroll
    for (int u = 0; u < DL; ++u) o[u] = 0.f;
#pragma unroll 8
    for (int j = 0; j < C; ++j) {
      float pjj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), j));
#pragma unroll
      for (int u = 0; u < DL; ++u) o[u] = fmaf(pjj, Vs[j][lane + 64 * u], o[u]);
    }
#pragma unroll
    for (int u = 0; u < DL; ++u) op[lane + 64 * u] = o[u];
    if (lane == 0) { mlp[0] = mx; mlp[1] = l; }
    __builtin_amdgcn_wave_barrier();
  }
}

// One workgroup per (row, q head); thread d owns head dim d.  Chunks merge
// in index order.  Writes the attention output as activation tiles.
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ o_part, const float* __restrict__ ml_part,
                                                        const int32_t* __restrict__ d_len, int rows, int max_len, int nq,
                                                        int nkv, int hd, int max_chunks, bf16_bits* __restrict__ ob,
                                                        const int32_t* gate) {
  if (gate && *gate == 0) return;
  const int m = blockIdx.x / nq, hq = blockIdx.x % nq;
  const int G = nq / nkv, h = hq / G, r = m * G + hq % G;
  int pos = *d_len + m;
  if (pos >= max_len) pos = max_len - 1;
  const int nch = pos / kAttnChunk + 1;
  const float* ml = ml_part + ((size_t)h * max_chunks * (kMaxRows * 8) + r) * 2;
  const size_t cstride = (size_t)kMaxRows * 8;
  float mx = -INFINITY;
  for (int c = 0; c < nch; ++c) mx = fmaxf(mx, ml[c * cstride * 2]);
  const int d = threadIdx.x;
  if (d >= hd) return;
  float L = 0.f, acc = 0.f;
  const float* op = o_part + ((size_t)h * max_chunks * cstride + r) * hd + d;
#pragma unroll 4
  for (int c = 0; c < nch; ++c) {
    float mc = ml[c * cstride * 2];
    float wgt = (mc == -INFINITY) ? 0.f : __expf(mc - mx);
    L = fmaf(wgt, ml[c * cstride * 2 + 1], L);
    acc = fmaf(wgt, op[c * cstride * hd], acc);
  }
  btile_put(ob, (nq * hd) >> 5, m, hq * hd + d, acc / L);
}

// ---------------------------------------------------------------------------
// Final reduction of the LM-head partials: argmax (lowest index on ties) and
// log-sum-exp per row; then the cache length advances by the row count.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lm_reduce_kernel(const float* __restrict__ part, int n_wg, int rows,
                                                        int32_t* __restrict__ argmax_out, float* __restrict__ lse_out,
                                                        int32_t* __restrict__ d_len, int32_t* err, const int32_t* gate) {
  if (gate && *gate == 0) return;
  const int m = blockIdx.x;
  const float* pp = part + (size_t)m * n_wg * 3;
  __shared__ float sb[256];
  __shared__ int si[256];
  __shared__ float ss[256];
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  bool bad = false;
  for (int i = threadIdx.x; i < n_wg; i += 256) {
    float v = pp[i * 3];
    int ix = __float_as_int(pp[i * 3 + 1]);
    if (!(fabsf(v) <= 3.0e38f)) bad = true;
    if (v > best || (v == best && ix < bidx)) { best = v; bidx = ix; }
  }
  sb[threadIdx.x] = best;
  si[threadIdx.x] = bidx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      float ob = sb[threadIdx.x + s];
      int oi = si[threadIdx.x + s];
      if (ob > sb[threadIdx.x] || (ob == sb[threadIdx.x] && oi < si[threadIdx.x])) {
        sb[threadIdx.x] = ob;
        si[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  const float gmax = sb[0];
  float se = 0.f;
  for (int i = threadIdx.x; i < n_wg; i += 256) se += pp[i * 3 + 2] * expf(pp[i * 3] - gmax);
  ss[threadIdx.x] = se;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) ss[threadIdx.x] += ss[threadIdx.x + s];
    __syncthreads();
  }
  if (bad) raise_error(err, kErrNonFinite);
  if (threadIdx.x == 0) {
    if (argmax_out) argmax_out[m] = si[0];
    if (lse_out) lse_out[m] = gmax + logf(ss[0]);
    if (m == 0) *d_len += rows;
  }
}

// ---------------------------------------------------------------------------
// Host launcher of one forward pass.
// ---------------------------------------------------------------------------
template <int NT>
static void launch_gemvs_layer(const FwdArgs& a, int l, GemvParams base) {
  const Dims& d = a.m->d;
  const LayerPtrs& L = a.m->layers[l];
  const WsPlan& pl = *a.plan;
  char* ws = a.ws;
  float* x = reinterpret_cast<float*>(ws + pl.x);
  bf16_bits* xb = reinterpret_cast<bf16_bits*>(ws + pl.xb);
  float* ss = reinterpret_cast<float*>(ws + pl.ss);
  float* q = reinterpret_cast<float*>(ws + pl.q);
  bf16_bits* ob = reinterpret_cast<bf16_bits*>(ws + pl.ob);
  bf16_bits* hb = reinterpret_cast<bf16_bits*>(ws + pl.hb);
  float* att_o = reinterpret_cast<float*>(ws + pl.att_o);
  float* att_ml = reinterpret_cast<float*>(ws + pl.att_ml);
  hipStream_t s = a.stream;

  // fused RMSNorm -> QKV -> RoPE -> K/V append
  GemvParams p = base;
  p.A = L.wqkv; p.B = reinterpret_cast<const bf16x8_t*>(xb); p.KB = d.H / 32; p.n_groups = d.qkv_rows() / 16;
  p.ss_in = ss; p.q_out = q; p.k_cache = a.c->k_layer(l); p.v_cache = a.c->v_layer(l);
  gemv_kernel<NT, 1, 4, Epi::QKV><<<p.n_groups, 256, 0, s>>>(p);

  // attention
  dim3 ag(pl.max_chunks, d.nkv);
  if (d.hd == 128)
    attn_partial_kernel<128><<<ag, 256, 0, s>>>(q, a.c->k_layer(l), a.c->v_layer(l), a.c->d_len, a.rows, a.c->max_len,
                                                 d.nq, d.nkv, att_o, att_ml, pl.max_chunks, a.gate);
  else
    attn_partial_kernel<64><<<ag, 256, 0, s>>>(q, a.c->k_layer(l), a.c->v_layer(l), a.c->d_len, a.rows, a.c->max_len,
                                                d.nq, d.nkv, att_o, att_ml, pl.max_chunks, a.gate);
  attn_merge_kernel<<<a.rows * d.nq, 128, 0, s>>>(att_o, att_ml, a.c->d_len, a.rows, a.c->max_len, d.nq, d.nkv, d.hd,
                                                  pl.max_chunks, ob, a.gate);

  // O projection + residual; next input is the MLP norm
  p = base;
  p.A = L.wo; p.B = reinterpret_cast<const bf16x8_t*>(ob); p.KB = d.qdim() / 32; p.n_groups = d.H / 16;
  p.x = x; p.gain_next = L.mlp_norm; p.xb_out = xb; p.ss_out = ss;
  gemv_kernel<NT, 1, 4, Epi::RESID><<<p.n_groups, 256, 0, s>>>(p);

  // RMSNorm -> gate/up -> SwiGLU
  p = base;
  p.A = L.wgu; p.B = reinterpret_cast<const bf16x8_t*>(xb); p.KB = d.H / 32; p.n_groups = d.F / 8;
  p.ss_in = ss; p.hb_out = hb;
  gemv_kernel<NT, 1, 4, Epi::SWIGLU><<<p.n_groups, 256, 0, s>>>(p);

  // down projection + residual; next input is the next layer's (or final) norm
  p = base;
  p.A = L.wdown; p.B = reinterpret_cast<const bf16x8_t*>(hb); p.KB = d.F / 32; p.n_groups = d.H / 16;
  p.x = x; p.gain_next = (l + 1 < d.L) ? a.m->layers[l + 1].attn_norm : a.m->final_norm; p.xb_out = xb; p.ss_out = ss;
  gemv_kernel<NT, 1, 8, Epi::RESID><<<p.n_groups, 512, 0, s>>>(p);
}

template <int NT>
static hipError_t launch_forward_nt(const FwdArgs& a) {
  const Dims& d = a.m->d;
  const WsPlan& pl = *a.plan;
  char* ws = a.ws;
  int32_t* err = reinterpret_cast<int32_t*>(ws + pl.err);
  float* x = reinterpret_cast<float*>(ws + pl.x);
  bf16_bits* xb = reinterpret_cast<bf16_bits*>(ws + pl.xb);
  float* ss = reinterpret_cast<float*>(ws + pl.ss);
  hipStream_t s = a.stream;

  embed_kernel<<<a.rows, 256, 0, s>>>(a.tokens, a.m->embed, a.m->layers[0].attn_norm, d.H, d.V, a.rows, x, xb, ss,
                                      a.c->d_len, a.c->max_len, err, a.gate);
  GemvParams base = {};
  base.rows = a.rows; base.gate = a.gate; base.err = err; base.H = d.H; base.eps = d.eps;
  base.rope = a.c->rope; base.d_len = a.c->d_len; base.max_len = a.c->max_len;
  base.nq = d.nq; base.nkv = d.nkv; base.hd = d.hd; base.F = d.F; base.V = d.V;
  for (int l = 0; l < d.L; ++l) launch_gemvs_layer<NT>(a, l, base);

  if (a.skip_head) return launch_advance(a.c->d_len, a.rows, a.gate, s);
  GemvParams p = base;
  p.A = a.m->lm_head; p.B = reinterpret_cast<const bf16x8_t*>(xb); p.KB = d.H / 32; p.n_groups = d.V / 16;
  p.ss_in = ss; p.logits = a.logits;
  float* lm_part = reinterpret_cast<float*>(ws + pl.lm_part);
  p.lm_part = lm_part;
  constexpr int LMR = 4;
  int wgs = (p.n_groups + LMR - 1) / LMR;
  gemv_kernel<NT, LMR, 1, Epi::LMHEAD><<<wgs, 64 * LMR, 0, s>>>(p);
  lm_reduce_kernel<<<a.rows, 256, 0, s>>>(lm_part, wgs, a.rows, a.argmax, a.lse, a.c->d_len, err, a.gate);
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

__global__ void advance_kernel(int32_t* d_len, int rows, const int32_t* gate) {
  if (gate && *gate == 0) return;
  if (threadIdx.x == 0) *d_len += rows;
}

hipError_t launch_advance(int32_t* d_len, int rows, const int32_t* gate, hipStream_t s) {
  advance_kernel<<<1, 64, 0, s>>>(d_len, rows, gate);
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
