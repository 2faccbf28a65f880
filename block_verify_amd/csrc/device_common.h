// Device-side layouts and helpers shared by the gfx950 kernels.
//
// Tile formats (all tiles are 1 KiB = 64 lanes x 16 bytes, the operand size
// of one v_mfma_f32_16x16x32_bf16):
//
//  * Weight tile (A operand): 16 output rows x 32 inputs of a linear weight.
//    Lane l holds 8 bf16 of row (l % 16), inputs 8*(l / 16) .. +7.  A matrix
//    with N rows (N % 16 == 0) and K inputs (K % 32 == 0) is stored as
//    [N/16 row groups][K/32 k-blocks][tile], so one row group streams as one
//    contiguous run and every wave-wide 16-byte load is a contiguous 1 KiB.
//
//  * Activation tile (B operand): 32 inputs x 16 columns.  Column c < 8 holds
//    the bf16 "hi" part of activation row 8*t + c, column c >= 8 its "lo"
//    remainder (x = hi + lo to ~16 significant bits).  Lane l holds 8 bf16 of
//    column (l % 16) at inputs 8*(l / 16) .. +7.  Layout
//    [NT column tiles][K/32 k-blocks][tile]; row m lives in tile m / 8.
//
//  * MFMA result: lane l, register r holds C[4*(l/16) + r][l % 16].  The
//    output for weight row i and activation row m is C[i][m%8] + C[i][m%8+8].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;

namespace sd {

constexpr int kTileBytes = 1024;
constexpr int kTileU16 = 512;       // bf16 elements per tile
constexpr int kColsPerTile = 8;     // activation rows per column tile
constexpr int kMaxRows = 32;        // rows per forward pass
constexpr int kMaxNT = kMaxRows / kColsPerTile;
// Draft trees: nodes of one tree (its forwards take at most kMaxRows of them
// at a time) and the 32-bit words of a node's ancestor mask.
constexpr int kMaxTreeNodes = 512;
constexpr int kTreeWords = kMaxTreeNodes / 32;

__device__ __forceinline__ float bf2f(bf16_bits b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float -> bf16, round to nearest even (the native gfx950 conversion).
__device__ __forceinline__ bf16_bits f2bf(float f) {
  return __builtin_bit_cast(bf16_bits, (__bf16)f);
}

// Activation operand tiles: one 1 KiB tile per (column tile t, k-block of
// 32 inputs) holds rows 8t..8t+7 as MFMA operand B; operand column col
// carries row col / 2, its hi part in even and its lo part in odd columns.
// The lane of column col and k-quarter s reads the 16-byte slot
// btile_slot(col, s) = 16 (col / 4) + 4 s + col % 4: every group of four
// lanes reads one 64-byte segment, and rows 2j and 2j + 1 fill bytes
// 256 j .. 256 j + 255, so a pass of M < 8 rows touches the first
// 256 ceil(M / 2) bytes of the tile.
constexpr int kBtileLo = 8;   // bf16 elements from a hi part to its lo part

__device__ __forceinline__ int btile_slot(int col, int s) { return 16 * (col >> 2) + 4 * s + (col & 3); }

// Position of activation (row m, input k) inside an activation tile buffer,
// in bf16 units; the "lo" element sits kBtileLo further.
__device__ __forceinline__ size_t btile_index(int KB, int m, int k) {
  int t = m >> 3, c = m & 7;
  int kb = k >> 5, s = (k >> 3) & 3, e = k & 7;
  return ((size_t)(t * KB + kb) * kTileU16) + (size_t)(btile_slot(2 * c, s) * 8 + e);
}

__device__ __forceinline__ void btile_put(bf16_bits* tiles, int KB, int m, int k, float v) {
  size_t i = btile_index(KB, m, k);
  bf16_bits hi = f2bf(v);
  bf16_bits lo = f2bf(v - bf2f(hi));
  tiles[i] = hi;
  tiles[i + kBtileLo] = lo;
}

// Cross-lane moves within 16-lane rows (DPP); control words of the GFX9
// DPP encoding: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_ror:8 = 0x128,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Value of lane (l ^ 1): the lo column next to a hi column of an MFMA result.
__device__ __forceinline__ float swap1(float v) { return dpp_f<0xB1>(v); }

// Sum over each 16-lane row in a fixed tree; every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

// Wave-wide sum / max: a fixed tree inside each 16-lane row, then the four
// row results in lane order.  Every lane gets the same value.
__device__ __forceinline__ float warp_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return ((readlane_f(v, 0) + readlane_f(v, 16)) + readlane_f(v, 32)) + readlane_f(v, 48);
}

__device__ __forceinline__ float warp_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Wave-wide (max, lowest index of the max).
__device__ __forceinline__ void warp_argmax(float& v, int& idx) {
#define SD_ARGMAX_STEP(CTRL)                                        \
  {                                                                 \
    float ov = dpp_f<CTRL>(v);                                      \
    int oi = dpp_i<CTRL>(idx);                                      \
    if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }      \
  }
  SD_ARGMAX_STEP(0xB1)
  SD_ARGMAX_STEP(0x4E)
  SD_ARGMAX_STEP(0x141)
  SD_ARGMAX_STEP(0x140)
#undef SD_ARGMAX_STEP
  float bv = readlane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(idx, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    float ov = readlane_f(v, 16 * r);
    int oi = __builtin_amdgcn_readlane(idx, 16 * r);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  v = bv;
  idx = bi;
}

// Sticky device error bits.
enum : int32_t {
  kErrCapacity = 1,     // a forward would pass the cache capacity
  kErrTrim = 2,         // trim above the current length
  kErrNonFinite = 4,    // non-finite logits
  kErrTable = 8,        // draft table / noise read past its end
  kErrOutput = 16,      // committed-token buffer full
  kErrSync = 32,        // a split-K hand-off waited past its bound
  kErrTree = 64,        // a tree row's parent is not an earlier row
};

__device__ __forceinline__ void raise_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace sd
