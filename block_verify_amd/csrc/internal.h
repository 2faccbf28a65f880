// Host-side internals shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/specdec.h"
#include "device_common.h"

namespace sd {

struct Dims {
  int L, H, nq, nkv, hd, F, V;
  float theta, eps;
  int wfmt;
  int qdim() const { return nq * hd; }
  int kvdim() const { return nkv * hd; }
  int qkv_rows() const { return (nq + 2 * nkv) * hd; }
  int group() const { return nq / nkv; }
};

int dims_from_desc(const specdec_model_desc* d, Dims* out);

// Byte offsets of every packed tensor inside the weight blob.
struct LayerOffsets {
  size_t attn_norm, wqkv, wo, mlp_norm, wgu, wdown;
  size_t s_wqkv, s_wo, s_wgu, s_wdown;   // 4-bit models: (scale, zero) arrays
};
struct BlobLayout {
  size_t embed, final_norm, lm_head, total;
  std::vector<LayerOffsets> layer;
};
BlobLayout blob_layout(const Dims& d);

struct LayerPtrs {
  const float* attn_norm;
  const float* mlp_norm;
  const bf16x8_t* wqkv;   // tiles, RoPE-paired row groups
  const bf16x8_t* wo;
  const bf16x8_t* wgu;    // tiles, gate/up interleaved by 8 rows
  const bf16x8_t* wdown;
  // 4-bit substitute weights (weight_format == SPECDEC_W_Q4G64): codes and
  // (scale, zero) pairs of each linear, in the 4-bit kernel's block order
  const uint8_t* q_wqkv;
  const uint8_t* q_wo;
  const uint8_t* q_wgu;
  const uint8_t* q_wdown;
  const uint8_t* s_wqkv;
  const uint8_t* s_wo;
  const uint8_t* s_wgu;
  const uint8_t* s_wdown;
};

}  // namespace sd

struct specdec_model {
  sd::Dims d;
  const bf16_bits* embed;
  const float* final_norm;
  const bf16x8_t* lm_head;
  std::vector<sd::LayerPtrs> layers;
};

// K is [nkv][lp][hd] per layer; V is kept transposed, [nkv][hd][lp], so the
// attention's P*V operand reads 8 consecutive keys of one head dim as 16
// contiguous bytes.  lp = max_len rounded up to kKvPad positions.
struct specdec_cache {
  sd::Dims d;
  bf16_bits* kv;      // [L][K|V][...]
  float2* rope;       // [max_len][hd/2] (cos, sin)
  int32_t* d_len;
  int max_len;
  int lp;
  bf16_bits* k_layer(int l) const { return kv + (size_t)l * 2 * d.nkv * lp * d.hd; }
  bf16_bits* v_layer(int l) const { return k_layer(l) + (size_t)d.nkv * lp * d.hd; }
};

namespace sd {

#ifndef SD_ATTN_CHUNK
#define SD_ATTN_CHUNK 64
#endif
constexpr int kAttnChunk = SD_ATTN_CHUNK;   // keys per attention chunk (64 or 128)
constexpr int kKvPad = 128;                 // cache positions are padded to a multiple of this
static_assert(kKvPad % kAttnChunk == 0, "chunks tile the padded cache");
constexpr int kWsHeader = 65536;   // error word + split-K launch sequence numbers
constexpr int kMaxSplit = 8;
constexpr int kMaxHidden = 4096;   // the largest hidden size a model may have
// K splits of the down projection: bf16 (tuned on the verify forward) and
// 4-bit (bounded by the activations the 4-bit kernel stages in LDS).
#ifndef SD_DOWN_SPLIT
#define SD_DOWN_SPLIT 2
#endif
constexpr int kDownSplit = SD_DOWN_SPLIT;

// With two K splits the producer takes kSplit0Share / 64 of the k-blocks
// (the finisher, which waits for its partials, the rest), as long as the
// finisher's waves still stream their share in one batch.
constexpr unsigned kSplit0Share = 30;

// Workspace plan for one model.
struct WsPlan {
  size_t err, cnt, x, xb, ss, qb, ob, hb, att_o, att_ml, part, lm_part, toks, logits, tree, total;
  int max_rows, nt, max_chunks, lm_wgs;
};
WsPlan ws_plan(const Dims& d, int max_rows, int max_len);

// Kernel launchers (kernels_forward.hip).
struct FwdArgs {
  const specdec_model* m;
  const specdec_cache* c;
  const int32_t* tokens;
  int rows;
  float* logits;
  int32_t* argmax;
  float* lse;
  char* ws;
  const WsPlan* plan;
  hipStream_t stream;
  const int32_t* gate;   // optional device flag: when *gate == 0 every kernel returns at once
  bool skip_head;        // prefill chunks before the last: no LM head, only the length advance
  int32_t* err = nullptr;   // sticky error word; null: the word at the workspace's start
  const int32_t* parents = nullptr;   // tree forward: each node's parent node (-1: none), else a causal block
  int tree_n0 = 0;                    // tree forward: the node of row 0 (nodes before it are in the cache)
};
hipError_t launch_forward(const FwdArgs& a);

// Row order of the packed linears.  Output row r of a weight goes to row
// group g, slot i (16 slots per group): PLAIN keeps the order; ROPE puts the
// rotate-half partners (d, d + hd/2) of a head in slots i and i + 8 of one
// group; GATE / UP interleave 8 gate rows and the 8 matching up rows.
enum PackKind { PACK_PLAIN = 0, PACK_ROPE = 1, PACK_GATE = 2, PACK_UP = 3 };

// 4-bit group-64 linears (kernels_q4.hip).  One workgroup covers at most
// kQ4MaxBlocks blocks of 128 inputs of a linear's K (the down projection
// splits its K over up to kMaxSplit workgroups).
constexpr int kQ4MaxBlocks = 32;
// Packed sizes of one 4-bit linear with N outputs and K inputs.
inline size_t q4_code_bytes(int N, int K) { return (size_t)N * ((K + 127) / 128) * 64; }
inline size_t q4_scale_bytes(int N, int K) { return (size_t)N * ((K + 127) / 128) * 8; }
enum class Q4Linear { QKV, O, GATE_UP, DOWN };
struct GemvParams;
hipError_t launch_q4_linear(Q4Linear which, const GemvParams& p, const uint8_t* codes, const uint8_t* scales, int K,
                            hipStream_t s);
hipError_t launch_pack_q4(const void* src, int rows, int K, int kind, int hd, int group_base, uint8_t* codes,
                          uint8_t* scales, hipStream_t s);
hipError_t launch_pack(const Dims& d, int index, const void* src, void* blob, const BlobLayout& lay, hipStream_t s);
hipError_t launch_trim(int32_t* d_len, int32_t new_len, const int32_t* d_base, int32_t* err, hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, hipStream_t s);
// Draft trees (kernels_tree.hip): selection of a construction step (the k
// best (leaf, token) pairs of r leaves' logits), its first and last steps,
// and the greedy acceptance (longest path, K/V compaction, commit).
hipError_t launch_tree_select(const float* logits, int r, int V, int k, float inv_t, int n0, int n_new,
                              float* scratch, int32_t* tokens, int32_t* parents, float* scores, hipStream_t s);
size_t tree_select_scratch_bytes(int r, int V, int k);
hipError_t launch_tree_root(const int32_t* root, const int32_t* d_len, int32_t* saved, int32_t* tokens,
                            int32_t* parents, float* scores, hipStream_t s);
hipError_t launch_tree_restore(int32_t* d_len, const int32_t* saved, hipStream_t s);
hipError_t launch_tree_accept(const specdec_cache* c, const int32_t* tokens, const int32_t* parents, int n,
                              const int32_t* argmax, int32_t* out_tokens, int32_t* out_count, int32_t* root,
                              int32_t* log, int log_cap, int32_t* err, hipStream_t s);

// Round kernels (kernels_round.hip).
struct RoundDev;  // defined in api.cpp
}  // namespace sd
