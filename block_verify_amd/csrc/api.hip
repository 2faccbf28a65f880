// C ABI of the block-verify path: validation, HBM layouts, orchestration.
// Kernels live in kernels_forward.hip and kernels_round.hip.
#include <math.h>
#include <string.h>

#include <cmath>

#include <new>
#include <vector>

#include "round_dev.h"

namespace {
thread_local int32_t g_last_hip = 0;

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return SPECDEC_OK;
  g_last_hip = (int32_t)e;
  return SPECDEC_EHIP;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

namespace sd {

int dims_from_desc(const specdec_model_desc* d, Dims* o) {
  if (!d || !o) return SPECDEC_EINVAL;
  Dims x;
  x.L = d->n_layers; x.H = d->hidden; x.nq = d->n_q_heads; x.nkv = d->n_kv_heads; x.hd = d->head_dim;
  x.F = d->ffn; x.V = d->vocab; x.theta = d->rope_theta; x.eps = d->rms_eps; x.wfmt = d->weight_format;
  if (x.L <= 0 || x.H <= 0 || x.nq <= 0 || x.nkv <= 0 || x.hd <= 0 || x.F <= 0 || x.V <= 0) return SPECDEC_EINVAL;
  if (!(x.theta > 0.f) || !(x.eps >= 0.f)) return SPECDEC_EINVAL;
  if (x.wfmt != SPECDEC_W_BF16 && x.wfmt != SPECDEC_W_Q4G64) return SPECDEC_EINVAL;
  if (x.hd != 64 && x.hd != 128) return SPECDEC_ESHAPE;
  if (x.nq % x.nkv != 0 || x.nq / x.nkv > 8) return SPECDEC_ESHAPE;
  if (x.H % 32 || x.F % 32 || x.qdim() % 32 || x.V % 16 || x.H % 16) return SPECDEC_ESHAPE;
  // the RMSNorm scale reads at most 256 per-16-feature partials per row
  if (x.H > kMaxHidden || x.V > (1 << 24)) return SPECDEC_ESHAPE;
  if (x.wfmt == SPECDEC_W_Q4G64) {
    if (x.H % 64 || x.qdim() % 64 || x.F % 64) return SPECDEC_ESHAPE;
    // a workgroup of the 4-bit product covers kQ4MaxBlocks blocks of 128 inputs
    // (kMaxSplit of them for the down projection)
    if ((x.H + 127) / 128 > kQ4MaxBlocks || (x.qdim() + 127) / 128 > kQ4MaxBlocks ||
        (x.F + 127) / 128 > kMaxSplit * kQ4MaxBlocks)
      return SPECDEC_ESHAPE;
  }
  *o = x;
  return SPECDEC_OK;
}

BlobLayout blob_layout(const Dims& d) {
  BlobLayout b;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  b.embed = take((size_t)d.V * d.H * 2);
  b.layer.resize(d.L);
  const bool q4 = d.wfmt == SPECDEC_W_Q4G64;
  for (int l = 0; l < d.L; ++l) {
    LayerOffsets& o = b.layer[l];
    o.attn_norm = take((size_t)d.H * 4);
    o.mlp_norm = take((size_t)d.H * 4);
    if (q4) {
      o.wqkv = take(q4_code_bytes(d.qkv_rows(), d.H));
      o.s_wqkv = take(q4_scale_bytes(d.qkv_rows(), d.H));
      o.wo = take(q4_code_bytes(d.H, d.qdim()));
      o.s_wo = take(q4_scale_bytes(d.H, d.qdim()));
      o.wgu = take(q4_code_bytes(2 * d.F, d.H));
      o.s_wgu = take(q4_scale_bytes(2 * d.F, d.H));
      o.wdown = take(q4_code_bytes(d.H, d.F));
      o.s_wdown = take(q4_scale_bytes(d.H, d.F));
    } else {
      o.wqkv = take((size_t)d.qkv_rows() * d.H * 2);
      o.wo = take((size_t)d.H * d.qdim() * 2);
      o.wgu = take((size_t)2 * d.F * d.H * 2);
      o.wdown = take((size_t)d.H * d.F * 2);
      o.s_wqkv = o.s_wo = o.s_wgu = o.s_wdown = 0;
    }
  }
  b.final_norm = take((size_t)d.H * 4);
  b.lm_head = take((size_t)d.V * d.H * 2);
  b.total = off;
  return b;
}

WsPlan ws_plan(const Dims& d, int max_rows, int max_len) {
  WsPlan p;
  p.max_rows = kMaxRows;
  p.nt = kMaxNT;
  p.max_chunks = (max_len + kAttnChunk - 1) / kAttnChunk;
  p.lm_wgs = d.V / 16;   // LM-head workgroups for the smallest launch shape (one row group each)
  (void)max_rows;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t R = kMaxRows;
  p.err = 0;
  p.cnt = 256;
  off = kWsHeader;
  p.x = take(R * d.H * 4);
  p.xb = take((size_t)kMaxNT * d.H * 32);
  p.ss = take(R * (d.H / 16) * 4);
  p.qb = take((size_t)d.nkv * (kMaxRows * 8 / 16) * (d.hd / 32) * 2 * 1024);
  p.ob = take((size_t)kMaxNT * d.qdim() * 32);
  p.hb = take((size_t)kMaxNT * d.F * 32);
  p.att_o = take((size_t)d.nkv * p.max_chunks * (R * 8) * d.hd * 4);
  p.att_ml = take((size_t)d.nkv * p.max_chunks * (R * 8) * 2 * 4);
  p.part = take((size_t)kMaxSplit * kMaxRows * d.H * 8);   // (value, tag) pairs
  p.lm_part = take(R * p.lm_wgs * 3 * 4);
  p.toks = take(R * 4 * 2);
  p.logits = take(R * (size_t)d.V * 4);
  p.tree = take((R + R * kTreeWords) * 4);   // tree forward: depth and ancestor mask per row
  p.total = off;
  return p;
}

RoundWsPlan round_ws_plan(int V, int k) {
  RoundWsPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t K1 = (size_t)kMaxK + 1;
  (void)k;
  p.flags = take(kNumFlags * 4);
  p.block = take(K1 * 4);
  p.repair_tok = take(4);
  p.rows_argmax = take(K1 * 4);
  p.rows_lse = take(K1 * 4);
  p.repair_argmax = take(4);
  p.repair_lse = take(4);
  p.q_lse = take(K1 * 4);
  p.snap = take(kNumSnap * 4);
  p.dbg = take((2 * kMaxK + 2) * 4);
  p.smax = take((size_t)n_slices(V) * 4);
  p.ssum = take((size_t)n_slices(V) * 4);
  p.sw = take((size_t)n_slices(V) * 8);
  p.sctl = take(4 * 4);
  p.t_lse = take(K1 * 4);
  p.tsmax = take(K1 * n_slices(V) * 4);
  p.tssum = take(K1 * n_slices(V) * 4);
  p.hcnt = take((size_t)n_slices(V) * kTruncBins * 4);
  p.hmass = take((size_t)n_slices(V) * kTruncBins * 8);
  p.trunc = take(sizeof(TruncState));
  p.draft_argmax = take(4);
  p.rows_logits = take(K1 * V * 4);
  p.saved_logits = take((size_t)V * 4);
  p.q_logits = take(K1 * V * 4);
  p.z = take((size_t)V * 4);
  p.draft_logits = take((size_t)V * 4);
  p.snap_logits = take((size_t)V * 4);
  p.total = off;
  return p;
}

hipError_t launch_copy_last(const FwdArgs& a, float* logits_dst, int32_t* argmax_dst, float* lse_dst);
hipError_t launch_advance(int32_t* d_len, int rows, int max_len, const int32_t* gate, hipStream_t s);

}  // namespace sd

using namespace sd;

struct specdec_round {
  specdec_round_desc desc;
  RoundDev dev;
  WsPlan tplan, dplan;
  int prompt_len;
  long calls;
  hipStream_t cap_stream;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
  // the whole round as one graph, replayed when no per-term events are
  // recorded (one launch per round instead of four)
  hipGraph_t fused_graph;
  hipGraphExec_t fused_exec;
};

extern "C" {

int32_t specdec_last_hip_error(void) { return g_last_hip; }

const char* specdec_status_str(int s) {
  switch (s) {
    case SPECDEC_OK: return "ok";
    case SPECDEC_EINVAL: return "invalid argument";
    case SPECDEC_ECAPACITY: return "capacity exceeded";
    case SPECDEC_ESHAPE: return "unsupported shape";
    case SPECDEC_EHIP: return "HIP runtime error";
    case SPECDEC_EDEVICE: return "device error flag set";
    case SPECDEC_EUNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

int32_t specdec_tensor_count(const specdec_model_desc* desc) {
  if (!desc || desc->n_layers <= 0) return 0;
  return 3 + 9 * desc->n_layers;
}

int specdec_weights_bytes(const specdec_model_desc* desc, size_t* bytes) {
  Dims d;
  int rc = dims_from_desc(desc, &d);
  if (rc) return rc;
  if (!bytes) return SPECDEC_EINVAL;
  *bytes = blob_layout(d).total;
  return SPECDEC_OK;
}

int specdec_weights_pack(const specdec_model_desc* desc, int32_t index, const void* d_src, void* d_blob, void* stream) {
  Dims d;
  int rc = dims_from_desc(desc, &d);
  if (rc) return rc;
  if (!d_src || !d_blob) return SPECDEC_EINVAL;
  if (index < 0 || index >= 3 + 9 * d.L) return SPECDEC_EINVAL;
  const BlobLayout lay = blob_layout(d);
  if (d.wfmt == SPECDEC_W_Q4G64 && index > 0 && index < 1 + 9 * d.L) {
    const int l = (index - 1) / 9, which = (index - 1) % 9;
    const LayerOffsets& o = lay.layer[l];
    uint8_t* blob = static_cast<uint8_t*>(d_blob);
    const int qg = d.qdim() / 16, kg = d.kvdim() / 16;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    switch (which) {
      case 1: e = launch_pack_q4(d_src, d.qdim(), d.H, PACK_ROPE, d.hd, 0, blob + o.wqkv, blob + o.s_wqkv, st); break;
      case 2: e = launch_pack_q4(d_src, d.kvdim(), d.H, PACK_ROPE, d.hd, qg, blob + o.wqkv, blob + o.s_wqkv, st); break;
      case 3:
        e = launch_pack_q4(d_src, d.kvdim(), d.H, PACK_PLAIN, d.hd, qg + kg, blob + o.wqkv, blob + o.s_wqkv, st);
        break;
      case 4: e = launch_pack_q4(d_src, d.H, d.qdim(), PACK_PLAIN, d.hd, 0, blob + o.wo, blob + o.s_wo, st); break;
      case 6: e = launch_pack_q4(d_src, d.F, d.H, PACK_GATE, d.hd, 0, blob + o.wgu, blob + o.s_wgu, st); break;
      case 7: e = launch_pack_q4(d_src, d.F, d.H, PACK_UP, d.hd, 0, blob + o.wgu, blob + o.s_wgu, st); break;
      case 8: e = launch_pack_q4(d_src, d.H, d.F, PACK_PLAIN, d.hd, 0, blob + o.wdown, blob + o.s_wdown, st); break;
      default: return hip_status(launch_pack(d, index, d_src, d_blob, lay, st));   // norms stay fp32 gains
    }
    return hip_status(e);
  }
  return hip_status(launch_pack(d, index, d_src, d_blob, lay, (hipStream_t)stream));
}

int specdec_model_create(const specdec_model_desc* desc, const void* d_blob, const specdec_model* share,
                         specdec_model** out) {
  Dims d;
  int rc = dims_from_desc(desc, &d);
  if (rc) return rc;
  if (!d_blob || !out) return SPECDEC_EINVAL;
  if (share && (share->d.H != d.H || share->d.V != d.V)) return SPECDEC_ESHAPE;
  BlobLayout lay = blob_layout(d);
  const char* b = static_cast<const char*>(d_blob);
  specdec_model* m = new (std::nothrow) specdec_model;
  if (!m) return SPECDEC_EINVAL;
  m->d = d;
  m->embed = share ? share->embed : reinterpret_cast<const bf16_bits*>(b + lay.embed);
  m->final_norm = share ? share->final_norm : reinterpret_cast<const float*>(b + lay.final_norm);
  m->lm_head = share ? share->lm_head : reinterpret_cast<const bf16x8_t*>(b + lay.lm_head);
  m->layers.resize(d.L);
  for (int l = 0; l < d.L; ++l) {
    const LayerOffsets& o = lay.layer[l];
    LayerPtrs& p = m->layers[l];
    memset(&p, 0, sizeof(p));
    p.attn_norm = reinterpret_cast<const float*>(b + o.attn_norm);
    p.mlp_norm = reinterpret_cast<const float*>(b + o.mlp_norm);
    p.wqkv = reinterpret_cast<const bf16x8_t*>(b + o.wqkv);
    p.wo = reinterpret_cast<const bf16x8_t*>(b + o.wo);
    p.wgu = reinterpret_cast<const bf16x8_t*>(b + o.wgu);
    p.wdown = reinterpret_cast<const bf16x8_t*>(b + o.wdown);
    if (d.wfmt == SPECDEC_W_Q4G64) {
      const uint8_t* ub = reinterpret_cast<const uint8_t*>(b);
      p.q_wqkv = ub + o.wqkv; p.s_wqkv = ub + o.s_wqkv;
      p.q_wo = ub + o.wo; p.s_wo = ub + o.s_wo;
      p.q_wgu = ub + o.wgu; p.s_wgu = ub + o.s_wgu;
      p.q_wdown = ub + o.wdown; p.s_wdown = ub + o.s_wdown;
    }
  }
  *out = m;
  return SPECDEC_OK;
}

void specdec_model_destroy(specdec_model* m) { delete m; }

int specdec_cache_bytes(const specdec_model_desc* desc, int32_t max_len, size_t* bytes) {
  Dims d;
  int rc = dims_from_desc(desc, &d);
  if (rc) return rc;
  if (!bytes || max_len <= 0) return SPECDEC_EINVAL;
  if (max_len > 65536) return SPECDEC_ECAPACITY;
  const size_t lp = ((size_t)max_len + kKvPad - 1) / kKvPad * kKvPad;
  size_t kv = align256((size_t)d.L * 2 * d.nkv * lp * d.hd * 2);
  size_t rope = align256((size_t)max_len * (d.hd / 2) * 8);
  *bytes = kv + rope;
  return SPECDEC_OK;
}

int specdec_cache_create(const specdec_model_desc* desc, void* d_mem, size_t bytes, int32_t max_len, int32_t* d_len,
                         specdec_cache** out) {
  Dims d;
  int rc = dims_from_desc(desc, &d);
  if (rc) return rc;
  size_t need;
  rc = specdec_cache_bytes(desc, max_len, &need);
  if (rc) return rc;
  if (!d_mem || !d_len || !out) return SPECDEC_EINVAL;
  if (bytes < need) return SPECDEC_ECAPACITY;
  specdec_cache* c = new (std::nothrow) specdec_cache;
  if (!c) return SPECDEC_EINVAL;
  c->d = d;
  c->kv = static_cast<bf16_bits*>(d_mem);
  const size_t lpad = ((size_t)max_len + kKvPad - 1) / kKvPad * kKvPad;
  size_t kv = align256((size_t)d.L * 2 * d.nkv * lpad * d.hd * 2);
  c->rope = reinterpret_cast<float2*>(static_cast<char*>(d_mem) + kv);
  c->d_len = d_len;
  c->max_len = max_len;
  c->lp = (max_len + kKvPad - 1) / kKvPad * kKvPad;
  // RoPE table in double precision on the host: angle = pos * theta^(-2i/d)
  const int half = d.hd / 2;
  std::vector<float2> tab((size_t)max_len * half);
  for (int i = 0; i < half; ++i) {
    double inv = pow((double)d.theta, -2.0 * i / (double)d.hd);
    for (int p = 0; p < max_len; ++p) {
      double a = (double)p * inv;
      tab[(size_t)p * half + i] = make_float2((float)cos(a), (float)sin(a));
    }
  }
  hipError_t e = hipMemcpy(c->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(d_len, 0, sizeof(int32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    delete c;
    return hip_status(e);
  }
  *out = c;
  return SPECDEC_OK;
}

void specdec_cache_destroy(specdec_cache* c) { delete c; }

int specdec_kv_trim(specdec_cache* c, int32_t new_len, int32_t* d_err, void* stream) {
  if (!c || new_len < 0 || new_len > c->max_len) return SPECDEC_EINVAL;
  return hip_status(launch_trim(c->d_len, new_len, nullptr, d_err, (hipStream_t)stream));
}

int specdec_workspace_bytes(const specdec_model_desc* desc, int32_t max_rows, int32_t max_len, size_t* bytes) {
  Dims d;
  int rc = dims_from_desc(desc, &d);
  if (rc) return rc;
  if (!bytes || max_rows <= 0 || max_len <= 0) return SPECDEC_EINVAL;
  if (max_rows > SPECDEC_MAX_ROWS) return SPECDEC_ECAPACITY;
  *bytes = ws_plan(d, max_rows, max_len).total;
  return SPECDEC_OK;
}

int specdec_workspace_init(void* d_ws, size_t ws_bytes, void* stream) {
  if (!d_ws || ws_bytes < (size_t)kWsHeader) return SPECDEC_EINVAL;
  // all of it: the error word, the split-K sequence numbers and the tags of
  // the split-K partials start at zero (a tag is never zero after a launch)
  return hip_status(hipMemsetAsync(d_ws, 0, ws_bytes, (hipStream_t)stream));
}

static int check_fwd(const specdec_model* m, const specdec_cache* c, int32_t rows, size_t ws_bytes, WsPlan* plan) {
  if (!m || !c) return SPECDEC_EINVAL;
  if (rows < 1 || rows > SPECDEC_MAX_ROWS) return SPECDEC_ECAPACITY;
  if (m->d.L != c->d.L || m->d.nkv != c->d.nkv || m->d.hd != c->d.hd) return SPECDEC_ESHAPE;
  *plan = ws_plan(m->d, rows, c->max_len);
  if (ws_bytes < plan->total) return SPECDEC_ECAPACITY;
  return SPECDEC_OK;
}

int specdec_decode_step(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, int32_t rows,
                        float* d_logits, int32_t* d_argmax, float* d_lse, void* d_ws, size_t ws_bytes, void* stream) {
  WsPlan plan;
  int rc = check_fwd(m, c, rows, ws_bytes, &plan);
  if (rc) return rc;
  if (!d_tokens || !d_ws) return SPECDEC_EINVAL;
  FwdArgs a;
  a.m = m; a.c = c; a.tokens = d_tokens; a.rows = rows;
  a.logits = d_logits ? d_logits : reinterpret_cast<float*>(static_cast<char*>(d_ws) + plan.logits);
  a.argmax = d_argmax; a.lse = d_lse; a.ws = static_cast<char*>(d_ws); a.plan = &plan;
  a.stream = (hipStream_t)stream; a.gate = nullptr; a.skip_head = false;
  return hip_status(launch_forward(a));
}

int specdec_tree_verify(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, const int32_t* d_parents,
                        int32_t n, float* d_logits, int32_t* d_argmax, float* d_lse, void* d_ws, size_t ws_bytes,
                        void* stream) {
  if (!m) return SPECDEC_EINVAL;
  if (n < 1 || n > SPECDEC_MAX_TREE) return SPECDEC_ECAPACITY;
  const int pass = kMaxRows;
  WsPlan plan;
  int rc = check_fwd(m, c, n < pass ? n : pass, ws_bytes, &plan);
  if (rc) return rc;
  if (!d_tokens || !d_parents || !d_ws) return SPECDEC_EINVAL;
  // passes of up to `pass` nodes in node order: a node's ancestors are
  // earlier nodes, so their K/V are in the cache when its pass runs
  for (int n0 = 0; n0 < n; n0 += pass) {
    FwdArgs a;
    a.m = m; a.c = c; a.tokens = d_tokens + n0; a.rows = n - n0 < pass ? n - n0 : pass;
    a.logits = d_logits ? d_logits + (size_t)n0 * m->d.V
                        : reinterpret_cast<float*>(static_cast<char*>(d_ws) + plan.logits);
    a.argmax = d_argmax ? d_argmax + n0 : nullptr;
    a.lse = d_lse ? d_lse + n0 : nullptr;
    a.ws = static_cast<char*>(d_ws); a.plan = &plan;
    a.stream = (hipStream_t)stream; a.gate = nullptr; a.skip_head = false;
    a.parents = d_parents; a.tree_n0 = n0;
    rc = hip_status(launch_forward(a));
    if (rc) return rc;
  }
  return SPECDEC_OK;
}

int specdec_tree_accept(specdec_cache* c, const int32_t* d_tokens, const int32_t* d_parents, int32_t n,
                        const int32_t* d_argmax, int32_t* d_out_tokens, int32_t* d_out_count, int32_t* d_root,
                        int32_t* d_log, int32_t log_cap, int32_t* d_err, void* stream) {
  if (!c || !d_tokens || !d_parents || !d_argmax || !d_out_tokens || !d_out_count || !d_err) return SPECDEC_EINVAL;
  if (n < 1 || n > SPECDEC_MAX_TREE) return SPECDEC_ECAPACITY;
  if (d_log && log_cap < 0) return SPECDEC_EINVAL;
  return hip_status(launch_tree_accept(c, d_tokens, d_parents, n, d_argmax, d_out_tokens, d_out_count, d_root, d_log,
                                       d_log ? log_cap : 0, d_err, (hipStream_t)stream));
}

int specdec_tree_draft(const specdec_model* draft, specdec_cache* c, const int32_t* d_root, int32_t k,
                       int32_t depth, float temperature, int32_t* d_tokens, int32_t* d_parents, float* d_scores,
                       void* d_ws, size_t ws_bytes, void* stream) {
  if (!draft || !c || !d_root || !d_tokens || !d_parents || !d_scores || !d_ws) return SPECDEC_EINVAL;
  if (k < 1 || k > SPECDEC_MAX_K || k > draft->d.V || depth < 1) return SPECDEC_EINVAL;
  if (1 + (long)k * depth > SPECDEC_MAX_TREE) return SPECDEC_ECAPACITY;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return SPECDEC_EINVAL;
  const int pass = kMaxRows;
  WsPlan plan;
  int rc = check_fwd(draft, c, k < pass ? k : pass, ws_bytes, &plan);
  if (rc) return rc;
  const int V = draft->d.V;
  char* ws = static_cast<char*>(d_ws);
  // the leaves' logits in the first SPECDEC_MAX_K rows of the workspace's
  // logits region, the selection's partials after them
  float* leaf = reinterpret_cast<float*>(ws + plan.logits);
  float* scratch = leaf + (size_t)SPECDEC_MAX_K * V;
  if (tree_select_scratch_bytes(k, V, k) > (size_t)(kMaxRows - SPECDEC_MAX_K) * V * sizeof(float))
    return SPECDEC_ECAPACITY;
  int32_t* saved = reinterpret_cast<int32_t*>(ws + plan.toks);
  hipStream_t s = (hipStream_t)stream;
  rc = hip_status(launch_tree_root(d_root, c->d_len, saved, d_tokens, d_parents, d_scores, s));
  const float inv_t = 1.0f / temperature;
  for (int st = 0; st < depth && !rc; ++st) {
    const int r = st == 0 ? 1 : k, n0 = st == 0 ? 0 : 1 + (st - 1) * k;
    for (int j0 = 0; j0 < r && !rc; j0 += pass) {
      FwdArgs a;
      a.m = draft; a.c = c; a.tokens = d_tokens + n0 + j0; a.rows = r - j0 < pass ? r - j0 : pass;
      a.logits = leaf + (size_t)j0 * V; a.argmax = nullptr; a.lse = nullptr;
      a.ws = ws; a.plan = &plan; a.stream = s; a.gate = nullptr; a.skip_head = false;
      a.parents = d_parents; a.tree_n0 = n0 + j0;
      rc = hip_status(launch_forward(a));
    }
    if (!rc)
      rc = hip_status(launch_tree_select(leaf, r, V, k, inv_t, n0, 1 + st * k, scratch, d_tokens, d_parents, d_scores,
                                         s));
  }
  if (!rc) rc = hip_status(launch_tree_restore(c->d_len, saved, s));
  return rc;
}

// ---------------------------------------------------------------------------
// The decode step without a workspace argument, for callers that cannot
// allocate.  Its scratch is a file-scope device array: each GPU the library
// runs on holds its own copy until the process ends.  In host code the
// array's name is not a device address; the address comes from
// hipGetSymbolAddress once per device (specdec_static_init) and only that
// pointer is passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
static void* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

int specdec_static_init(void* stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return SPECDEC_EUNSUPPORTED;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_status(e);
  if (!ptr) return SPECDEC_EHIP;
  // the split-K launch sequence numbers and partial tags start at zero
  zero_fill_kernel<<<1024, 256, 0, (hipStream_t)stream>>>(static_cast<uint4*>(ptr), kStaticScratchBytes / 16);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_status(e);
  g_scratch_ptr[dev] = ptr;
  return SPECDEC_OK;
}

int specdec_decode_step_noalloc(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, int32_t rows,
                                float* d_logits, int32_t* d_argmax, float* d_lse, int32_t* d_err, void* stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices || !g_scratch_ptr[dev]) return SPECDEC_EINVAL;   // specdec_static_init first
  WsPlan plan;
  int rc = check_fwd(m, c, rows, kStaticScratchBytes, &plan);   // ECAPACITY past the scratch's size
  if (rc) return rc;
  if (!d_tokens || !d_err) return SPECDEC_EINVAL;
  char* ws = static_cast<char*>(g_scratch_ptr[dev]);
  FwdArgs a;
  a.m = m; a.c = c; a.tokens = d_tokens; a.rows = rows;
  a.logits = d_logits ? d_logits : reinterpret_cast<float*>(ws + plan.logits);
  a.argmax = d_argmax; a.lse = d_lse; a.ws = ws; a.plan = &plan;
  a.stream = (hipStream_t)stream; a.gate = nullptr; a.skip_head = false; a.err = d_err;
  return hip_status(launch_forward(a));
}

int specdec_prefill(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, int32_t n, int32_t chunk,
                    float* d_last_logits, int32_t* d_last_argmax, float* d_last_lse, void* d_ws, size_t ws_bytes,
                    void* stream) {
  WsPlan plan;
  int rc = check_fwd(m, c, 1, ws_bytes, &plan);
  if (rc) return rc;
  if (!d_tokens || !d_ws || n <= 0 || chunk <= 0) return SPECDEC_EINVAL;
  if (n > c->max_len) return SPECDEC_ECAPACITY;
  if (chunk > SPECDEC_MAX_ROWS) chunk = SPECDEC_MAX_ROWS;
  char* ws = static_cast<char*>(d_ws);
  for (int off = 0; off < n; off += chunk) {
    int rows = n - off < chunk ? n - off : chunk;
    bool last = off + rows >= n;
    FwdArgs a;
    a.m = m; a.c = c; a.tokens = d_tokens + off; a.rows = rows;
    a.logits = reinterpret_cast<float*>(ws + plan.logits);
    a.argmax = reinterpret_cast<int32_t*>(ws + plan.toks);
    a.lse = reinterpret_cast<float*>(ws + plan.toks + SPECDEC_MAX_ROWS * 4);
    a.ws = ws; a.plan = &plan; a.stream = (hipStream_t)stream; a.gate = nullptr;
    a.skip_head = !last;
    hipError_t e = launch_forward(a);
    if (e == hipSuccess && last) e = launch_copy_last(a, d_last_logits, d_last_argmax, d_last_lse);
    if (e != hipSuccess) return hip_status(e);
  }
  return SPECDEC_OK;
}

int specdec_check(const void* d_ws, int32_t* bits, void* stream) {
  if (!d_ws) return SPECDEC_EINVAL;
  int32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, d_ws, sizeof(int32_t), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  if (bits) *bits = h;
  return h ? SPECDEC_EDEVICE : SPECDEC_OK;
}

// ------------------------------------------------------------------ rounds

int specdec_round_state_bytes(int32_t cap, size_t* bytes) {
  if (!bytes || cap <= 0) return SPECDEC_EINVAL;
  *bytes = sizeof(specdec_round_state) + (size_t)cap * 4;
  return SPECDEC_OK;
}

int specdec_round_ws_bytes(const specdec_model_desc* target, int32_t k, size_t* bytes) {
  Dims d;
  int rc = dims_from_desc(target, &d);
  if (rc) return rc;
  if (!bytes || k < 1 || k > SPECDEC_MAX_K) return SPECDEC_EINVAL;
  *bytes = round_ws_plan(d.V, k).total;
  return SPECDEC_OK;
}

int specdec_round_create(const specdec_round_desc* desc, specdec_round** out) {
  if (!desc || !out || !desc->target || !desc->target_cache || !desc->d_state || !desc->d_ws || !desc->d_round_ws)
    return SPECDEC_EINVAL;
  const specdec_round_desc& q = *desc;
  if (q.k < 1 || q.k > SPECDEC_MAX_K) return SPECDEC_EINVAL;
  if (q.state_cap <= 0) return SPECDEC_EINVAL;
  if (q.mode != SPECDEC_GREEDY && q.mode != SPECDEC_STOCHASTIC && q.mode != SPECDEC_RELAXED) return SPECDEC_EINVAL;
  if (q.schedule != SPECDEC_SCHEDULE_A && q.schedule != SPECDEC_SCHEDULE_B) return SPECDEC_EINVAL;
  if (q.draft_source < SPECDEC_DRAFT_TABLE || q.draft_source > SPECDEC_DRAFT_Q4_SELF) return SPECDEC_EINVAL;
  const Dims& d = q.target->d;
  const int rows = q.k + (q.schedule == SPECDEC_SCHEDULE_B ? 1 : 0);
  if (rows > SPECDEC_MAX_ROWS) return SPECDEC_ECAPACITY;
  if (q.schedule == SPECDEC_SCHEDULE_B && !q.bonus) return SPECDEC_EINVAL;
  if (q.mode == SPECDEC_STOCHASTIC && (q.schedule != SPECDEC_SCHEDULE_A || q.draft_source != SPECDEC_DRAFT_NOISY_SELF))
    return SPECDEC_EUNSUPPORTED;
  if (q.mode != SPECDEC_STOCHASTIC && q.draft_source == SPECDEC_DRAFT_NOISY_SELF) return SPECDEC_EINVAL;
  if (q.mode == SPECDEC_STOCHASTIC) {
    if (!(q.temperature > 0.f) || !isfinite(q.temperature)) return SPECDEC_EINVAL;
    if (q.top_k < 0 || q.top_k > d.V || !(q.top_p > 0.f && q.top_p <= 1.f)) return SPECDEC_EINVAL;
    if (((q.top_k > 0 && q.top_k < d.V) || q.top_p < 1.f) && d.V > (1 << kKeyIndexBits)) return SPECDEC_EUNSUPPORTED;
  }
  if (q.mode == SPECDEC_RELAXED && !(q.relax_delta >= 0.f)) return SPECDEC_EINVAL;
  if ((q.draft_source == SPECDEC_DRAFT_TABLE || q.draft_source == SPECDEC_DRAFT_MODEL) &&
      (!q.d_draft_table || q.table_len <= 0))
    return SPECDEC_EINVAL;
  if (q.draft_source == SPECDEC_DRAFT_NOISY_SELF && (!q.d_noise || q.noise_rows <= 0)) return SPECDEC_EINVAL;
  if (q.draft_source == SPECDEC_DRAFT_MODEL) {
    if (!q.draft || !q.draft_cache || !q.d_draft_ws) return SPECDEC_EINVAL;
    if (q.draft->d.V != d.V) return SPECDEC_ESHAPE;
  }
  if (q.draft_source == SPECDEC_DRAFT_Q4_SELF) {
    if (!q.draft || q.draft_cache) return SPECDEC_EINVAL;
    if (q.schedule != SPECDEC_SCHEDULE_A) return SPECDEC_EUNSUPPORTED;
    const Dims& e = q.draft->d;
    if (e.L != d.L || e.H != d.H || e.V != d.V || e.nkv != d.nkv || e.nq != d.nq || e.hd != d.hd || e.F != d.F)
      return SPECDEC_ESHAPE;
  }
  specdec_round* r = new (std::nothrow) specdec_round;
  if (!r) return SPECDEC_EINVAL;
  r->desc = q;
  r->prompt_len = 0;
  r->calls = 0;
  r->cap_stream = nullptr;
  r->fused_graph = nullptr;
  r->fused_exec = nullptr;
  if (q.events && q.n_events < 5) { delete r; return SPECDEC_EINVAL; }
  r->tplan = ws_plan(d, rows, q.target_cache->max_len);
  if (q.ws_bytes < r->tplan.total) { delete r; return SPECDEC_ECAPACITY; }
  if (q.draft_source == SPECDEC_DRAFT_MODEL) {
    r->dplan = ws_plan(q.draft->d, 1, q.draft_cache->max_len);
    if (q.draft_ws_bytes < r->dplan.total) { delete r; return SPECDEC_ECAPACITY; }
  }
  RoundWsPlan rp = round_ws_plan(d.V, q.k);
  if (q.round_ws_bytes < rp.total) { delete r; return SPECDEC_ECAPACITY; }
  char* w = static_cast<char*>(q.d_round_ws);
  RoundDev& v = r->dev;
  memset(&v, 0, sizeof(v));
  v.state = q.d_state;
  v.flags = reinterpret_cast<int32_t*>(w + rp.flags);
  v.block = reinterpret_cast<int32_t*>(w + rp.block);
  v.repair_tok = reinterpret_cast<int32_t*>(w + rp.repair_tok);
  v.rows_argmax = reinterpret_cast<int32_t*>(w + rp.rows_argmax);
  v.rows_lse = reinterpret_cast<float*>(w + rp.rows_lse);
  v.rows_logits = reinterpret_cast<float*>(w + rp.rows_logits);
  v.saved_logits = reinterpret_cast<float*>(w + rp.saved_logits);
  v.repair_argmax = reinterpret_cast<int32_t*>(w + rp.repair_argmax);
  v.repair_lse = reinterpret_cast<float*>(w + rp.repair_lse);
  v.q_logits = reinterpret_cast<float*>(w + rp.q_logits);
  v.q_lse = reinterpret_cast<float*>(w + rp.q_lse);
  v.z = reinterpret_cast<float*>(w + rp.z);
  v.draft_logits = reinterpret_cast<float*>(w + rp.draft_logits);
  v.draft_argmax = reinterpret_cast<int32_t*>(w + rp.draft_argmax);
  v.snap_logits = reinterpret_cast<float*>(w + rp.snap_logits);
  v.snap = reinterpret_cast<int32_t*>(w + rp.snap);
  v.dbg = reinterpret_cast<float*>(w + rp.dbg);
  v.smax = reinterpret_cast<float*>(w + rp.smax);
  v.ssum = reinterpret_cast<float*>(w + rp.ssum);
  v.sw = reinterpret_cast<double*>(w + rp.sw);
  v.sctl = reinterpret_cast<int32_t*>(w + rp.sctl);
  v.t_lse = reinterpret_cast<float*>(w + rp.t_lse);
  v.tsmax = reinterpret_cast<float*>(w + rp.tsmax);
  v.tssum = reinterpret_cast<float*>(w + rp.tssum);
  v.hcnt = reinterpret_cast<int32_t*>(w + rp.hcnt);
  v.hmass = reinterpret_cast<uint64_t*>(w + rp.hmass);
  v.trunc = reinterpret_cast<TruncState*>(w + rp.trunc);
  v.t_len = q.target_cache->d_len;
  v.d_len = q.draft_source == SPECDEC_DRAFT_MODEL ? q.draft_cache->d_len : nullptr;
  v.err = static_cast<int32_t*>(q.d_ws);
  v.table = q.d_draft_table;
  v.table_len = q.table_len;
  v.noise = q.d_noise;
  v.noise_rows = q.noise_rows;
  v.seed = q.philox_seed;
  v.k = q.k; v.V = d.V; v.bonus = q.bonus ? 1 : 0; v.schedule = q.schedule; v.draft_source = q.draft_source;
  v.mode = q.mode;
  v.state_cap = q.state_cap;
  v.inv_t = q.mode == SPECDEC_STOCHASTIC ? 1.0f / q.temperature : 1.0f;
  v.top_k = q.mode == SPECDEC_STOCHASTIC ? q.top_k : 0;
  v.top_p = q.mode == SPECDEC_STOCHASTIC ? q.top_p : 1.0f;
  v.relax_delta = q.mode == SPECDEC_RELAXED ? q.relax_delta : 0.0f;
  *out = r;
  return SPECDEC_OK;
}

void specdec_round_destroy(specdec_round* r) {
  if (!r) return;
  for (auto x : r->execs) (void)hipGraphExecDestroy(x);
  for (auto g : r->graphs) (void)hipGraphDestroy(g);
  if (r->fused_exec) (void)hipGraphExecDestroy(r->fused_exec);
  if (r->fused_graph) (void)hipGraphDestroy(r->fused_graph);
  if (r->cap_stream) (void)hipStreamDestroy(r->cap_stream);
  delete r;
}

static hipError_t fwd(const specdec_round* r, bool draft, const int32_t* toks, int rows, float* logits,
                      int32_t* argmax, float* lse, const int32_t* gate, hipStream_t s) {
  const specdec_round_desc& q = r->desc;
  FwdArgs a;
  const bool own_draft = draft && q.draft_source == SPECDEC_DRAFT_MODEL;
  a.m = draft ? q.draft : q.target;
  a.c = own_draft ? q.draft_cache : q.target_cache;
  a.tokens = toks; a.rows = rows; a.logits = logits; a.argmax = argmax; a.lse = lse;
  a.ws = static_cast<char*>(own_draft ? q.d_draft_ws : q.d_ws);
  a.plan = own_draft ? &r->dplan : &r->tplan;
  a.stream = s; a.gate = gate; a.skip_head = false;
  return launch_forward(a);
}

int specdec_round_prefill(specdec_round* r, const int32_t* d_prompt, int32_t n, int32_t chunk, void* stream) {
  if (!r || !d_prompt || n <= 0 || chunk <= 0) return SPECDEC_EINVAL;
  const specdec_round_desc& q = r->desc;
  const bool B = q.schedule == SPECDEC_SCHEDULE_B;
  const int rows = q.k + (B ? 1 : 0);
  // room for the prompt and at least one round (specdec_round_reset checks the whole job)
  int need = n + 2 * rows + 2;
  if (need > q.target_cache->max_len) return SPECDEC_ECAPACITY;
  if (B && n < 2) return SPECDEC_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const RoundDev& v = r->dev;
  int32_t* err = static_cast<int32_t*>(q.d_ws);
  hipError_t e = launch_trim(q.target_cache->d_len, 0, nullptr, err, s);
  if (e == hipSuccess && q.draft_source == SPECDEC_DRAFT_MODEL) e = launch_trim(q.draft_cache->d_len, 0, nullptr, err, s);
  if (e != hipSuccess) return hip_status(e);
  int rc = specdec_prefill(q.target, q.target_cache, d_prompt, B ? n - 1 : n, chunk, v.saved_logits, v.repair_argmax,
                           v.repair_lse, q.d_ws, q.ws_bytes, stream);
  if (rc) return rc;
  if (q.draft_source == SPECDEC_DRAFT_MODEL) {
    rc = specdec_prefill(q.draft, q.draft_cache, d_prompt, n, chunk, v.draft_logits, v.draft_argmax, nullptr,
                         q.d_draft_ws, q.draft_ws_bytes, stream);
    if (rc) return rc;
  }
  r->prompt_len = n;
  e = launch_snapshot(v, B ? d_prompt + n - 1 : nullptr, s);
  if (e == hipSuccess) e = launch_reset(v, 0, s);
  return hip_status(e);
}

int specdec_round_reset(specdec_round* r, int32_t n_target, void* stream) {
  if (!r || n_target < 0) return SPECDEC_EINVAL;
  if (r->prompt_len == 0) return SPECDEC_EINVAL;
  const specdec_round_desc& q = r->desc;
  if ((size_t)n_target + q.k + 1 > (size_t)q.state_cap) return SPECDEC_ECAPACITY;
  int rows = q.k + (q.schedule == SPECDEC_SCHEDULE_B ? 1 : 0);
  // every round commits at least one token; positions used stay below
  // prompt + n_target + rows + 1
  if (r->prompt_len + n_target + 2 * rows + 2 > q.target_cache->max_len) return SPECDEC_ECAPACITY;
  return hip_status(launch_reset(r->dev, n_target, (hipStream_t)stream));
}

// A round is four segments: 0 round start + draft provision, 1 block verify,
// 2 acceptance + trim, 3 repair.  Per-term events sit between segments.
static hipError_t enqueue_segment(specdec_round* r, hipStream_t s, int seg);

static hipError_t record_mark(specdec_round* r, hipStream_t s, long call, int i) {
  const specdec_round_desc& q = r->desc;
  const int ring = q.events ? (q.n_events / 5) * 5 : 0;
  if (!ring) return hipSuccess;
  const int eb = (int)((call * 5) % ring);
  return hipEventRecord((hipEvent_t)q.events[eb + i], s);
}

static hipError_t enqueue_round(specdec_round* r, hipStream_t s) {
  const long call = r->calls++;
  hipError_t e = hipSuccess;
  for (int seg = 0; seg < 4 && e == hipSuccess; ++seg) {
    e = record_mark(r, s, call, seg);
    if (e == hipSuccess) e = enqueue_segment(r, s, seg);
  }
  if (e == hipSuccess) e = record_mark(r, s, call, 4);
  return e;
}

int specdec_verify_round(specdec_round* r, void* stream) {
  if (!r) return SPECDEC_EINVAL;
  if (r->prompt_len == 0) return SPECDEC_EINVAL;
  return hip_status(enqueue_round(r, (hipStream_t)stream));
}

int specdec_round_graph(specdec_round* r) {
  if (!r) return SPECDEC_EINVAL;
  if (r->prompt_len == 0) return SPECDEC_EINVAL;
  hipError_t e = hipSuccess;
  if (!r->cap_stream) e = hipStreamCreateWithFlags(&r->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_status(e);
  for (auto x : r->execs) (void)hipGraphExecDestroy(x);
  for (auto g : r->graphs) (void)hipGraphDestroy(g);
  r->execs.clear();
  r->graphs.clear();
  if (r->fused_exec) (void)hipGraphExecDestroy(r->fused_exec);
  if (r->fused_graph) (void)hipGraphDestroy(r->fused_graph);
  r->fused_exec = nullptr;
  r->fused_graph = nullptr;
  for (int seg = 0; seg < 4; ++seg) {
    e = hipStreamBeginCapture(r->cap_stream, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) break;
    hipError_t e2 = enqueue_segment(r, r->cap_stream, seg);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(r->cap_stream, &g);
    if (e2 != hipSuccess) e = e2;
    if (e != hipSuccess) { if (g) (void)hipGraphDestroy(g); break; }
    hipGraphExec_t x = nullptr;
    e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) { (void)hipGraphDestroy(g); break; }
    r->graphs.push_back(g);
    r->execs.push_back(x);
  }
  if (e == hipSuccess) {
    // the four segments back to back in one capture
    e = hipStreamBeginCapture(r->cap_stream, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      hipError_t e2 = hipSuccess;
      for (int seg = 0; seg < 4 && e2 == hipSuccess; ++seg) e2 = enqueue_segment(r, r->cap_stream, seg);
      hipGraph_t g = nullptr;
      e = hipStreamEndCapture(r->cap_stream, &g);
      if (e2 != hipSuccess) e = e2;
      if (e == hipSuccess) e = hipGraphInstantiate(&r->fused_exec, g, nullptr, nullptr, 0);
      if (g && e == hipSuccess) r->fused_graph = g;
      else if (g) (void)hipGraphDestroy(g);
    }
  }
  if (e != hipSuccess) {
    for (auto x : r->execs) (void)hipGraphExecDestroy(x);
    for (auto g : r->graphs) (void)hipGraphDestroy(g);
    r->execs.clear();
    r->graphs.clear();
    if (r->fused_exec) (void)hipGraphExecDestroy(r->fused_exec);
    r->fused_exec = nullptr;
  }
  return hip_status(e);
}

int specdec_round_graph_launch(specdec_round* r, int32_t n_rounds, void* stream) {
  if (!r || r->execs.size() != 4 || n_rounds < 0) return SPECDEC_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const specdec_round_desc& q = r->desc;
  const bool timed = q.events && (q.n_events / 5) * 5 > 0;
  if (!timed && r->fused_exec) {
    for (int i = 0; i < n_rounds; ++i) {
      ++r->calls;
      hipError_t e = hipGraphLaunch(r->fused_exec, s);
      if (e != hipSuccess) return hip_status(e);
    }
    return SPECDEC_OK;
  }
  for (int i = 0; i < n_rounds; ++i) {
    const long call = r->calls++;
    hipError_t e = hipSuccess;
    for (int seg = 0; seg < 4 && e == hipSuccess; ++seg) {
      e = record_mark(r, s, call, seg);
      if (e == hipSuccess) e = hipGraphLaunch(r->execs[(size_t)seg], s);
    }
    if (e == hipSuccess) e = record_mark(r, s, call, 4);
    if (e != hipSuccess) return hip_status(e);
  }
  return SPECDEC_OK;
}

static hipError_t enqueue_segment(specdec_round* r, hipStream_t s, int seg) {
  const specdec_round_desc& q = r->desc;
  const RoundDev& v = r->dev;
  const bool B = q.schedule == SPECDEC_SCHEDULE_B;
  const int k = q.k;
  const int32_t* open = v.flags + kFlagOpen;
  const int32_t* rep = v.flags + kFlagRepair;
  hipError_t e = hipSuccess;
  if (seg == 0) {
    e = launch_round_start(v, s);
    if (e == hipSuccess && q.draft_source == SPECDEC_DRAFT_MODEL) {
      for (int j = 0; j < k && e == hipSuccess; ++j)
        e = fwd(r, true, v.block + (B ? 1 : 0) + j, 1, v.draft_logits, v.draft_argmax, nullptr, open, s);
    } else if (e == hipSuccess && q.draft_source == SPECDEC_DRAFT_NOISY_SELF) {
      e = launch_draft_sample(v, v.saved_logits, 0, s);
      for (int j = 1; j < k && e == hipSuccess; ++j) {
        e = fwd(r, false, v.block + j - 1, 1, v.z, nullptr, nullptr, open, s);
        if (e == hipSuccess) e = launch_draft_sample(v, v.z, j, s);
      }
      if (e == hipSuccess && k > 1) e = launch_rewind(v, v.t_len, k - 1, s);
    } else if (e == hipSuccess && q.draft_source == SPECDEC_DRAFT_Q4_SELF) {
      for (int j = 1; j < k && e == hipSuccess; ++j)
        e = fwd(r, true, v.block + j - 1, 1, v.draft_logits, v.block + j, nullptr, open, s);
      if (e == hipSuccess && k > 1) e = launch_rewind(v, v.t_len, k - 1, s);
    }
  } else if (seg == 1) {
    e = fwd(r, false, v.block, k + (B ? 1 : 0), v.rows_logits, v.rows_argmax, v.rows_lse, open, s);
  } else if (seg == 2) {
    e = q.mode == SPECDEC_STOCHASTIC ? launch_accept_stochastic(v, s) : launch_accept_greedy(v, s);
  } else {
    if (!B) {
      e = fwd(r, false, v.repair_tok, 1, v.saved_logits, v.repair_argmax, v.repair_lse, rep, s);
      if (e == hipSuccess) e = launch_repair_done(v, s);
      // without the bonus a fully accepted round keeps its last verify row as saved_next
      if (e == hipSuccess && !q.bonus) e = launch_copy_saved(v, s);
    }
    if (e == hipSuccess && q.draft_source == SPECDEC_DRAFT_MODEL)
      e = fwd(r, true, v.repair_tok, 1, v.draft_logits, v.draft_argmax, nullptr, rep, s);
  }
  return e;
}

int specdec_round_debug_view(const specdec_round* r, int32_t which, void** d_ptr, size_t* bytes) {
  if (!r || !d_ptr || !bytes) return SPECDEC_EINVAL;
  const RoundDev& v = r->dev;
  const size_t V = (size_t)v.V;
  switch (which) {
    case 0: *d_ptr = v.saved_logits; *bytes = V * 4; break;
    case 1: *d_ptr = v.rows_logits; *bytes = (size_t)(v.k + 1) * V * 4; break;
    case 2: *d_ptr = v.q_logits; *bytes = (size_t)v.k * V * 4; break;
    case 3: *d_ptr = v.block; *bytes = (size_t)(v.k + 1) * 4; break;
    case 4: *d_ptr = v.dbg; *bytes = (2 * kMaxK + 2) * 4; break;
    default: return SPECDEC_EINVAL;
  }
  return SPECDEC_OK;
}

int specdec_stream_read(const void* d_buf, size_t bytes, int32_t workgroups, uint32_t* d_sink, void* stream) {
  if (!d_buf || !d_sink || bytes == 0 || bytes % 16 || workgroups < 1 || workgroups > 65536) return SPECDEC_EINVAL;
  return hip_status(launch_stream_read(d_buf, bytes, workgroups, d_sink, (hipStream_t)stream));
}

// Test hook: Philox4x64-10 words for n (counter, key) pairs (device arrays).
int specdec_philox4x64(const uint64_t* d_ctr, const uint64_t* d_key, int32_t n, uint64_t* d_out, void* stream) {
  if (!d_ctr || !d_key || !d_out || n <= 0) return SPECDEC_EINVAL;
  return hip_status(launch_philox_words(d_ctr, d_key, n, d_out, (hipStream_t)stream));
}

}  // extern "C"
