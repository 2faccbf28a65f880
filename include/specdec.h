/* specdec.h - C ABI of the MI355X (gfx950) block-verify speculative decoding path.
 *
 * What the path computes is defined by these pages:
 *  - "SpecDec-Context-Scaling 项目解读" (richardf123.github.io): section 2.2 (a
 *    self-built forward serving prefill, decode and block verification; an
 *    independent KV-cache API with trim and repair for the target and draft
 *    caches), section 3 (the greedy round: k drafts, one block forward,
 *    longest-prefix acceptance, replacement, bonus), section 3.1 (row
 *    alignment: saved_next verifies d_1, rows[j-1] verifies d_(j+1)),
 *    section 3.2 (cache length == committed tokens; trim to t+m, then repair
 *    to t+m+1), section 2.1 (chunked prefill).
 *  - the wmrh.cn speculative-decoding explainer, section 2.2, and
 *    "mini-infer系统实战-13" (smarter.xin), modified rejection sampling section
 *    (accept with min(1, p/q), resample from norm(max(0, p-q)), bonus on full
 *    acceptance).
 *  - "SubSpec" summary (jjl357.github.io), sections 4.1.1-4.1.3 (4-bit group-64
 *    substitute draft sharing embedding, LM head and the KV cache) and 4.2
 *    (the context-aware draft tree, sharpened with temperature 0.2, verified
 *    in one tree-causal target pass).
 *  - "SpecDec-Context-Scaling 项目解读", section 7.2 (acceptance relaxed by a
 *    logit gap), and the wmrh.cn explainer, sections 3.3, 4.2 and 8
 *    (temperature, and top-k / top-p applied after the accept test).
 *
 * Conventions for every entry point:
 *  - Pointers prefixed d_ are device pointers (hipMalloc or a framework's
 *    device allocation).  The caller owns every buffer; the library keeps
 *    non-owning references inside its handles and never frees them.  Buffers
 *    must outlive the handles that reference them.
 *  - After the *_create calls the library performs no device allocation.
 *  - `stream` is a hipStream_t passed as void*.  Calls enqueue work on it and
 *    return without synchronising unless stated.
 *  - Return value: SPECDEC_OK (0) or a negative specdec_status.  Errors that
 *    can be decided from host-visible values are returned synchronously and
 *    nothing is enqueued.  Violations only the device can see (a trim above
 *    the current length, a forward past the cache capacity, a draft table
 *    read past its end, non-finite logits) set bits of a sticky device error
 *    word (the SPECDEC_DERR_* bits) instead of faulting; the affected writes
 *    are skipped.  specdec_check() reads and reports that word.
 *  - The library never aborts, exits or prints.
 *  - Handles are not thread-safe; use one stream per handle set.  Results
 *    are bitwise deterministic for fixed inputs, and a row's results do not
 *    depend on how many rows share its forward pass.
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPECDEC_OK = 0,
  SPECDEC_EINVAL = -1,      /* NULL pointer, bad enum, bad size */
  SPECDEC_ECAPACITY = -2,   /* rows / length beyond what the buffers were sized for */
  SPECDEC_ESHAPE = -3,      /* model dimensions the kernels do not support */
  SPECDEC_EHIP = -4,        /* a HIP runtime call failed (see specdec_last_hip_error) */
  SPECDEC_EDEVICE = -5,     /* the sticky device error word is non-zero */
  SPECDEC_EUNSUPPORTED = -6 /* valid request this build does not implement */
} specdec_status;

/* Bits of the sticky device error word. */
enum {
  SPECDEC_DERR_CAPACITY = 1,   /* a forward would pass the cache capacity (writes skipped) */
  SPECDEC_DERR_TRIM = 2,       /* trim above the current length (length unchanged) */
  SPECDEC_DERR_NONFINITE = 4,  /* non-finite logits */
  SPECDEC_DERR_TABLE = 8,      /* draft table or noise read past its end */
  SPECDEC_DERR_OUTPUT = 16,    /* committed-token buffer full (tokens dropped) */
  SPECDEC_DERR_SYNC = 32,      /* a split-K hand-off inside a forward waited past its bound */
  SPECDEC_DERR_TREE = 64       /* a tree node's parent is not an earlier node (the node is taken as a root) */
};

enum { SPECDEC_W_BF16 = 0, SPECDEC_W_Q4G64 = 1 };
/* Acceptance rules.  GREEDY: a draft passes when it is the target's argmax
 * ("SpecDec-Context-Scaling 项目解读", sections 3 and 3.1).  STOCHASTIC:
 * modified rejection sampling (wmrh.cn explainer, section 2.2).  RELAXED: a
 * draft passes when its target logit trails the target's top-1 logit by at
 * most relax_delta (same SpecDec page, section 7.2; lossy: the output is no
 * longer the target's greedy decode). */
enum { SPECDEC_GREEDY = 0, SPECDEC_STOCHASTIC = 1, SPECDEC_RELAXED = 2 };
enum { SPECDEC_SCHEDULE_A = 0, SPECDEC_SCHEDULE_B = 1 };
enum { SPECDEC_DRAFT_TABLE = 0, SPECDEC_DRAFT_MODEL = 1, SPECDEC_DRAFT_NOISY_SELF = 2, SPECDEC_DRAFT_Q4_SELF = 3 };

/* Largest number of rows one forward pass takes (prefill runs in passes of
 * at most this many rows). */
#define SPECDEC_MAX_ROWS 32
/* Largest number of drafts per round. */
#define SPECDEC_MAX_K 16

/* Decoder dimensions.  Pre-norm RMSNorm decoder with rotate-half RoPE,
 * grouped-query attention (query head h reads kv head h / (n_q/n_kv)),
 * SwiGLU MLP, untied LM head, no biases.  Supported: hidden, q_dim and ffn
 * multiples of 32 (64 for q4), hidden <= 4096, head_dim 64 or 128, n_q a
 * multiple of n_kv, n_q / n_kv <= 8, vocab a multiple of 16 and <= 2^24. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rope_theta, rms_eps;
  int32_t weight_format; /* SPECDEC_W_BF16, or SPECDEC_W_Q4G64 for 4-bit linears */
} specdec_model_desc;

typedef struct specdec_model specdec_model;
typedef struct specdec_cache specdec_cache;
typedef struct specdec_round specdec_round;

/* ---------------------------------------------------------------- weights */

/* Canonical tensor order, index i: 0 embed [V][H]; per layer l the indices
 * 1+9l .. 9+9l are attn_norm [H], wq [n_q*hd][H], wk [n_kv*hd][H],
 * wv [n_kv*hd][H], wo [H][n_q*hd], mlp_norm [H], wgate [F][H], wup [F][H],
 * wdown [H][F]; then final_norm [H], lm_head [V][H].  Linear weights are
 * [out][in] row-major. */
int32_t specdec_tensor_count(const specdec_model_desc* desc);

/* Bytes of the packed weight blob (the library's own HBM layout: MFMA-tile
 * ordered linears, fp32 norm gains, row-major bf16 embedding). */
int specdec_weights_bytes(const specdec_model_desc* desc, size_t* bytes);

/* Pack canonical tensor `index` into the blob on `stream`.
 * BF16 models: d_src is the row-major bf16 tensor (device memory).
 * Q4G64 models: for linear tensors other than lm_head, d_src points to the
 * packed codes uint8 [out][in/2] (even input in the low nibble) immediately
 * followed by fp16 scale [out][in/64] and fp16 zero [out][in/64] (weight =
 * (code - zero) * scale); other tensors are bf16 as above.  d_src may be
 * freed after the stream has passed this call. */
int specdec_weights_pack(const specdec_model_desc* desc, int32_t index, const void* d_src,
                         void* d_blob, void* stream);

/* Model handle over a packed blob.  `share` (may be NULL) names a model whose
 * embedding, final norm and LM head this one uses instead of its own (the
 * substitute draft); then those tensors need not be packed here. */
int specdec_model_create(const specdec_model_desc* desc, const void* d_blob, const specdec_model* share,
                         specdec_model** out);
void specdec_model_destroy(specdec_model* m);

/* ------------------------------------------------------------------ cache */

/* Bytes of a KV cache of `max_len` positions (at most 65536).  With
 * lp = max_len rounded up to 128, each layer holds bf16 K as
 * [kv head][lp][head_dim] followed by bf16 V transposed as
 * [kv head][head_dim][lp]; then the fp32 RoPE table [max_len][head_dim/2]
 * of (cos, sin). */
int specdec_cache_bytes(const specdec_model_desc* desc, int32_t max_len, size_t* bytes);

/* Cache handle over `d_mem` (cache_bytes).  `d_len` is a caller-owned
 * device int32 holding the current length (committed positions); the
 * library reads and updates it on the device only.  This call writes the
 * RoPE table (synchronous copy) and sets *d_len = 0. */
int specdec_cache_create(const specdec_model_desc* desc, void* d_mem, size_t bytes, int32_t max_len,
                         int32_t* d_len, specdec_cache** out);
void specdec_cache_destroy(specdec_cache* c);

/* Trim the cache to new_len positions (device-checked: new_len <= length,
 * else SPECDEC_DERR_TRIM and the length is left as is).  No data moves. */
int specdec_kv_trim(specdec_cache* c, int32_t new_len, int32_t* d_err, void* stream);

/* -------------------------------------------------------------- workspace */

/* Bytes of the scratch workspace one forward pass needs for up to max_rows
 * rows against a cache of max_len positions.  The workspace also holds the
 * sticky device error word at offset 0 (int32). */
int specdec_workspace_bytes(const specdec_model_desc* desc, int32_t max_rows, int32_t max_len, size_t* bytes);

/* Zero the whole workspace (ws_bytes) on `stream`: the error word, the
 * launch sequence numbers of the split-K row groups and the tags of the
 * split-K partials.  Required once before the first forward; later forwards
 * keep these consistent themselves.  Forwards that share one workspace must
 * not overlap (enqueue them on one stream). */
int specdec_workspace_init(void* d_ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------- forwards */

/* One forward pass of `rows` tokens (1..SPECDEC_MAX_ROWS) at positions
 * length .. length+rows-1: appends their K/V, then length += rows.
 * d_tokens int32 [rows] (device).  Outputs (any may be NULL): d_logits fp32
 * [rows][vocab], d_argmax int32 [rows] (lowest index on ties), d_lse fp32
 * [rows] (log-sum-exp of the row).  This is the decode step (rows = 1) and
 * the block verify (rows = k or k+1). */
int specdec_decode_step(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, int32_t rows,
                        float* d_logits, int32_t* d_argmax, float* d_lse, void* d_ws, size_t ws_bytes,
                        void* stream);

/* ------------------------------------------------------------- draft tree
 * The context-aware draft tree of the "SubSpec" summary (jjl357.github.io,
 * section 4.2), verified by the target in tree-causal forwards.  Block
 * layout: node 0 is the root (the round's pending token: the last committed
 * token, whose K/V is not yet cached), nodes 1 .. n-1 the draft nodes;
 * d_parents int32 [n] holds each node's parent (an earlier node), -1 for the
 * root.  At cache length t, node i occupies slot t + i and runs at position
 * t + depth(i). */
#define SPECDEC_MAX_TREE 512

/* Tree verify: the target's forward of all n (1..SPECDEC_MAX_TREE) nodes at
 * the current length t.  Node i attends to the cached positions 0 .. t-1 and
 * to its ancestors-or-self only, and appends its K/V at slot t + i; then
 * length = t + n.  The nodes run in passes of up to SPECDEC_MAX_ROWS in node
 * order, so a tree wider than a pass costs one weight stream per pass.  d_logits fp32 [n][V], d_argmax int32 [n] and
 * d_lse fp32 [n] as for specdec_decode_step (any may be NULL; d_argmax is
 * what specdec_tree_accept reads).  A chain (d_parents = -1, 0, 1, ...)
 * computes exactly the block verify.  A parent that is not an earlier node
 * sets SPECDEC_DERR_TREE (the node is taken as a root). */
int specdec_tree_verify(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, const int32_t* d_parents,
                        int32_t n, float* d_logits, int32_t* d_argmax, float* d_lse, void* d_ws, size_t ws_bytes,
                        void* stream);

/* Greedy acceptance of a verified tree (right after specdec_tree_verify of
 * the same n nodes, so the length is t + n).  From the root, the first child
 * in node order whose token is the target's argmax at the current node
 * continues the accepted path; the walk stops at a node with no such child.
 * The path's K/V move to slots t+1 .. t+m (every layer), the root stays at
 * slot t, the length becomes t + 1 + m.  d_out_tokens int32 [n] receives the
 * path's tokens then the target's choice at its end (the next pending
 * token), *d_out_count = m + 1.  Optional (NULL to skip): d_root receives
 * the next pending token; d_log int32 [1 + log_cap] is a job log whose
 * d_log[0] counts the tokens stored from d_log[1]: the committed tokens are
 * appended (tokens past log_cap are dropped and set SPECDEC_DERR_OUTPUT).
 * A length below n sets SPECDEC_DERR_TRIM in *d_err and changes nothing. */
int specdec_tree_accept(specdec_cache* c, const int32_t* d_tokens, const int32_t* d_parents, int32_t n,
                        const int32_t* d_argmax, int32_t* d_out_tokens, int32_t* d_out_count, int32_t* d_root,
                        int32_t* d_log, int32_t log_cap, int32_t* d_err, void* stream);

/* Tree construction by a draft that shares the target's cache (the
 * substitute draft: same layers, kv heads and head dim).  At the current
 * length t (every committed token but the pending root *d_root), `depth`
 * steps: the first feeds the root, each later one the k nodes the previous
 * step chose (tree-causal, at slots t + node); after each step every (leaf,
 * token) pair scores the leaf's cumulative log probability plus
 * log softmax(z / temperature)[token] of the leaf's draft logits z, and the
 * k best pairs become the next nodes (ties: the lower leaf node, then the
 * lower token id).  The pages sharpen with temperature 0.2.  Outputs in
 * block layout, n = 1 + k * depth nodes: d_tokens and d_parents int32 [n],
 * d_scores fp32 [n] (cumulative log probabilities, 0 at the root; step s
 * writes nodes 1 + k (s-1) .. k s in rank order).  k in 1..SPECDEC_MAX_K,
 * n <= SPECDEC_MAX_TREE, temperature finite and > 0.  d_ws is a workspace
 * of the draft (its leaf logits and the selection's partials live there).
 * On return the length is t again; the draft's K/V of the fed nodes stay in
 * the slots past it until the verify of the tree overwrites them. */
int specdec_tree_draft(const specdec_model* draft, specdec_cache* c, const int32_t* d_root, int32_t k,
                       int32_t depth, float temperature, int32_t* d_tokens, int32_t* d_parents, float* d_scores,
                       void* d_ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid device allocation): the decode step
 * above without a workspace argument.  Its scratch (activations, attention
 * and LM-head partials, split-K hand-off words) is a device array of
 * 128 MiB inside the library, one per GPU, held until the process ends; a
 * forward whose workspace (specdec_workspace_bytes) exceeds it returns
 * SPECDEC_ECAPACITY.  Device-detected errors are OR-ed into the caller's
 * device int32 *d_err (required; the caller clears it).  Other arguments as
 * for specdec_decode_step.  Every call on one GPU shares that GPU's array
 * and keeps the last call's contents: calls that overlap on one GPU (two
 * streams, two threads) race; enqueue them on one stream.  No device memory
 * is allocated or freed.  specdec_static_init must have run on the current
 * device first (SPECDEC_EINVAL otherwise). */
int specdec_decode_step_noalloc(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, int32_t rows,
                                float* d_logits, int32_t* d_argmax, float* d_lse, int32_t* d_err, void* stream);

/* Set-up of specdec_decode_step_noalloc on the current device: looks up the
 * device address of the library's scratch array and clears it (a fill
 * kernel on `stream`, not captured: call it once per device outside any
 * graph capture, before the first allocation-free step).  Calling it again
 * clears the array again. */
int specdec_static_init(void* stream);

/* Prefill `n` tokens in passes of `chunk` rows (chunk clipped to
 * SPECDEC_MAX_ROWS), starting at the current length.  Writes the last row's
 * logits / argmax / lse (any may be NULL). */
int specdec_prefill(const specdec_model* m, specdec_cache* c, const int32_t* d_tokens, int32_t n, int32_t chunk,
                    float* d_last_logits, int32_t* d_last_argmax, float* d_last_lse, void* d_ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ round */

/* Device-resident round state, followed in memory by int32 tokens[cap]
 * (the committed tokens in order). */
typedef struct {
  int32_t n_committed;     /* tokens committed so far */
  int32_t round;           /* rounds run */
  int32_t m_last;          /* drafts accepted in the last round */
  int32_t last_tok;        /* last committed token (repaired under A, pending under B) */
  int32_t saved_argmax;    /* argmax of saved_next (schedule A) */
  float saved_lse;         /* log-sum-exp of saved_next (schedule A) */
  int32_t accepted_total;  /* sum of m over rounds */
  int32_t cap;             /* capacity of the token array */
  int32_t n_target;        /* rounds become no-ops once n_committed >= n_target */
  int32_t reserved[7];
} specdec_round_state;

typedef struct {
  const specdec_model* target;
  specdec_cache* target_cache;
  const specdec_model* draft;   /* DRAFT_MODEL: independent draft; DRAFT_Q4_SELF: substitute draft; else NULL */
  specdec_cache* draft_cache;   /* DRAFT_MODEL only (own cache); NULL otherwise */
  int32_t k;                    /* drafts per round, 1..SPECDEC_MAX_K (DRAFT_Q4_SELF: the depth D) */
  int32_t mode;                 /* SPECDEC_GREEDY | SPECDEC_STOCHASTIC | SPECDEC_RELAXED */
  int32_t bonus;                /* 1: bonus token on full acceptance; 0: a fully accepted round
                                   commits the k drafts only, and the last verify row becomes the
                                   next round's saved_next (schedule A only) */
  int32_t schedule;             /* SPECDEC_SCHEDULE_A | SPECDEC_SCHEDULE_B */
  int32_t draft_source;         /* SPECDEC_DRAFT_* */
  const int32_t* d_draft_table; /* TABLE / MODEL: drafts by generated index, int32 [table_len] */
  int32_t table_len;
  const float* d_noise;         /* NOISY_SELF: fp32 [noise_rows][vocab] logit noise by generated index */
  int32_t noise_rows;
  uint64_t philox_seed;         /* STOCHASTIC: Philox4x64-10 key word 0 */
  specdec_round_state* d_state; /* device state + tokens (specdec_round_state_bytes) */
  void* d_ws;                   /* target workspace (rows >= k+1) */
  size_t ws_bytes;
  void* d_draft_ws;             /* draft workspace (DRAFT_MODEL, DRAFT_Q4_SELF) */
  size_t draft_ws_bytes;
  void* d_round_ws;             /* round scratch (specdec_round_ws_bytes) */
  size_t round_ws_bytes;
  int32_t state_cap;            /* capacity of the state's token array (specdec_round_state_bytes(cap)) */
  void* const* events;          /* optional hipEvent_t ring for per-term timing, or NULL */
  int32_t n_events;             /* ring size (>= 5); each round records 5 events in order:
                                   start, after draft provision, after verify, after accept,
                                   after repair; round i uses entries 5*i .. 5*i+4 modulo the ring */
  /* STOCHASTIC only (wmrh.cn explainer, sections 3.3, 4.2 and 8): draft and
   * target distributions are softmax(logits / temperature); the accept test
   * and the residual run on these untruncated distributions; top_k / top_p
   * truncate only the distribution the round's last token is drawn from (the
   * residual after a rejection, the bonus row after full acceptance): entries
   * ranked by weight (ties: lower index first), the first top_k kept, then
   * the shortest leading run of those holding top_p of their mass.
   * temperature > 0 (1: plain softmax); top_k 0 = off, else 1..vocab;
   * top_p in (0, 1], 1 = off.  Truncation needs vocab <= 2^18
   * (SPECDEC_EUNSUPPORTED beyond). */
  float temperature;
  int32_t top_k;
  float top_p;
  float relax_delta;            /* RELAXED only: the logit gap to the top-1 a draft may have (>= 0) */
} specdec_round_desc;

int specdec_round_state_bytes(int32_t cap, size_t* bytes);
int specdec_round_ws_bytes(const specdec_model_desc* target, int32_t k, size_t* bytes);

/* Validate the descriptor and build a round handle (host memory only). */
int specdec_round_create(const specdec_round_desc* desc, specdec_round** out);
void specdec_round_destroy(specdec_round* r);

/* Prefill `d_prompt` (int32 [n], device) into the round's caches in passes
 * of `chunk` rows and snapshot the post-prefill state.  The caches are
 * first trimmed to 0.  Schedule A prefills all n tokens into the target and
 * keeps the last row as saved_next; schedule B prefills n-1 tokens and
 * leaves prompt[n-1] pending.  An independent draft model prefills all n.
 * SPECDEC_ECAPACITY unless the target cache holds n + 2 * (verify rows) + 2
 * positions (the prompt and one round); specdec_round_reset checks the
 * whole job. */
int specdec_round_prefill(specdec_round* r, const int32_t* d_prompt, int32_t n, int32_t chunk, void* stream);

/* Return to the post-prefill snapshot: trim every cache back to its
 * post-prefill length, restore saved_next / the pending token, zero the
 * counters and set n_target (rounds stop committing once n_committed >=
 * n_target).  Enqueued on `stream`; cheap (no forward). */
int specdec_round_reset(specdec_round* r, int32_t n_target, void* stream);

/* Enqueue one speculative round: draft provision, block verify, acceptance,
 * trim of every cache to t+m and repair to t+m+1 (schedule A) or the
 * pending-token form (schedule B).  No host synchronisation; once
 * n_committed >= n_target the round's kernels return without work. */
int specdec_verify_round(specdec_round* r, void* stream);

/* Capture the round (exactly the work of specdec_verify_round) as HIP
 * graphs owned by the round handle: four segment graphs (round start +
 * draft provision, block verify, acceptance + trim, repair) and one graph
 * of the whole round.  Every dynamic value a round uses (lengths, tokens,
 * counters) lives in device memory, so one set of graphs serves every
 * position.  Captures on an internal stream; no device memory is
 * allocated. */
int specdec_round_graph(specdec_round* r);

/* Enqueue `n_rounds` rounds on `stream` as graph replays.  With a per-term
 * event ring configured, each round replays the four segment graphs with the
 * ring's events recorded between them, exactly as specdec_verify_round
 * records them; without one, each round is one launch of the whole-round
 * graph (the same kernels, one launch instead of four). */
int specdec_round_graph_launch(specdec_round* r, int32_t n_rounds, void* stream);

/* Device views of a round's internal buffers, for inspection by tests:
 * which = 0 saved_next logits fp32 [V] (schedule A; overwritten by the repair),
 * 1 verify logits fp32 [k+1][V], 2 noisy draft logits z + noise fp32 [k][V],
 * 3 verify block tokens int32 [k+1], 4 the last stochastic round's
 * (ratio, u_accept) pairs fp32 [2*SPECDEC_MAX_K] then (u_resample, m).
 * Returns the pointer and the byte size; nothing is copied. */
int specdec_round_debug_view(const specdec_round* r, int32_t which, void** d_ptr, size_t* bytes);

/* Read the device error word of `d_ws` (synchronises `stream`): returns
 * SPECDEC_OK or SPECDEC_EDEVICE and stores the bits in *bits (may be NULL). */
int specdec_check(const void* d_ws, int32_t* bits, void* stream);

/* The last hipError_t seen by a failing call on this thread. */
int32_t specdec_last_hip_error(void);

/* Philox4x64-10 output words for n (counter[4], key[2]) pairs: device
 * arrays ctr uint64 [n][4], key uint64 [n][2], out uint64 [n][4].  The same
 * generator draws the stochastic round's uniforms. */
int specdec_philox4x64(const uint64_t* d_ctr, const uint64_t* d_key, int32_t n, uint64_t* d_out, void* stream);
const char* specdec_status_str(int status);

/* Measurement helper, not a step of the path: read `bytes` (a multiple of
 * 16) of device memory at d_buf once, with the same non-temporal 16-byte
 * loads the weight stream uses, by `workgroups` (1..65536) workgroups of
 * 256 threads, on `stream`.  d_sink is a device uint32 the kernel may write
 * (keeps the loads live).  Timing this read over a buffer far larger than
 * the caches gives the measured stream-read ceiling that achieved HBM
 * bandwidth is reported against next to the published peak. */
int specdec_stream_read(const void* d_buf, size_t bytes, int32_t workgroups, uint32_t* d_sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H */
