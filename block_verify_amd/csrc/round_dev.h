// Device-visible description of one speculative round (passed by value to
// the round kernels) and the launchers of kernels_round.hip.
#pragma once

#include "internal.h"

namespace sd {

constexpr int kMaxK = SPECDEC_MAX_K;
// Rows sampled by inverse CDF are cut into slices of kSliceElems entries,
// one 256-thread workgroup each.
constexpr int kSliceElems = 1024;
inline __host__ __device__ int n_slices(int V) { return (V + kSliceElems - 1) / kSliceElems; }

enum { kFlagOpen = 0, kFlagRepair = 1, kFlagCopySaved = 2, kNumFlags = 4 };

// Truncation of the post-acceptance sample (top-k, then top-p) selects by a
// 49-bit key per vocabulary entry: the fp32 weight's bits (non-negative, so
// ordered like the values) above 18 bits of (2^18 - 1 - index), so a larger
// key is a larger weight, or an equal weight at a lower index.  A radix
// select over the key in 8-bit digits resolves one digit per pass.
constexpr int kKeyIndexBits = 18;
constexpr int kKeyBits = 31 + kKeyIndexBits;
constexpr int kTruncPasses = (kKeyBits + 7) / 8;
constexpr int kTruncBins = 256;
// Bin masses are sums of the fp32 weights in fixed point (units of 2^-60;
// every weight is at most 1 and their total stays below 2^63), so a bin's
// mass is the same whatever order its entries are added in.
constexpr double kMassScale = 1152921504606846976.0;   // 2^60
// Select state in device memory: the key prefix resolved so far, the count
// (top-k) or mass (top-p, fixed point) still to cover below the bins taken,
// the top-k threshold key (0 when top-k is off) and the final threshold key.
struct TruncState {
  uint64_t prefix;
  int64_t need;
  uint64_t target;
  uint64_t kthresh;
  uint64_t thresh;
  int32_t active;    // 0: no sample this round (or truncation off)
  int32_t done;      // the current stage's threshold is settled (later passes of the stage return at once)
};
enum { kSnapTLen = 0, kSnapDLen = 1, kSnapArgmax = 2, kSnapLse = 3, kSnapLast = 4, kNumSnap = 8 };

struct RoundDev {
  specdec_round_state* state;
  int32_t* flags;          // [kNumFlags]; gates of the round's forwards
  int32_t* block;          // verify block tokens [k + 1]
  int32_t* repair_tok;     // [1]
  int32_t* rows_argmax;    // [k + 1]
  float* rows_lse;         // [k + 1]
  float* rows_logits;      // [k + 1][V]
  float* saved_logits;     // [V] saved_next (schedule A)
  int32_t* repair_argmax;  // [1]
  float* repair_lse;       // [1]
  float* q_logits;         // [k][V] noisy draft logits
  float* q_lse;            // [k]
  float* z;                // [V] logits of the noisy-draft steps
  float* draft_logits;     // [V] scratch for draft-model steps
  int32_t* draft_argmax;   // [1]
  float* snap_logits;      // [V]
  int32_t* snap;           // [kNumSnap]
  float* dbg;              // [2 * kMaxK + 2] ratios / uniforms of the last stochastic round
  float* smax;             // [slices] per-slice max of a sampled row
  float* ssum;             // [slices] per-slice sum of exp(x - slice max)
  double* sw;              // [slices] per-slice sum of the sampling weights
  int32_t* sctl;           // [4] sampler control: accepted count m, weight mode
  float* t_lse;            // [k + 1] log-sum-exp of the tempered target rows (temperature != 1)
  float* tsmax;            // [(k + 1) * slices] per-slice max of the tempered target rows
  float* tssum;            // [(k + 1) * slices] per-slice sum of exp(x - slice max)
  int32_t* hcnt;           // [slices][kTruncBins] truncation histogram: counts
  uint64_t* hmass;         // [slices][kTruncBins] truncation histogram: masses (fixed point)
  TruncState* trunc;       // truncation select state
  int32_t* t_len;
  int32_t* d_len;          // independent draft's cache length, or null
  int32_t* err;
  const int32_t* table;
  int table_len;
  const float* noise;
  int noise_rows;
  uint64_t seed;
  int k, V, bonus, schedule, draft_source, mode, state_cap;
  float inv_t;             // 1 / temperature (stochastic mode)
  int top_k;               // truncation of the post-acceptance sample: 0 = off
  float top_p;             // 1 = off
  float relax_delta;       // relaxed greedy mode: the logit gap a draft may trail the top-1 by
};

// Round scratch layout inside d_round_ws.
struct RoundWsPlan {
  size_t flags, block, repair_tok, rows_argmax, rows_lse, repair_argmax, repair_lse, q_lse, snap, dbg;
  size_t smax, ssum, sw, sctl, t_lse, tsmax, tssum, hcnt, hmass, trunc;
  size_t rows_logits, saved_logits, q_logits, z, draft_logits, draft_argmax, snap_logits, total;
};
RoundWsPlan round_ws_plan(int V, int k);

hipError_t launch_round_start(const RoundDev& r, hipStream_t s);
hipError_t launch_accept_greedy(const RoundDev& r, hipStream_t s);
hipError_t launch_repair_done(const RoundDev& r, hipStream_t s);
hipError_t launch_rewind(const RoundDev& r, int32_t* len, int n, hipStream_t s);
hipError_t launch_snapshot(const RoundDev& r, const int32_t* last, hipStream_t s);
hipError_t launch_reset(const RoundDev& r, int32_t n_target, hipStream_t s);
hipError_t launch_draft_sample(const RoundDev& r, const float* z, int j, hipStream_t s);
hipError_t launch_accept_stochastic(const RoundDev& r, hipStream_t s);
hipError_t launch_copy_saved(const RoundDev& r, hipStream_t s);
hipError_t launch_philox_words(const uint64_t* ctr, const uint64_t* key, int n, uint64_t* out, hipStream_t s);

}  // namespace sd
