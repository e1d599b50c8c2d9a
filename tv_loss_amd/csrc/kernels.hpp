// Internal interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace mtp {

// Vectors of 16 bytes each thread holds per row and layer in the verify main
// kernel: 16 bf16 or 12 fp32 values per row (chunks of 4096 or 3072 elements), so that the
// current layer, the previous one (waiting for its row statistics) and the next
// one in flight fit in 128 VGPRs.
constexpr int kVerifyNVBf16 = 2;
constexpr int kVerifyNVF32 = 3;
constexpr int kMaxRowsPerSeq = 9;  // gamma + 1 with gamma <= 8
// Workgroups per CU the verify main kernel is compiled for (one wave per SIMD
// each): 4 (128 VGPRs) keeps one layer's e values in registers and two chunks in
// flight, for both dtypes and both acceptance rules, without spilling.
constexpr int kVerifyBlocksPerCU = 4;

// Counters sit 16 ints (64 bytes) apart so clusters do not share a line.
constexpr int kCounterStride = 16;

// Row status bits (same values as the public header's MTP_ROW_*).
constexpr int kRowBadToken = 1;
constexpr int kRowBadTarget = 2;
constexpr int kRowBadDraft = 4;
constexpr int kRowResidualEmpty = 8;
constexpr int kRowSyncTimeout = 16;

// Division by a runtime-invariant d >= 1 for numerators 0 <= n < 2^31 with one
// high multiply (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): n / d = (mulhi(n, lo) + n hi) >> s.  For d >= 2,
// s = ceil(log2 d) - 1 and lo = ceil(2^(32+s) / d) < 2^32, hi = 0; the error term
// n (lo d - 2^(32+s)) < 2^31 d <= 2^(32+s) keeps the floor exact.  d = 1: lo = 0,
// hi = 1, s = 0.
struct FastDiv {
  uint32_t lo, hi, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  if (d <= 1) return FastDiv{0u, 1u, 0u};
  int l = 0;
  while ((1ull << l) < d) ++l;
  const uint32_t s = (uint32_t)(l - 1);
  const uint64_t m = ((1ull << (32 + s)) + d - 1) / d;
  return FastDiv{(uint32_t)m, 0u, s};
}

__device__ __forceinline__ int fast_div(int n, const FastDiv& f) {
  return (int)((__umulhi((uint32_t)n, f.lo) + (uint32_t)n * f.hi) >> f.s);
}

// Contiguous item ranges for S persistent super-groups of C workgroups each.  The
// grid's workgroups reach the compute units in launch order, one per unit and
// dispatch round, so super-group s (workgroups sC .. sC + C - 1) has its last
// workgroup in round r(s) = ((s + 1) C - 1) / W, W the workgroups per round (the
// compute-unit count).  Waves of a later round lose issue arbitration to the older
// ones on their unit and run measurably slower, so the host gives the super-groups
// of round r `items` items each, except the last `short_by` of them, which take one
// fewer (plan_round_split).  Returns the first item of super-group s (the total for
// s = S).
constexpr int kMaxRounds = 8;
struct RoundSplit {
  int W;                       // workgroups per round; 0: strided items; -1: split by thirds
  int rounds;
  int items[kMaxRounds], short_by[kMaxRounds];
};

__device__ __forceinline__ int round_first_sg(int r, int C, int W) { return (r * W + C) / C - 1; }

__device__ __forceinline__ int round_split_base(const RoundSplit& rs, int s, int S, int C) {
  int base = 0;
  for (int r = 0; r < rs.rounds; ++r) {
    const int lo = min(S, round_first_sg(r, C, rs.W)), hi = min(S, round_first_sg(r + 1, C, rs.W));
    const int full = (hi - lo) - rs.short_by[r];   // super-groups of the round with all items
    const int k = min(max(s, lo), hi) - lo;        // super-groups of the round before s
    base += k * rs.items[r] - max(0, k - full);
  }
  return base;
}

struct VerifyArgs {
  const void* target; int64_t t_stride;   // row (b, k) of [B, G+1, V] at (b*(G+1)+k)*t_stride
  const void* draft;  int64_t d_stride;   // row (b, k) of [B, G, V]   at (b*G+k)*d_stride
  const int32_t* tokens;                  // [B, G]; unused by target-only verify
  int B, G;
  int64_t V;
  uint64_t seed, offset;
  uint8_t* accept; int32_t* accepted_len; int32_t* next_token;
  int32_t* row_token; float* overlap; float* tv; float* entropy; int32_t* row_status;
  // target-only verify: greedy draft tokens [B, G], p at them, RS/TO boundary flags
  int32_t* draft_token; float* p_yhat; uint8_t* rs_better;
  // Gumbel-max verify: 1 / temperature (1 otherwise)
  float inv_temp;
  // bounded waits give up after this many ticks of the 100 MHz counter
  uint64_t wait_limit;
  // workspace sections: error word, pass-1 records [group][chunk][3 or 4 words],
  // pass-2 sums [group][chunk][wave] = (residual or p mass, overlap) as two floats,
  // target-only: p mass without the greedy token [group][chunk][wave]; Gumbel-max:
  // each wave's (largest key, index + 1) of the residual and of p [group][chunk][wave][2]
  uint32_t* err; uint64_t* part1; uint64_t* part2; float* part3; uint64_t* gkeys;
  RowSplit sp;
  int ngroups;
  int sgroups, layers;   // super-groups (all co-resident), groups per super-group
  FastDiv div_b, div_g1; // division by B and by gamma + 1
  RoundSplit split;      // contiguous item ranges per super-group (see verify_main)
};

// Verify modes: rejection sampling with inverse-CDF samples; target-only (greedy
// draft tokens, no tokens input); rejection sampling at a temperature with
// Gumbel-max samples.
constexpr int kVerifyRejection = 0;
constexpr int kVerifyTargetOnly = 1;
constexpr int kVerifyGumbel = 2;

int verify_vec_per_thread(int dt);
hipError_t launch_verify(const VerifyArgs& a, int dt, int mode, hipStream_t stream);
hipError_t verify_occupancy(int dt, int mode, int* blocks_per_cu);
int verify_record_words(int mode);
// Gumbel-max tokens of `rows` logit rows: argmax_v (x_v L - log2 E_v), E the
// elements' exponential variates.  keys: [rows][gumbel_sample_chunks_per_row] words.
int gumbel_sample_chunks_per_row(int dt, int64_t V);
hipError_t launch_gumbel_sample(const void* logits, int64_t row_stride, int dt, int rows, int64_t V, float L,
                                uint64_t seed, uint64_t offset, int32_t* tokens, uint64_t* keys,
                                hipStream_t stream);

// ---------------------------------------------------------------------------
// End-to-end TV loss.  Head k of position t compares draft row
// draft + t*d_pos + k*d_head with target row target + t*t_pos + k*t_head
// (t_head = 0: one target row shared by all heads).
struct TvArgs {
  const void* target; int64_t t_pos, t_head;
  const void* draft;  int64_t d_pos, d_head;
  int T, G;
  int64_t V;
  // forward outputs
  float* loss; float* pos_loss; float* saved;
  // backward
  const float* saved_in; const float* grad_loss;
  void* grad; int64_t g_pos, g_head; int grad_dt;
  // forward workspace: error word, log-sum-exp partials [t][chunk][rows] as
  // (ref, z), overlap and S partials [t][chunk][2 gamma], per-position losses [t];
  // the fused forward + backward also: overlap / S records [t][chunk][gamma]
  uint32_t* err; uint64_t* part1; float* part2; float* pos_ws; uint64_t* part3;
  RowSplit sp;
  int sgroups;   // single-read forward: super-groups of sp.nchunks workgroups, all resident
  RoundSplit split;   // their contiguous position ranges (split.W = 0: t = sg + i sgroups)
  // top-K path: the target of head k at position t is given by K entries, indices
  // idx and logits val at t*k_pos + k*k_head + j (k_head = 0: shared by the heads)
  const int32_t* idx; const float* val; int64_t k_pos, k_head; int K;
  // bounded waits give up after this many ticks of the 100 MHz counter
  uint64_t wait_limit;
};

constexpr int kTvSavedStride = 4;   // saved[t, k, :] = (lse_p, lse_q, alpha, S)
constexpr int kTvMaxHeads = 8;

int tv_fwd_vec_per_thread(int dt, int G, bool shared);
int tv_fwd_part1_words(int G, bool shared);
hipError_t launch_tv_fwd(const TvArgs& a, int dt, bool shared, hipStream_t stream);
// single-read forward (rows held on chip between the two passes): applies when a
// position has at most kTvPipeMaxRows rows; vectors per thread and row (0: does not
// apply), main-kernel workgroups per CU, launch (main, finish, mean).  The workspace
// holds the records part1 [t][chunk][rows] (64-bit words) and part2 [t][chunk][2 gamma].
constexpr int kTvPipeMaxRows = 5;
int tv_pipe_vec_per_thread(int dt, int G, bool shared);
hipError_t tv_pipe_occupancy(int dt, int G, bool shared, int* blocks_per_cu);
hipError_t launch_tv_pipe_fwd(const TvArgs& a, int dt, bool shared, hipStream_t stream);
// fused forward + backward (same shapes as the single-read forward): launch (main,
// finish, mean) and main-kernel occupancy; the workspace holds the normaliser
// records part1 [t][chunk][rows], the overlap / S records part3 [t][chunk][gamma]
// and the per-position losses
hipError_t tv_fused_occupancy(int dt, int grad_dt, int G, bool shared, int* blocks_per_cu);
hipError_t launch_tv_fused(const TvArgs& a, int dt, bool shared, hipStream_t stream);
int tv_bwd_vec_per_thread(int dt);   // top-K backward
int tv_bwd_full_vec_per_thread(int dt, int G, bool shared);
hipError_t launch_tv_bwd(const TvArgs& a, int dt, bool shared, hipStream_t stream);
// top-K path: forward (draft log-sum-exp partials, per-position finish over the K
// entries, mean) and backward; the workspace holds part1 [t][chunk][gamma] and pos_ws
int tv_topk_fwd_vec_per_thread(int dt, int G);
hipError_t launch_tv_topk_fwd(const TvArgs& a, int dt, hipStream_t stream);
hipError_t launch_tv_topk_bwd(const TvArgs& a, int dt, hipStream_t stream);

}  // namespace mtp
