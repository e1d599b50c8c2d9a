// Rejection-sampling verification of MTP draft tokens over the full vocabulary.
//
// What is computed (Bebop pages: paperlayer.ai Sec. 2 "Acceptance methods",
// Sec. 3 "Rejection Sampling", App. G.1 "Multinomial Draft Sampling"; rainbus
// prerequisites "Rejection Sampling", "Total Variation Distance", "Entropy"):
// for sequence b and draft position k < gamma,
//   p = softmax(target row), q = softmax(draft row),
//   accept_k = u_k < min(1, p(y_k) / q(y_k)),
//   overlap_k = sum_v min(p_v, q_v) = 1 - TV_k,   TV_k = sum_v max(0, p_v - q_v),
//   H(p) = -sum_v p_v ln p_v   (also for the bonus row k = gamma),
// and every row draws its sample by inverse CDF over r in vocabulary order,
// r = max(0, p - q) for k < gamma and r = p for the bonus row; the sequence emits
// the sample of row n_b, n_b being the number of leading accepts.
//
// One kernel, verify_main.  It streams every logit once.  A "group" is one row of
// one sequence: (target row, draft row) for k < gamma, or the bonus target row
// alone.  Each group is split along the vocabulary into C chunks of 4096 elements
// (3072 for fp32); C workgroups form a super-group that walks a list of groups
// ("layers"), chunk c of every group going to workgroup c, and each wave of a
// workgroup owns a contiguous segment of the chunk.  All super-groups are resident
// at once.  The two passes over a chunk are software-pipelined across layers, so
// that no workgroup waits on its cluster:
//   layer i:  row statistics and pass 2 of group i - 2: its C records were polled
//             a layer ago; merged in one fixed order they give the row
//             log-sum-exps, and each wave sums r = p - min(p, q) and min(p, q)
//             (p alone for a bonus row) over its segment from the e values held
//             in LDS, and publishes them as a self-announcing pass-2 word;
//             group i - 1's e values move from registers to LDS;
//             unpack the chunk of group i (its loads went out two layers ago),
//             poll group i - 1's records and issue the loads of group i + 2;
//             pass 1 on group i: per-wave log-sum-exp partials (both rows, plus
//             the entropy moment of the target), combined over the workgroup and
//             published as one self-announcing record.
// Records and pass-2 words use device-scope loads and stores, so a super-group may
// span XCDs.
//
// The finish runs in the same kernel: a workgroup whose layers are done takes a
// sequence, one wave per row.  A wave waits for the row's records and merges them
// (lse, entropy, the acceptance test, which needs p(y) and q(y) only), then waits
// for its pass-2 words, scans the chunk masses, then the segment masses of the
// owner chunk in vocabulary order, re-reads the single 1024-element segment
// holding t = u' * sum r and finishes the inverse CDF in it.  The sequence's
// accepted length and next token are formed in LDS.  It also clears what the
// layers wrote for the row, so the workspace is all zeros again when the call ends.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mtp {

// Chunk record of pass 1: (ref_p, z_p), (ref_q, z_q), (y_p, 1), and for target-only
// verify a fourth word, the chunk's largest draft logit and its vocabulary index + 1.
// The z's carry the sign bit as a marker (and the index is at least 1), so no word of
// a published record is 0.  rec_bytes is the record stride.
template <bool TO>
constexpr int rec_bytes() { return TO ? 32 : 24; }
constexpr int kArgmaxWord = 3;

// Row statistics from the C records of a group.  Lane l holds the partial of
// record l and merges records l + 64, l + 128, ... into it in that order; the wave
// then merges the lanes.  Both kernels use these functions, so both derive the same
// bits for a row.
__device__ __forceinline__ Lse lane_records(Lse acc, __amdgpu_buffer_rsrc_t rs, int C, int st, int word,
                                            bool with_y) {
  const int lane = threadIdx.x & 63;
  for (int c = lane + 64; c < C; c += 64) {
    const uint64_t w = rec_load(rs, c * st + word * 8);
    const float y = with_y ? unpack_lo(rec_load(rs, c * st + 16)) : 0.f;
    acc = lse_merge(acc, Lse{unpack_lo(w), unmark(unpack_hi(w)), y});
  }
  return acc;
}

struct RowStats {
  Lse p, q;
};

// Words 0-2 of record `lane` (clamped into the row, so the loads are unconditional
// and can go out early); lanes past the last record ignore them.
struct RecWords {
  uint64_t w0, w1, w2;
};
__device__ __forceinline__ RecWords rec_words(__amdgpu_buffer_rsrc_t rs, int C, int st) {
  const int l = min((int)(threadIdx.x & 63), C - 1);
  return RecWords{rec_load(rs, l * st), rec_load(rs, l * st + 8), rec_load(rs, l * st + 16)};
}

__device__ __forceinline__ RowStats merge_records(const RecWords& r, __amdgpu_buffer_rsrc_t rs, int C, int st,
                                                  bool pair) {
  const int lane = threadIdx.x & 63;
  Lse a[2] = {lse_empty(), lse_empty()};
  if (lane < C) {
    a[0] = Lse{unpack_lo(r.w0), unmark(unpack_hi(r.w0)), unpack_lo(r.w2)};
    if (pair) a[1] = Lse{unpack_lo(r.w1), unmark(unpack_hi(r.w1)), 0.f};
  }
  a[0] = lane_records(a[0], rs, C, st, 0, true);
  if (pair) a[1] = lane_records(a[1], rs, C, st, 1, false);
  wave_merge<2, 1>(a);
  return RowStats{a[0], a[1]};
}

// ---- argmax of the draft logits (target-only verify) --------------------------
__device__ __forceinline__ uint64_t pack_argmax(float m, uint32_t idx) {
  return pack2(m, __uint_as_float(min(idx, 0xfffffffeu) + 1u));
}
__device__ __forceinline__ uint32_t argmax_index(uint64_t w) { return __float_as_uint(unpack_hi(w)) - 1u; }

// (m, idx) absorbs (m2, idx2) if m2 is larger, or equal with a smaller index; a NaN
// m2 never wins.
__device__ __forceinline__ void argmax_fold(float& m, uint32_t& idx, float m2, uint32_t idx2) {
  const bool take = m2 > m || (m2 == m && idx2 < idx);
  m = take ? m2 : m;
  idx = take ? idx2 : idx;
}

// Wave argmax: the largest m over the lanes (NaN ignored), the smallest idx among
// the lanes that hold it.  The same bits in every lane.
__device__ __forceinline__ void wave_argmax(float& m, uint32_t& idx) {
  const float M = wave_maximum(m);
  const uint32_t cand = m == M ? idx : 0xffffffffu;
  m = M;
  idx = wave_min_u32(cand);
}

// The chunk argmax words of a group merged over its C records, in record order per
// lane then over the wave: the vocabulary index of the largest draft logit.
// A wait that timed out gives kNoArgmax.
constexpr uint32_t kNoArgmax = 0xffffffffu;

__device__ __forceinline__ uint32_t poll_argmax(uint64_t v, __amdgpu_buffer_rsrc_t rs, int C, int st,
                                                uint32_t* err, uint64_t limit) {
  float m = kNegInf;
  uint32_t idx = 0xffffffffu;
  const bool timed_out = poll_words(v, rs, C, st, kArgmaxWord, err, limit,
                                    [&](bool, uint64_t w) { argmax_fold(m, idx, unpack_lo(w), argmax_index(w)); });
  wave_argmax(m, idx);
  return timed_out ? kNoArgmax : idx;
}

__device__ __forceinline__ uint32_t merge_argmax(__amdgpu_buffer_rsrc_t rs, int C, int st) {
  const int lane = threadIdx.x & 63;
  float m = kNegInf;
  uint32_t idx = 0xffffffffu;
  for (int c = lane; c < C; c += 64) {
    const uint64_t w = rec_load(rs, c * st + kArgmaxWord * 8);
    argmax_fold(m, idx, unpack_lo(w), argmax_index(w));
  }
  wave_argmax(m, idx);
  return idx;
}

// ---------------------------------------------------------------------------
template <int DT, int NV, int MODE>
__device__ __forceinline__ void finish_row(const VerifyArgs& a, int b, int k, int* flag_sh, int* token_sh,
                                           uint64_t limit);

// The finish's waits are for the other workgroups' last layers (not for a record
// of the exchange), so they are bounded by at least this many ticks of the 100 MHz
// counter (one second), whatever the exchange's own bound.
constexpr uint64_t kFinishWaitFloor = 100000000ull;

template <int DT, int NV, int MODE>
__global__ __launch_bounds__(kBlock, kVerifyBlocksPerCU) void verify_main(VerifyArgs a) {
  constexpr bool TO = MODE == kVerifyTargetOnly, GM = MODE == kVerifyGumbel;
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NE = NV * PV;
  constexpr int NQ = NE / 4;              // 16-byte LDS slots per row and thread
  constexpr int kSegVec = NV * 64;
  const int C = a.sp.nchunks;
  const int slot = blockIdx.x;
  const int sg = slot / C, c = slot - sg * C;
  const int S = a.sgroups;
  const int B = a.B, G = a.G, G1 = G + 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = threadIdx.x;
  // the rows' bookkeeping is one task per wave (combine and publish p, the same for
  // q, poll p's records, poll q's), so that none of it runs back to back on one
  // wave; the roles rotate over the workgroups so that they spread over the SIMDs
  const int wp = (slot + c) & (kWaves - 1), wq = wp ^ 1;   // combine and publish p / q
  const int rp = wp ^ 2, rq = wp ^ 3;                     // poll p / q records

  // Items are rows w = 0 .. N - 1 taken k-major (all k = 0 rows first), each
  // super-group a contiguous range, by one of two splits the host picks:
  //  - by dispatch round (round_split_base), when the super-groups have many items
  //    each: what a later round loses per item then adds up over the layers;
  //  - with few items each, the middle and last thirds of the super-groups take one
  //    and two items fewer than the first: the last ones end well before the others
  //    and, as they host the finish (below), have the rows' statistics merged by
  //    the time the last pass-2 words arrive.
  // With fewer than four items per super-group, super-group sg takes w = sg + i S.
  if (sg >= a.ngroups) return;
  const int N = a.ngroups;
  int nl = (N - 1 - sg) / S + 1, base = -1;
  if (a.split.W > 0) {
    base = round_split_base(a.split, sg, S, C);
    nl = round_split_base(a.split, sg + 1, S, C) - base;
  } else if (a.split.W < 0) {
    const int s1 = (S + 2) / 3, s2 = (2 * S + 2) / 3;
    const int Sd = (S - s1) + (S - s2);                 // items the later thirds give up
    const int H = (N + Sd) / S, R = N + Sd - H * S;
    nl = H - (sg >= s1) - (sg >= s2) + (sg < R);
    base = sg * H - max(0, sg - s1) - max(0, sg - s2) + min(sg, R);
  }
  auto group_of = [&](int i) {
    const int w = base >= 0 ? base + i : sg + i * S;
    const int k = fast_div(w, a.div_b);
    return (w - k * B) * G1 + k;
  };
  auto is_pair = [&](int g) { return g - fast_div(g, a.div_g1) * G1 < G; };
  auto trow_of = [&](int g) {
    return reinterpret_cast<const char*>(a.target) + (int64_t)g * a.t_stride * Elem<DT>::kBytes;
  };
  auto drow_of = [&](int g) {   // a bonus row has no draft row: its target row again
    const int b = fast_div(g, a.div_g1), k = g - b * G1;
    return k < G ? reinterpret_cast<const char*>(a.draft) + (int64_t)(b * G + k) * a.d_stride * Elem<DT>::kBytes
                 : trow_of(g);
  };
  constexpr int kSt = rec_bytes<TO>();
  auto rsrc_rec = [&](int g) { return rsrc_of(a.part1 + (int64_t)g * C * (kSt / 8)); };
  const float L = GM ? kLog2e * a.inv_temp : kLog2e;   // logit -> base-2 exponent scale

  // vector indices fit in 32 bits (V <= 2^30)
  const int vpc = (int)a.sp.vec_per_chunk, nvec = (int)a.sp.nvec, nfull = (int)a.sp.nvec_full;
  const int vbeg = c * vpc;
  const int vend = min(vbeg + vpc, nvec);
  const int s0 = vbeg + wave * kSegVec;      // this wave's segment
  const int v0 = s0 + lane;
  const int lim = min(vend, nfull);
  const bool full = s0 + kSegVec <= lim;
  const int last = nfull - 1;
  const int tail = nfull;
  const int V = (int)a.V;

  // e values of the item two layers back, waiting for their row statistics:
  // thread t owns slots [row][q][t] (16 bytes each), so a wave's accesses are
  // contiguous and no thread touches another's slots
  __shared__ float4 held[2][NQ][kBlock];
  // double-buffered by layer parity: a wave may run one layer ahead of another
  __shared__ float part_sh[2][2][kWaves * 3];
  // row statistics of the item in pass 2, the normaliser being 2^ref z: (ref, z, 1/z)
  __shared__ float st_sh[2][2][3];
  // target-only: per-wave argmax of the draft logits (pass 1), the row's argmax (pass 2)
  __shared__ float am_sh[2][kWaves];
  __shared__ uint32_t ai_sh[2][kWaves];
  __shared__ uint32_t yhat_sh[2];

  // the chunks of items i + 1 and i + 2 are in flight while item i is processed;
  // every prefetch issues the same number of loads (see issue_seg_fixed).  A
  // prefetch past the end of the list (live false) names an item of the list (the
  // window below only ever holds such items) and reads at offset 0.
  const int row_bytes = (int)min(a.V * Elem<DT>::kBytes, (int64_t)0x7fffffff);
  auto prefetch = [&](RawChunk<NV, 2>& rb, int g, bool live) {
    const char* const rows[2] = {trow_of(g), drow_of(g)};
    issue_seg_fixed<DT, NV, 2>(rb, rows, v0, last, live, row_bytes);
  };
  RawChunk<NV, 2> rawA, rawB;
  // groups of items i, i + 1 of the current layer (past the end: an earlier item).
  // Layers -2 and -1 only issue the loads of items 0 and 1, from the same code as
  // every later prefetch, so the loop is entered with no load outstanding and the
  // compiler's count of outstanding loads at the loop head stays exact: each unpack
  // then waits for its own chunk only, not for the one issued after it.
  int g_0 = group_of(0), g_p1 = g_0;
  int g_m2 = 0, g_m1 = 0;          // groups of items i - 2 and i - 1
  bool pair_m2 = false, pair_m1 = false;
  uint64_t wpoll = 0ull;                     // this lane's polled record word
  uint64_t wpoll_am = 0ull;                  // ... and its argmax word (target-only)
  float x[2][NE];                            // item i - 1's e values between layers
  float xref[2] = {0.f, 0.f};                // ... and this wave's references for them
  float href[2] = {0.f, 0.f};                // references of the item held in LDS
  float xz = 0.f, hz = 0.f;                  // this wave's p mass (e units) of each

  // Layer i: statistics and pass 2 of item i - 2 (held in LDS), item i - 1 moves
  // from registers to LDS, item i is unpacked from buffer i & 1, the poll for item
  // i - 1's records and the loads of item i + 2 (into the same buffer) go out, pass
  // 1 of item i.
  auto layer = [&](int i, RawChunk<NV, 2>& rb) __attribute__((always_inline)) {
    // this wave's role, derived again in every layer (opaque to the compiler), so
    // that the role tests are not hoisted out of the loop as 64-bit masks that
    // would hold scalar registers through it: 0 combines p, 1 q; 2 polls p, 3 q
    int role = wave ^ wp, c_l = c;
    asm volatile("" : "+s"(role), "+s"(c_l));
    // ---- row statistics of item i - 2 (polled a layer ago) ---------------------
    if (i >= 2 && i - 2 < nl) {
      const bool pair2 = pair_m2;
      // the bookkeeping waves run at raised priority: the layer waits for them
      if (role == 2 || (role == 3 && pair2)) {
        __builtin_amdgcn_s_setprio(3);
        const int row = role == 2 ? 0 : 1;
        // Waiting for every load in flight first (the next item's chunk included)
        // measured faster than testing the words as soon as their own load is back:
        // the test comes later and finds a record missing less often, and a reload
        // waits for those loads anyway.
        wait_vmem_all();
        // a wait that timed out gives NaN statistics (and no greedy token), which
        // pass 2 turns into NaN partials: the finish reports such rows as failed
        const Lse st = poll_row(wpoll, rsrc_rec(g_m2), C, kSt, row, a.err, a.wait_limit);
        if (lane == 0) {
          st_sh[i & 1][row][0] = st.ref;
          st_sh[i & 1][row][1] = st.z;
          st_sh[i & 1][row][2] = __builtin_amdgcn_rcpf(st.z);
        }
        if (TO && row == 1) {
          const uint32_t yh = poll_argmax(wpoll_am, rsrc_rec(g_m2), C, kSt, a.err, a.wait_limit);
          if (lane == 0) yhat_sh[i & 1] = yh;
        }
        __builtin_amdgcn_s_setprio(0);
      }
      __syncthreads();
      // ---- pass 2 of item i - 2 ------------------------------------------------
      // In this wave's e units p = sa e_p and q = sb e_q, sa = 2^(href_p - ref_p) / z_p
      // and sb likewise.  The difference of references is exact for every wave whose
      // largest logit is near the row's (two floats within a factor of 2), so the
      // ratio rho = sb / sa = 2^(dq - dp) z_p / z_q carries a few roundings of its own
      // (the reciprocal 1 / z_q to within one unit).  (Through the logarithms
      // ref + log2 z instead, rho would inherit their rounding, about 2^-24 times
      // their size: an error common to every element that the cancellation in p - q
      // magnifies in the residual's shape.)  While rho is at most 2^64,
      // max(0, p - q) = sa max(0, e_p - rho e_q) (one fused multiply-add; e_p <= 1,
      // so the max is the [0, 1] output clamp, free) and the overlap is the wave's p
      // mass minus the residual, both summed in pass 1's order, so disjoint supports
      // give an overlap of exactly 0.  A larger rho (q outweighs p here by more than
      // 2^64) works in q's units instead.
      const float* const sp = st_sh[i & 1][0];
      const float* const sq = st_sh[i & 1][1];
      const float dp = href[0] - sp[0];   // -inf: no p mass here
      const float sa = fast_exp2(dp) * sp[2];
      // log2 of sa for the Gumbel-max keys (whose comparisons within the row cancel
      // the log2 z_p term) and the target-only test below
      const float la = dp - fast_log2(sp[1]);
      float rm = 0.f, om = 0.f;
      if (!pair2) {
        rm = sa * hz;
      } else if (dp != kNegInf) {
        const float dq = href[1] - sq[0];
        const float zr = z_ratio(sp[1], sq[1], sq[2]);   // z_p / z_q
        const float rho = fast_exp2(dq - dp) * zr;     // +inf past 2^128
        float r0 = -0.f, r1 = -0.f;   // -0 + x = x: the first additions fold away
        if (!(rho > 0x1p64f)) {
#pragma unroll
          for (int qi = 0; qi < NQ; ++qi) {
            const float4 ea = held[0][qi][t], eb = held[1][qi][t];
            const float va[4] = {ea.x, ea.y, ea.z, ea.w}, vb[4] = {eb.x, eb.y, eb.z, eb.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float d = clamp01(__builtin_fmaf(-rho, vb[e], va[e]));   // <= va <= 1
              if (e & 1) r1 += d; else r0 += d;
            }
          }
          const float rw = wave_total(r0 + r1);
          rm = sa * rw;
          om = sa * fmaxf(hz - rw, 0.f);
        } else {
          const float rr = fast_exp2(dp - dq) * z_ratio(sq[1], sp[1], sp[2]), sb = fast_exp2(dq) * sq[2];   // rr = 1 / rho
          float o0 = -0.f, o1 = -0.f;
#pragma unroll 1
          for (int qi = 0; qi < NQ; ++qi) {
            const float4 ea = held[0][qi][t], eb = held[1][qi][t];
            const float va[4] = {ea.x, ea.y, ea.z, ea.w}, vb[4] = {eb.x, eb.y, eb.z, eb.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float d = clamp01(__builtin_fmaf(rr, va[e], -vb[e]));    // <= rr va <= 1
              const float m = __builtin_elementwise_minimum(rr * va[e], vb[e]);
              if (e & 1) { r1 += d; o1 += m; } else { r0 += d; o0 += m; }
            }
          }
          rm = sb * wave_total(r0 + r1);
          om = sb * wave_total(o0 + o1);
        }
      }
      // statistics that are NaN (a timed-out wait, or a row without a finite
      // normaliser) make the partials NaN, whatever the sums above gave
      const bool poison = !(sp[1] == sp[1]) || (pair2 && !(sq[1] == sq[1])) ||
                          (TO && pair2 && yhat_sh[i & 1] == kNoArgmax);
      if (poison) rm = om = __builtin_nanf("");
      // (om >= 0 or NaN carries the sign bit as a marker: a published word is non-zero)
      if (lane == 0) put_word(a.part2 + ((int64_t)g_m2 * C + c_l) * kWaves + wave, pack2(rm, mark(om)));
      if constexpr (GM) {
        // Gumbel-max keys of this wave's segment, key = w / E (the exponential race,
        // E the element's exponential variate): w = the residual for a pair row, w = p
        // for a bonus row (a pair row whose residual turns out empty samples p by the
        // inverse CDF in the finish instead).  Each thread keeps its best as a
        // (numerator, E) pair compared by cross-multiplication, in increasing index
        // order (strict >, so the smaller index stays on equal keys); the wave then
        // compares log2 keys.
        float np = 0.f, ep = 1.f, nr = 0.f, er = 1.f;
        uint32_t ip = 0xffffffffu, ir = 0xffffffffu;
        float lr = la;   // log2 of the residual's unit
        if (la != kNegInf) {
          const uint64_t crow = a.offset + (uint64_t)g_m2;
          const float dq = href[1] - sq[0];
          const float lb = dq - fast_log2(sq[1]);
          const bool p_units = !(lb - la > 64.f);
          // rho = sb / sa as in the residual above
          const float fq = p_units ? fast_exp2(dq - dp) * z_ratio(sp[1], sq[1], sq[2]) : 1.f,
                      fp = p_units ? 1.f : fast_exp2(dp - dq) * z_ratio(sq[1], sp[1], sp[2]);
          lr = p_units ? la : lb;
          // two 16-byte slots at a time: unrolled further, the Philox rounds would
          // hold the registers that the items in flight need (scratch spills)
          auto keys = [&](auto kind) __attribute__((always_inline)) {
            constexpr int K = decltype(kind)::value;   // 0: p, 1: residual in p's units, 2: in q's
#pragma unroll 2
            for (int qi = 0; qi < NQ; ++qi) {
              const float4 ea = held[0][qi][t];
              const float va[4] = {ea.x, ea.y, ea.z, ea.w};
              float vb[4] = {0.f, 0.f, 0.f, 0.f};
              if constexpr (K > 0) {
                const float4 eb = held[1][qi][t];
                vb[0] = eb.x; vb[1] = eb.y; vb[2] = eb.z; vb[3] = eb.w;
              }
              const uint32_t gi0 = (uint32_t)(v0 + (4 * qi / PV) * 64) * PV + (4 * qi) % PV;   // 4-aligned
              float E[4];
              expo4(a.seed, crow, gi0 >> 2, E);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if constexpr (K == 0) {
                  const bool tp = va[e] * ep > np * E[e];
                  np = tp ? va[e] : np;
                  ep = tp ? E[e] : ep;
                  ip = tp ? gi0 + e : ip;
                } else {
                  // <= fp va <= 1; fp = 1 in p's units
                  const float d = clamp01(__builtin_fmaf(-fq, vb[e], K == 1 ? va[e] : fp * va[e]));
                  const bool tr = d * er > nr * E[e];
                  nr = tr ? d : nr;
                  er = tr ? E[e] : er;
                  ir = tr ? gi0 + e : ir;
                }
              }
            }
          };
          if (!pair2) keys(std::integral_constant<int, 0>{});
          else if (p_units) keys(std::integral_constant<int, 1>{});
          else keys(std::integral_constant<int, 2>{});
        }
        float kp = np > 0.f ? la + fast_log2(np) - fast_log2(ep) : kNegInf;
        float kr = nr > 0.f ? lr + fast_log2(nr) - fast_log2(er) : kNegInf;
        wave_argmax(kp, ip);
        if (pair2) wave_argmax(kr, ir);
        if (lane == 0) {
          uint64_t* gk = a.gkeys + (((int64_t)g_m2 * C + c) * kWaves + wave) * 2;
          put_word(gk, pack_argmax(kr, ir));
          put_word(gk + 1, pack_argmax(kp, ip));
        }
      }
      if constexpr (TO) {
        if (pair2) {
          // target-only: this wave's p mass without the greedy draft token (the
          // residual a rejected row samples), re-summed only by the wave holding it
          const uint32_t yh = yhat_sh[i & 1];
          const uint32_t ylo = (uint32_t)s0 * PV;
          float pex = sa * hz;
          if (la != kNegInf && yh >= ylo && yh - ylo < (uint32_t)(kSegVec * PV)) {
            float m0 = -0.f, m1 = -0.f;
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
              const float4 ea = held[0][qi][t];
              const float va[4] = {ea.x, ea.y, ea.z, ea.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int ii = 4 * qi + e;
                const uint32_t gi = (uint32_t)(v0 + (ii / PV) * 64) * PV + ii % PV;
                const float v = gi == yh ? 0.f : va[e];
                if (e & 1) m1 += v; else m0 += v;
              }
            }
            pex = sa * wave_total(m0 + m1);
          }
          if (lane == 0) st_coherent(a.part3 + ((int64_t)g_m2 * C + c) * kWaves + wave, mark(pex));
        }
      }
    }
    // ---- item i - 1 moves to LDS (own slots only) ------------------------------
    if (i >= 1 && i - 1 < nl) {
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        held[0][qi][t] = make_float4(x[0][4 * qi], x[0][4 * qi + 1], x[0][4 * qi + 2], x[0][4 * qi + 3]);
        held[1][qi][t] = make_float4(x[1][4 * qi], x[1][4 * qi + 1], x[1][4 * qi + 2], x[1][4 * qi + 3]);
      }
      href[0] = xref[0];
      href[1] = xref[1];
      hz = xz;
    }

    // ---- item i: unpack, then the poll for item i - 1 and the loads of i + 2 ----
    const bool pair = is_pair(g_0);
    if (i >= 0 && i < nl) {
      const char* const rows[2] = {trow_of(g_0), drow_of(g_0)};
      // both rows always (a bonus item's second row is its target row again, which
      // pass 1 then ignores), so that every load of the buffer is consumed before
      // the buffer is refilled and x[1] has one definition on every path (a
      // bonus-only branch around its unpack costs more register copies at the join
      // than the unpack saves); the bounds pass through an empty asm so that the
      // masks of the partial segment path are derived there, not kept live across
      // the loop
      int lim_l = lim, tail_l = tail, vend_l = vend, V_l = V;
      asm volatile("" : "+s"(lim_l), "+s"(tail_l), "+s"(vend_l), "+s"(V_l));
      unpack_seg<DT, NV, 2>(rb, rows, v0, full, lim_l, tail_l, vend_l, V_l, x);
    }
    // the poll goes out before the prefetch, so that waiting for it (a layer
    // later) does not wait for the prefetch
    if (i >= 1 && i <= nl && role >= 2 && lane < C) {
      const __amdgpu_buffer_rsrc_t rs = rsrc_rec(g_m1);
      wpoll = rec_load(rs, lane * kSt + (role == 2 ? 0 : 8));
      if (TO && role == 3) wpoll_am = rec_load(rs, lane * kSt + kArgmaxWord * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int g_p2 = i + 2 < nl ? group_of(i + 2) : g_0;
    prefetch(rb, g_p2, i + 2 < nl);
    __builtin_amdgcn_sched_barrier(0);

    if (i >= 0 && i < nl) {
      // ---- pass 1 of item i: wave partials, combined and published --------------
      // (raised priority up to the barrier: the combine and the next layer wait on it)
      __builtin_amdgcn_s_setprio(1);
      Lse pt[2];
      float am = 0.f;   // target-only: this wave's largest draft logit and its index
      uint32_t ai = 0;
      if (TO && pair) {
        float bm = x[1][NE - 1];
        int bi = NE - 1;
#pragma unroll
        for (int ii = NE - 2; ii >= 0; --ii) {   // downwards with >=: the smallest index wins ties
          const bool tk = x[1][ii] >= bm;
          bm = tk ? x[1][ii] : bm;
          bi = tk ? ii : bi;
        }
        am = bm;
        ai = (uint32_t)(v0 + (bi / PV) * 64) * PV + bi % PV;
        wave_argmax(am, ai);
      }
      if (pair) {
        wave_pass1<NE, 2, 1>(x, pt, L);
      } else {
        wave_pass1<NE, 1, 1>(*reinterpret_cast<float(*)[1][NE]>(&x[0]), *reinterpret_cast<Lse(*)[1]>(&pt[0]), L);
        pt[1] = lse_empty();
      }
      xref[0] = pt[0].ref;
      xref[1] = pt[1].ref;
      xz = pt[0].z;
      if (lane == 0) {
        float* ps = part_sh[i & 1][0];
        ps[wave * 3 + 0] = pt[0].ref; ps[wave * 3 + 1] = pt[0].z; ps[wave * 3 + 2] = pt[0].y;
        ps = part_sh[i & 1][1];
        ps[wave * 3 + 0] = pt[1].ref; ps[wave * 3 + 1] = pt[1].z; ps[wave * 3 + 2] = 0.f;
        if (TO) {
          am_sh[i & 1][wave] = am;
          ai_sh[i & 1][wave] = ai;
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      if (role < 2) __builtin_amdgcn_s_setprio(3);
      if (role == 0) {
        const Lse p = merge_lds<kWaves, true>(part_sh[i & 1][0]);
        if (lane == 0) {
          const __amdgpu_buffer_rsrc_t rs = rsrc_rec(g_0);
          rec_store(rs, c_l * kSt, pack2(p.ref, mark(p.z)));
          rec_store(rs, c_l * kSt + 16, pack2(p.y, 1.f));
        }
      } else if (role == 1) {
        const Lse q = merge_lds<kWaves, false>(part_sh[i & 1][1]);
        if (lane == 0) {
          const __amdgpu_buffer_rsrc_t rs = rsrc_rec(g_0);
          rec_store(rs, c_l * kSt + 8, pack2(q.ref, mark(q.z)));
          if (TO && pair) {   // the chunk's argmax over the four waves
            float m = am_sh[i & 1][0];
            uint32_t idx = ai_sh[i & 1][0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) argmax_fold(m, idx, am_sh[i & 1][w], ai_sh[i & 1][w]);
            rec_store(rs, c_l * kSt + kArgmaxWord * 8, pack_argmax(m, idx));
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    // ---- shift the item window -------------------------------------------------
    g_m2 = g_m1;
    pair_m2 = pair_m1;
    g_m1 = g_0;
    pair_m1 = pair;
    g_0 = g_p1;
    g_p1 = g_p2;
  };

  // nl + 4 layers from -2, rounded up to an even count so that both halves of the
  // loop body always run (the buffers then keep their registers across iterations)
  for (int i = -2; i < nl + 2; i += 2) {
    layer(i, rawA);
    layer(i + 1, rawB);
  }

  // ---- the finish: the workgroup j places from the end of the grid (j = S C - 1 -
  // blockIdx.x), its layers done, finishes sequences j, j + S C, ...: wave w takes
  // rows w, w + kWaves, ... of the sequence, then thread 0 forms the accepted length
  // and the next token.  With the item split above the last super-groups have the
  // fewest items and end first, so their workgroups merge a sequence's records
  // while the other super-groups still run, and wait only for its pass-2 words.
  __shared__ int flag_sh[kMaxRowsPerSeq], token_sh[kMaxRowsPerSeq];
  const uint64_t flimit = a.wait_limit > kFinishWaitFloor ? a.wait_limit : kFinishWaitFloor;
  for (int b = S * C - 1 - slot; b < B; b += S * C) {
    for (int k = wave; k < G1; k += kWaves) finish_row<DT, NV, MODE>(a, b, k, flag_sh, token_sh, flimit);
    __syncthreads();
    if (t == 0) {
      int n = 0;
      while (n < G && flag_sh[n] == 1) ++n;
      a.accepted_len[b] = n;
      a.next_token[b] = token_sh[n];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// The finish of a sequence: the main kernel's workgroups run it once their layers
// are done, one wave per row.

// The cumulative sums of the inverse CDF run in float64 (chunk, segment and
// element prefixes alike): their rounding then stays far below that of the float32
// masses they add up, so a token differs from the exact inverse CDF's only where t
// lies within the masses' own rounding of a boundary.

// A lane's double moved by a DPP control (both halves), 0 where there is no source.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_or_zero_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over the wave in lane order (the float32 wave_incl_sum's
// steps on doubles); lane 63 holds the total.
__device__ __forceinline__ double wave_incl_sum_f64(double v) {
  v += dpp_or_zero_f64<0x111>(v);
  v += dpp_or_zero_f64<0x112>(v);
  v += dpp_or_zero_f64<0x114>(v);
  v += dpp_or_zero_f64<0x118>(v);
  v += dpp_or_zero_f64<0x142, 0xa>(v);
  v += dpp_or_zero_f64<0x143, 0xc>(v);
  return v;
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The previous lane's value (0 in lane 0): a DPP wave shift right by one lane.
__device__ __forceinline__ double lane_before(double incl) {
  return dpp_or_zero_f64<0x138>(incl);
}

// log2 z for a positive float z, accurate to a few units of 2^-24 in absolute terms
// even where log2 z is large: z = m 2^k with m in [1, 2) exactly, log2 z = k +
// log2 m, the float32 log2 of m (a value in [0, 1)) carrying the only rounding.
__device__ __forceinline__ double log2_split(float z) {
  int k = 0;
  const float m = 2.f * __builtin_frexpf(z, &k);   // z = m 2^(k - 1), m in [1, 2)
  return (double)(k - 1) + (double)fast_log2(m);
}

// Inverse CDF of one wave segment (NV blocks of 64 vectors, PV values per lane per
// block, vocabulary order block-major then lane-major): the index (within the
// segment) of the first value whose running mass exceeds t; if none, the last
// index with positive mass; -1 if the segment has no mass.  The running masses are
// float64 sums: each lane's prefixes of its PV values (a tree, log2 PV deep), the
// wave's exclusive prefix of the lane totals, and the blocks before; the blocks'
// wave scans are independent of each other.
template <int NV, int PV>
__device__ __forceinline__ int wave_inverse_cdf(const float (&v)[NV][PV], double t) {
  const int lane = threadIdx.x & 63;
  double pre[NV][PV], incl[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int e = 0; e < PV; ++e) pre[j][e] = (double)v[j][e];
    // in place, highest index first, so each step reads the previous step's values
#pragma unroll
    for (int d = 1; d < PV; d *= 2)
#pragma unroll
      for (int e = PV - 1; e >= d; --e) pre[j][e] += pre[j][e - d];
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) incl[j] = wave_incl_sum_f64(pre[j][PV - 1]);
  double base = 0.0;
  int best = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const double cum0 = base + lane_before(incl[j]);
    // the running masses only grow, so the lane's first crossing is the smallest
    // index that crosses: scanned downwards, the last one found
    int bj = 0x7fffffff;
#pragma unroll
    for (int e = PV - 1; e >= 0; --e)
      if (v[j][e] > 0.f && cum0 + pre[j][e] > t) bj = (j * 64 + lane) * PV + e;
    best = min(best, bj);
#pragma unroll
    for (int e = 0; e < PV; ++e)
      if (v[j][e] > 0.f) lastpos = (j * 64 + lane) * PV + e;
    base += readlane_d(incl[j], 63);
  }
  best = (int)wave_min_u32((uint32_t)best);
  lastpos = (int)wave_max_u32((uint32_t)(lastpos + 1)) - 1;
  // blocks are scanned in order, so the smallest crossing index is the first one
  return best != 0x7fffffff ? best : lastpos;
}

// Scan of masses m(0..n-1) in order: lane l owns [l*K, l*K + K).  Returns the
// total, the first index whose running mass exceeds u' * total (else the last
// index with mass, with start = -inf) and the mass before it.  Every lane of the
// wave gets the same result.
struct Scan {
  double total;
  int owner;
  double start;
};

template <typename MassFn>
__device__ __forceinline__ Scan wave_scan_owner(int n, float u_prime, MassFn mass) {
  const int lane = threadIdx.x & 63;
  const int K = (n + 63) / 64;
  const int c0 = lane * K, c1 = min(n, c0 + K);
  double block = 0.0;
  int last_pos = -1;
  for (int c = c0; c < c1; ++c) {
    const float m = mass(c);
    block += (double)m;
    if (m > 0.f) last_pos = c;
  }
  const double incl = wave_incl_sum_f64(block);
  const double excl = lane_before(incl);
  Scan r;
  r.total = readlane_d(incl, 63);
  const double t = (double)u_prime * r.total;
  r.owner = -1;
  r.start = -__builtin_huge_val();
  const uint64_t hit = __ballot(c0 < c1 && incl > t);
  if (hit != 0ull && r.total > 0.0) {
    const int l = __builtin_ctzll(hit);
    double run = readlane_d(excl, l);
    const int a0 = l * K, a1 = min(n, a0 + K);
    for (int c = a0; c < a1; ++c) {
      const double m = (double)mass(c);
      if (r.owner < 0 && run + m > t) { r.owner = c; r.start = run; }
      run += m;
    }
  }
  if (r.owner < 0) {   // rounding left t past every boundary: last index with mass
    const uint64_t pos = __ballot(last_pos >= 0);
    r.owner = pos ? readlane_i(last_pos, 63 - __builtin_clzll(pos)) : 0;
    r.start = -__builtin_huge_val();  // t - start = +inf: the owner takes its last positive element
  }
  return r;
}

// Row (b, k) of the finish, by one wave (k wave-uniform, so the record descriptor
// built from it is scalar).  It first waits until every word the row needs is
// published: the pass-2 words of all its chunks and waves (written last, each after
// its workgroup had polled the row's records), the records themselves, and the
// Gumbel-max keys or the masses without the greedy token.  The wait is bounded by
// `limit` ticks; one that gives up sets the error word and reports the row as timed
// out.  Writes the row's outputs and its acceptance flag and token to flag_sh[k],
// token_sh[k].
template <int DT, int NV, int MODE>
__device__ __forceinline__ void finish_row(const VerifyArgs& a, int b, int k, int* flag_sh, int* token_sh,
                                           uint64_t limit) {
  constexpr bool TO = MODE == kVerifyTargetOnly, GM = MODE == kVerifyGumbel;
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int kSegVec = NV * 64;
  // chunks per lane whose pass-2 words are kept in registers: one (rows of up to 64
  // chunks, 262,144 bf16 logits, have no more per lane; a lane's further chunks are
  // read again from memory), as more registers here spill the finish's live values
  constexpr int KC = 1;
  const int C = a.sp.nchunks;
  const int G = a.G, G1 = G + 1;
  const int lane = threadIdx.x & 63;
  const int g = b * G1 + k;
  const bool pair = k < G;

  const char* trow = reinterpret_cast<const char*>(a.target) + (int64_t)g * a.t_stride * Elem<DT>::kBytes;
  const char* drow = reinterpret_cast<const char*>(a.draft) + (int64_t)(b * G + (pair ? k : 0)) * a.d_stride * Elem<DT>::kBytes;
  constexpr int kSt = rec_bytes<TO>();
  const float L = GM ? kLog2e * a.inv_temp : kLog2e;   // logit -> base-2 exponent scale
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.part1 + (int64_t)g * C * (kSt / 8));
  uint64_t* p2 = a.part2 + (int64_t)g * C * kWaves;
  // the row's pass-2 words through a buffer descriptor: 32-bit offsets, so that no
  // 64-bit address per lane stays live through the finish
  const __amdgpu_buffer_rsrc_t rs2 = rsrc_of(p2);
  auto p2_word = [&](int i) { return rec_load(rs2, i * 8); };
  // target-only pair rows sample p without the greedy token: its per-wave masses
  float* p3 = TO ? a.part3 + (int64_t)g * C * kWaves : nullptr;
  const bool to_pair = TO && pair;

  // lane l owns chunks [l K, l K + K); the pass-2 words of its first KC are kept
  const int K = (C + 63) / 64;
  const int c0 = lane * K, c1 = min(C, c0 + K);
  float seg[KC][kWaves], om_sum = 0.f, tv_sum = 0.f;
#pragma unroll
  for (int i = 0; i < KC; ++i)
#pragma unroll
    for (int w = 0; w < kWaves; ++w) seg[i][w] = 0.f;
  // the given draft token and its two logits do not depend on the other
  // workgroups: their loads go out before the wait
  int y = 0;
  bool y_ok = false;
  float ay = 0.f, by = 0.f;
  if constexpr (!TO) {
    y = a.tokens[b * G + min(k, G - 1)];
    y_ok = pair && y >= 0 && y < a.V;
    const int yc = y_ok ? y : 0;
    ay = load_one<DT>(trow, yc);
    by = load_one<DT>(drow, yc);
  }
  float u, up;
  row_uniforms(a.seed, a.offset, (uint64_t)g, &u, &up);

  // A bounded wait: `test` loads words and tells whether this lane's are all
  // published; a timeout sets the error word and returns true.
  auto wait_words = [&](auto&& test) -> bool {
    uint64_t t0 = 0;
    for (;;) {
      const bool ready = test();
      if (__ballot(!ready) == 0ull) return false;
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      if (t0 == 0) t0 = now;
      if (now - t0 > limit) {
        if (lane == 0) __hip_atomic_fetch_or(a.err, kErrSyncTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  };

  // ---- phase 1: the records, complete some two layers before the pass-2 words:
  // the row statistics and the acceptance test's log ratio ----------------------
  RecWords rw;
  const bool wto_rec = wait_words([&]() {
    rw = rec_words(rs, C, kSt);   // record `lane`'s words, kept
    bool ready = lane >= C || (rw.w0 != 0ull && rw.w1 != 0ull && rw.w2 != 0ull);
    if (to_pair && lane < C) ready &= rec_load(rs, lane * kSt + kArgmaxWord * 8) != 0ull;
    for (int cc = lane + 64; cc < C; cc += 64) {
#pragma unroll
      for (int w = 0; w < 3; ++w) ready &= rec_load(rs, cc * kSt + w * 8) != 0ull;
      if (to_pair) ready &= rec_load(rs, cc * kSt + kArgmaxWord * 8) != 0ull;
    }
    return ready;
  });
  const RowStats st = merge_records(rw, rs, C, kSt, pair);
  const float lse2_p = lse_log2(st.p);
  const float lse2_q = pair ? lse_log2(st.q) : 0.f;
  const bool bad_p = !wto_rec && !(__builtin_isfinite(lse2_p));
  const bool bad_q = !wto_rec && pair && !(__builtin_isfinite(lse2_q));
  const bool stats_ok = !wto_rec && !bad_p && !bad_q;
  // target-only: the greedy draft token from the records, then p at it
  if constexpr (TO) {
    y = pair ? (int)merge_argmax(rs, C, kSt) : 0;
    y_ok = pair && y >= 0 && y < a.V;
    ay = y_ok ? load_one<DT>(trow, y) : 0.f;
  }
  // The acceptance test in the base-2 log domain, in float64, from the row
  // statistics (ref, z) the main kernel summed with the same logit scale L:
  //   u < p(y) / q(y)  <=>  log2 u < (a_y - b_y) L - (lse2_p - lse2_q),
  // lse2 = ref + log2 z.  Taken in float32, the two base-2 log-sum-exps (about
  // 17 at V = 151936) would each round by up to 1e-6; here every term keeps the
  // accuracy of the float32 sums z (log2 z split into exponent and mantissa),
  // and log2 u (u on a 2^-24 grid) carries one float32 rounding.  Target-only
  // verify tests log2 u < log2 p(y) = a_y L - lse2_p instead.
  const double Ld = (double)L;
  const double l2p = stats_ok ? (double)st.p.ref + log2_split(st.p.z) : 0.0;
  double lu = u > 0.f ? (double)fast_log2(u) : -__builtin_huge_val();
  double lratio = 0.0;
  if (TO) lratio = (double)ay * Ld - l2p;
  else if (pair && stats_ok)
    lratio = ((double)ay - (double)by) * Ld - (l2p - ((double)st.q.ref + log2_split(st.q.z)));
  // the entropy needs only the pass-1 records: valid after a timed-out wait for the
  // pass-2 words too
  const float entropy = bad_p || wto_rec ? __builtin_nanf("") : kLn2 * (fast_log2(st.p.z) - st.p.y / st.p.z);
  // formed here, while the other workgroups still run, not where they are used
  float ent_v = entropy;
  asm volatile("" : "+v"(lratio), "+v"(lu), "+v"(up), "+v"(ent_v));

  // ---- phase 2: the pass-2 words, and the Gumbel-max keys or the masses without
  // the greedy token; each poll keeps the pass-2 words of the lane's first KC chunks
  // and only tests the others (they are read again below) -------------------------
  const uint64_t* gk = GM ? a.gkeys + (int64_t)g * C * kWaves * 2 : nullptr;
  uint64_t pw[KC][kWaves];
  const bool wto_p2 = wait_words([&]() {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < KC; ++i)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        pw[i][w] = p2_word(min(c0 + i, C - 1) * kWaves + w);
        ready &= !(c0 + i < c1) || pw[i][w] != 0ull;
      }
    for (int cc = c0 + KC; cc < c1; ++cc)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) ready &= p2_word(cc * kWaves + w) != 0ull;
    if (to_pair)
      for (int i = lane; i < C * kWaves; i += 64) ready &= __float_as_uint(ld_coherent(p3 + i)) != 0u;
    if (GM)
      for (int i = lane; i < C * kWaves * 2; i += 64) ready &= get_word(gk + i) != 0ull;
    return ready;
  });
  const bool wto = wto_rec || wto_p2;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    if (c0 + i < c1) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint64_t v = pw[i][w];
        seg[i][w] = to_pair ? unmark(ld_coherent(p3 + (int64_t)(c0 + i) * kWaves + w)) : unpack_lo(v);
        om_sum += unmark(unpack_hi(v));
        tv_sum += unpack_lo(v);
      }
    }
  }
  for (int cc = c0 + KC; cc < c1; ++cc)
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint64_t v = p2_word(cc * kWaves + w);
      om_sum += unmark(unpack_hi(v));
      tv_sum += unpack_lo(v);
    }

  // chunk mass (residual, or p for a bonus row) and its segment masses
  auto seg_mass = [&](int cc, int w) {   // any chunk, from memory
    return to_pair ? unmark(ld_coherent(p3 + (int64_t)cc * kWaves + w))
                   : unpack_lo(p2_word(cc * kWaves + w));
  };
  auto chunk_mass_own = [&](int cc) {    // a chunk of this lane's block
    const int i = cc - c0;
    float m = 0.f;
    if (i < KC) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) m += seg[i][w];
    } else {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) m += seg_mass(cc, w);
    }
    return m;
  };
  // ---- the chunk scan: it needs only the pass-2 masses and u', so it runs as soon
  // as they are in, on whatever they hold (a row found bad below discards it) ------
  bool empty_res = false;
  Scan sc{0.0, 0, 0.0};
  float oseg[kWaves] = {0.f, 0.f, 0.f, 0.f};   // segment masses of the owner chunk
  if constexpr (!GM) {
    // block sums in lane order, prefix over lanes, then the owner lane walks its block
    double blk = 0.0;
    int last_pos = -1;
    for (int cc = c0; cc < c1; ++cc) {
      const float m = chunk_mass_own(cc);
      blk += (double)m;
      if (m > 0.f) last_pos = cc;
    }
    const double incl = wave_incl_sum_f64(blk);
    const double excl = lane_before(incl);
    sc.total = readlane_d(incl, 63);
    const double tt = (double)up * sc.total;
    sc.owner = -1;
    sc.start = -__builtin_huge_val();
    int ol = -1;
    const uint64_t hit = __ballot(c0 < c1 && incl > tt);
    if (hit != 0ull && sc.total > 0.0) {
      ol = __builtin_ctzll(hit);
      double run = excl;
      int own = -1;
      double st0 = -__builtin_huge_val();
      for (int cc = c0; cc < c1; ++cc) {
        const double m = (double)chunk_mass_own(cc);
        if (own < 0 && run + m > tt) { own = cc; st0 = run; }
        run += m;
      }
      sc.owner = readlane_i(own, ol);
      sc.start = readlane_d(st0, ol);
    }
    if (sc.owner < 0) {   // rounding left t past every boundary: last chunk with mass
      const uint64_t pos = __ballot(last_pos >= 0);
      ol = pos ? 63 - __builtin_clzll(pos) : 0;
      sc.owner = pos ? readlane_i(last_pos, ol) : 0;
      sc.start = -__builtin_huge_val();
    }
    // the owner chunk's segment masses, from the lane that holds them
    const int oi = sc.owner - ol * K;
    if (oi >= 0 && oi < KC) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < KC; ++i) v = i == oi ? seg[i][w] : v;
        oseg[w] = readlane_f(v, ol);
      }
    } else {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) oseg[w] = seg_mass(sc.owner, w);
    }
  }
  // Where the residual has mass, and for a bonus row, the owner segment follows from
  // the owner chunk's segment masses: its loads go out right away, ahead of the
  // checks below.
  const int vpc = (int)a.sp.vec_per_chunk, nvec = (int)a.sp.nvec, nfull = (int)a.sp.nvec_full;
  auto pick_segment = [&](double tl, int& os, double& seg_start) {
    os = -1;
    seg_start = -__builtin_huge_val();
    double run = 0.0;
    int lastpos = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const double m = (double)oseg[i];
      if (m > 0.0) lastpos = i;
      if (os < 0 && run + m > tl) { os = i; seg_start = run; }
      run += m;
    }
    if (os < 0) os = lastpos;
  };
  auto issue_segment = [&](int oc, int sgm, bool q_rows, RawChunk<NV, 2>& raw) {
    const int s0 = oc * vpc + sgm * kSegVec;
    const char* const rows[2] = {trow, q_rows ? drow : trow};
    issue_seg<DT, NV, 2>(raw, rows, s0 + lane, nfull - 1);
  };
  const bool pre = !GM && !(pair && !(sc.total > 0.0));
  RawChunk<NV, 2> raw_pre;
  int os_pre = 0;
  double start_pre = 0.0;
  if (pre) {
    pick_segment((double)up * sc.total - sc.start, os_pre, start_pre);
    issue_segment(sc.owner, os_pre, !TO && pair, raw_pre);
  }

  // the row's pass-2 partials: NaN (with finite statistics) where a bounded wait of
  // a workgroup for the row statistics timed out
  float ot[2] = {om_sum, tv_sum};
  wave_reduce<false, 2>(ot);
  const bool timed_out = wto || (!(bad_p || bad_q) && !(ot[0] == ot[0] && ot[1] == ot[1]));
  const bool bad = bad_p || bad_q || timed_out;

  auto pmass = [&](int cc) {   // mass of p in chunk cc, from its record
    const uint64_t w0 = rec_load(rs, cc * kSt);
    const float z = unmark(unpack_hi(w0));
    return z > 0.f ? z * fast_exp2(unpack_lo(w0) - lse2_p) : 0.f;
  };

  float alpha = 0.f;
  if (!bad && pair) {
    alpha = ot[0];
    tv_sum = ot[1];
    if (GM ? !(tv_sum > 0.f) : !(sc.total > 0.0)) {   // the residual has no mass: sample from p
      empty_res = true;
      if (!GM) sc = wave_scan_owner(C, up, pmass);
    }
  }
  // TV: the residual mass (the scan's total for rejection sampling)
  const float r_tot = TO || GM ? tv_sum : pair && !empty_res ? (float)sc.total : 0.f;
  bool use_q = !TO && pair && !empty_res;
  const bool drop_y = to_pair && !empty_res && y_ok;   // target-only residual: p without y

  // ---- owner segment inside the owner chunk, then the inverse CDF in it ------
  int token = -1;
  if (GM && !bad) {
    // Gumbel-max: the largest key over the row's waves, of the residual for a pair
    // row (unless it is empty or no residual key is finite: then the inverse CDF of
    // p below), of p for a bonus row
    float m = kNegInf;
    uint32_t idx = 0xffffffffu;
    auto best = [&](int slot) {
      m = kNegInf;
      idx = 0xffffffffu;
      for (int i = lane; i < C * kWaves; i += 64) {
        const uint64_t w = get_word(gk + i * 2 + slot);
        argmax_fold(m, idx, unpack_lo(w), argmax_index(w));
      }
      wave_argmax(m, idx);
    };
    if (pair && !empty_res) {
      best(0);
      empty_res = !(m > kNegInf);
    }
    if (!pair) best(1);
    token = !(pair && empty_res) && m > kNegInf && idx < (uint32_t)a.V ? (int)idx : -1;
  }
  // the owner segment inside the owner chunk, then the inverse CDF in it
  const float zr = pair ? z_ratio(st.p.z, st.q.z, __builtin_amdgcn_rcpf(st.q.z)) : 1.f,
              rzp = __builtin_amdgcn_rcpf(st.p.z);
  // have_raw: the owner segment and its loads are the ones issued above
  auto sample_owner = [&](bool have_raw) -> int {
    const int oc = sc.owner;
    const int obeg = oc * vpc;
    const int oend = min(obeg + vpc, nvec);
    const int lim = min(oend, nfull);
    // this lane's values of wave segment s: p, or max(0, p - q) for a non-empty residual
    auto seg_values = [&](int s, float (&v)[NV][PV], bool use_pre) {
      const int s0 = obeg + s * kSegVec;
      const char* const rows[2] = {trow, use_q ? drow : trow};
      RawChunk<NV, 2> raw;
      if (use_pre) raw = raw_pre;
      else issue_segment(oc, s, use_q, raw);
      float x[2][NV * PV];
      unpack_seg<DT, NV, 2>(raw, rows, s0 + lane, s0 + kSegVec <= lim, lim, nfull, oend, (int)a.V, x);
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < PV; ++e) {
          if (use_q) {
            // in the row's units e = 2^(x L - ref): max(0, p - q) = max(0, e_p - zr e_q) / z_p,
            // zr = z_p / z_q, the ratio pass 2 forms the residual with
            const float ep = fast_exp2(__builtin_fmaf(x[0][j * PV + e], L, -st.p.ref));
            const float eq = fast_exp2(__builtin_fmaf(x[1][j * PV + e], L, -st.q.ref));
            v[j][e] = fmaxf(__builtin_fmaf(-zr, eq, ep), 0.f) * rzp;
          } else {
            const float p = fast_exp2(__builtin_fmaf(x[0][j * PV + e], L, -lse2_p));
            v[j][e] = drop_y && (s0 + lane + j * 64) * PV + e == y ? 0.f : p;
          }
        }
    };
    const double tl = (double)up * sc.total - sc.start;
    int os = -1;
    double seg_start = -__builtin_huge_val();
    float v[NV][PV];
    if (pair && empty_res) {
      // segment masses of p are not recorded for a pair row: measure them (rare)
      double run = 0.0;
      for (int s = 0; s < kWaves && os < 0; ++s) {
        seg_values(s, v, false);
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int e = 0; e < PV; ++e) m += v[j][e];
        const double md = (double)wave_total(m);
        if (run + md > tl) { os = s; seg_start = run; }
        run += md;
      }
      if (os < 0) os = kWaves - 1;
      have_raw = false;
    } else if (have_raw) {
      os = os_pre;
      seg_start = start_pre;
    } else {
      pick_segment(tl, os, seg_start);
    }
    seg_values(os, v, have_raw);
    const int loc = wave_inverse_cdf<NV, PV>(v, tl - seg_start);
    return loc >= 0 ? (obeg + os * kSegVec) * PV + loc : -1;
  };
  if (GM && !bad && pair && empty_res) {
    // a Gumbel-max pair row whose residual is empty samples p by the inverse CDF
    // with the row's u' (the main kernel forms p's keys for bonus rows only)
    use_q = false;
    sc = wave_scan_owner(C, up, pmass);
    token = sample_owner(false);
  }
  if (!bad && !GM) {
    token = sample_owner(pre);
    if (token < 0 && use_q) {
      // a residual made of rounding alone (p and q equal up to float32 rounding):
      // its mass from pass 2 was positive, but the owner segment's values, formed
      // again from the logits, have none; the row samples p, like an empty residual
      empty_res = true;
      use_q = false;
      sc = wave_scan_owner(C, up, pmass);
      token = sample_owner(false);
    }
  }

  if (lane == 0) {
    int status = 0;
    if (bad_p) status |= kRowBadTarget;
    if (bad_q) status |= kRowBadDraft;
    if (timed_out) status |= kRowSyncTimeout;
    if (empty_res) status |= kRowResidualEmpty;
    int flag = 0;
    const float nan = __builtin_nanf("");
    if (pair) {
      if (TO) {
        // target-only: accept the greedy token with probability p(y); the RS/TO
        // boundary TV < 1 - p(y)
        const double lpy = lratio;
        const float py = y_ok && !bad ? fast_exp2((float)lpy) : nan;
        if (y_ok && !bad) flag = lpy >= 0.0 || lu < lpy ? 1 : 0;   // p(y) = 1: u < 1 always
        a.draft_token[b * G + k] = y_ok && !bad ? y : -1;
        if (a.p_yhat) a.p_yhat[b * G + k] = py;
        if (a.rs_better) a.rs_better[b * G + k] = (uint8_t)(y_ok && !bad && r_tot < 1.f - py ? 1 : 0);
      } else if (!y_ok) {
        status |= kRowBadToken;
      } else if (!bad) {
        const double d = lratio;
        if (d == d) flag = d >= 0.0 || lu < d ? 1 : 0;   // ratio >= 1: u < 1 always
      }
      a.accept[b * G + k] = (uint8_t)flag;
      if (a.overlap) a.overlap[b * G + k] = bad ? nan : alpha;
      if (a.tv) a.tv[b * G + k] = bad ? nan : r_tot;
    }
    if (a.entropy) a.entropy[g] = ent_v;
    if (a.row_token) a.row_token[g] = token;
    if (a.row_status) a.row_status[g] = status;
    flag_sh[k] = flag;
    token_sh[k] = token;
  }
  // clear this row's records and pass-2 words for the next call (the wave has read
  // them all): a call leaves every workspace word it wrote at zero.  Last, so that
  // nothing in the row waits for these stores to complete
  for (int cc = lane; cc < C; cc += 64) {
#pragma unroll
    for (int w = 0; w < kSt / 8; ++w) rec_store(rs, cc * kSt + w * 8, 0ull);
  }
  for (int i = lane; i < C * kWaves; i += 64) rec_store(rs2, i * 8, 0ull);
  if (to_pair)
    for (int i = lane; i < C * kWaves; i += 64) st_coherent(p3 + i, 0.f);
  if (GM)
    for (int i = lane; i < C * kWaves * 2; i += 64) put_word(a.gkeys + (int64_t)g * C * kWaves * 2 + i, 0ull);
}

// ---------------------------------------------------------------------------
// Gumbel-max tokens of logit rows (draft sampling at a temperature): row r emits
// argmax_v (x_v L - log2 E_v) with E the element's exponential variate (counter
// offset + r; L = log2(e) / T), the smallest index among equal keys, -1 if no key
// is finite.  A row is cut into chunks of kSampleVec 16-byte vectors, one
// workgroup each (thread t takes vectors t, t + 256, ...), which writes its best
// (key, index + 1) word; gumbel_sample_finish reduces a row's words, one wave per row.
// two vectors per thread (4096 bf16 logits per workgroup): measured faster than
// one, four or eight
constexpr int kSampleVecPerThread = 2;
constexpr int kSampleVec = kBlock * kSampleVecPerThread;

template <int DT>
__global__ __launch_bounds__(kBlock) void gumbel_sample_chunks(const char* logits, int64_t row_bytes, int64_t V,
                                                               int nchunks, float L, uint64_t seed, uint64_t offset,
                                                               uint64_t* keys) {
  constexpr int PV = Elem<DT>::kPerVec;
  const int r = blockIdx.x / nchunks, c = blockIdx.x - r * nchunks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const char* row = logits + (int64_t)r * row_bytes;
  const int64_t nvec = (V + PV - 1) / PV;
  const uint64_t crow = offset + (uint64_t)r;
  const int64_t vb = (int64_t)c * kSampleVec + threadIdx.x;
  // all of this thread's loads first; a vector past the row's end stays unused
  u32x4 w[kSampleVecPerThread];
#pragma unroll
  for (int j = 0; j < kSampleVecPerThread; ++j) {
    const int64_t v = vb + (int64_t)j * kBlock;
    if ((v + 1) * PV <= V) w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + v);
  }
  float km = kNegInf;
  uint32_t ki = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < kSampleVecPerThread; ++j) {
    const int64_t v = vb + (int64_t)j * kBlock;
    if (v >= nvec) break;
    float x[PV];
    if ((v + 1) * PV <= V) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (DT == kBF16) {
          x[2 * h] = bf16_lo(w[j][h]);
          x[2 * h + 1] = bf16_hi(w[j][h]);
        } else {
          x[h] = __uint_as_float(w[j][h]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < PV; ++e) x[e] = v * PV + e < V ? load_one<DT>(row, v * PV + e) : kNegInf;
    }
#pragma unroll
    for (int h = 0; h < PV / 4; ++h) {
      float E[4];
      expo4(seed, crow, (uint32_t)(v * PV / 4 + h), E);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the thread visits its elements in increasing index order, so a strict >
        // keeps the smaller index on equal keys (and a NaN key never wins); a row
        // whose keys are all -inf yields no token, whatever index is kept
        const float kv = __builtin_fmaf(x[4 * h + e], L, -fast_log2(E[e]));
        const bool tk = kv > km;
        km = tk ? kv : km;
        ki = tk ? (uint32_t)(v * PV + 4 * h + e) : ki;
      }
    }
  }
  wave_argmax(km, ki);
  __shared__ float m_sh[kWaves];
  __shared__ uint32_t i_sh[kWaves];
  if (lane == 0) {
    m_sh[wave] = km;
    i_sh[wave] = ki;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = m_sh[0];
    uint32_t idx = i_sh[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) argmax_fold(m, idx, m_sh[q], i_sh[q]);
    keys[blockIdx.x] = pack_argmax(m, idx);
  }
}

// Each wave clears its row's words after reading them: the workspace is left zeroed,
// as the verify kernels leave theirs, so that the two can share one.
__global__ __launch_bounds__(kBlock) void gumbel_sample_finish(uint64_t* keys, int rows, int nchunks, int64_t V,
                                                               int32_t* tokens) {
  const int r = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= rows) return;
  float m = kNegInf;
  uint32_t idx = 0xffffffffu;
  for (int i = lane; i < nchunks; i += 64) {
    uint64_t* const p = keys + (int64_t)r * nchunks + i;
    const uint64_t w = *p;
    *p = 0ull;
    argmax_fold(m, idx, unpack_lo(w), argmax_index(w));
  }
  wave_argmax(m, idx);
  if (lane == 0) tokens[r] = m > kNegInf && idx < (uint32_t)V ? (int32_t)idx : -1;
}

int gumbel_sample_chunks_per_row(int dt, int64_t V) {
  const int pv = dt == kBF16 ? Elem<kBF16>::kPerVec : Elem<kF32>::kPerVec;
  const int64_t nvec = (V + pv - 1) / pv;
  return (int)((nvec + kSampleVec - 1) / kSampleVec);
}

hipError_t launch_gumbel_sample(const void* logits, int64_t row_stride, int dt, int rows, int64_t V, float L,
                                uint64_t seed, uint64_t offset, int32_t* tokens, uint64_t* keys,
                                hipStream_t stream) {
  const char* base = reinterpret_cast<const char*>(logits);
  const int nch = gumbel_sample_chunks_per_row(dt, V);
  const dim3 grid((unsigned)((int64_t)rows * nch));
  if (dt == kBF16)
    hipLaunchKernelGGL(gumbel_sample_chunks<kBF16>, grid, dim3(kBlock), 0, stream, base, row_stride * 2, V, nch, L,
                       seed, offset, keys);
  else
    hipLaunchKernelGGL(gumbel_sample_chunks<kF32>, grid, dim3(kBlock), 0, stream, base, row_stride * 4, V, nch, L,
                       seed, offset, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gumbel_sample_finish, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kBlock), 0, stream,
                     keys, rows, nch, V, tokens);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <int DT, int NV, int MODE>
static hipError_t launch(const VerifyArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.sgroups * a.sp.nchunks;
  hipLaunchKernelGGL((verify_main<DT, NV, MODE>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

int verify_vec_per_thread(int dt) { return dt == kBF16 ? kVerifyNVBf16 : kVerifyNVF32; }

int verify_record_words(int mode) { return (mode == kVerifyTargetOnly ? rec_bytes<true>() : rec_bytes<false>()) / 8; }

template <int MODE>
static hipError_t launch_mode(const VerifyArgs& a, int dt, hipStream_t stream) {
  return dt == kBF16 ? launch<kBF16, kVerifyNVBf16, MODE>(a, stream) : launch<kF32, kVerifyNVF32, MODE>(a, stream);
}

hipError_t launch_verify(const VerifyArgs& a, int dt, int mode, hipStream_t stream) {
  switch (mode) {
    case kVerifyTargetOnly: return launch_mode<kVerifyTargetOnly>(a, dt, stream);
    case kVerifyGumbel: return launch_mode<kVerifyGumbel>(a, dt, stream);
    default: return launch_mode<kVerifyRejection>(a, dt, stream);
  }
}

template <int MODE>
static hipError_t occupancy_mode(int dt, int* n) {
  return dt == kBF16
             ? hipOccupancyMaxActiveBlocksPerMultiprocessor(n, verify_main<kBF16, kVerifyNVBf16, MODE>, kBlock, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(n, verify_main<kF32, kVerifyNVF32, MODE>, kBlock, 0);
}

hipError_t verify_occupancy(int dt, int mode, int* blocks_per_cu) {
  switch (mode) {
    case kVerifyTargetOnly: return occupancy_mode<kVerifyTargetOnly>(dt, blocks_per_cu);
    case kVerifyGumbel: return occupancy_mode<kVerifyGumbel>(dt, blocks_per_cu);
    default: return occupancy_mode<kVerifyRejection>(dt, blocks_per_cu);
  }
}

}  // namespace mtp
