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
// Two kernels.
//
// verify_main streams every logit once.  A "group" is one row of one sequence:
// (target row, draft row) for k < gamma, or the bonus target row alone.  Each
// group is split along the vocabulary into C chunks of 4096 elements; C workgroups
// form a super-group that walks a list of groups ("layers"), chunk c of every group
// going to workgroup c, and each wave of a workgroup owns a contiguous segment of
// 1024 elements of the chunk.  The two passes over a chunk are software-pipelined
// across layers, so that no workgroup waits on its cluster:
//   layer i:  unpack the chunk of group i (its loads were issued a layer earlier)
//             and issue the loads of group i + 1;
//             pass 1 on group i: per-wave log-sum-exp partials (both rows, plus
//             the entropy moment of the target), combined over the workgroup and
//             published as one self-announcing record;
//             pass 2 on group i - 1, whose values are still in registers: the C
//             records of that group were published a layer ago, so polling them
//             finds them ready; merged (same order everywhere) they give the row
//             log-sum-exps, and each wave sums r = p - min(p, q) and min(p, q)
//             (p alone for a bonus row) over its segment.
// A super-group's workgroups run on one XCD (workgroup i runs on XCD i mod 8).
//
// verify_finish runs one workgroup per sequence, one wave per row.  A wave merges
// the row's records again (lse, entropy), scans the chunk masses, then the segment
// masses of the owner chunk in vocabulary order, re-reads the single 1024-element
// segment holding t = u' * sum r and finishes the inverse CDF in it.  The row's
// acceptance flag needs p(y) and q(y) only.  The sequence's accepted length and
// next token are formed in LDS.  It also clears what the main kernel wrote, so the
// workspace is all zeros again when the call ends.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mtp {

// Chunk record of pass 1 (three words): (ref_p, z_p), (ref_q, z_q), (y_p, 1); the
// z's carry the sign bit as a marker so that no word of a published record is 0.
constexpr int kRecWords = 3;

__device__ __forceinline__ Lse rec_p(uint64_t w0, uint64_t w2) {
  return Lse{unpack_lo(w0), unmark(unpack_hi(w0)), unpack_lo(w2)};
}
__device__ __forceinline__ Lse rec_q(uint64_t w1) { return Lse{unpack_lo(w1), unmark(unpack_hi(w1)), 0.f}; }

// Row statistics of a group from its C records: lane l merges records l, l + 64,
// ... in that order, then the wave merges the lanes.  Used by both kernels, so
// both derive the same bits.  `w` holds the words of record l (first batch).
struct RowStats {
  Lse p, q;
};

template <bool kY>
__device__ __forceinline__ RowStats merge_records(const uint64_t (&w)[kRecWords], __amdgpu_buffer_rsrc_t rs, int C,
                                                  bool pair) {
  const int lane = threadIdx.x & 63;
  Lse ap = lse_empty(), aq = lse_empty();
  if (lane < C) {
    ap = rec_p(w[0], w[2]);
    if (pair) aq = rec_q(w[1]);
  }
  for (int c = lane + 64; c < C; c += 64) {   // further batches: already known to be ready
    const uint64_t w0 = rec_load(rs, c * 24), w1 = rec_load(rs, c * 24 + 8), w2 = rec_load(rs, c * 24 + 16);
    ap = lse_merge(ap, rec_p(w0, w2));
    if (pair) aq = lse_merge(aq, rec_q(w1));
  }
  RowStats s;
  s.p = wave_merge<kY>(ap);
  s.q = pair ? wave_merge<false>(aq) : lse_empty();
  return s;
}

// Wait until every record of the group is published.  `w` holds this lane's words
// of record `lane` as loaded earlier; lanes whose words are not all non-zero load
// again.  Records beyond the first 64 are polled the same way.  Bounded by the
// spin limit (a timeout sets the error word and returns).
__device__ __forceinline__ void poll_records(uint64_t (&w)[kRecWords], __amdgpu_buffer_rsrc_t rs, int C,
                                             uint32_t* err) {
  const int lane = threadIdx.x & 63;
  uint64_t t0 = 0;
  for (int c0 = 0; c0 < C; c0 += 64) {
    const int c = c0 + lane;
    uint64_t v0 = w[0], v1 = w[1], v2 = w[2];
    if (c0 > 0 && c < C) { v0 = rec_load(rs, c * 24); v1 = rec_load(rs, c * 24 + 8); v2 = rec_load(rs, c * 24 + 16); }
    bool ready = !(c < C) || (v0 != 0ull && v1 != 0ull && v2 != 0ull);
    for (int it = 0; __ballot(!ready) != 0ull; ++it) {
      if (t0 == 0) t0 = __builtin_amdgcn_s_memrealtime();
      __builtin_amdgcn_s_sleep(1);
      if (!ready) {
        v0 = rec_load(rs, c * 24); v1 = rec_load(rs, c * 24 + 8); v2 = rec_load(rs, c * 24 + 16);
        ready = v0 != 0ull && v1 != 0ull && v2 != 0ull;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimitTicks) {
        if (lane == 0) __hip_atomic_fetch_or(err, kErrSyncTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    if (c0 == 0) { w[0] = v0; w[1] = v1; w[2] = v2; }
  }
}

// ---------------------------------------------------------------------------
template <int DT, int NV>
__global__ __launch_bounds__(kBlock, kVerifyBlocksPerCU) void verify_main(VerifyArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NE = NV * PV;
  constexpr int NQ = NE / 4;              // 16-byte LDS slots per row and thread
  constexpr int kSegVec = NV * 64;
  const int C = a.sp.nchunks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int sg = slot / C, c = slot - sg * C;
  const int S = a.sgroups;
  const int B = a.B, G = a.G, G1 = G + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int leader = (slot + c) & (kWaves - 1);   // spreads the leader role over the SIMDs

  // item i of this super-group is w = (i S + sg) 8 + xcd; items run over rows
  // k-major (all k = 0 rows first), so every stream sees the same mix of pair and
  // bonus groups
  const int64_t first = (int64_t)sg * 8 + xcd;
  if (first >= a.ngroups) return;
  const int nl = (int)((a.ngroups - 1 - first) / ((int64_t)S * 8)) + 1;
  auto group_of = [&](int i) {
    const int w = (i * S + sg) * 8 + xcd;
    const int k = w / B;
    return (w - k * B) * G1 + k;
  };

  const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
  const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);
  const int64_t s0 = vbeg + (int64_t)wave * kSegVec;      // this wave's segment
  const int64_t v0 = s0 + lane;
  const int64_t lim = min(vend, a.sp.nvec_full);
  const bool full = s0 + kSegVec <= lim;
  const int64_t last = a.sp.nvec_full - 1;
  const int64_t tail = a.sp.nvec_full;

  // e values of the previous layer, waiting for their row statistics: thread t owns
  // slots [row][q][t] (16 bytes each), so the accesses of a wave are contiguous
  __shared__ float4 held[2][NQ][kBlock];
  __shared__ float part_sh[2][kWaves * 3];
  __shared__ float lse_sh[2];

  auto trow_of = [&](int g) {
    return reinterpret_cast<const char*>(a.target) + (int64_t)g * a.t_stride * Elem<DT>::kBytes;
  };
  auto drow_of = [&](int g) {
    const int b = g / G1, k = g - b * G1;
    return reinterpret_cast<const char*>(a.draft) + (int64_t)(b * G + (k < G ? k : 0)) * a.d_stride * Elem<DT>::kBytes;
  };
  auto is_pair = [&](int g) { return g % G1 < G; };

  RawChunk<NV, 2> raw;
  {
    const int g = group_of(0);
    const char* const rows[2] = {trow_of(g), drow_of(g)};
    issue_seg<DT, NV, 2>(raw, rows, v0, last, is_pair(g) ? 2 : 1);
  }

  uint64_t w[kRecWords] = {0ull, 0ull, 0ull};
  float held_ref[2] = {kNegInf, kNegInf};   // this wave's references of the held layer
  float x[2][NE];

  for (int i = 0; i <= nl; ++i) {
    const int gp = i >= 1 ? group_of(i - 1) : 0;
    const bool pair_p = is_pair(gp);
    const __amdgpu_buffer_rsrc_t rs_prev = rsrc_of(a.part1 + (int64_t)gp * C * kRecWords);
    const int g = i < nl ? group_of(i) : 0;
    const bool pair = is_pair(g);
    if (i < nl) {
      const char* const rows[2] = {trow_of(g), drow_of(g)};
      unpack_seg<DT, NV, 2>(raw, rows, v0, full, lim, tail, vend, a.V, x, pair ? 2 : 1);
    }
    // the leader's poll of the previous item's records goes out before the
    // prefetch, so that waiting for it does not wait for the prefetch
    if (i >= 1 && wave == leader && lane < C) {
      w[0] = rec_load(rs_prev, lane * 24);
      w[1] = rec_load(rs_prev, lane * 24 + 8);
      w[2] = rec_load(rs_prev, lane * 24 + 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < nl) {
      const int gn = group_of(i + 1);
      const char* const rows[2] = {trow_of(gn), drow_of(gn)};
      issue_seg<DT, NV, 2>(raw, rows, v0, last, is_pair(gn) ? 2 : 1);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- pass 1 of item i ----------------------------------------------------
    float ref_a = kNegInf, ref_b = kNegInf;
    if (i < nl) {
      const Lse pa = wave_pass1<NE, true>(x[0]);
      ref_a = pa.ref;
      Lse pb = lse_empty();
      if (pair) pb = wave_pass1<NE, false>(x[1]);
      ref_b = pb.ref;
      if (lane == 0) {
        part_sh[0][wave * 3 + 0] = pa.ref; part_sh[0][wave * 3 + 1] = pa.z; part_sh[0][wave * 3 + 2] = pa.y;
        part_sh[1][wave * 3 + 0] = pb.ref; part_sh[1][wave * 3 + 1] = pb.z; part_sh[1][wave * 3 + 2] = pb.y;
      }
    }
    __syncthreads();
    if (wave == leader) {
      if (i < nl) {
        const Lse p = merge_lds<kWaves, true>(part_sh[0]);
        const Lse q = pair ? merge_lds<kWaves, false>(part_sh[1]) : lse_empty();
        if (lane == 0) {
          const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.part1 + (int64_t)g * C * kRecWords);
          rec_store(rs, c * 24, pack2(p.ref, mark(p.z)));
          rec_store(rs, c * 24 + 8, pack2(q.ref, mark(q.z)));
          rec_store(rs, c * 24 + 16, pack2(p.y, 1.f));
        }
      }
      if (i >= 1) {
        poll_records(w, rs_prev, C, a.err);
        const RowStats st = merge_records<false>(w, rs_prev, C, pair_p);
        if (lane == 0) {
          lse_sh[0] = lse_log2(st.p);
          lse_sh[1] = pair_p ? lse_log2(st.q) : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- pass 2 of item i - 1, from LDS ----------------------------------------
    const int t = threadIdx.x;
    if (i >= 1) {
      const float sa = fast_exp2(held_ref[0] - lse_sh[0]);
      float rm = 0.f, om = 0.f;
      if (pair_p) {
        const float sb = fast_exp2(held_ref[1] - lse_sh[1]);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
          const float4 ea = held[0][qi][t], eb = held[1][qi][t];
          const float va[4] = {ea.x, ea.y, ea.z, ea.w}, vb[4] = {eb.x, eb.y, eb.z, eb.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma clang fp contract(off)
            const float p = va[e] * sa, q = vb[e] * sb;
            const float m = fminf(p, q);
            rm += p - m;   // = max(0, p - q) exactly
            om += m;
          }
        }
      } else {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
          const float4 ea = held[0][qi][t];
          rm += ea.x * sa;
          rm += ea.y * sa;
          rm += ea.z * sa;
          rm += ea.w * sa;
        }
      }
      rm = wave_total(rm);
      om = pair_p ? wave_total(om) : 0.f;
      if (lane == 0) a.part2[((int64_t)gp * C + c) * kWaves + wave] = pack2(rm, om);
    }
    // ---- hold item i's e values for the next layer (own slots only) ------------
    if (i < nl) {
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi)
        held[0][qi][t] = make_float4(x[0][4 * qi], x[0][4 * qi + 1], x[0][4 * qi + 2], x[0][4 * qi + 3]);
      if (pair) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi)
          held[1][qi][t] = make_float4(x[1][4 * qi], x[1][4 * qi + 1], x[1][4 * qi + 2], x[1][4 * qi + 3]);
      }
      held_ref[0] = ref_a;
      held_ref[1] = ref_b;
    }
  }
}

// ---------------------------------------------------------------------------
// verify_finish: one workgroup per sequence, wave k handles row (b, k).

// Inverse CDF of one wave segment (NV blocks of 64 vectors, PV values per lane per
// block, vocabulary order block-major then lane-major): the index (within the
// segment) of the first value whose running mass exceeds t; if none, the last
// index with positive mass; -1 if the segment has no mass.
template <int NV, int PV>
__device__ __forceinline__ int wave_inverse_cdf(const float (&v)[NV][PV], float t) {
  const int lane = threadIdx.x & 63;
  float base = 0.f;
  int best = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < PV; ++e) s += v[j][e];
    float incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    const float ex = __shfl_up(incl, 1, 64);
    float cum = base + (lane == 0 ? 0.f : ex);
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      if (v[j][e] > 0.f) {
        cum += v[j][e];
        const int idx = (j * 64 + lane) * PV + e;
        if (best == 0x7fffffff && cum > t) best = idx;
        lastpos = idx;
      }
    }
    base += __shfl(incl, 63, 64);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    best = min(best, __shfl_xor(best, o, 64));
    lastpos = max(lastpos, __shfl_xor(lastpos, o, 64));
  }
  // blocks are scanned in order, so the smallest crossing index is the first one
  return best != 0x7fffffff ? best : lastpos;
}

// Scan of masses m(0..n-1) in order: lane l owns [l*K, l*K + K).  Returns the
// total, the first index whose running mass exceeds u' * total (else the last
// index with mass, with start = -inf) and the mass before it.  Every lane of the
// wave gets the same result.
struct Scan {
  float total;
  int owner;
  float start;
};

template <typename MassFn>
__device__ __forceinline__ Scan wave_scan_owner(int n, float u_prime, MassFn mass) {
  const int lane = threadIdx.x & 63;
  const int K = (n + 63) / 64;
  const int c0 = lane * K, c1 = min(n, c0 + K);
  float block = 0.f;
  int last_pos = -1;
  for (int c = c0; c < c1; ++c) {
    const float m = mass(c);
    block += m;
    if (m > 0.f) last_pos = c;
  }
  float incl = block;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const float ex = __shfl_up(incl, 1, 64);
  const float excl = lane == 0 ? 0.f : ex;
  Scan r;
  r.total = __shfl(incl, 63, 64);
  const float t = u_prime * r.total;
  r.owner = -1;
  r.start = kNegInf;
  const uint64_t hit = __ballot(c0 < c1 && incl > t);
  if (hit != 0ull && r.total > 0.f) {
    const int l = __builtin_ctzll(hit);
    float run = __shfl(excl, l, 64);
    const int a0 = l * K, a1 = min(n, a0 + K);
    for (int c = a0; c < a1; ++c) {
      const float m = mass(c);
      if (r.owner < 0 && run + m > t) { r.owner = c; r.start = run; }
      run += m;
    }
  }
  if (r.owner < 0) {   // rounding left t past every boundary: last index with mass
    const uint64_t pos = __ballot(last_pos >= 0);
    r.owner = pos ? __shfl(last_pos, 63 - __builtin_clzll(pos), 64) : 0;
    r.start = kNegInf;  // t - start = +inf: the owner takes its last positive element
  }
  return r;
}

template <int DT, int NV>
__global__ void verify_finish(VerifyArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int kSegVec = NV * 64;
  const int C = a.sp.nchunks;
  const int G = a.G, G1 = G + 1;
  const int b = blockIdx.x;
  const int k = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = b * G1 + k;
  const bool pair = k < G;
  __shared__ int flag_sh[kMaxRowsPerSeq], token_sh[kMaxRowsPerSeq];

  const char* trow = reinterpret_cast<const char*>(a.target) + (int64_t)g * a.t_stride * Elem<DT>::kBytes;
  const char* drow = reinterpret_cast<const char*>(a.draft) + (int64_t)(b * G + (pair ? k : 0)) * a.d_stride * Elem<DT>::kBytes;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.part1 + (int64_t)g * C * kRecWords);
  uint64_t* p2 = a.part2 + (int64_t)g * C * kWaves;

  // ---- row statistics from the pass-1 records ---------------------------------
  uint64_t w[kRecWords] = {0ull, 0ull, 0ull};
  if (lane < C) { w[0] = rec_load(rs, lane * 24); w[1] = rec_load(rs, lane * 24 + 8); w[2] = rec_load(rs, lane * 24 + 16); }
  const RowStats st = merge_records<true>(w, rs, C, pair);
  const float lse2_p = lse_log2(st.p);
  const float lse2_q = pair ? lse_log2(st.q) : 0.f;
  const bool bad_p = !(__builtin_isfinite(lse2_p));
  const bool bad_q = pair && !(__builtin_isfinite(lse2_q));
  const bool bad = bad_p || bad_q;
  float u, up;
  row_uniforms(a.seed, a.offset, (uint64_t)g, &u, &up);

  // chunk sums of the pass-2 words: (residual or p mass, overlap)
  auto chunk_mass = [&](int cc) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) m += unpack_lo(p2[(int64_t)cc * kWaves + i]);
    return m;
  };
  auto pmass = [&](int cc) {   // mass of p in chunk cc, from its record
    const uint64_t w0 = rec_load(rs, cc * 24);
    const float z = unmark(unpack_hi(w0));
    return z > 0.f ? z * fast_exp2(unpack_lo(w0) - lse2_p) : 0.f;
  };

  float alpha = 0.f;
  bool empty_res = false;
  Scan sc{0.f, 0, 0.f};
  if (!bad) {
    sc = wave_scan_owner(C, up, chunk_mass);
    if (pair) {
      float om = 0.f;
      for (int cc = lane; cc < C; cc += 64) {
#pragma unroll
        for (int i = 0; i < kWaves; ++i) om += unpack_hi(p2[(int64_t)cc * kWaves + i]);
      }
      alpha = wave_total(om);
      if (!(sc.total > 0.f)) {   // the residual has no mass: sample from p
        empty_res = true;
        sc = wave_scan_owner(C, up, pmass);
      }
    }
  }
  const float r_tot = pair && !empty_res ? sc.total : 0.f;
  const bool use_q = pair && !empty_res;

  // ---- owner segment inside the owner chunk, then the inverse CDF in it ------
  int token = -1;
  if (!bad) {
    const int oc = sc.owner;
    const int64_t obeg = (int64_t)oc * a.sp.vec_per_chunk;
    const int64_t oend = min(obeg + a.sp.vec_per_chunk, a.sp.nvec);
    // this lane's values of wave segment s: p, or max(0, p - q) for a non-empty residual
    auto seg_values = [&](int s, float (&v)[NV][PV]) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int64_t vi = obeg + (int64_t)s * kSegVec + j * 64 + lane;
#pragma unroll
        for (int e = 0; e < PV; ++e) {
          const int64_t idx = vi * PV + e;
          float xa = kNegInf, xb = kNegInf;
          if (vi < oend && idx < a.V) {
            xa = load_one<DT>(trow, idx);
            if (use_q) xb = load_one<DT>(drow, idx);
          }
          const float p = fast_exp2(__builtin_fmaf(xa, kLog2e, -lse2_p));
          if (use_q) {
            const float q = fast_exp2(__builtin_fmaf(xb, kLog2e, -lse2_q));
            v[j][e] = fmaxf(p - q, 0.f);
          } else {
            v[j][e] = p;
          }
        }
      }
    };
    const float tl = up * sc.total - sc.start;
    int os = -1;
    float seg_start = kNegInf;
    float v[NV][PV];
    if (pair && empty_res) {
      // segment masses of p are not recorded for a pair row: measure them (rare)
      float run = 0.f;
      for (int s = 0; s < kWaves && os < 0; ++s) {
        seg_values(s, v);
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int e = 0; e < PV; ++e) m += v[j][e];
        m = wave_total(m);
        if (run + m > tl) { os = s; seg_start = run; }
        run += m;
      }
      if (os < 0) os = kWaves - 1;
    } else {
      float run = 0.f;
      int lastpos = 0;
      for (int i = 0; i < kWaves; ++i) {
        const float m = unpack_lo(p2[(int64_t)oc * kWaves + i]);
        if (m > 0.f) lastpos = i;
        if (os < 0 && run + m > tl) { os = i; seg_start = run; }
        run += m;
      }
      if (os < 0) os = lastpos;
    }
    seg_values(os, v);
    const int loc = wave_inverse_cdf<NV, PV>(v, tl - seg_start);
    if (loc >= 0) token = (int)((obeg + (int64_t)os * kSegVec) * PV + loc);
  }

  // clear this row's records and pass-2 words for the next call (the wave has read
  // them all): a call leaves every workspace word it wrote at zero
  for (int cc = lane; cc < C; cc += 64) {
    rec_store(rs, cc * 24, 0ull);
    rec_store(rs, cc * 24 + 8, 0ull);
    rec_store(rs, cc * 24 + 16, 0ull);
  }
  for (int64_t i = lane; i < (int64_t)C * kWaves; i += 64) p2[i] = 0ull;

  if (lane == 0) {
    int status = 0;
    if (bad_p) status |= kRowBadTarget;
    if (bad_q) status |= kRowBadDraft;
    if (empty_res) status |= kRowResidualEmpty;
    int flag = 0;
    const float nan = __builtin_nanf("");
    if (pair) {
      const int y = a.tokens[b * G + k];
      if (y < 0 || y >= a.V) {
        status |= kRowBadToken;
      } else if (!bad) {
        const float ay = load_one<DT>(trow, y), by = load_one<DT>(drow, y);
        const float d = __builtin_fmaf(ay, kLog2e, -lse2_p) - __builtin_fmaf(by, kLog2e, -lse2_q);
        if (d == d) flag = u < fminf(1.f, fast_exp2(d)) ? 1 : 0;
      }
      a.accept[b * G + k] = (uint8_t)flag;
      if (a.overlap) a.overlap[b * G + k] = bad ? nan : alpha;
      if (a.tv) a.tv[b * G + k] = bad ? nan : r_tot;
    }
    if (a.entropy) a.entropy[g] = bad_p ? nan : kLn2 * (fast_log2(st.p.z) - st.p.y / st.p.z);
    if (a.row_token) a.row_token[g] = token;
    if (a.row_status) a.row_status[g] = status;
    flag_sh[k] = flag;
    token_sh[k] = token;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < G && flag_sh[n] == 1) ++n;
    a.accepted_len[b] = n;
    a.next_token[b] = token_sh[n];
  }
}

// ---------------------------------------------------------------------------
template <int DT, int NV>
static hipError_t launch(const VerifyArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.sgroups * a.sp.nchunks * 8;
  hipLaunchKernelGGL((verify_main<DT, NV>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_finish<DT, NV>), dim3((unsigned)a.B), dim3(64 * (a.G + 1)), 0, stream, a);
  return hipGetLastError();
}

int verify_vec_per_thread(int dt) { return dt == kBF16 ? kVerifyNVBf16 : kVerifyNVF32; }

hipError_t launch_verify(const VerifyArgs& a, int dt, hipStream_t stream) {
  if (dt == kBF16) return launch<kBF16, kVerifyNVBf16>(a, stream);
  return launch<kF32, kVerifyNVF32>(a, stream);
}

hipError_t verify_occupancy(int dt, int* blocks_per_cu) {
  if (dt == kBF16)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, verify_main<kBF16, kVerifyNVBf16>, kBlock, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, verify_main<kF32, kVerifyNVF32>, kBlock, 0);
}

}  // namespace mtp
