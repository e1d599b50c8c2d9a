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
// group is split along the vocabulary into C chunks; C workgroups form a
// super-group that processes one group after another ("layers") in lockstep,
// chunk c of every group going to the same workgroup.  Per layer a workgroup
//   - unpacks its chunk (loaded during the previous layer) and immediately puts
//     the next layer's loads in flight,
//   - computes its chunk's log-sum-exp partials (both rows, and the entropy
//     moment of the target) and publishes them as one self-announcing record,
//   - polls the C records of its group (the only wait; it overlaps the prefetch)
//     and merges them in one fixed order,
//   - computes from registers the residual masses r = max(0, p - q) (the masses
//     of p for a bonus row) of its 4*NV segments (each 512 contiguous elements)
//     and stores them.
// All workgroups of a super-group sit on one XCD (workgroup i runs on XCD i mod 8)
// and are dispatched together, so a super-group only needs its own C workgroups
// to be co-resident.
//
// verify_finish runs one workgroup per sequence, one wave per row.  A wave merges
// the row's records again (lse, entropy), scans the chunk masses and then the
// segment masses of the owner chunk in vocabulary order, re-reads the single
// 512-element segment holding t = u' * sum r and finishes the inverse CDF in it.
// The row's acceptance flag needs p(y) and q(y) only.  The sequence's accepted
// length and next token are then formed in LDS.  It also clears the records, so
// the workspace is all zeros again when the call ends.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mtp {

// Per-thread log-sum-exp partial of NE logits; x is overwritten with
// 2^(x log2 e - ref).  With kEntropy the moment y is accumulated as well.
template <int NE, bool kEntropy>
__device__ __forceinline__ Lse thread_lse(float (&x)[NE]) {
  float m = x[0];
#pragma unroll
  for (int i = 1; i < NE; ++i) m = fmaxf(m, x[i]);
  const bool empty = !(m > kNegInf);          // all -inf (NaN-only also lands here)
  const float ref = empty ? 0.f : m * kLog2e;
  float z = 0.f, y = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const float t = __builtin_fmaf(x[i], kLog2e, -ref);
    const float e = fast_exp2(t);
    z += e;
    if constexpr (kEntropy) y = __builtin_fmaf(e, fmaxf(t, -300.f), y);
    x[i] = e;
  }
  if (empty && z == 0.f) return lse_empty();  // NaN inputs keep z = NaN
  return Lse{ref, z, y};
}

// max(0, p - q) with p = ea * sa and q = eb * sb, without FMA contraction.
__device__ __forceinline__ float residual_of(float ea, float sa, float eb, float sb) {
#pragma clang fp contract(off)
  const float p = ea * sa, q = eb * sb;
  return fmaxf(p - q, 0.f);
}

// Chunk record of pass 1 (three words): (ref_p, z_p), (ref_q, z_q), (y_p, 1).
__device__ __forceinline__ void put_p1(uint64_t* rec, const Lse& p, const Lse& q) {
  put_word(rec + 0, pack2(p.ref, mark(p.z)));
  put_word(rec + 1, pack2(q.ref, mark(q.z)));
  put_word(rec + 2, pack2(p.y, 1.f));
}

__device__ __forceinline__ Lse rec_p(const uint64_t (&w)[3]) {
  return Lse{unpack_lo(w[0]), unmark(unpack_hi(w[0])), unpack_lo(w[2])};
}
__device__ __forceinline__ Lse rec_q(const uint64_t (&w)[3]) {
  return Lse{unpack_lo(w[1]), unmark(unpack_hi(w[1])), 0.f};
}

struct RowLse {
  float lse2_p, lse2_q;
};

// Wave 0 polls the C pass-1 records of the group and merges them in one fixed
// order; log2-sum-exp of both rows is broadcast through LDS.
__device__ __forceinline__ RowLse merge_group(const uint64_t* p1, int C, bool pair, float* lds, uint32_t* err) {
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    Lse ap = lse_empty(), aq = lse_empty();
    for (int c0 = 0; c0 < C; c0 += 64) {
      uint64_t w[3];
      wave_poll<3>(p1, c0, C, w, err);
      if (c0 + lane < C) {
        ap = lse_merge(ap, rec_p(w));
        if (pair) aq = lse_merge(aq, rec_q(w));
      }
    }
    ap = wave_lse(ap);
    aq = wave_lse(aq);
    if (lane == 0) {
      lds[0] = lse_log2(ap);
      lds[1] = pair ? lse_log2(aq) : 0.f;
    }
  }
  __syncthreads();
  RowLse r{lds[0], lds[1]};
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
template <int DT, int NV>
__global__ __launch_bounds__(kBlock, kVerifyBlocksPerCU) void verify_main(VerifyArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NE = NV * PV;
  constexpr int NSEG = NV * kWaves;
  const int C = a.sp.nchunks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int sg = slot / C, c = slot - sg * C;
  const int G = a.G, G1 = G + 1;
  // layer i of this super-group handles group (sg + i * S) * 8 + xcd
  int nl = 0;
  while (nl < a.layers && (int64_t)(sg + nl * a.sgroups) * 8 + xcd < a.ngroups) ++nl;
  if (nl == 0) return;

  __shared__ float lds[3 * kWaves * 2];
  const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
  const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // the rows of group g: target (b, k) and, for k < gamma, draft (b, k)
  auto trow_of = [&](int g) {
    return reinterpret_cast<const char*>(a.target) + (int64_t)g * a.t_stride * Elem<DT>::kBytes;
  };
  auto drow_of = [&](int g) {
    const int b = g / G1, k = g - b * G1;
    return reinterpret_cast<const char*>(a.draft) + (int64_t)(b * G + (k < G ? k : 0)) * a.d_stride * Elem<DT>::kBytes;
  };
  auto is_pair = [&](int g) { return g % G1 < G; };
  auto issue = [&](RawChunk<NV, 2>& raw, int g) {
    const char* const rows[2] = {trow_of(g), drow_of(g)};
    issue_rows<DT, NV, 2>(raw, rows, vbeg, a.sp, is_pair(g) ? 2 : 1);
  };

  RawChunk<NV, 2> raw;
  issue(raw, sg * 8 + xcd);

  for (int i = 0; i < nl; ++i) {
    const int g = (sg + i * a.sgroups) * 8 + xcd;
    const bool pair = is_pair(g);
    float x[2][NE];
    {
      const char* const rows[2] = {trow_of(g), drow_of(g)};
      unpack_rows<DT, NV, 2>(raw, rows, vbeg, vend, a.sp, a.V, x, pair ? 2 : 1);
    }
    if (i + 1 < nl) issue(raw, (sg + (i + 1) * a.sgroups) * 8 + xcd);   // prefetch the next layer

    // ---- pass 1: chunk log-sum-exp partials, published as one record -------
    Lse parts[2] = {thread_lse<NE, true>(x[0]), lse_empty()};
    const float ref_a = parts[0].ref;
    float ref_b = 0.f;
    if (pair) {
      parts[1] = thread_lse<NE, false>(x[1]);
      ref_b = parts[1].ref;
    }
    block_lse<2>(parts, lds);
    uint64_t* p1 = a.part1 + (int64_t)g * C * 3;
    if (threadIdx.x == 0) put_p1(p1 + (int64_t)c * 3, parts[0], parts[1]);
    const RowLse L = merge_group(p1, C, pair, lds, a.err);

    // ---- pass 2: segment masses from registers -------------------------------
    const float sa = fast_exp2(ref_a - L.lse2_p);
    const float sb = pair ? fast_exp2(ref_b - L.lse2_q) : 0.f;
    float segm[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        const int idx = j * PV + e;
        acc += pair ? residual_of(x[0][idx], sa, x[1][idx], sb) : x[0][idx] * sa;
      }
      segm[j] = wave_sum(acc);
    }
    if (lane == 0) {
      float* seg = a.seg + ((int64_t)g * C + c) * NSEG;
#pragma unroll
      for (int j = 0; j < NV; ++j) st_coherent(seg + j * kWaves + wave, segm[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// verify_finish: one workgroup per sequence, wave k handles row (b, k).

// Inverse CDF of one segment held by a wave (PV values per lane, vocabulary order
// lane-major): smallest index whose running mass exceeds t; if none, the last
// index with positive mass; -1 if the segment has no mass.
template <int PV>
__device__ __forceinline__ int wave_inverse_cdf(const float (&v)[PV], float t) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < PV; ++e) s += v[e];
  float incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  const float ex = __shfl_up(incl, 1, 64);
  float cum = lane == 0 ? 0.f : ex;
  int best = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int e = 0; e < PV; ++e) {
    if (v[e] > 0.f) {
      cum += v[e];
      const int idx = lane * PV + e;
      if (best == 0x7fffffff && cum > t) best = idx;
      lastpos = idx;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    best = min(best, __shfl_xor(best, o, 64));
    lastpos = max(lastpos, __shfl_xor(lastpos, o, 64));
  }
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
  constexpr int NSEG = NV * kWaves;
  const int C = a.sp.nchunks;
  const int G = a.G, G1 = G + 1;
  const int b = blockIdx.x;
  const int k = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = b * G1 + k;
  const bool pair = k < G;
  __shared__ int flag_sh[kMaxRowsPerSeq], token_sh[kMaxRowsPerSeq];

  const char* trow = reinterpret_cast<const char*>(a.target) + (int64_t)g * a.t_stride * Elem<DT>::kBytes;
  const char* drow = reinterpret_cast<const char*>(a.draft) + (int64_t)(b * G + (pair ? k : 0)) * a.d_stride * Elem<DT>::kBytes;
  uint64_t* p1 = a.part1 + (int64_t)g * C * 3;
  const float* seg = a.seg + (int64_t)g * C * NSEG;

  // ---- row statistics from the pass-1 records ---------------------------------
  Lse ap = lse_empty(), aq = lse_empty();
  for (int c = lane; c < C; c += 64) {
    const uint64_t w[3] = {get_word(p1 + (int64_t)c * 3), get_word(p1 + (int64_t)c * 3 + 1),
                           get_word(p1 + (int64_t)c * 3 + 2)};
    ap = lse_merge(ap, rec_p(w));
    if (pair) aq = lse_merge(aq, rec_q(w));
  }
  ap = wave_lse(ap);
  aq = wave_lse(aq);
  const float lse2_p = lse_log2(ap);
  const float lse2_q = pair ? lse_log2(aq) : 0.f;
  const bool bad_p = !(__builtin_isfinite(lse2_p));
  const bool bad_q = pair && !(__builtin_isfinite(lse2_q));
  const bool bad = bad_p || bad_q;
  float u, up;
  row_uniforms(a.seed, a.offset, (uint64_t)g, &u, &up);

  auto pmass = [&](int c) {   // mass of p in chunk c, from its record
    const uint64_t w = get_word(p1 + (int64_t)c * 3);
    const float z = unmark(unpack_hi(w));
    return z > 0.f ? z * fast_exp2(unpack_lo(w) - lse2_p) : 0.f;
  };
  auto chunk_seg_mass = [&](int c) {
    const float* s = seg + (int64_t)c * NSEG;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < NSEG; ++i) m += ld_coherent(s + i);
    return m;
  };

  float alpha = 0.f;
  bool empty_res = false;
  Scan sc{0.f, 0, 0.f};
  if (!bad) {
    sc = wave_scan_owner(C, up, chunk_seg_mass);
    if (pair) {
      float pm = 0.f;
      for (int c = lane; c < C; c += 64) pm += pmass(c);
      alpha = wave_sum(pm) - sc.total;
      if (!(sc.total > 0.f)) {   // the residual has no mass: sample from p
        empty_res = true;
        sc = wave_scan_owner(C, up, pmass);
      }
    }
  }
  const float r_tot = pair && !empty_res ? sc.total : 0.f;

  // ---- owner segment inside the owner chunk, then the inverse CDF in it ------
  int token = -1;
  if (!bad) {
    const int oc = sc.owner;
    const int64_t obeg = (int64_t)oc * a.sp.vec_per_chunk;
    const int64_t oend = min(obeg + a.sp.vec_per_chunk, a.sp.nvec);
    // this lane's values in segment s (p, or max(0, p - q) for a non-empty residual)
    auto seg_values = [&](int s, float (&v)[PV]) {
      const int j = s / kWaves, w = s - j * kWaves;
      const int64_t vi = obeg + (int64_t)j * kBlock + w * 64 + lane;
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        const int64_t idx = vi * PV + e;
        float xa = kNegInf, xb = kNegInf;
        if (vi < oend && idx < a.V) {
          xa = load_one<DT>(trow, idx);
          if (pair && !empty_res) xb = load_one<DT>(drow, idx);
        }
        const float p = fast_exp2(__builtin_fmaf(xa, kLog2e, -lse2_p));
        if (pair && !empty_res) {
          const float q = fast_exp2(__builtin_fmaf(xb, kLog2e, -lse2_q));
          v[e] = fmaxf(p - q, 0.f);
        } else {
          v[e] = p;
        }
      }
    };
    const float tl = up * sc.total - sc.start;
    int os = -1;
    float seg_start = kNegInf;
    if (empty_res) {
      // segment masses of p are not recorded for a pair row: measure them (rare)
      float run = 0.f;
      for (int s = 0; s < NSEG && os < 0; ++s) {
        float v[PV];
        seg_values(s, v);
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < PV; ++e) m += v[e];
        m = wave_sum(m);
        if (run + m > tl) { os = s; seg_start = run; }
        run += m;
      }
      if (os < 0) os = NSEG - 1;
    } else {
      const float* s = seg + (int64_t)oc * NSEG;
      float run = 0.f;
      int lastpos = 0;
      for (int i = 0; i < NSEG; ++i) {
        const float m = ld_coherent(s + i);
        if (m > 0.f) lastpos = i;
        if (os < 0 && run + m > tl) { os = i; seg_start = run; }
        run += m;
      }
      if (os < 0) os = lastpos;
    }
    float v[PV];
    seg_values(os, v);
    const int loc = wave_inverse_cdf<PV>(v, tl - seg_start);
    if (loc >= 0) {
      const int j = os / kWaves, w = os - j * kWaves;
      token = (int)((obeg + (int64_t)j * kBlock + w * 64) * PV + loc);
    }
  }

  // clear this row's records and segment masses for the next call (the wave has
  // read them all): a call leaves every workspace word it wrote at zero
  for (int c = lane; c < C; c += 64) {
    put_word(p1 + (int64_t)c * 3, 0ull);
    put_word(p1 + (int64_t)c * 3 + 1, 0ull);
    put_word(p1 + (int64_t)c * 3 + 2, 0ull);
  }
  for (int64_t i = lane; i < (int64_t)C * NSEG; i += 64) st_coherent(const_cast<float*>(seg) + i, 0.f);

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
    if (a.entropy) a.entropy[g] = bad_p ? nan : kLn2 * (fast_log2(ap.z) - ap.y / ap.z);
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
