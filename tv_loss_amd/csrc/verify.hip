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
// Layout of the work.  A "group" is one row of one sequence: (target row, draft
// row) for k < gamma, or the bonus target row alone.  Each group is split along
// the vocabulary into C chunks, one workgroup each; a chunk is read from HBM once
// into registers.  The workgroups of a group form a cluster (all on one XCD:
// workgroup i runs on XCD i mod 8) that exchanges partials through the workspace
// with device-coherent loads and stores:
//   1. every workgroup publishes its chunk's log-sum-exp partials (both rows, and
//      the entropy moment of the target) and waits for the cluster -- the only
//      wait; each then merges all C partials in one fixed order -> lse, H;
//   2. pair groups: every workgroup publishes its chunk's overlap and residual
//      mass from registers and leaves, except the last to publish, which scans
//      the residual masses in chunk order, finds the chunk holding
//      t = u' * sum r, and finishes the inverse CDF inside it (from its own
//      registers, or by reading that chunk again);
//      bonus groups: the masses of p per chunk come from step 1, so the chunk
//      holding t finishes the inverse CDF from its registers;
//   3. the row's finisher writes its outputs; the last row of a sequence to
//      finish writes the accepted length and the next token.
// The last user of every counter, partial and record slot clears it, so the
// workspace is all zeros again when the kernel ends.
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

// max(0, p - q) as p - min(p, q), with p = e_a * s_a and q = e_b * s_b.  FMA
// contraction is off so that every evaluation (the pass-2 sums and the inverse
// CDF, possibly in another workgroup) produces the same bits.
__device__ __forceinline__ void pq_residual(float ea, float sa, float eb, float sb, float* p, float* mn,
                                            float* r) {
#pragma clang fp contract(off)
  const float pp = ea * sa, qq = eb * sb;
  const float m = fminf(pp, qq);
  *p = pp;
  *mn = m;
  *r = pp - m;
}

// Prefix structure over per-chunk masses: lane l owns chunks [l*K, l*K + K).
struct ChunkScan {
  float total;     // sum of all masses
  int owner;       // chunk holding t
  float start;     // mass before the owner chunk
};

// Every lane computes the same result.  mass(c) supplies chunk c's mass.
template <typename MassFn>
__device__ __forceinline__ ChunkScan scan_chunks(int C, float u_prime, MassFn mass) {
  const int lane = threadIdx.x & 63;
  const int K = (C + 63) / 64;
  const int c0 = lane * K, c1 = min(C, c0 + K);
  float block = 0.f;
  int last_pos = -1;
  for (int c = c0; c < c1; ++c) {
    const float m = mass(c);
    block += m;
    if (m > 0.f) last_pos = c;
  }
  // inclusive scan over lanes (Hillis-Steele), deterministic
  float incl = block;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  const float excl_lane = __shfl_up(incl, 1, 64);
  const float excl = lane == 0 ? 0.f : excl_lane;
  ChunkScan r;
  r.total = __shfl(incl, 63, 64);
  const float t = u_prime * r.total;
  const uint64_t hit = __ballot(c0 < c1 && incl > t);
  if (hit != 0ull && r.total > 0.f) {
    const int l = __builtin_ctzll(hit);
    // walk the winning lane's chunks, accumulating in the same order
    const float lane_start = __shfl(excl, l, 64);
    float run = lane_start;
    int owner = -1;
    float start = lane_start;
    const int a0 = l * K, a1 = min(C, a0 + K);
    for (int c = a0; c < a1; ++c) {
      const float m = mass(c);
      const float nxt = run + m;
      if (owner < 0 && nxt > t) { owner = c; start = run; }
      run = nxt;
    }
    r.owner = owner;
    r.start = start;
    if (owner < 0) {   // rounding: the lane's last chunk with mass, from its end
      int lastc = a0;
      for (int c = a0; c < a1; ++c)
        if (mass(c) > 0.f) lastc = c;
      r.owner = lastc;
      r.start = kNegInf;
    }
  } else {
    // rounding left t past every boundary (or no mass): last chunk with mass
    const uint64_t pos = __ballot(last_pos >= 0);
    if (pos != 0ull) {
      const int l = 63 - __builtin_clzll(pos);
      r.owner = __shfl(last_pos, l, 64);
    } else {
      r.owner = 0;
    }
    r.start = kNegInf;   // t_local = +inf: the owner takes its last positive element
  }
  return r;
}

// Inverse CDF inside the owner chunk: smallest local index whose running mass
// exceeds t_local; if none, the last index with positive mass; -1 if no mass.
// v holds this thread's NV*PV masses in (j, e) order.
template <int NV, int PV>
__device__ __forceinline__ int chunk_inverse_cdf(const float (&v)[NV * PV], float t_local, float* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float s[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < PV; ++e) acc += v[j * PV + e];
    s[j] = acc;
  }
  // exclusive scan over threads, per iteration j
  float incl[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    incl[j] = s[j];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float n = __shfl_up(incl[j], o, 64);
      if (lane >= o) incl[j] += n;
    }
  }
  __syncthreads();
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < NV; ++j) lds[j * kWaves + wave] = incl[j];
  }
  __syncthreads();
  float off = 0.f;
  int best = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const float* wt = lds + j * kWaves;
    float woff = 0.f;
    for (int w = 0; w < wave; ++w) woff += wt[w];
    const float ex_lane = __shfl_up(incl[j], 1, 64);
    const float start = off + (woff + (lane == 0 ? 0.f : ex_lane));
    float cum = start;
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      const float val = v[j * PV + e];
      if (val > 0.f) {
        cum += val;
        const int idx = (j * kBlock + tid) * PV + e;
        if (best == 0x7fffffff && cum > t_local) best = idx;
        lastpos = idx;
      }
    }
    off += (wt[0] + wt[1]) + (wt[2] + wt[3]);
  }
  // block min of best, block max of lastpos
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    best = min(best, __shfl_xor(best, o, 64));
    lastpos = max(lastpos, __shfl_xor(lastpos, o, 64));
  }
  __syncthreads();
  int* li = reinterpret_cast<int*>(lds);
  if (lane == 0) { li[wave] = best; li[kWaves + wave] = lastpos; }
  __syncthreads();
  best = min(min(li[0], li[1]), min(li[2], li[3]));
  lastpos = max(max(li[4], li[5]), max(li[6], li[7]));
  return best != 0x7fffffff ? best : lastpos;
}

// Workspace record per row, read by the sequence finaliser.
struct RowRec { int flag; int token; };

// Row statistics every workgroup of a group derives from the chunk partials.
struct RowLse {
  Lse p, q;
  float lse2_p, lse2_q;
  bool bad_p, bad_q;
};

// Wave 0 merges the C chunk partials (coherent loads) in a fixed order; the
// result is broadcast through LDS.  Identical in every workgroup of the group.
__device__ __forceinline__ RowLse merge_group(const float* p1, int C, bool pair, float* lds) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    Lse ap = lse_empty(), aq = lse_empty();
    for (int c = lane; c < C; c += 64) {
      const float* q = p1 + (int64_t)c * 8;
      ap = lse_merge(ap, Lse{ld_coherent(q), ld_coherent(q + 1), ld_coherent(q + 2)});
      if (pair) aq = lse_merge(aq, Lse{ld_coherent(q + 3), ld_coherent(q + 4), 0.f});
    }
    ap = wave_lse(ap);
    aq = wave_lse(aq);
    if (lane == 0) {
      lds[0] = ap.ref; lds[1] = ap.z; lds[2] = ap.y;
      lds[3] = aq.ref; lds[4] = aq.z; lds[5] = aq.y;
    }
  }
  __syncthreads();
  RowLse r;
  r.p = Lse{lds[0], lds[1], lds[2]};
  r.q = Lse{lds[3], lds[4], lds[5]};
  __syncthreads();
  r.lse2_p = lse_log2(r.p);
  r.bad_p = !(__builtin_isfinite(r.lse2_p));
  r.lse2_q = pair ? lse_log2(r.q) : 0.f;
  r.bad_q = pair && !(__builtin_isfinite(r.lse2_q));
  return r;
}

// The sequence finaliser: every row's finisher records (flag, token) and arrives
// on the sequence counter; the last of the gamma+1 writes n_b and the next token,
// then clears the records and the counter.  Called by one thread.
__device__ __forceinline__ void finish_row(const VerifyArgs& a, int b, int g, int flag, int token) {
  const int G = a.G, G1 = G + 1;
  int* rec = a.rec;
  st_coherent(rec + 2 * g, flag);
  st_coherent(rec + 2 * g + 1, token);
  int* scnt = a.seq_cnt + (int64_t)b * kCounterStride;
  const int old = arrive(scnt);
  if (old == G) {
    int n = 0;
    while (n < G && ld_coherent(rec + 2 * (b * G1 + n)) == 1) ++n;
    a.accepted_len[b] = n;
    a.next_token[b] = ld_coherent(rec + 2 * (b * G1 + n) + 1);
    for (int k = 0; k < G1; ++k) {
      st_coherent(rec + 2 * (b * G1 + k), 0);
      st_coherent(rec + 2 * (b * G1 + k) + 1, 0);
    }
    reset_counter(scnt);
  }
}

template <int DT, int NV>
__global__ __launch_bounds__(kBlock) void verify_kernel(VerifyArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NE = NV * PV;
  const int C = a.sp.nchunks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int lg = slot / C, c = slot - lg * C;
  const int g = lg * 8 + xcd;
  if (g >= a.ngroups) return;
  const int G = a.G, G1 = G + 1;
  const int b = g / G1, k = g - b * G1;
  const bool pair = k < G;

  __shared__ float lds[64];
  __shared__ int flag_sh;

  float xa[NE], xb[NE];
  const char* trow = reinterpret_cast<const char*>(a.target) + (int64_t)g * a.t_stride * Elem<DT>::kBytes;
  const char* drow = reinterpret_cast<const char*>(a.draft) + (int64_t)(b * G + k) * a.d_stride * Elem<DT>::kBytes;
  {
    const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
    const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);
    load_chunk<DT, NV>(trow, vbeg, vend, a.sp, a.V, xa);
    if (pair) load_chunk<DT, NV>(drow, vbeg, vend, a.sp, a.V, xb);
  }

  // ---- pass 1: chunk log-sum-exp partials ----------------------------------
  Lse parts[2] = {thread_lse<NE, true>(xa), lse_empty()};
  const float ref_a = parts[0].ref;
  float ref_b = 0.f;
  if (pair) {
    parts[1] = thread_lse<NE, false>(xb);
    ref_b = parts[1].ref;
  }
  block_lse<2>(parts, lds);
  float* p1 = a.part1 + (int64_t)g * C * 8;
  float* p2 = a.part2 + (int64_t)g * C * 2;
  int* cnt = a.grp_cnt + (int64_t)g * kCounterStride;
  if (threadIdx.x == 0) {
    float* mine = p1 + (int64_t)c * 8;
    st_coherent(mine + 0, parts[0].ref); st_coherent(mine + 1, parts[0].z); st_coherent(mine + 2, parts[0].y);
    st_coherent(mine + 3, parts[1].ref); st_coherent(mine + 4, parts[1].z);
    arrive(cnt);
  }
  block_wait(cnt, C, a.err);
  const RowLse L = merge_group(p1, C, pair, lds);
  const bool bad = L.bad_p || (pair && L.bad_q);
  const float sa = fast_exp2(ref_a - L.lse2_p);            // p_i = xa[i] * sa
  const float sb = pair ? fast_exp2(ref_b - L.lse2_q) : 0.f;
  float u, up;
  row_uniforms(a.seed, a.offset, (uint64_t)g, &u, &up);
  auto pmass = [&](int cc) {                                // target mass of chunk cc
    const float* q = p1 + (int64_t)cc * 8;
    const float z = ld_coherent(q + 1);
    return z > 0.f ? z * fast_exp2(ld_coherent(q) - L.lse2_p) : 0.f;
  };

  ChunkScan sc;
  float alpha_tot = 0.f, r_tot = 0.f;
  bool empty_res = false;
  if (pair) {
    // ---- pass 2: overlap and residual mass from registers -----------------
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      float p, mn, r;
      pq_residual(xa[i], sa, xb[i], sb, &p, &mn, &r);
      acc[0] += mn;
      acc[1] += r;
    }
    block_sum<2>(acc, lds);
    if (threadIdx.x == 0) {
      st_coherent(p2 + 2 * c, acc[0]);
      st_coherent(p2 + 2 * c + 1, acc[1]);
      flag_sh = arrive(cnt) == 2 * C - 1;
    }
    __syncthreads();
    if (!flag_sh) return;
    // ---- the last workgroup of the group finishes the row ------------------
    const int lane = threadIdx.x & 63;
    float al = 0.f;
    for (int cc = lane; cc < C; cc += 64) al += ld_coherent(p2 + 2 * cc);
    alpha_tot = wave_sum(al);
    sc = scan_chunks(C, up, [&](int cc) { return ld_coherent(p2 + 2 * cc + 1); });
    r_tot = sc.total;
    if (!(r_tot > 0.f) && !bad) {
      empty_res = true;
      sc = scan_chunks(C, up, pmass);
    }
  } else {
    sc = scan_chunks(C, up, pmass);
    // departure: the last workgroup to leave clears the group's partials
    if (threadIdx.x == 0) flag_sh = arrive(cnt) == 2 * C - 1;
    __syncthreads();
    if (flag_sh) {
      block_zero(p1, (int64_t)C * 8);
      if (threadIdx.x == 0) reset_counter(cnt);
    }
    if (bad) sc.owner = 0;
    if (c != sc.owner) return;
  }
  if (bad) sc.owner = 0;

  // ---- inverse CDF inside the owner chunk -----------------------------------
  int token = -1;
  if (!bad) {
    const int oc = sc.owner;
    const int64_t obeg = (int64_t)oc * a.sp.vec_per_chunk;
    if (pair && oc != c) {
      // the owner chunk is another workgroup's: read it again and recompute the
      // same per-thread values that workgroup summed
      const int64_t oend = min(obeg + a.sp.vec_per_chunk, a.sp.nvec);
      load_chunk<DT, NV>(trow, obeg, oend, a.sp, a.V, xa);
      load_chunk<DT, NV>(drow, obeg, oend, a.sp, a.V, xb);
      const Lse ta = thread_lse<NE, true>(xa);
      const Lse tb = thread_lse<NE, false>(xb);
      const float sa2 = fast_exp2(ta.ref - L.lse2_p), sb2 = fast_exp2(tb.ref - L.lse2_q);
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        float p, mn, r;
        pq_residual(xa[i], sa2, xb[i], sb2, &p, &mn, &r);
        xa[i] = empty_res ? p : r;
      }
    } else if (pair) {
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        float p, mn, r;
        pq_residual(xa[i], sa, xb[i], sb, &p, &mn, &r);
        xa[i] = empty_res ? p : r;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NE; ++i) xa[i] *= sa;
    }
    const float t_local = up * sc.total - sc.start;
    const int loc = chunk_inverse_cdf<NV, PV>(xa, t_local, lds);
    token = loc >= 0 ? (int)(obeg * PV + loc) : -1;
  }
  if (pair) {   // the finishing workgroup clears the group's partials
    block_zero(p1, (int64_t)C * 8);
    block_zero(p2, (int64_t)C * 2);
  }
  if (threadIdx.x != 0) return;
  if (pair) reset_counter(cnt);

  int status = 0;
  if (L.bad_p) status |= kRowBadTarget;
  if (pair && L.bad_q) status |= kRowBadDraft;
  if (empty_res) status |= kRowResidualEmpty;
  int flag = 0;
  const float nan = __builtin_nanf("");
  if (pair) {
    const int y = a.tokens[b * G + k];
    if (y < 0 || y >= a.V) {
      status |= kRowBadToken;
    } else if (!bad) {
      const float ay = load_one<DT>(trow, y), by = load_one<DT>(drow, y);
      const float d = __builtin_fmaf(ay, kLog2e, -L.lse2_p) - __builtin_fmaf(by, kLog2e, -L.lse2_q);
      if (d == d) flag = u < fminf(1.f, fast_exp2(d)) ? 1 : 0;
    }
    a.accept[b * G + k] = (uint8_t)flag;
    if (a.overlap) a.overlap[b * G + k] = bad ? nan : alpha_tot;
    if (a.tv) a.tv[b * G + k] = bad ? nan : r_tot;
  }
  if (a.entropy) a.entropy[g] = L.bad_p ? nan : kLn2 * (fast_log2(L.p.z) - L.p.y / L.p.z);
  if (a.row_token) a.row_token[g] = token;
  if (a.row_status) a.row_status[g] = status;
  finish_row(a, b, g, flag, token);
}

template <int DT, int NV>
static hipError_t launch(const VerifyArgs& a, hipStream_t stream) {
  const int C = a.sp.nchunks;
  const int64_t per_xcd = (a.ngroups + 7) / 8;
  const int64_t grid = per_xcd * C * 8;
  hipLaunchKernelGGL((verify_kernel<DT, NV>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

int verify_vec_per_thread(int dt) { return dt == kBF16 ? kVerifyNVBf16 : kVerifyNVF32; }

hipError_t launch_verify(const VerifyArgs& a, int dt, hipStream_t stream) {
  if (dt == kBF16) return launch<kBF16, kVerifyNVBf16>(a, stream);
  return launch<kF32, kVerifyNVF32>(a, stream);
}

hipError_t verify_occupancy(int dt, int* blocks_per_cu) {
  if (dt == kBF16)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, verify_kernel<kBF16, kVerifyNVBf16>, kBlock, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, verify_kernel<kF32, kVerifyNVF32>, kBlock, 0);
}

}  // namespace mtp
