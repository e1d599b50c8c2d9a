// End-to-end multi-step TV loss: forward and backward.
//
// What is computed (Bebop pages: paperlayer.ai Sec. 4 "End-to-end TV loss",
// App. A "Derivation of TV Loss Gradient", App. F "Fused TV Loss Kernel";
// rainbus "Method steps" and "Technical novelty"):
//   alpha_{t,k} = clamp(sum_v min(p_v, q_v), 0, 1),  S_{t,k} = sum_v 1[q_v <= p_v] q_v,
//   l_t = -sum_{k=1..gamma} prod_{j<=k} alpha_{t,j},  L = (1/T) sum_t l_t,
// and, with p detached and an upstream scalar g,
//   dL/dz_{t,j,v} = w_{t,j} q_v (1[q_v <= p_v] - S_{t,j}),
//   w_{t,j} = -(g/T) sum_{k>=j} prod_{i<=k, i!=j} alpha_{t,i}.
//
// Forward: three streaming kernels, no cross-workgroup waits.  tv_fwd_lse reads
// chunk c of every row of position t (one workgroup per (t, c)) and writes the
// chunk's log-sum-exp partial of each row.  tv_fwd_stats merges the partials of its
// position's rows (every workgroup of the position derives the same bits), reads
// the chunk again and writes the chunk's overlap and S partials of every head; the
// indicator and the minimum are taken on log-probabilities, min(p, q) =
// 2^min(log2 p, log2 q), so one exponential per head and element suffices.
// tv_fwd_finish (one wave per position) sums the partials in a fixed order and
// writes l_t and the saved statistics; tv_fwd_mean writes the mean.  Every logit is
// read twice; the partials take a few bytes per chunk.
// Backward: pure streaming; each workgroup reads one chunk of the target and draft
// rows of one position plus the saved statistics, and writes the gradient chunk.
// The indicator is evaluated on logits, z_v - a_v <= lse_q - lse_p, so no
// exponential of the target is needed.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mtp {

// Vectors per thread and row for the forward kernels: 16 bf16 or 8 fp32 values
// per row and thread for up to four rows, fewer vectors when there are more rows
// (at least one).
template <int NR>
constexpr int fwd_nv(int per_vec) {
  const int nv = (per_vec == 8 ? 64 : 32) / (NR * per_vec);
  return nv < 1 ? 1 : nv;
}

template <int G, bool SHARED>
struct FwdShape {
  static constexpr int NT = SHARED ? 1 : G;   // target rows
  static constexpr int NR = NT + G;           // target rows, then the G draft rows
};

// Row bases of position t: targets first, then drafts.
template <int DT, int NT, int G>
__device__ __forceinline__ void fwd_rows(const TvArgs& a, int t, const char* (&rows)[NT + G]) {
  const char* tb = reinterpret_cast<const char*>(a.target);
  const char* db = reinterpret_cast<const char*>(a.draft);
#pragma unroll
  for (int r = 0; r < NT; ++r) rows[r] = tb + ((int64_t)t * a.t_pos + (int64_t)r * a.t_head) * Elem<DT>::kBytes;
#pragma unroll
  for (int k = 0; k < G; ++k) rows[NT + k] = db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes;
}

// This workgroup's chunk of every row of position t, widened to fp32 (-inf outside
// the chunk and the row).  Each wave owns a contiguous segment of NV * 64 vectors.
template <int DT, int NV, int NR>
__device__ __forceinline__ void fwd_load(const TvArgs& a, const char* const (&rows)[NR], int c,
                                         float (&x)[NR][NV * Elem<DT>::kPerVec]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int vpc = (int)a.sp.vec_per_chunk, nvec = (int)a.sp.nvec, nfull = (int)a.sp.nvec_full;
  const int vbeg = c * vpc;
  const int vend = min(vbeg + vpc, nvec);
  const int s0 = vbeg + wave * NV * 64;
  const int lim = min(vend, nfull);
  RawChunk<NV, NR> raw;
  issue_seg<DT, NV, NR>(raw, rows, s0 + lane, nfull - 1);
  unpack_seg<DT, NV, NR>(raw, rows, s0 + lane, s0 + NV * 64 <= lim, lim, nfull, vend, (int)a.V, x);
}

// Pass 1: chunk log-sum-exp partials of every row, part1[t][c][r] = (ref, z).
template <int DT, int G, bool SHARED>
__global__ __launch_bounds__(kBlock) void tv_fwd_lse(TvArgs a) {
  constexpr int NR = FwdShape<G, SHARED>::NR;
  constexpr int NV = fwd_nv<NR>(Elem<DT>::kPerVec);
  constexpr int NE = NV * Elem<DT>::kPerVec;
  const int C = a.sp.nchunks;
  const int t = blockIdx.x / C, c = blockIdx.x - t * C;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  __shared__ float part_sh[NR][kWaves * 3];
  const char* rows[NR];
  fwd_rows<DT, FwdShape<G, SHARED>::NT, G>(a, t, rows);
  float x[NR][NE];
  fwd_load<DT, NV, NR>(a, rows, c, x);
  Lse pt[NR];
  wave_pass1<NE, NR, 0>(x, pt);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      part_sh[r][wave * 3 + 0] = pt[r].ref;
      part_sh[r][wave * 3 + 1] = pt[r].z;
      part_sh[r][wave * 3 + 2] = 0.f;
    }
  }
  __syncthreads();
  if (threadIdx.x < NR) {
    const Lse m = merge_lds<kWaves, false>(part_sh[threadIdx.x]);
    reinterpret_cast<float2*>(a.part1)[((int64_t)t * C + c) * NR + threadIdx.x] = make_float2(m.ref, m.z);
  }
}

// log2-sum-exp of row r of position t from its C chunk partials: lane l merges
// chunks l, l + 64, ... in order, then the wave merges the lanes.  tv_fwd_stats and
// tv_fwd_finish both use it, so both derive the same bits.
template <int NR>
__device__ __forceinline__ float fwd_row_lse2(const TvArgs& a, int t, int r) {
  const int C = a.sp.nchunks;
  const int lane = threadIdx.x & 63;
  const float2* p1 = reinterpret_cast<const float2*>(a.part1) + (int64_t)t * C * NR + r;
  Lse acc[1] = {lse_empty()};
  for (int c = lane; c < C; c += 64) {
    const float2 w = p1[(int64_t)c * NR];
    const Lse v{w.x, w.y, 0.f};
    acc[0] = c == lane ? v : lse_merge(acc[0], v);
  }
  wave_merge<1, 0>(acc);
  return lse_log2(acc[0]);
}

// Pass 2: chunk partials of the overlap sum_v min(p, q) and of S = sum_v 1[q <= p] q
// for every head, part2[t][c][2k] = overlap, [2k + 1] = S.
template <int DT, int G, bool SHARED>
__global__ __launch_bounds__(kBlock) void tv_fwd_stats(TvArgs a) {
  constexpr int NT = FwdShape<G, SHARED>::NT;
  constexpr int NR = FwdShape<G, SHARED>::NR;
  constexpr int NV = fwd_nv<NR>(Elem<DT>::kPerVec);
  constexpr int NE = NV * Elem<DT>::kPerVec;
  const int C = a.sp.nchunks;
  const int t = blockIdx.x / C, c = blockIdx.x - t * C;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  __shared__ float lse_sh[NR];
  __shared__ float acc_sh[2 * G][kWaves];
  const char* rows[NR];
  fwd_rows<DT, NT, G>(a, t, rows);
  float x[NR][NE];
  fwd_load<DT, NV, NR>(a, rows, c, x);
  for (int r = wave; r < NR; r += kWaves) {
    const float l = fwd_row_lse2<NR>(a, t, r);
    if (lane == 0) lse_sh[r] = l;
  }
  __syncthreads();
  float al[G], sk[G];
#pragma unroll
  for (int k = 0; k < G; ++k) al[k] = sk[k] = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    float u[NT];
#pragma unroll
    for (int r = 0; r < NT; ++r) u[r] = __builtin_fmaf(x[r][i], kLog2e, -lse_sh[r]);   // log2 p
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float uk = u[SHARED ? 0 : k];
      const float v = __builtin_fmaf(x[NT + k][i], kLog2e, -lse_sh[NT + k]);        // log2 q
      // min(p, q) and 1[q <= p] q; a NaN log-probability (a row without a
      // normaliser) propagates into both sums
      const float m = fast_exp2(__builtin_elementwise_minimum(uk, v));
      al[k] += m;
      sk[k] += v > uk ? 0.f : m;
    }
  }
#pragma unroll
  for (int k = 0; k < G; ++k) {
    al[k] = wave_total(al[k]);
    sk[k] = wave_total(sk[k]);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < G; ++k) {
      acc_sh[2 * k][wave] = al[k];
      acc_sh[2 * k + 1][wave] = sk[k];
    }
  }
  __syncthreads();
  if (threadIdx.x < 2 * G) {
    const float* v = acc_sh[threadIdx.x];
    a.part2[((int64_t)t * C + c) * 2 * G + threadIdx.x] = (v[0] + v[1]) + (v[2] + v[3]);
  }
}

// One wave per position: row log-sum-exps, the overlap and S of every head, l_t and
// the saved statistics.  Clears the partials it read, so the workspace is all
// zeros again when the call ends.
constexpr int kFinishWaves = 4;

template <int G, bool SHARED>
__global__ __launch_bounds__(64 * kFinishWaves) void tv_fwd_finish(TvArgs a) {
  constexpr int NT = FwdShape<G, SHARED>::NT;
  constexpr int NR = FwdShape<G, SHARED>::NR;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kFinishWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int C = a.sp.nchunks;
  float lse2[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) lse2[r] = fwd_row_lse2<NR>(a, t, r);
  float* p2 = a.part2 + (int64_t)t * C * 2 * G;
  float tot[2 * G];
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) tot[k] = 0.f;
  for (int c = lane; c < C; c += 64) {
#pragma unroll
    for (int k = 0; k < 2 * G; ++k) tot[k] += p2[(int64_t)c * 2 * G + k];
  }
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) tot[k] = wave_total(tot[k]);
  // a call leaves every workspace word it wrote at zero
  float2* p1 = reinterpret_cast<float2*>(a.part1) + (int64_t)t * C * NR;
  for (int i = lane; i < C * NR; i += 64) p1[i] = make_float2(0.f, 0.f);
  for (int i = lane; i < C * 2 * G; i += 64) p2[i] = 0.f;
  if (lane == 0) {
    float prod = 1.f, l = 0.f;
    float* sv = a.saved + (int64_t)t * G * kTvSavedStride;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float ov = tot[2 * k];   // NaN (a row without a normaliser) stays NaN
      const float al = ov != ov ? ov : fminf(fmaxf(ov, 0.f), 1.f);
      prod *= al;
      l -= prod;
      sv[k * kTvSavedStride + 0] = lse2[SHARED ? 0 : k] * kLn2;
      sv[k * kTvSavedStride + 1] = lse2[NT + k] * kLn2;
      sv[k * kTvSavedStride + 2] = al;
      sv[k * kTvSavedStride + 3] = tot[2 * k + 1];
    }
    if (a.pos_loss) a.pos_loss[t] = l;
    a.pos_ws[t] = l;
  }
}

// The mean over positions, in one fixed order; clears the per-position losses.
__global__ __launch_bounds__(kBlock) void tv_fwd_mean(TvArgs a) {
  __shared__ float lds[kWaves];
  float sum[1] = {0.f};
  // eight loads in flight per step, added in the same order as one at a time
  int i = threadIdx.x;
  for (; i + 7 * kBlock < a.T; i += 8 * kBlock) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = a.pos_ws[i + j * kBlock];
#pragma unroll
    for (int j = 0; j < 8; ++j) sum[0] += v[j];
  }
  for (; i < a.T; i += kBlock) sum[0] += a.pos_ws[i];
  block_sum<1>(sum, lds);
  for (int i = threadIdx.x; i < a.T; i += kBlock) a.pos_ws[i] = 0.f;
  if (threadIdx.x == 0) a.loss[0] = sum[0] / (float)a.T;
}

// ---------------------------------------------------------------------------
// Single-read forward.  The two passes above read every logit twice; this path
// reads it once.  Super-groups of C workgroups, all resident at once, walk their
// positions t = sg, sg + S, ... in layers; workgroup c of a super-group takes chunk
// c of every row of each of its positions, and each wave owns a contiguous segment
// of the chunk.  Layer i:
//   * the records of position i - 2 (polled a layer ago) give each row's base-2
//     log-sum-exp; every wave forms the overlap and S partials of every head over
//     its segment from the e values it holds in LDS;
//   * the e values of position i - 1 move from registers to LDS;
//   * the chunk of position i is unpacked (its loads went out two layers ago), the
//     poll of position i - 1's records and the loads of position i + 2 go out;
//   * pass 1 of position i: every lane's sums of e against its wave's largest logit
//     go to LDS; wave r merges row r over the workgroup (lanes first, across the
//     waves, then one wave sum) and publishes it as one self-announcing record word;
//     the lanes' overlap and S partials of position i - 2 are added up the same way,
//     wave w taking the values w, w + 4, ...
// In a wave's own units p = sa e_p and q = sb e_q (e <= 1, taken against the wave's
// largest logit of the row).  For head k, with rho = sb / sa <= 1:
//   min(p, q) = sa min(e_p, rho e_q),  1[q <= p] q = sa 1[rho e_q <= e_p] rho e_q,
// and with rho > 1 the same in q's units (sb, e_q and e_p / rho), so no scale
// overflows.  tv_pipe_finish (one wave per position) merges the records in the
// order the poll used, sums the partials, writes the saved statistics and l_t, and
// clears what it read.  Record words: (ref, z with the sign bit set), never zero.
constexpr int kPipeFloats = 64;   // logits per thread and position (all rows) in flight

// Pass 1 of R rows with the sums left per lane: row r's reference is the wave's
// largest logit M (ref = M L rounded up, so e <= 1; -inf for a wave holding only
// -inf), x[r] is overwritten with e = 2^(x L - ref) and z[r] is this lane's sum of
// its e values.
template <int NE, int R>
__device__ __forceinline__ void lane_pass1(float (&x)[R][NE], float (&ref)[R], float (&z)[R], float L) {
  float M[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float m = x[r][0];
#pragma unroll
    for (int i = 1; i < NE; ++i) m = fmaximum(m, x[r][i]);
    M[r] = m;
  }
  wave_reduce<true, R>(M);
  float sh[R], z0[R], z1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    sh[r] = M[r] > kNegInf ? ref_up(M[r], L) : 0.f;   // 0 keeps -inf - sh = -inf
    z0[r] = z1[r] = -0.f;                       // -0 + e = e: the first addition folds away
  }
#pragma unroll
  for (int i = 0; i < NE; ++i) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float e = fast_exp2(__builtin_fmaf(x[r][i], L, -sh[r]));
      if (i & 1) z1[r] += e; else z0[r] += e;
      x[r][i] = e;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    z[r] = z0[r] + z1[r];
    ref[r] = M[r] > kNegInf ? sh[r] : kNegInf;
  }
}

template <int NR>
constexpr int pipe_nv(int per_vec) {
  const int nv = kPipeFloats / (NR * per_vec);
  return nv < 1 ? 1 : nv;
}

template <int G, bool SHARED>
constexpr bool pipe_fits() { return FwdShape<G, SHARED>::NR <= kTvPipeMaxRows; }

template <int DT, int G, bool SHARED>
__global__ __launch_bounds__(kBlock, 2) void tv_pipe_main(TvArgs a) {
  constexpr int NT = FwdShape<G, SHARED>::NT;
  constexpr int NR = FwdShape<G, SHARED>::NR;
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NV = pipe_nv<NR>(PV);
  constexpr int NE = NV * PV;
  constexpr int NQ = NE / 4;                       // 16-byte LDS slots per row and thread
  constexpr int kSegVec = NV * 64;
  constexpr int RW = (NR + kWaves - 1) / kWaves;   // rows whose records one wave polls / publishes
  constexpr int kSt = NR * 8;                      // record stride (bytes) per chunk
  const int C = a.sp.nchunks;
  const int slot = blockIdx.x;
  const int sg = slot / C, c = slot - sg * C;
  const int S = a.sgroups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  if (sg >= a.T) return;
  // positions t = sg + i S, or the contiguous range the host sized for this
  // super-group's dispatch round (round_split_base)
  int nl = (a.T - 1 - sg) / S + 1, base = -1;
  if (a.split.W > 0) {
    base = round_split_base(a.split, sg, S, C);
    nl = round_split_base(a.split, sg + 1, S, C) - base;
  }
  auto pos_of = [&](int i) { return base >= 0 ? base + i : sg + i * S; };
  auto rsrc_rec = [&](int t) { return rsrc_of(a.part1 + (int64_t)t * C * NR); };

  const int vpc = (int)a.sp.vec_per_chunk, nvec = (int)a.sp.nvec, nfull = (int)a.sp.nvec_full;
  const int vbeg = c * vpc;
  const int vend = min(vbeg + vpc, nvec);
  const int s0 = vbeg + wave * kSegVec;
  const int v0 = s0 + lane;
  const int lim = min(vend, nfull);
  const bool full = s0 + kSegVec <= lim;
  const int last = nfull - 1;
  const int tail = nfull;
  const int V = (int)a.V;
  const int row_bytes = (int)min(a.V * Elem<DT>::kBytes, (int64_t)0x7fffffff);

  constexpr int KW = (2 * G + kWaves - 1) / kWaves;   // pass-2 values each wave adds up
  __shared__ float4 held[NR][NQ][kBlock];      // e values of the position two layers back
  __shared__ float ref_sh[2][NR][kWaves];       // pass-1 wave references, by layer parity
  __shared__ float z_sh[2][NR][kBlock];         // pass-1 lane sums in their wave's units
  __shared__ float st_sh[2][NR][3];             // row normalisers 2^ref z of the position in pass 2: (ref, z, 1/z)
  __shared__ float red_sh[2 * G][kBlock];       // pass-2 lane partials (overlap, S per head)

  auto prefetch = [&](RawChunk<NV, NR>& rb, int t, bool live) {
    const char* rows[NR];
    fwd_rows<DT, NT, G>(a, t, rows);
    issue_seg_fixed<DT, NV, NR>(rb, rows, v0, last, live, row_bytes);
  };
  RawChunk<NV, NR> rawA, rawB;
  // Layers -2 and -1 only issue the loads of positions 0 and 1, from the same code
  // as every later prefetch, so the loop is entered with no load outstanding and
  // the compiler's count of outstanding loads at the loop head stays exact: each
  // unpack then waits for its own chunk only, not for the one issued after it.
  int t_0 = sg, t_p1 = sg;
  int t_m2 = 0, t_m1 = 0;
  uint64_t wpoll[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) wpoll[j] = 0ull;
  float x[NR][NE];
  float xref[NR], href[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) xref[r] = href[r] = 0.f;

  auto layer = [&](int i, RawChunk<NV, NR>& rb) __attribute__((always_inline)) {
    const int par = i & 1;
    // the wave index passes through an empty asm in every layer, so that the tests
    // on it are made here instead of being hoisted out of the loop as 64-bit masks
    // that hold scalar registers through it
    int wv = wave;
    asm volatile("" : "+s"(wv));
    const bool do2 = i >= 2 && i - 2 < nl;
    // ---- row statistics of position i - 2 (polled a layer ago) ---------------
    if (do2) {
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int r = wv + j * kWaves;
        if (r < NR) {
          __builtin_amdgcn_s_setprio(3);
          const Lse st = poll_row(wpoll[j], rsrc_rec(t_m2), C, kSt, r, a.err, a.wait_limit);
          if (lane == 0) {
            st_sh[par][r][0] = st.ref;
            st_sh[par][r][1] = st.z;
            st_sh[par][r][2] = __builtin_amdgcn_rcpf(st.z);
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }
      __syncthreads();
      // pass 2 runs at raised priority (2), then the move and the unpack (1); pass 1
      // runs at the base priority and the record work at 3 (measured faster than
      // pass 2, the move and the unpack at the base priority, than pass 2 at 3, and
      // than pass 1 at 1 or 2)
      __builtin_amdgcn_s_setprio(2);
      // ---- pass 2 of position i - 2: overlap and S partials of every head ----
      // In a wave's units p = sa e_p, q = sb e_q (e <= 1).  Working in q's units with
      // rho = sa / sb, the residual of q over p, r = max(0, e_q - rho e_p) <= e_q <= 1,
      // is one fused multiply-add with the [0, 1] output clamp, and
      //   overlap = sum min(rho e_p, e_q) = zq - sum r,
      //   S = sum_{q <= p} e_q = zq - sum_{r > 0} e_q,
      // where zq is this lane's pass-1 sum of e_q (so disjoint supports give exactly
      // 0 and identical rows exactly zq).  The indicator 1[r > 0] is r * 2^126
      // clamped: exactly 1 for every normal r (only a subnormal r, a difference
      // below 2^-126 of the wave's largest q, gives a fraction); a tie (r = 0)
      // counts as q <= p.  Four operations per element and head.  When p outweighs
      // q here by more than 2^100 the same sums run in p's units: r' = max(0, rho'
      // e_q - e_p), rho' = sb / sa, overlap = rho' zq - sum r', S = rho' (zq -
      // sum_{r' > 0} e_q).  The units come from the rows' normalisers 2^ref z:
      // sa = 2^(href_p - ref_p) / z_p, sb likewise, so rho = 2^(dp - dq) z_q / z_p
      // carries a few roundings of its own (the differences of references are exact
      // for every wave near the row's largest logit), not those of the normalisers'
      // logarithms, which the cancellation in min(p, q) would magnify.
      constexpr float kIndScale = 0x1p126f;
      float res[2 * G];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int rt = SHARED ? 0 : k, rq = NT + k;
        const float* const stp = st_sh[par][rt];
        const float* const stq = st_sh[par][rq];
        const float dp = href[rt] - stp[0];            // -inf: no p mass here
        const float dq = href[rq] - stq[0];            // -inf: no q mass here
        const float zq = z_sh[par][rq][tid];           // this lane's pass-1 sum of e_q
        // sums start at -0, so that the first addition folds away (-0 + x = x)
        float r0 = -0.f, r1 = -0.f, c0 = -0.f, c1 = -0.f;
        float ov, sv;
        const float rho_q = fast_exp2(dp - dq) * z_ratio(stq[1], stp[1], stp[2]);   // sa / sb; NaN for a bad row
        if (dp == kNegInf || dq == kNegInf) {
          ov = sv = 0.f;                                 // one of p, q has no mass here
        } else if (rho_q <= 0x1p100f) {                  // q units
          const float rho = rho_q;
#pragma unroll
          for (int qi = 0; qi < NQ; ++qi) {
            const float4 ep4 = held[rt][qi][tid], eq4 = held[rq][qi][tid];
            const float ep[4] = {ep4.x, ep4.y, ep4.z, ep4.w}, eq[4] = {eq4.x, eq4.y, eq4.z, eq4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float r = clamp01(__builtin_fmaf(-rho, ep[e], eq[e]));
              const float ind = clamp01(r * kIndScale);
              if (e & 1) { r1 += r; c1 = __builtin_fmaf(ind, eq[e], c1); }
              else { r0 += r; c0 = __builtin_fmaf(ind, eq[e], c0); }
            }
          }
          const float sb = fast_exp2(dq) * stq[2];
          ov = sb * (zq - (r0 + r1));
          sv = sb * (zq - (c0 + c1));
        } else if (rho_q > 0x1p100f) {                   // p units (q is comparatively tiny)
          const float rho = fast_exp2(dq - dp) * z_ratio(stp[1], stq[1], stq[2]);
#pragma unroll 1
          for (int qi = 0; qi < NQ; ++qi) {
            const float4 ep4 = held[rt][qi][tid], eq4 = held[rq][qi][tid];
            const float ep[4] = {ep4.x, ep4.y, ep4.z, ep4.w}, eq[4] = {eq4.x, eq4.y, eq4.z, eq4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float r = clamp01(__builtin_fmaf(rho, eq[e], -ep[e]));
              const float ind = clamp01(r * kIndScale);
              if (e & 1) { r1 += r; c1 = __builtin_fmaf(ind, eq[e], c1); }
              else { r0 += r; c0 = __builtin_fmaf(ind, eq[e], c0); }
            }
          }
          const float sa = fast_exp2(dp) * stp[2];
          ov = sa * (rho * zq - (r0 + r1));
          sv = sa * rho * (zq - (c0 + c1));
        } else {
          ov = sv = __builtin_nanf("");                  // a NaN statistic propagates
        }
        res[2 * k] = ov;
        res[2 * k + 1] = sv;
      }
#pragma unroll
      for (int k = 0; k < 2 * G; ++k) red_sh[k][tid] = res[k];
    }
    __builtin_amdgcn_s_setprio(1);
    // ---- position i - 1 moves to LDS (own slots only) --------------------------
    if (i >= 1 && i - 1 < nl) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi)
          held[r][qi][tid] = make_float4(x[r][4 * qi], x[r][4 * qi + 1], x[r][4 * qi + 2], x[r][4 * qi + 3]);
        href[r] = xref[r];
      }
    }
    // ---- position i: unpack, then the poll for i - 1 and the loads of i + 2 ------
    if (i >= 0 && i < nl) {
      const char* rows[NR];
      fwd_rows<DT, NT, G>(a, t_0, rows);
      int lim_l = lim, tail_l = tail, vend_l = vend, V_l = V;
      asm volatile("" : "+s"(lim_l), "+s"(tail_l), "+s"(vend_l), "+s"(V_l));
      unpack_seg<DT, NV, NR>(rb, rows, v0, full, lim_l, tail_l, vend_l, V_l, x);
    }
    if (i >= 1 && i <= nl && lane < C) {
      const __amdgpu_buffer_rsrc_t rs = rsrc_rec(t_m1);
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int r = wv + j * kWaves;
        if (r < NR) wpoll[j] = rec_load(rs, lane * kSt + r * 8);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    const int t_p2 = i + 2 < nl ? pos_of(i + 2) : t_0;
    prefetch(rb, t_p2, i + 2 < nl);
    __builtin_amdgcn_sched_barrier(0);

    if (i >= 0 && i < nl) {
      // ---- pass 1 of position i (base priority) ------------------------------
      float zl[NR];
      lane_pass1<NE, NR>(x, xref, zl, kLog2e);
#pragma unroll
      for (int r = 0; r < NR; ++r) z_sh[par][r][tid] = zl[r];
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) ref_sh[par][r][wv] = xref[r];
      }
    }
    if ((i >= 0 && i < nl) || do2) __syncthreads();
    if (i >= 0 && i < nl) {
      __builtin_amdgcn_s_setprio(3);
      const __amdgpu_buffer_rsrc_t rs = rsrc_rec(t_0);
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int r = wv + j * kWaves;
        if (r < NR) {
          // row r over the workgroup: each lane rescales its four waves' sums to the
          // largest reference, then one wave sum
          float rf[kWaves], R = kNegInf;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            rf[w] = ref_sh[par][r][w];
            R = fmaximum(R, rf[w]);
          }
          const float Rf = finite_ref(R);
          float zs = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) zs = __builtin_fmaf(z_sh[par][r][w * 64 + lane], fast_exp2(rf[w] - Rf), zs);
          const float Z = wave_total(zs);
          if (lane == 0) rec_store(rs, c * kSt + r * 8, pack2(R, mark(Z)));
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (do2) {
      // the chunk's overlap and S partials of position i - 2: wave w adds up values
      // w, w + 4, ... over the lanes (the four waves' lanes first), in a fixed order
      float v[KW];
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const int k = min(wv + j * kWaves, 2 * G - 1);
        v[j] = (red_sh[k][lane] + red_sh[k][lane + 64]) + (red_sh[k][lane + 128] + red_sh[k][lane + 192]);
      }
      wave_reduce<false, KW>(v);
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < KW; ++j) {
          const int k = wv + j * kWaves;
          if (k < 2 * G) a.part2[((int64_t)t_m2 * C + c) * 2 * G + k] = v[j];
        }
      }
    }
    // ---- shift the position window ---------------------------------------------
    t_m2 = t_m1;
    t_m1 = t_0;
    t_0 = t_p1;
    t_p1 = t_p2;
  };

  // nl + 4 layers from -2, rounded up to an even count so that both buffers keep
  // their registers across iterations
  for (int i = -2; i < nl + 2; i += 2) {
    layer(i, rawA);
    layer(i + 1, rawB);
  }
}

// One wave per position: the row log-sum-exps from the records (merged as the poll
// merged them), the overlap and S of every head from the chunk partials, l_t and the
// saved statistics.  Clears the records and partials it read.
template <int G, bool SHARED>
__global__ __launch_bounds__(64 * kFinishWaves) void tv_pipe_finish(TvArgs a) {
  constexpr int NT = FwdShape<G, SHARED>::NT;
  constexpr int NR = FwdShape<G, SHARED>::NR;
  constexpr int kSt = NR * 8;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kFinishWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int C = a.sp.nchunks;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.part1 + (int64_t)t * C * NR);
  // every row's first record word and the first partials go out at once (clamped
  // into the position, so the loads are unconditional); lanes past the last chunk
  // ignore them
  const int lc = min(lane, C - 1);
  float* p2 = a.part2 + (int64_t)t * C * 2 * G;
  uint64_t v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) v[r] = rec_load(rs, lc * kSt + r * 8);
  float pre[2 * G];
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) pre[k] = p2[(int64_t)lc * 2 * G + k];
  float lse2[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r)
    lse2[r] = lse_log2(poll_row(lane < C ? v[r] : 0ull, rs, C, kSt, r, a.err, a.wait_limit));
  float tot[2 * G];
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) tot[k] = lane < C ? pre[k] : 0.f;
  for (int cc = lane + 64; cc < C; cc += 64) {
#pragma unroll
    for (int k = 0; k < 2 * G; ++k) tot[k] += p2[(int64_t)cc * 2 * G + k];
  }
  wave_reduce<false, 2 * G>(tot);
  uint64_t* rec = a.part1 + (int64_t)t * C * NR;
  for (int i = lane; i < C * NR; i += 64) rec[i] = 0ull;
  for (int i = lane; i < C * 2 * G; i += 64) p2[i] = 0.f;
  if (lane == 0) {
    float prod = 1.f, l = 0.f;
    float* sv = a.saved + (int64_t)t * G * kTvSavedStride;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float ov = tot[2 * k];   // NaN (a row without a normaliser) stays NaN
      const float al = ov != ov ? ov : fminf(fmaxf(ov, 0.f), 1.f);
      prod *= al;
      l -= prod;
      sv[k * kTvSavedStride + 0] = lse2[SHARED ? 0 : k] * kLn2;
      sv[k * kTvSavedStride + 1] = lse2[NT + k] * kLn2;
      sv[k * kTvSavedStride + 2] = al;
      sv[k * kTvSavedStride + 3] = tot[2 * k + 1];
    }
    if (a.pos_loss) a.pos_loss[t] = l;
    a.pos_ws[t] = l;
  }
}

// ---------------------------------------------------------------------------
constexpr int kBwdNVBf16 = 4;
constexpr int kBwdNVF32 = 8;

template <int GDT, int PV>
__device__ __forceinline__ void store_grad(char* row, int64_t vi, const RowSplit& sp, int64_t V,
                                           const float* gv) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  if (vi < sp.nvec_full) {
    if constexpr (GDT == kBF16) {
      uint32_t w[PV / 2];
#pragma unroll
      for (int e = 0; e < PV / 2; ++e)
        w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{gv[2 * e], gv[2 * e + 1]}), b2));
      if constexpr (PV == 8) {
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(row) + vi);
      } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(row) + vi);
      }
    } else {
#pragma unroll
      for (int h = 0; h < PV / 4; ++h) {
        u32x4 o{__float_as_uint(gv[4 * h]), __float_as_uint(gv[4 * h + 1]), __float_as_uint(gv[4 * h + 2]),
                __float_as_uint(gv[4 * h + 3])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(row) + vi * (PV / 4) + h);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      const int64_t idx = vi * PV + e;
      if (idx < V) {
        if constexpr (GDT == kBF16) {
          const __bf16 h = (__bf16)gv[e];
          reinterpret_cast<uint16_t*>(row)[idx] = __builtin_bit_cast(uint16_t, h);
        } else {
          reinterpret_cast<float*>(row)[idx] = gv[e];
        }
      }
    }
  }
}

// Vectors per thread and row for the backward: 32 bf16 or 16 fp32 values per row
// and thread for up to four rows (fewer with more rows, at least one vector).
template <int NR>
constexpr int bwd_nv(int per_vec) {
  const int nv = (per_vec == 8 ? 128 : 64) / (NR * per_vec);
  return nv < 1 ? 1 : nv;
}

template <int G>
static int bwd_nv_for(int dt, bool shared) {
  const int pv = dt == kBF16 ? 8 : 4;
  return shared ? bwd_nv<FwdShape<G, true>::NR>(pv) : bwd_nv<FwdShape<G, false>::NR>(pv);
}

// One workgroup per (position, chunk).  The chunk of every row of the position
// (target row(s), then the G draft rows) is put in flight at once, then the
// gradient of each head is formed and stored: one memory round trip per
// workgroup, and the stores of one head overlap the arithmetic of the next.
template <int DT, int GDT, int G, bool SHARED>
__global__ __launch_bounds__(kBlock) void tv_bwd_kernel(TvArgs a) {
  constexpr int NT = FwdShape<G, SHARED>::NT;
  constexpr int NR = FwdShape<G, SHARED>::NR;
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NV = bwd_nv<NR>(PV);
  constexpr int NE = NV * PV;
  const int C = a.sp.nchunks;
  const int t = blockIdx.x / C, c = blockIdx.x - (blockIdx.x / C) * C;
  const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
  const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);

  const char* rows[NR];
  fwd_rows<DT, NT, G>(a, t, rows);
  float x[NR][NE];
  load_rows<DT, NV, NR>(rows, vbeg, vend, a.sp, a.V, x);

  // end-to-end weights of this position
  const float* sv = a.saved_in + (int64_t)t * G * kTvSavedStride;
  float alpha[G];
#pragma unroll
  for (int k = 0; k < G; ++k) alpha[k] = sv[k * kTvSavedStride + 2];
  const float gscale = -a.grad_loss[0] / (float)a.T;

  char* gb = reinterpret_cast<char*>(a.grad);
  constexpr int gbytes = GDT == kBF16 ? 2 : 4;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    float wsum = 0.f;
#pragma unroll
    for (int kk = k; kk < G; ++kk) {
      float prod = 1.f;
#pragma unroll
      for (int i = 0; i <= kk; ++i)
        if (i != k) prod *= alpha[i];
      wsum += prod;
    }
    const float w = gscale * wsum;
    const float lse_p = sv[k * kTvSavedStride + 0], lse_q = sv[k * kTvSavedStride + 1];
    const float S = sv[k * kTvSavedStride + 3];
    const float delta = lse_q - lse_p;
    const float lq2 = lse_q * kLog2e;
    const float c1 = w * (1.f - S), c0 = -w * S;
    const float(&xt)[NE] = x[SHARED ? 0 : k];
    const float(&xd)[NE] = x[NT + k];
    float gr[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const bool ind = (xd[i] - xt[i]) <= delta;
      const float q = fast_exp2(__builtin_fmaf(xd[i], kLog2e, -lq2));
      gr[i] = q * (ind ? c1 : c0);
    }
    char* grow = gb + ((int64_t)t * a.g_pos + (int64_t)k * a.g_head) * gbytes;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t vi = vbeg + (int64_t)j * kBlock + threadIdx.x;
      if (vi < vend) store_grad<GDT, PV>(grow, vi, a.sp, a.V, gr + j * PV);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused forward + backward (paperlayer App. F "Fused TV Loss Kernel": the backward
// reuses quantities the forward computed; rainbus "Method steps": the fused
// kernel keeps the memory peak down).  With the upstream scalar g known before
// the call, one sweep over the logits gives the loss, the saved statistics and
// the gradient: every logit is read once and every gradient element written once.
//
// The single-read forward's pipeline (super-groups of C workgroups, chunk c of
// every row of a position per workgroup, records of the row normalisers, pass 2
// from the e values held on chip two layers after pass 1) gains a second exchange
// and a gradient phase.  Layer i:
//   * gradient of position i - 3: every wave reads the position's overlap and S
//     totals (merged by the waves from the chunks' records in one fixed order),
//     forms the end-to-end weights and writes g_v = w q_v (1[q_v <= p_v] - S) for
//     its segment of every head from the values s_v it kept since pass 2;
//   * pass 2 of position i - 2 (as in the forward) also keeps, per draft element,
//     s_v = +e_q where q_v <= p_v and -e_q where q_v > p_v (e_q in the wave's q
//     units sb): the gradient needs q_v = sb |s_v| and the indicator, the sign.
//     The test is r > 0 for the residual r = max(0, e_q - rho e_p) (a compare
//     and a select; a tie counts as q <= p), and S comes from the sum of the s
//     values: S = sb (zq + sum s) / 2.  The chunk's overlap and S partials (summed
//     over the waves) are published at once as one self-announcing record per
//     head;
//   * the e values of position i - 1 move to LDS, position i is unpacked, the
//     record polls of positions i - 1 (normalisers) and i - 2 (overlap, S) and
//     the loads of position i + 1 go out, pass 1 of position i and its records.
// The overlap/S records of a position are polled a layer after they are
// published and used a layer later; the s values live in registers for one
// layer.  tv_fused_finish (one wave per position) writes the saved statistics
// and l_t from the same records, merged in the same order, and clears them.
template <int G>
struct FusedRec {
  // record word of (chunk, head): (overlap partial, S partial with the sign bit as
  // a marker: S >= 0, so a published word is never zero)
  static constexpr int kStride = G * 8;
};

// The overlap and S totals of head k from the chunks' records: lane l folds record
// l, then l + 64, ... in that order, then the wave sums the lanes (the same bits in
// every lane and every workgroup).  `v` is this lane's first word, loaded earlier.
// NaN totals if the wait timed out.
template <int G>
__device__ __forceinline__ void fused_totals(uint64_t v, __amdgpu_buffer_rsrc_t rs, int C, int k, uint32_t* err,
                                             uint64_t limit, float& alpha, float& S) {
  float ac = 0.f, sc = 0.f;
  const bool timed_out = poll_words(v, rs, C, FusedRec<G>::kStride, k, err, limit, [&](bool first, uint64_t w) {
    const float aw = unpack_lo(w), sw = unmark(unpack_hi(w));
    ac = first ? aw : ac + aw;
    sc = first ? sw : sc + sw;
  });
  if ((threadIdx.x & 63) >= C) ac = sc = 0.f;
  float t[2] = {ac, sc};
  wave_reduce<false, 2>(t);
  alpha = timed_out ? __builtin_nanf("") : t[0];
  S = timed_out ? __builtin_nanf("") : t[1];
}

// This thread's gradient values of one head's segment (NV vectors of PV values,
// vector v0 + 64 j), stored to row `row`: full vectors as one 16-byte (bf16) or
// PV/4 16-byte (fp32) non-temporal stores, the row's partial last vector element by
// element; vectors past the chunk or the row are skipped.
template <int GDT, int NV, int PV>
__device__ __forceinline__ void fused_store(char* row, int v0, int vend, const RowSplit& sp, int64_t V,
                                            const float (&g)[NV * PV]) {
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = v0 + j * 64;
    if (vi < vend) store_grad<GDT, PV>(row, vi, sp, V, g + j * PV);
  }
}

template <int DT, int GDT, int G, bool SHARED>
__global__ __launch_bounds__(kBlock, 2) void tv_fused_main(TvArgs a) {
  constexpr int NT = FwdShape<G, SHARED>::NT;
  constexpr int NR = FwdShape<G, SHARED>::NR;
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NV = pipe_nv<NR>(PV);
  constexpr int NE = NV * PV;
  constexpr int NQ = NE / 4;
  constexpr int kSegVec = NV * 64;
  constexpr int RW = (NR + kWaves - 1) / kWaves;
  constexpr int kSt = NR * 8;
  constexpr int kSt2 = FusedRec<G>::kStride;
  static_assert(G <= kWaves, "one wave per head merges the overlap / S records");
  const int C = a.sp.nchunks;
  const int slot = blockIdx.x;
  const int sg = slot / C, c = slot - sg * C;
  const int S = a.sgroups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  if (sg >= a.T) return;
  // positions t = sg + i S, or the contiguous range the host sized for this
  // super-group's dispatch round (round_split_base)
  int nl = (a.T - 1 - sg) / S + 1, base = -1;
  if (a.split.W > 0) {
    base = round_split_base(a.split, sg, S, C);
    nl = round_split_base(a.split, sg + 1, S, C) - base;
  }
  auto pos_of = [&](int i) { return base >= 0 ? base + i : sg + i * S; };
  auto rsrc_rec = [&](int t) { return rsrc_of(a.part1 + (int64_t)t * C * NR); };
  auto rsrc_rec2 = [&](int t) { return rsrc_of(a.part3 + (int64_t)t * C * G); };

  const int vpc = (int)a.sp.vec_per_chunk, nvec = (int)a.sp.nvec, nfull = (int)a.sp.nvec_full;
  const int vbeg = c * vpc;
  const int vend = min(vbeg + vpc, nvec);
  const int s0 = vbeg + wave * kSegVec;
  const int v0 = s0 + lane;
  const int lim = min(vend, nfull);
  const bool full = s0 + kSegVec <= lim;
  const int last = nfull - 1;
  const int tail = nfull;
  const int V = (int)a.V;
  const int row_bytes = (int)min(a.V * Elem<DT>::kBytes, (int64_t)0x7fffffff);
  const float gscale = -a.grad_loss[0] / (float)a.T;
  char* gb = reinterpret_cast<char*>(a.grad);
  constexpr int gbytes = GDT == kBF16 ? 2 : 4;

  __shared__ float4 held[NR][NQ][kBlock];      // e values of the position two layers back
  __shared__ float ref_sh[2][NR][kWaves];       // pass-1 wave references, by layer parity
  __shared__ float z_sh[2][NR][kBlock];         // pass-1 lane sums in their wave's units
  __shared__ float st_sh[NR][3];                // row normalisers 2^ref z of the position in pass 2: (ref, z, 1/z)
  __shared__ float red_sh[2 * G][kBlock];       // pass-2 lane partials (overlap, S per head)
  __shared__ float tot_sh[2 * G];               // overlap and S totals of the gradient's position

  auto prefetch = [&](int t, bool live, RawChunk<NV, NR>& rb) {
    const char* rows[NR];
    fwd_rows<DT, NT, G>(a, t, rows);
    issue_seg_fixed<DT, NV, NR>(rb, rows, v0, last, live, row_bytes);
  };
  RawChunk<NV, NR> raw;
  uint64_t wpoll[RW], wpoll2 = 0ull;
#pragma unroll
  for (int j = 0; j < RW; ++j) wpoll[j] = 0ull;
  float x[NR][NE];
  float xref[NR], href[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) xref[r] = href[r] = 0.f;
  float sv[G][NE];   // signed q values kept from pass 2 for the gradient
  float sbg[G];      // their q units (log2) per head
#pragma unroll
  for (int k = 0; k < G; ++k) sbg[k] = 0.f;

  // Layer -1 only issues the loads of position 0 (from the same code as every
  // later prefetch); layer i unpacks position i, whose loads went out a layer ago.
  for (int i = -1; i < nl + 3; ++i) {
    const bool dog = i >= 3 && i - 3 < nl;   // gradient of position i - 3
    const bool do2 = i >= 2 && i - 2 < nl;   // pass 2 of position i - 2
    const bool do1 = i >= 0 && i < nl;       // pass 1 of position i
    const int t_g = pos_of(i - 3), t_2 = pos_of(i - 2), t_1 = pos_of(i - 1), t_0 = pos_of(i);
    // ---- record polls issued a layer ago: overlap / S totals, row normalisers --
    if (dog || do2) {
      __builtin_amdgcn_s_setprio(3);
      if (dog && wave < G) {
        float al, s;
        fused_totals<G>(wpoll2, rsrc_rec2(t_g), C, wave, a.err, a.wait_limit, al, s);
        if (lane == 0) {
          tot_sh[2 * wave] = al;
          tot_sh[2 * wave + 1] = s;
        }
      }
      if (do2) {
#pragma unroll
        for (int j = 0; j < RW; ++j) {
          const int r = wave + j * kWaves;
          if (r < NR) {
            const Lse st = poll_row(wpoll[j], rsrc_rec(t_2), C, kSt, r, a.err, a.wait_limit);
            if (lane == 0) {
              st_sh[r][0] = st.ref;
              st_sh[r][1] = st.z;
              st_sh[r][2] = __builtin_amdgcn_rcpf(st.z);
            }
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
    }
    // ---- gradient of position i - 3 ------------------------------------------
    if (dog) {
      float al[G], Sk[G];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const float ov = tot_sh[2 * k];   // NaN (a row without a normaliser) stays NaN
        al[k] = ov != ov ? ov : fminf(fmaxf(ov, 0.f), 1.f);
        Sk[k] = tot_sh[2 * k + 1];
      }
#pragma unroll
      for (int k = 0; k < G; ++k) {
        // w_k = -(g / T) sum_{m >= k} prod_{j <= m, j != k} alpha_j
        float wsum = 0.f;
#pragma unroll
        for (int m = k; m < G; ++m) {
          float prod = 1.f;
#pragma unroll
          for (int j = 0; j <= m; ++j)
            if (j != k) prod *= al[j];
          wsum += prod;
        }
        const float qs = gscale * wsum * sbg[k];   // w sb
        const float cp = qs * (1.f - Sk[k]), cn = qs * Sk[k];
        float gv[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) gv[e] = sv[k][e] * (sv[k][e] >= 0.f ? cp : cn);
        char* grow = gb + ((int64_t)t_g * a.g_pos + (int64_t)k * a.g_head) * gbytes;
        fused_store<GDT, NV, PV>(grow, v0, vend, a.sp, a.V, gv);
      }
    }
    // ---- pass 2 of position i - 2 ---------------------------------------------
    if (do2) {
      float res[2 * G];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int rt = SHARED ? 0 : k, rq = NT + k;
        // units as in the single-read forward: sa = 2^(href_p - ref_p) / z_p, sb likewise
        const float dp = href[rt] - st_sh[rt][0];        // -inf: no p mass here
        const float dq = href[rq] - st_sh[rq][0];        // -inf: no q mass here
        const float zq = z_sh[i & 1][rq][tid];
        float r0 = -0.f, r1 = -0.f, c0 = -0.f, c1 = -0.f;
        float ov, svp;
        const float sb = fast_exp2(dq) * st_sh[rq][2];
        const float rho_q = fast_exp2(dp - dq) * z_ratio(st_sh[rq][1], st_sh[rt][1], st_sh[rt][2]);   // sa / sb; NaN for a bad row
        sbg[k] = sb;
        if (dq == kNegInf) {                             // no q mass here: no gradient
          ov = svp = 0.f;
#pragma unroll
          for (int e = 0; e < NE; ++e) sv[k][e] = 0.f;
        } else if (dp == kNegInf) {                      // no p mass: every q > p
          ov = svp = 0.f;
#pragma unroll
          for (int qi = 0; qi < NQ; ++qi) {
            const float4 eq4 = held[rq][qi][tid];
            sv[k][4 * qi] = -eq4.x; sv[k][4 * qi + 1] = -eq4.y; sv[k][4 * qi + 2] = -eq4.z; sv[k][4 * qi + 3] = -eq4.w;
          }
        } else if (rho_q <= 0x1p100f) {                  // q units
          const float rho = rho_q;
#pragma unroll
          for (int qi = 0; qi < NQ; ++qi) {
            const float4 ep4 = held[rt][qi][tid], eq4 = held[rq][qi][tid];
            const float ep[4] = {ep4.x, ep4.y, ep4.z, ep4.w}, eq[4] = {eq4.x, eq4.y, eq4.z, eq4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float r = clamp01(__builtin_fmaf(-rho, ep[e], eq[e]));
              const float s = r > 0.f ? -eq[e] : eq[e];   // q > p: -e_q, else e_q
              sv[k][4 * qi + e] = s;
              if (e & 1) { r1 += r; c1 += s; }
              else { r0 += r; c0 += s; }
            }
          }
          // sum s = sum_{q <= p} e_q - sum_{q > p} e_q, so S = sb (zq + sum s) / 2
          ov = sb * (zq - (r0 + r1));
          svp = 0.5f * sb * (zq + (c0 + c1));
        } else if (rho_q > 0x1p100f) {                   // p units (q is comparatively tiny)
          const float rho = fast_exp2(dq - dp) * z_ratio(st_sh[rt][1], st_sh[rq][1], st_sh[rq][2]);
#pragma unroll
          for (int qi = 0; qi < NQ; ++qi) {
            const float4 ep4 = held[rt][qi][tid], eq4 = held[rq][qi][tid];
            const float ep[4] = {ep4.x, ep4.y, ep4.z, ep4.w}, eq[4] = {eq4.x, eq4.y, eq4.z, eq4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float r = clamp01(__builtin_fmaf(rho, eq[e], -ep[e]));
              const float s = r > 0.f ? -eq[e] : eq[e];
              sv[k][4 * qi + e] = s;
              if (e & 1) { r1 += r; c1 += s; }
              else { r0 += r; c0 += s; }
            }
          }
          const float sa = fast_exp2(dp) * st_sh[rt][2];
          ov = sa * (rho * zq - (r0 + r1));
          svp = 0.5f * sa * rho * (zq + (c0 + c1));
        } else {
          ov = svp = __builtin_nanf("");                 // a NaN statistic propagates
#pragma unroll
          for (int e = 0; e < NE; ++e) sv[k][e] = __builtin_nanf("");
        }
        res[2 * k] = ov;
        res[2 * k + 1] = svp;
      }
#pragma unroll
      for (int k = 0; k < 2 * G; ++k) red_sh[k][tid] = res[k];
      __syncthreads();
      // the chunk's overlap and S partials: wave k sums head k over the four
      // waves' lanes (in a fixed order) and publishes them as one record word
      if (wave < G) {
        float v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float* rr = red_sh[2 * wave + h];
          v[h] = (rr[lane] + rr[lane + 64]) + (rr[lane + 128] + rr[lane + 192]);
        }
        wave_reduce<false, 2>(v);
        if (lane == 0) rec_store(rsrc_rec2(t_2), c * kSt2 + wave * 8, pack2(v[0], mark(v[1])));
      }
    }
    // ---- position i - 1 moves to LDS (own slots only) --------------------------
    if (i >= 1 && i - 1 < nl) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi)
          held[r][qi][tid] = make_float4(x[r][4 * qi], x[r][4 * qi + 1], x[r][4 * qi + 2], x[r][4 * qi + 3]);
        href[r] = xref[r];
      }
    }
    // ---- position i: unpack; record polls; the loads of position i + 1 --------
    if (do1) {
      const char* rows[NR];
      fwd_rows<DT, NT, G>(a, t_0, rows);
      int lim_l = lim, tail_l = tail, vend_l = vend, V_l = V;
      asm volatile("" : "+s"(lim_l), "+s"(tail_l), "+s"(vend_l), "+s"(V_l));
      unpack_seg<DT, NV, NR>(raw, rows, v0, full, lim_l, tail_l, vend_l, V_l, x);
    }
    if (i >= 1 && i <= nl && lane < C) {
      const __amdgpu_buffer_rsrc_t rs = rsrc_rec(t_1);
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int r = wave + j * kWaves;
        if (r < NR) wpoll[j] = rec_load(rs, lane * kSt + r * 8);
      }
    }
    if (do2 && wave < G && lane < C) wpoll2 = rec_load(rsrc_rec2(t_2), lane * kSt2 + wave * 8);
    __builtin_amdgcn_sched_barrier(0);
    prefetch(i + 1 < nl ? pos_of(i + 1) : sg, i + 1 < nl, raw);
    __builtin_amdgcn_sched_barrier(0);
    // ---- pass 1 of position i ------------------------------------------------
    if (do1) {
      __builtin_amdgcn_s_setprio(1);
      float zl[NR];
      lane_pass1<NE, NR>(x, xref, zl, kLog2e);
#pragma unroll
      for (int r = 0; r < NR; ++r) z_sh[i & 1][r][tid] = zl[r];
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) ref_sh[i & 1][r][wave] = xref[r];
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      __builtin_amdgcn_s_setprio(3);
      const __amdgpu_buffer_rsrc_t rs = rsrc_rec(t_0);
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int r = wave + j * kWaves;
        if (r < NR) {
          float rf[kWaves], R = kNegInf;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            rf[w] = ref_sh[i & 1][r][w];
            R = fmaximum(R, rf[w]);
          }
          const float Rf = finite_ref(R);
          float zs = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w)
            zs = __builtin_fmaf(z_sh[i & 1][r][w * 64 + lane], fast_exp2(rf[w] - Rf), zs);
          const float Z = wave_total(zs);
          if (lane == 0) rec_store(rs, c * kSt + r * 8, pack2(R, mark(Z)));
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
  }
}

// One wave per position: row log-sum-exps from the normaliser records, overlap and
// S totals from the overlap / S records (merged as the main kernel merged them, so
// the saved statistics are the ones its gradient used), l_t; clears the records.
template <int G, bool SHARED>
__global__ __launch_bounds__(64 * kFinishWaves) void tv_fused_finish(TvArgs a) {
  constexpr int NT = FwdShape<G, SHARED>::NT;
  constexpr int NR = FwdShape<G, SHARED>::NR;
  constexpr int kSt = NR * 8;
  constexpr int kSt2 = FusedRec<G>::kStride;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kFinishWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int C = a.sp.nchunks;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.part1 + (int64_t)t * C * NR);
  const __amdgpu_buffer_rsrc_t rs2 = rsrc_of(a.part3 + (int64_t)t * C * G);
  const int lc = min(lane, C - 1);
  uint64_t v[NR], v2[G];
#pragma unroll
  for (int r = 0; r < NR; ++r) v[r] = rec_load(rs, lc * kSt + r * 8);
#pragma unroll
  for (int k = 0; k < G; ++k) v2[k] = rec_load(rs2, lc * kSt2 + k * 8);
  float lse2[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r)
    lse2[r] = lse_log2(poll_row(lane < C ? v[r] : 0ull, rs, C, kSt, r, a.err, a.wait_limit));
  float al[G], Sk[G];
#pragma unroll
  for (int k = 0; k < G; ++k) fused_totals<G>(lane < C ? v2[k] : 0ull, rs2, C, k, a.err, a.wait_limit, al[k], Sk[k]);
  uint64_t* rec = a.part1 + (int64_t)t * C * NR;
  for (int i = lane; i < C * NR; i += 64) rec[i] = 0ull;
  uint64_t* rec2 = a.part3 + (int64_t)t * C * G;
  for (int i = lane; i < C * G; i += 64) rec2[i] = 0ull;
  if (lane == 0) {
    float prod = 1.f, l = 0.f;
    float* sv = a.saved + (int64_t)t * G * kTvSavedStride;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float ov = al[k];
      const float alc = ov != ov ? ov : fminf(fmaxf(ov, 0.f), 1.f);
      prod *= alc;
      l -= prod;
      sv[k * kTvSavedStride + 0] = lse2[SHARED ? 0 : k] * kLn2;
      sv[k * kTvSavedStride + 1] = lse2[NT + k] * kLn2;
      sv[k * kTvSavedStride + 2] = alc;
      sv[k * kTvSavedStride + 3] = Sk[k];
    }
    if (a.pos_loss) a.pos_loss[t] = l;
    a.pos_ws[t] = l;
  }
}

// ---------------------------------------------------------------------------
template <int DT, bool SHARED, int G>
static hipError_t launch_fwd_g(const TvArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.T * a.sp.nchunks;
  hipLaunchKernelGGL((tv_fwd_lse<DT, G, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tv_fwd_stats<DT, G, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((tv_fwd_finish<G, SHARED>), dim3((unsigned)((a.T + kFinishWaves - 1) / kFinishWaves)),
                     dim3(64 * kFinishWaves), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tv_fwd_mean, dim3(1), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

template <int DT, bool SHARED>
static hipError_t launch_fwd_dt(const TvArgs& a, hipStream_t stream) {
  switch (a.G) {
    case 1: return launch_fwd_g<DT, SHARED, 1>(a, stream);
    case 2: return launch_fwd_g<DT, SHARED, 2>(a, stream);
    case 3: return launch_fwd_g<DT, SHARED, 3>(a, stream);
    case 4: return launch_fwd_g<DT, SHARED, 4>(a, stream);
    case 5: return launch_fwd_g<DT, SHARED, 5>(a, stream);
    case 6: return launch_fwd_g<DT, SHARED, 6>(a, stream);
    case 7: return launch_fwd_g<DT, SHARED, 7>(a, stream);
    case 8: return launch_fwd_g<DT, SHARED, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tv_fwd(const TvArgs& a, int dt, bool shared, hipStream_t stream) {
  if (dt == kBF16) return shared ? launch_fwd_dt<kBF16, true>(a, stream) : launch_fwd_dt<kBF16, false>(a, stream);
  return shared ? launch_fwd_dt<kF32, true>(a, stream) : launch_fwd_dt<kF32, false>(a, stream);
}

// ---- single-read forward: launch, vectors per thread, occupancy --------------
template <int DT, bool SHARED, int G>
static hipError_t launch_pipe_g(const TvArgs& a, hipStream_t stream) {
  if constexpr (!pipe_fits<G, SHARED>()) {
    return hipErrorInvalidValue;
  } else {
    const int64_t grid = (int64_t)a.sgroups * a.sp.nchunks;
    hipLaunchKernelGGL((tv_pipe_main<DT, G, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tv_pipe_finish<G, SHARED>), dim3((unsigned)((a.T + kFinishWaves - 1) / kFinishWaves)),
                       dim3(64 * kFinishWaves), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(tv_fwd_mean, dim3(1), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
  }
}

template <int DT, bool SHARED, int G>
static hipError_t occupancy_pipe_g(int* n) {
  if constexpr (!pipe_fits<G, SHARED>()) {
    *n = 0;
    return hipErrorInvalidValue;
  } else {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, tv_pipe_main<DT, G, SHARED>, kBlock, 0);
  }
}

template <int DT, bool SHARED>
static hipError_t pipe_dispatch(int G, const TvArgs* a, hipStream_t stream, int* occ) {
  switch (G) {
#define MTP_PIPE_CASE(g) \
    case g: return a ? launch_pipe_g<DT, SHARED, g>(*a, stream) : occupancy_pipe_g<DT, SHARED, g>(occ);
    MTP_PIPE_CASE(1) MTP_PIPE_CASE(2) MTP_PIPE_CASE(3) MTP_PIPE_CASE(4)
    MTP_PIPE_CASE(5) MTP_PIPE_CASE(6) MTP_PIPE_CASE(7) MTP_PIPE_CASE(8)
#undef MTP_PIPE_CASE
  }
  return hipErrorInvalidValue;
}

static hipError_t pipe_any(int dt, bool shared, int G, const TvArgs* a, hipStream_t stream, int* occ) {
  if (dt == kBF16) return shared ? pipe_dispatch<kBF16, true>(G, a, stream, occ) : pipe_dispatch<kBF16, false>(G, a, stream, occ);
  return shared ? pipe_dispatch<kF32, true>(G, a, stream, occ) : pipe_dispatch<kF32, false>(G, a, stream, occ);
}

int tv_pipe_vec_per_thread(int dt, int G, bool shared) {
  const int nr = (shared ? 1 : G) + G;
  if (nr > kTvPipeMaxRows) return 0;
  const int pv = dt == kBF16 ? 8 : 4;
  const int nv = kPipeFloats / (nr * pv);
  return nv < 1 ? 1 : nv;
}

hipError_t tv_pipe_occupancy(int dt, int G, bool shared, int* blocks_per_cu) {
  return pipe_any(dt, shared, G, nullptr, nullptr, blocks_per_cu);
}

hipError_t launch_tv_pipe_fwd(const TvArgs& a, int dt, bool shared, hipStream_t stream) {
  return pipe_any(dt, shared, a.G, &a, stream, nullptr);
}

// ---- fused forward + backward: launch, occupancy ------------------------------
template <int DT, int GDT, bool SHARED, int G>
static hipError_t fused_g(const TvArgs* a, hipStream_t stream, int* occ) {
  if constexpr (!pipe_fits<G, SHARED>() || G > kWaves) {
    if (occ) *occ = 0;
    return hipErrorInvalidValue;
  } else {
    if (!a) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, tv_fused_main<DT, GDT, G, SHARED>, kBlock, 0);
    const int64_t grid = (int64_t)a->sgroups * a->sp.nchunks;
    hipLaunchKernelGGL((tv_fused_main<DT, GDT, G, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, *a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tv_fused_finish<G, SHARED>), dim3((unsigned)((a->T + kFinishWaves - 1) / kFinishWaves)),
                       dim3(64 * kFinishWaves), 0, stream, *a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(tv_fwd_mean, dim3(1), dim3(kBlock), 0, stream, *a);
    return hipGetLastError();
  }
}

template <int DT, int GDT, bool SHARED>
static hipError_t fused_dispatch(int G, const TvArgs* a, hipStream_t stream, int* occ) {
  switch (G) {
    case 1: return fused_g<DT, GDT, SHARED, 1>(a, stream, occ);
    case 2: return fused_g<DT, GDT, SHARED, 2>(a, stream, occ);
    case 3: return fused_g<DT, GDT, SHARED, 3>(a, stream, occ);
    case 4: return fused_g<DT, GDT, SHARED, 4>(a, stream, occ);
  }
  if (occ) *occ = 0;
  return hipErrorInvalidValue;
}

static hipError_t fused_any(int dt, int gdt, bool shared, int G, const TvArgs* a, hipStream_t stream, int* occ) {
  if (dt == kBF16) {
    if (gdt == kBF16)
      return shared ? fused_dispatch<kBF16, kBF16, true>(G, a, stream, occ)
                    : fused_dispatch<kBF16, kBF16, false>(G, a, stream, occ);
    return shared ? fused_dispatch<kBF16, kF32, true>(G, a, stream, occ)
                  : fused_dispatch<kBF16, kF32, false>(G, a, stream, occ);
  }
  if (gdt == kBF16)
    return shared ? fused_dispatch<kF32, kBF16, true>(G, a, stream, occ)
                  : fused_dispatch<kF32, kBF16, false>(G, a, stream, occ);
  return shared ? fused_dispatch<kF32, kF32, true>(G, a, stream, occ) : fused_dispatch<kF32, kF32, false>(G, a, stream, occ);
}

hipError_t tv_fused_occupancy(int dt, int grad_dt, int G, bool shared, int* blocks_per_cu) {
  return fused_any(dt, grad_dt, shared, G, nullptr, nullptr, blocks_per_cu);
}

hipError_t launch_tv_fused(const TvArgs& a, int dt, bool shared, hipStream_t stream) {
  return fused_any(dt, a.grad_dt, shared, a.G, &a, stream, nullptr);
}

template <int G>
static int nv_for(int dt, bool shared) {
  const int pv = dt == kBF16 ? 8 : 4;
  return shared ? fwd_nv<FwdShape<G, true>::NR>(pv) : fwd_nv<FwdShape<G, false>::NR>(pv);
}

int tv_fwd_vec_per_thread(int dt, int G, bool shared) {
  switch (G) {
    case 1: return nv_for<1>(dt, shared);
    case 2: return nv_for<2>(dt, shared);
    case 3: return nv_for<3>(dt, shared);
    case 4: return nv_for<4>(dt, shared);
    case 5: return nv_for<5>(dt, shared);
    case 6: return nv_for<6>(dt, shared);
    case 7: return nv_for<7>(dt, shared);
    default: return nv_for<8>(dt, shared);
  }
}

int tv_fwd_part1_words(int G, bool shared) { return (shared ? 1 : G) + G; }

int tv_bwd_vec_per_thread(int dt) { return dt == kBF16 ? kBwdNVBf16 : kBwdNVF32; }

int tv_bwd_full_vec_per_thread(int dt, int G, bool shared) {
  switch (G) {
    case 1: return bwd_nv_for<1>(dt, shared);
    case 2: return bwd_nv_for<2>(dt, shared);
    case 3: return bwd_nv_for<3>(dt, shared);
    case 4: return bwd_nv_for<4>(dt, shared);
    case 5: return bwd_nv_for<5>(dt, shared);
    case 6: return bwd_nv_for<6>(dt, shared);
    case 7: return bwd_nv_for<7>(dt, shared);
    default: return bwd_nv_for<8>(dt, shared);
  }
}

template <int DT, int GDT, bool SHARED, int G>
static hipError_t launch_bwd_g(const TvArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.T * a.sp.nchunks;
  hipLaunchKernelGGL((tv_bwd_kernel<DT, GDT, G, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int GDT, bool SHARED>
static hipError_t launch_bwd3(const TvArgs& a, hipStream_t stream) {
  switch (a.G) {
    case 1: return launch_bwd_g<DT, GDT, SHARED, 1>(a, stream);
    case 2: return launch_bwd_g<DT, GDT, SHARED, 2>(a, stream);
    case 3: return launch_bwd_g<DT, GDT, SHARED, 3>(a, stream);
    case 4: return launch_bwd_g<DT, GDT, SHARED, 4>(a, stream);
    case 5: return launch_bwd_g<DT, GDT, SHARED, 5>(a, stream);
    case 6: return launch_bwd_g<DT, GDT, SHARED, 6>(a, stream);
    case 7: return launch_bwd_g<DT, GDT, SHARED, 7>(a, stream);
    case 8: return launch_bwd_g<DT, GDT, SHARED, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <int DT, int GDT>
static hipError_t launch_bwd2(const TvArgs& a, bool shared, hipStream_t stream) {
  return shared ? launch_bwd3<DT, GDT, true>(a, stream) : launch_bwd3<DT, GDT, false>(a, stream);
}

hipError_t launch_tv_bwd(const TvArgs& a, int dt, bool shared, hipStream_t stream) {
  if (dt == kBF16)
    return a.grad_dt == kBF16 ? launch_bwd2<kBF16, kBF16>(a, shared, stream) : launch_bwd2<kBF16, kF32>(a, shared, stream);
  return a.grad_dt == kBF16 ? launch_bwd2<kF32, kBF16>(a, shared, stream) : launch_bwd2<kF32, kF32>(a, shared, stream);
}

// ---------------------------------------------------------------------------
// Top-K path (paperlayer App. F: an optional top-K path keeps O(K) of the target).
// The target of head k at position t is given by K entries (vocabulary index I_j,
// logit A_j); it stands for the target truncated to them and renormalised,
// p_j = 2^(A_j log2 e - lse2_A).  With q the full softmax of the draft row,
//   alpha = clamp(sum_j min(p_j, q_{I_j}), 0, 1),  S = sum_j 1[q_{I_j} <= p_j] q_{I_j},
//   dL/dz_v = w q_v (c_v - S),  c_v = #{j : I_j = v, q_v <= p_j},
// entry by entry (an index outside [0, V) carries no mass; repeated indices count
// separately).  Forward: topk_fwd_lse streams the draft rows once (chunk
// log-sum-exp partials, one workgroup per (t, chunk)); topk_fwd_finish (one wave
// per position) merges them, takes the K entries' log-sum-exp, gathers the K draft
// logits and forms alpha and S; tv_fwd_mean averages.  Backward: one workgroup per
// (t, chunk) counts the chunk's entries whose indicator holds in LDS, then streams
// the draft chunk and writes the gradient.
template <int DT, int G>
__global__ __launch_bounds__(kBlock) void topk_fwd_lse(TvArgs a) {
  constexpr int NV = fwd_nv<G>(Elem<DT>::kPerVec);
  constexpr int NE = NV * Elem<DT>::kPerVec;
  const int C = a.sp.nchunks;
  const int t = blockIdx.x / C, c = blockIdx.x - t * C;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  __shared__ float part_sh[G][kWaves * 3];
  const char* db = reinterpret_cast<const char*>(a.draft);
  const char* rows[G];
#pragma unroll
  for (int k = 0; k < G; ++k) rows[k] = db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes;
  float x[G][NE];
  fwd_load<DT, NV, G>(a, rows, c, x);
  Lse pt[G];
  wave_pass1<NE, G, 0>(x, pt);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < G; ++k) {
      part_sh[k][wave * 3 + 0] = pt[k].ref;
      part_sh[k][wave * 3 + 1] = pt[k].z;
      part_sh[k][wave * 3 + 2] = 0.f;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const Lse m = merge_lds<kWaves, false>(part_sh[threadIdx.x]);
    reinterpret_cast<float2*>(a.part1)[((int64_t)t * C + c) * G + threadIdx.x] = make_float2(m.ref, m.z);
  }
}

template <int DT, int G>
__global__ __launch_bounds__(64 * kFinishWaves) void topk_fwd_finish(TvArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kFinishWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int C = a.sp.nchunks;
  const int K = a.K;
  const int64_t V = a.V;
  const char* db = reinterpret_cast<const char*>(a.draft);
  float al[G], ss[G], l2a[G], l2q[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    l2q[k] = fwd_row_lse2<G>(a, t, k);
    const int32_t* ii = a.idx + (int64_t)t * a.k_pos + (int64_t)k * a.k_head;
    const float* vv = a.val + (int64_t)t * a.k_pos + (int64_t)k * a.k_head;
    // log2-sum-exp of the K target logits (entries out of range count as -inf)
    float m = kNegInf;
    for (int j = lane; j < K; j += 64) {
      const int32_t i = ii[j];
      m = fmaxf(m, i >= 0 && i < V ? vv[j] : kNegInf);
    }
    m = wave_maximum(m);
    const float ref = m * kLog2e;
    float z = 0.f;
    for (int j = lane; j < K; j += 64) {
      const int32_t i = ii[j];
      if (i >= 0 && i < V) z += fast_exp2(__builtin_fmaf(vv[j], kLog2e, -ref));
    }
    z = wave_total(z);
    l2a[k] = ref + fast_log2(z);
    // the entries' overlap and S, on base-2 log-probabilities
    const char* drow = db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes;
    float ov = 0.f, s = 0.f;
    for (int j = lane; j < K; j += 64) {
      const int32_t i = ii[j];
      if (i >= 0 && i < V) {
        const float lq = __builtin_fmaf(load_one<DT>(drow, i), kLog2e, -l2q[k]);
        const float lp = __builtin_fmaf(vv[j], kLog2e, -l2a[k]);
        ov += fast_exp2(fminf(lq, lp));
        if (lq <= lp) s += fast_exp2(lq);
      }
    }
    ov = wave_total(ov);
    s = wave_total(s);
    // no finite normaliser on either side (no entry in range, NaN or -inf rows)
    const bool bad = !__builtin_isfinite(l2a[k]) || !__builtin_isfinite(l2q[k]);
    al[k] = bad ? __builtin_nanf("") : fminf(fmaxf(ov, 0.f), 1.f);
    ss[k] = bad ? __builtin_nanf("") : s;
  }
  // a call leaves every workspace word it wrote at zero
  float2* p1 = reinterpret_cast<float2*>(a.part1) + (int64_t)t * C * G;
  for (int i = lane; i < C * G; i += 64) p1[i] = make_float2(0.f, 0.f);
  if (lane == 0) {
    float prod = 1.f, l = 0.f;
    float* sv = a.saved + (int64_t)t * G * kTvSavedStride;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      prod *= al[k];
      l -= prod;
      sv[k * kTvSavedStride + 0] = l2a[k] * kLn2;
      sv[k * kTvSavedStride + 1] = l2q[k] * kLn2;
      sv[k * kTvSavedStride + 2] = al[k];
      sv[k * kTvSavedStride + 3] = ss[k];
    }
    if (a.pos_loss) a.pos_loss[t] = l;
    a.pos_ws[t] = l;
  }
}

template <int DT, int GDT>
__global__ __launch_bounds__(kBlock) void topk_bwd_kernel(TvArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NV = DT == kBF16 ? kBwdNVBf16 : kBwdNVF32;
  constexpr int NE = NV * PV;
  constexpr int kMap = kBlock * NE;           // the largest chunk, in elements
  __shared__ __align__(16) float cnt[kMap];   // indicator counts of the chunk's elements
  const int C = a.sp.nchunks;
  const int t = blockIdx.x / C, c = blockIdx.x - (blockIdx.x / C) * C;
  const int G = a.G, K = a.K;
  const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
  const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);
  const int64_t ebeg = vbeg * PV, eend = min(vend * PV, a.V);
  for (int i = threadIdx.x; i < kMap; i += kBlock) cnt[i] = 0.f;

  const float* sv = a.saved_in + (int64_t)t * G * kTvSavedStride;
  float alpha[kTvMaxHeads];
  for (int k = 0; k < G; ++k) alpha[k] = sv[k * kTvSavedStride + 2];
  const float gscale = -a.grad_loss[0] / (float)a.T;

  const char* db = reinterpret_cast<const char*>(a.draft);
  char* gb = reinterpret_cast<char*>(a.grad);
  constexpr int gbytes = GDT == kBF16 ? 2 : 4;
  for (int k = 0; k < G; ++k) {
    const char* drow = db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes;
    const char* const rows[1] = {drow};
    RawChunk<NV, 1> raw;
    issue_rows<DT, NV, 1>(raw, rows, vbeg, a.sp);   // the chunk's loads go out first
    float wsum = 0.f;
    for (int kk = k; kk < G; ++kk) {
      float prod = 1.f;
      for (int i = 0; i <= kk; ++i)
        if (i != k) prod *= alpha[i];
      wsum += prod;
    }
    const float w = gscale * wsum;
    const float lse_a = sv[k * kTvSavedStride + 0], lse_q = sv[k * kTvSavedStride + 1];
    const float S = sv[k * kTvSavedStride + 3];
    const float dl = lse_q - lse_a;
    const int32_t* ii = a.idx + (int64_t)t * a.k_pos + (int64_t)k * a.k_head;
    const float* vv = a.val + (int64_t)t * a.k_pos + (int64_t)k * a.k_head;
    __syncthreads();   // the map is clear (initial zeroing or the previous head's reset)
    // log q_v <= log p_j  <=>  z_v - A_j <= lse_q - lse_A
    for (int j = threadIdx.x; j < K; j += kBlock) {
      const int64_t i = ii[j];
      if (i >= ebeg && i < eend && load_one<DT>(drow, i) - vv[j] <= dl) atomicAdd(&cnt[i - ebeg], 1.f);
    }
    __syncthreads();
    float x[1][NE], gr[NE];
    unpack_rows<DT, NV, 1>(raw, rows, vbeg, vend, a.sp, a.V, x);
    const float lq2 = lse_q * kLog2e;
    const float c0 = -w * S;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float cv[PV];
      const float4* cp = reinterpret_cast<const float4*>(cnt + (j * kBlock + threadIdx.x) * PV);
#pragma unroll
      for (int h = 0; h < PV / 4; ++h) {
        const float4 f = cp[h];
        cv[4 * h] = f.x; cv[4 * h + 1] = f.y; cv[4 * h + 2] = f.z; cv[4 * h + 3] = f.w;
      }
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        const float q = fast_exp2(__builtin_fmaf(x[0][j * PV + e], kLog2e, -lq2));
        gr[j * PV + e] = q * __builtin_fmaf(w, cv[e], c0);
      }
    }
    char* grow = gb + ((int64_t)t * a.g_pos + (int64_t)k * a.g_head) * gbytes;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t vi = vbeg + (int64_t)j * kBlock + threadIdx.x;
      if (vi < vend) store_grad<GDT, PV>(grow, vi, a.sp, a.V, gr + j * PV);
    }
    __syncthreads();   // every thread has read the map
    for (int j = threadIdx.x; j < K; j += kBlock) {
      const int64_t i = ii[j];
      if (i >= ebeg && i < eend) cnt[i - ebeg] = 0.f;
    }
  }
}

template <int DT, int G>
static hipError_t launch_topk_fwd_g(const TvArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.T * a.sp.nchunks;
  hipLaunchKernelGGL((topk_fwd_lse<DT, G>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_fwd_finish<DT, G>), dim3((unsigned)((a.T + kFinishWaves - 1) / kFinishWaves)),
                     dim3(64 * kFinishWaves), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tv_fwd_mean, dim3(1), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_topk_fwd_dt(const TvArgs& a, hipStream_t stream) {
  switch (a.G) {
    case 1: return launch_topk_fwd_g<DT, 1>(a, stream);
    case 2: return launch_topk_fwd_g<DT, 2>(a, stream);
    case 3: return launch_topk_fwd_g<DT, 3>(a, stream);
    case 4: return launch_topk_fwd_g<DT, 4>(a, stream);
    case 5: return launch_topk_fwd_g<DT, 5>(a, stream);
    case 6: return launch_topk_fwd_g<DT, 6>(a, stream);
    case 7: return launch_topk_fwd_g<DT, 7>(a, stream);
    case 8: return launch_topk_fwd_g<DT, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tv_topk_fwd(const TvArgs& a, int dt, hipStream_t stream) {
  return dt == kBF16 ? launch_topk_fwd_dt<kBF16>(a, stream) : launch_topk_fwd_dt<kF32>(a, stream);
}

int tv_topk_fwd_vec_per_thread(int dt, int G) {
  const int pv = dt == kBF16 ? 8 : 4;
  switch (G) {
    case 1: return fwd_nv<1>(pv);
    case 2: return fwd_nv<2>(pv);
    case 3: return fwd_nv<3>(pv);
    case 4: return fwd_nv<4>(pv);
    case 5: return fwd_nv<5>(pv);
    case 6: return fwd_nv<6>(pv);
    case 7: return fwd_nv<7>(pv);
    default: return fwd_nv<8>(pv);
  }
}

template <int DT, int GDT>
static hipError_t launch_topk_bwd2(const TvArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.T * a.sp.nchunks;
  hipLaunchKernelGGL((topk_bwd_kernel<DT, GDT>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_tv_topk_bwd(const TvArgs& a, int dt, hipStream_t stream) {
  if (dt == kBF16)
    return a.grad_dt == kBF16 ? launch_topk_bwd2<kBF16, kBF16>(a, stream) : launch_topk_bwd2<kBF16, kF32>(a, stream);
  return a.grad_dt == kBF16 ? launch_topk_bwd2<kF32, kBF16>(a, stream) : launch_topk_bwd2<kF32, kF32>(a, stream);
}

}  // namespace mtp
