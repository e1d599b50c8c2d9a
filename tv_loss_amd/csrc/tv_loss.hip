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
// Forward: C workgroups split each position's rows along the vocabulary and sweep
// the positions in layers (tv_fwd_main).  Per layer a workgroup keeps its chunk of
// the target row(s) and of the gamma draft rows in registers while the next
// layer's chunk is in flight, publishes its log-sum-exp partials as a
// self-announcing record, polls its siblings' records, and computes its overlap
// and S partials from registers.  tv_fwd_finish (one wave per position) sums the
// partials in a fixed order and writes l_t and the saved statistics; tv_fwd_mean
// writes the mean.  Every logit is read from HBM once.
// Backward: pure streaming; each workgroup reads one chunk of the target and draft
// rows of one position plus the saved statistics, and writes the gradient chunk.
// The indicator is evaluated on logits, z_v - a_v <= lse_q - lse_p, so no
// exponential of the target is needed.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mtp {

template <int NE>
__device__ __forceinline__ Lse thread_lse_plain(float (&x)[NE]) {
  float m = x[0];
#pragma unroll
  for (int i = 1; i < NE; ++i) m = fmaxf(m, x[i]);
  const bool empty = !(m > kNegInf);
  const float ref = empty ? 0.f : m * kLog2e;
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const float e = fast_exp2(__builtin_fmaf(x[i], kLog2e, -ref));
    z += e;
    x[i] = e;
  }
  if (empty && z == 0.f) return lse_empty();
  return Lse{ref, z, 0.f};
}

// Wave 0 polls the C pass-1 records (NR words (ref, z) each) of the position and
// merges them in one fixed order; log2-sum-exp per row is broadcast through LDS.
template <int NR>
__device__ __forceinline__ void merge_rows(const uint64_t* p1, int C, float (&lse2)[NR], float* lds,
                                           uint32_t* err) {
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    Lse acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = lse_empty();
    for (int c0 = 0; c0 < C; c0 += 64) {
      uint64_t w[NR];
      wave_poll<NR>(p1, c0, C, w, err);
      if (c0 + lane < C) {
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = lse_merge(acc[r], Lse{unpack_lo(w[r]), unmark(unpack_hi(w[r])), 0.f});
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const Lse m = wave_lse(acc[r]);
      if (lane == 0) lds[r] = lse_log2(m);
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r) lse2[r] = lds[r];
  __syncthreads();
}

// Vectors per thread and row: about 64 bf16 or 32 fp32 values per thread in all
// (their raw words for the next layer are in flight at the same time).
template <int G>
constexpr int fwd_nv(int per_vec, bool shared) {
  const int rows = (shared ? 1 : G) + G;
  const int budget = per_vec == 8 ? 64 : 32;
  const int nv = budget / (rows * per_vec);
  return nv < 1 ? 1 : nv;
}

// Forward main kernel: super-groups of C workgroups sweep the positions of their
// XCD in layers (position (sg + i * S) * 8 + xcd at layer i), prefetching the next
// layer's chunk; per layer one record poll, then the chunk's overlap and S
// partials from registers.
template <int DT, int G, bool SHARED>
__global__ __launch_bounds__(kBlock, kTvFwdBlocksPerCU) void tv_fwd_main(TvArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NV = fwd_nv<G>(PV, SHARED);
  constexpr int NE = NV * PV;
  constexpr int NT = SHARED ? 1 : G;
  constexpr int NR = NT + G;
  const int C = a.sp.nchunks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int sg = slot / C, c = slot - sg * C;
  int nl = 0;
  while (nl < a.layers && (int64_t)(sg + nl * a.sgroups) * 8 + xcd < a.T) ++nl;
  if (nl == 0) return;
  const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
  const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);

  __shared__ float lds[3 * kWaves * NR + 2 * kWaves * G];

  auto rows_of = [&](int t, const char* (&rows)[NR]) {
    const char* tb = reinterpret_cast<const char*>(a.target);
    const char* db = reinterpret_cast<const char*>(a.draft);
#pragma unroll
    for (int r = 0; r < NT; ++r) rows[r] = tb + ((int64_t)t * a.t_pos + (int64_t)r * a.t_head) * Elem<DT>::kBytes;
#pragma unroll
    for (int k = 0; k < G; ++k) rows[NT + k] = db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes;
  };

  RawChunk<NV, NR> raw;
  {
    const char* rows[NR];
    rows_of(sg * 8 + xcd, rows);
    issue_rows<DT, NV, NR>(raw, rows, vbeg, a.sp);
  }
  for (int i = 0; i < nl; ++i) {
    const int t = (sg + i * a.sgroups) * 8 + xcd;
    const char* rows[NR];
    rows_of(t, rows);
    float x[NR][NE];
    unpack_rows<DT, NV, NR>(raw, rows, vbeg, vend, a.sp, a.V, x);
    if (i + 1 < nl) {   // prefetch the next layer's chunk
      const char* nrows[NR];
      rows_of((sg + (i + 1) * a.sgroups) * 8 + xcd, nrows);
      issue_rows<DT, NV, NR>(raw, nrows, vbeg, a.sp);
    }

    // ---- pass 1 --------------------------------------------------------------
    Lse parts[NR];
    float refs[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) { parts[r] = thread_lse_plain<NE>(x[r]); refs[r] = parts[r].ref; }
    block_lse<NR>(parts, lds);
    uint64_t* p1 = a.part1 + (int64_t)t * C * NR;
    if (threadIdx.x == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) put_word(p1 + (int64_t)c * NR + r, pack2(parts[r].ref, mark(parts[r].z)));
    }
    float lse2[NR];
    merge_rows<NR>(p1, C, lse2, lds, a.err);

    // ---- pass 2: overlap and S from registers ------------------------------
    float s[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) s[r] = fast_exp2(refs[r] - lse2[r]);
    float acc[2 * G];
#pragma unroll
    for (int k = 0; k < 2 * G; ++k) acc[k] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const float p0 = x[0][e] * s[0];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const float p = SHARED ? p0 : x[SHARED ? 0 : k][e] * s[SHARED ? 0 : k];
        const float q = x[NT + k][e] * s[NT + k];
        const bool ind = q <= p;
        acc[2 * k] += ind ? q : p;
        acc[2 * k + 1] += ind ? q : 0.f;
      }
    }
    block_sum<2 * G>(acc, lds);
    if (threadIdx.x == 0) {
      float* mine = a.part2 + ((int64_t)t * C + c) * 2 * G;
#pragma unroll
      for (int k = 0; k < 2 * G; ++k) st_coherent(mine + k, acc[k]);
    }
  }
}

// Forward finish: one wave per position sums the chunk partials in a fixed order
// and writes the position's statistics, then clears the position's records.
constexpr int kFinishWaves = 4;

template <int G, bool SHARED>
__global__ __launch_bounds__(64 * kFinishWaves) void tv_fwd_finish(TvArgs a) {
  constexpr int NT = SHARED ? 1 : G;
  constexpr int NR = NT + G;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kFinishWaves + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int C = a.sp.nchunks;
  uint64_t* p1 = a.part1 + (int64_t)t * C * NR;
  const float* p2 = a.part2 + (int64_t)t * C * 2 * G;
  Lse acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = lse_empty();
  float tot[2 * G];
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) tot[k] = 0.f;
  for (int c = lane; c < C; c += 64) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint64_t w = get_word(p1 + (int64_t)c * NR + r);
      acc[r] = lse_merge(acc[r], Lse{unpack_lo(w), unmark(unpack_hi(w)), 0.f});
    }
#pragma unroll
    for (int k = 0; k < 2 * G; ++k) tot[k] += ld_coherent(p2 + (int64_t)c * 2 * G + k);
  }
  float lse2[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) lse2[r] = lse_log2(wave_lse(acc[r]));
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) tot[k] = wave_sum(tot[k]);
  // a call leaves every workspace word it wrote at zero
  for (int c = lane; c < C; c += 64) {
#pragma unroll
    for (int r = 0; r < NR; ++r) put_word(p1 + (int64_t)c * NR + r, 0ull);
#pragma unroll
    for (int k = 0; k < 2 * G; ++k) st_coherent(const_cast<float*>(p2) + (int64_t)c * 2 * G + k, 0.f);
  }
  if (lane == 0) {
    float prod = 1.f, l = 0.f;
    float* sv = a.saved + (int64_t)t * G * kTvSavedStride;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float al = fminf(fmaxf(tot[2 * k], 0.f), 1.f);
      prod *= al;
      l -= prod;
      sv[k * kTvSavedStride + 0] = lse2[SHARED ? 0 : k] * kLn2;
      sv[k * kTvSavedStride + 1] = lse2[NT + k] * kLn2;
      sv[k * kTvSavedStride + 2] = al;
      sv[k * kTvSavedStride + 3] = tot[2 * k + 1];
    }
    if (a.pos_loss) a.pos_loss[t] = l;
    st_coherent(a.pos_ws + t, l);
  }
}

// The mean over positions, in one fixed order.
__global__ __launch_bounds__(kBlock) void tv_fwd_mean(TvArgs a) {
  __shared__ float lds[kWaves];
  float sum[1] = {0.f};
  for (int i = threadIdx.x; i < a.T; i += kBlock) sum[0] += ld_coherent(a.pos_ws + i);
  block_sum<1>(sum, lds);
  for (int i = threadIdx.x; i < a.T; i += kBlock) st_coherent(a.pos_ws + i, 0.f);
  if (threadIdx.x == 0) a.loss[0] = sum[0] / (float)a.T;
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

template <int DT, int GDT, bool SHARED>
__global__ __launch_bounds__(kBlock) void tv_bwd_kernel(TvArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NV = DT == kBF16 ? kBwdNVBf16 : kBwdNVF32;
  constexpr int NE = NV * PV;
  const int C = a.sp.nchunks;
  const int t = blockIdx.x / C, c = blockIdx.x - (blockIdx.x / C) * C;
  const int G = a.G;
  const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
  const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);

  // end-to-end weights of this position
  const float* sv = a.saved_in + (int64_t)t * G * kTvSavedStride;
  float alpha[kTvMaxHeads];
  for (int k = 0; k < G; ++k) alpha[k] = sv[k * kTvSavedStride + 2];
  const float gscale = -a.grad_loss[0] / (float)a.T;

  const char* tb = reinterpret_cast<const char*>(a.target);
  const char* db = reinterpret_cast<const char*>(a.draft);
  char* gb = reinterpret_cast<char*>(a.grad);
  constexpr int gbytes = GDT == kBF16 ? 2 : 4;
  float xv[2][NE], gr[NE];
  float (&xt)[NE] = xv[0];
  float (&xd)[NE] = xv[1];
  if (SHARED) {
    const char* const rows[1] = {tb + (int64_t)t * a.t_pos * Elem<DT>::kBytes};
    load_rows<DT, NV, 1>(rows, vbeg, vend, a.sp, a.V, *reinterpret_cast<float(*)[1][NE]>(&xv[0]));
  }
  for (int k = 0; k < G; ++k) {
    const char* drow = db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes;
    if (!SHARED) {
      const char* const rows[2] = {tb + ((int64_t)t * a.t_pos + (int64_t)k * a.t_head) * Elem<DT>::kBytes, drow};
      load_rows<DT, NV, 2>(rows, vbeg, vend, a.sp, a.V, xv);
    } else {
      const char* const rows[1] = {drow};
      load_rows<DT, NV, 1>(rows, vbeg, vend, a.sp, a.V, *reinterpret_cast<float(*)[1][NE]>(&xv[1]));
    }
    float wsum = 0.f;
    for (int kk = k; kk < G; ++kk) {
      float prod = 1.f;
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
template <int DT, bool SHARED, int G>
static hipError_t launch_fwd_g(const TvArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.sgroups * a.sp.nchunks * 8;
  hipLaunchKernelGGL((tv_fwd_main<DT, G, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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

int tv_fwd_vec_per_thread(int dt, int G, bool shared) {
  switch (G) {
    case 1: return fwd_nv<1>(dt == kBF16 ? 8 : 4, shared);
    case 2: return fwd_nv<2>(dt == kBF16 ? 8 : 4, shared);
    case 3: return fwd_nv<3>(dt == kBF16 ? 8 : 4, shared);
    case 4: return fwd_nv<4>(dt == kBF16 ? 8 : 4, shared);
    case 5: return fwd_nv<5>(dt == kBF16 ? 8 : 4, shared);
    case 6: return fwd_nv<6>(dt == kBF16 ? 8 : 4, shared);
    case 7: return fwd_nv<7>(dt == kBF16 ? 8 : 4, shared);
    default: return fwd_nv<8>(dt == kBF16 ? 8 : 4, shared);
  }
}

int tv_fwd_part1_words(int G, bool shared) { return (shared ? 1 : G) + G; }

template <int DT, bool SHARED, int G>
static hipError_t occ_g(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, tv_fwd_main<DT, G, SHARED>, kBlock, 0);
}

template <int DT, bool SHARED>
static hipError_t occ_dt(int G, int* n) {
  switch (G) {
    case 1: return occ_g<DT, SHARED, 1>(n);
    case 2: return occ_g<DT, SHARED, 2>(n);
    case 3: return occ_g<DT, SHARED, 3>(n);
    case 4: return occ_g<DT, SHARED, 4>(n);
    case 5: return occ_g<DT, SHARED, 5>(n);
    case 6: return occ_g<DT, SHARED, 6>(n);
    case 7: return occ_g<DT, SHARED, 7>(n);
    case 8: return occ_g<DT, SHARED, 8>(n);
  }
  return hipErrorInvalidValue;
}

hipError_t tv_fwd_occupancy(int dt, int G, bool shared, int* n) {
  if (dt == kBF16) return shared ? occ_dt<kBF16, true>(G, n) : occ_dt<kBF16, false>(G, n);
  return shared ? occ_dt<kF32, true>(G, n) : occ_dt<kF32, false>(G, n);
}

int tv_bwd_vec_per_thread(int dt) { return dt == kBF16 ? kBwdNVBf16 : kBwdNVF32; }

template <int DT, int GDT, bool SHARED>
static hipError_t launch_bwd3(const TvArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.T * a.sp.nchunks;
  hipLaunchKernelGGL((tv_bwd_kernel<DT, GDT, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
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

}  // namespace mtp
