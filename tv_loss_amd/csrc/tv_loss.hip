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
// Forward: one cluster per position t.  Each workgroup keeps one vocabulary chunk
// of the target row(s) and of the gamma draft rows in registers, publishes its
// log-sum-exp partials, waits for the cluster, then computes its overlap and S
// partials from registers.  The last workgroup of the cluster reduces them in a
// fixed order and writes l_t and the saved statistics; the last position to
// finish writes the mean.  Every logit is read from HBM once.
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

// Wave 0 merges the C chunk partials (ref, z) of NR rows with coherent loads in a
// fixed order and broadcasts log2-sum-exp per row through LDS.
template <int NR>
__device__ __forceinline__ void merge_rows(const float* p1, int C, float (&lse2)[NR], float* lds) {
  constexpr int P1S = 2 * NR;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      Lse acc = lse_empty();
      for (int c = lane; c < C; c += 64) {
        const float* q = p1 + (int64_t)c * P1S + 2 * r;
        acc = lse_merge(acc, Lse{ld_coherent(q), ld_coherent(q + 1), 0.f});
      }
      acc = wave_lse(acc);
      if (lane == 0) lds[r] = lse_log2(acc);
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r) lse2[r] = lds[r];
  __syncthreads();
}

template <int G>
constexpr int fwd_nv(int per_vec, bool shared) {
  const int rows = (shared ? 1 : G) + G;
  const int nv = 64 / (rows * per_vec);
  return nv < 1 ? 1 : nv;
}

template <int DT, int G, bool SHARED>
__global__ __launch_bounds__(kBlock) void tv_fwd_kernel(TvArgs a) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr int NV = fwd_nv<G>(PV, SHARED);
  constexpr int NE = NV * PV;
  constexpr int NT = SHARED ? 1 : G;
  constexpr int NR = NT + G;
  constexpr int P1S = 2 * NR;
  const int C = a.sp.nchunks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int lg = slot / C, c = slot - lg * C;
  const int t = lg * 8 + xcd;
  if (t >= a.T) return;
  const int64_t vbeg = (int64_t)c * a.sp.vec_per_chunk;
  const int64_t vend = min(vbeg + a.sp.vec_per_chunk, a.sp.nvec);

  __shared__ float lds[3 * kWaves * NR + 2 * kWaves * G];
  __shared__ int last_in_cluster, last_position;

  float xt[NT][NE], xd[G][NE];
  const char* tb = reinterpret_cast<const char*>(a.target);
  const char* db = reinterpret_cast<const char*>(a.draft);
#pragma unroll
  for (int r = 0; r < NT; ++r)
    load_chunk<DT, NV>(tb + ((int64_t)t * a.t_pos + (int64_t)r * a.t_head) * Elem<DT>::kBytes,
                       vbeg, vend, a.sp, a.V, xt[r]);
#pragma unroll
  for (int k = 0; k < G; ++k)
    load_chunk<DT, NV>(db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes,
                       vbeg, vend, a.sp, a.V, xd[k]);

  // ---- pass 1 ----------------------------------------------------------------
  Lse parts[NR];
  float refs[NR];
#pragma unroll
  for (int r = 0; r < NT; ++r) { parts[r] = thread_lse_plain<NE>(xt[r]); refs[r] = parts[r].ref; }
#pragma unroll
  for (int k = 0; k < G; ++k) { parts[NT + k] = thread_lse_plain<NE>(xd[k]); refs[NT + k] = parts[NT + k].ref; }
  block_lse<NR>(parts, lds);
  float* p1 = a.part1 + (int64_t)t * C * P1S;
  int* cnt = a.grp_cnt + (int64_t)t * kCounterStride;
  if (threadIdx.x == 0) {
    float* mine = p1 + (int64_t)c * P1S;
#pragma unroll
    for (int r = 0; r < NR; ++r) { st_coherent(mine + 2 * r, parts[r].ref); st_coherent(mine + 2 * r + 1, parts[r].z); }
    arrive(cnt);
  }
  block_wait(cnt, C, a.err);
  float lse2[NR];
  merge_rows<NR>(p1, C, lse2, lds);

  // ---- pass 2: overlap and S from registers ----------------------------------
  float s[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) s[r] = fast_exp2(refs[r] - lse2[r]);
  float acc[2 * G];
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) acc[k] = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const float p0 = xt[0][i] * s[0];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float p = SHARED ? p0 : xt[SHARED ? 0 : k][i] * s[SHARED ? 0 : k];
      const float q = xd[k][i] * s[NT + k];
      const bool ind = q <= p;
      acc[2 * k] += ind ? q : p;
      acc[2 * k + 1] += ind ? q : 0.f;
    }
  }
  block_sum<2 * G>(acc, lds);
  float* p2 = a.part2 + (int64_t)t * C * 2 * G;
  if (threadIdx.x == 0) {
    float* mine = p2 + (int64_t)c * 2 * G;
#pragma unroll
    for (int k = 0; k < 2 * G; ++k) st_coherent(mine + k, acc[k]);
    const int old = arrive(cnt);
    last_in_cluster = old == 2 * C - 1;
  }
  __syncthreads();
  if (!last_in_cluster) return;

  // ---- last workgroup of the cluster: position statistics --------------------
  const int lane = threadIdx.x & 63;
  float tot[2 * G];
#pragma unroll
  for (int k = 0; k < 2 * G; ++k) {
    float v = 0.f;
    for (int cc = lane; cc < C; cc += 64) v += ld_coherent(p2 + (int64_t)cc * 2 * G + k);
    tot[k] = wave_sum(v);
  }
  __syncthreads();   // every wave has read the partials: clear them for the next call
  block_zero(p1, (int64_t)C * P1S);
  block_zero(p2, (int64_t)C * 2 * G);
  if (threadIdx.x == 0) {
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
    reset_counter(cnt);
    const int old = arrive(a.glob_cnt);
    last_position = old == a.T - 1;
  }
  __syncthreads();
  if (!last_position) return;
  float sum[1] = {0.f};
  for (int i = threadIdx.x; i < a.T; i += kBlock) sum[0] += ld_coherent(a.pos_ws + i);
  block_sum<1>(sum, lds);
  block_zero(a.pos_ws, a.T);
  if (threadIdx.x == 0) {
    a.loss[0] = sum[0] / (float)a.T;
    reset_counter(a.glob_cnt);
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
  float xt[NE], xd[NE], gr[NE];
  if (SHARED) load_chunk<DT, NV>(tb + (int64_t)t * a.t_pos * Elem<DT>::kBytes, vbeg, vend, a.sp, a.V, xt);
  for (int k = 0; k < G; ++k) {
    if (!SHARED)
      load_chunk<DT, NV>(tb + ((int64_t)t * a.t_pos + (int64_t)k * a.t_head) * Elem<DT>::kBytes, vbeg, vend,
                         a.sp, a.V, xt);
    load_chunk<DT, NV>(db + ((int64_t)t * a.d_pos + (int64_t)k * a.d_head) * Elem<DT>::kBytes, vbeg, vend,
                       a.sp, a.V, xd);
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
  const int C = a.sp.nchunks;
  const int64_t grid = (int64_t)((a.T + 7) / 8) * C * 8;
  hipLaunchKernelGGL((tv_fwd_kernel<DT, G, SHARED>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
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
  const int pv = dt == kBF16 ? 8 : 4;
  const int rows = (shared ? 1 : G) + G;
  const int nv = 64 / (rows * pv);
  return nv < 1 ? 1 : nv;
}

int tv_fwd_part1_stride(int G, bool shared) { return 2 * ((shared ? 1 : G) + G); }

template <int DT, bool SHARED, int G>
static hipError_t occ_g(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, tv_fwd_kernel<DT, G, SHARED>, kBlock, 0);
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
