// Device building blocks shared by the verify and TV-loss kernels (gfx950, wave64).
//
//  * 16-byte row streaming with bf16 -> fp32 unpacking (a bf16 is the top half of
//    a binary32, so widening is a shift or a mask);
//  * the online log-sum-exp partial (reference, sum, entropy moment) and its
//    order-independent merge;
//  * wave butterflies and 256-thread block reductions that leave every lane with
//    bitwise-identical results (so every workgroup of a cluster derives the
//    same row statistics from the same partials);
//  * the cluster exchange: publish / arrive / bounded wait at agent scope;
//  * Philox4x32-10 (Salmon et al., SC'11) for the verify uniforms.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

constexpr int kBlock = 256;           // threads per workgroup: 4 wave64s
constexpr int kWaves = kBlock / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// dtype codes (match the C ABI)
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

template <int DT> struct Elem;
template <> struct Elem<kF32> { static constexpr int kPerVec = 4; static constexpr int kBytes = 4; };
template <> struct Elem<kBF16> { static constexpr int kPerVec = 8; static constexpr int kBytes = 2; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// x clamped to [0, 1]: folds into the producing instruction's output clamp (which
// also turns a NaN into 0)
__device__ __forceinline__ float clamp01(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 1.f); }

// The reference of a pass-1 partial: m L moved up past its rounding.  r = fl(m L)
// lies within half a unit in the last place of the exact product, and
// fl(r + |r| 2^-23) lies one or two units above r (toward +inf for either sign), so
// every logit x <= m has x L - ref < 0 exactly in the fused multiply-add and
// e = 2^(x L - ref) <= 1 (the pass-2 sums rely on it: their maxima are [0, 1] output
// clamps).  Where |r| < 2^-103 the increment underflows and x L - ref is within a
// subnormal of 0, whose exp2 is 1 in float32.  +-inf and NaN pass through.
__device__ __forceinline__ float ref_up(float m, float L) {
  const float r = m * L;
  return __builtin_fmaf(__builtin_fabsf(r), 0x1p-23f, r);
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// The ratio z_a / z_b of two normalisers from the reciprocal rz_b = 1 / z_b (one
// unit of rounding), and exactly 1 for equal normalisers, so that two rows of the
// same logits get exactly the same units (p = q exactly there).
__device__ __forceinline__ float z_ratio(float za, float zb, float rzb) { return za == zb ? 1.f : za * rzb; }

// Geometry of one row split into `nchunks` chunks of whole 16-byte vectors.
struct RowSplit {
  int64_t nvec;        // vectors covering the row (the last may be partial)
  int64_t nvec_full;   // vectors lying entirely inside the row
  int64_t vec_per_chunk;
  int nchunks;
};

// balanced: chunks of equal size (each a little under the capacity); otherwise
// every chunk but the last is full, so that only the last chunk has partly filled
// wave segments.
__host__ __device__ inline RowSplit make_split(int64_t V, int per_vec, int vec_per_thread, bool balanced = true) {
  RowSplit s;
  s.nvec = (V + per_vec - 1) / per_vec;
  s.nvec_full = V / per_vec;
  const int64_t cap = (int64_t)kBlock * vec_per_thread;
  s.nchunks = (int)((s.nvec + cap - 1) / cap);
  s.vec_per_chunk = balanced ? (s.nvec + s.nchunks - 1) / s.nchunks : cap;
  return s;
}

// Loading a chunk of R rows: this thread's NV 16-byte vectors per row.  Element
// (j, e) of the thread is vocabulary index (vbeg + j*kBlock + tid) * PV + e.
//
// issue_rows() puts every load of every row in flight at once (unconditional, at
// addresses clamped into the row), so a chunk costs one memory round trip and can
// be prefetched while earlier data is processed.  unpack_rows() turns the raw
// words into floats, -inf outside the chunk or the row; the row's partial last
// vector, if the chunk holds it, is read element by element.
template <int NV, int R>
struct RawChunk {
  u32x4 v[R][NV];
};

template <int DT, int NV, int R>
__device__ __forceinline__ void issue_rows(RawChunk<NV, R>& raw, const char* const (&rows)[R], int64_t vbeg,
                                           const RowSplit& sp) {
  const int tid = threadIdx.x;
  if (sp.nvec_full > 0) {
    const int64_t last = sp.nvec_full - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int64_t vi = min(vbeg + (int64_t)j * kBlock + tid, last);
        raw.v[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows[r]) + vi);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < NV; ++j) raw.v[r][j] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int DT, int NV, int R>
__device__ __forceinline__ void unpack_rows(const RawChunk<NV, R>& raw, const char* const (&rows)[R], int64_t vbeg,
                                            int64_t vend, const RowSplit& sp, int64_t V,
                                            float (&x)[R][NV * Elem<DT>::kPerVec]) {
  constexpr int PV = Elem<DT>::kPerVec;
  // a masked word reads as -inf in every element it holds
  constexpr uint32_t kMasked = DT == kBF16 ? 0xFF80FF80u : 0xFF800000u;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = vbeg + (int64_t)j * kBlock + tid;
    const bool full = vi < vend && vi < sp.nvec_full;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t word = full ? raw.v[r][j][w] : kMasked;
        if constexpr (DT == kBF16) {
          x[r][j * PV + 2 * w] = bf16_lo(word);
          x[r][j * PV + 2 * w + 1] = bf16_hi(word);
        } else {
          x[r][j * PV + w] = __uint_as_float(word);
        }
      }
    }
  }
  // the row's partial last vector (V not a multiple of PV), if this chunk holds it
  const int64_t tail = sp.nvec_full;
  if (sp.nvec != sp.nvec_full && vbeg <= tail && tail < vend) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (vbeg + (int64_t)j * kBlock + tid == tail) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int e = 0; e < PV; ++e) {
            const int64_t idx = tail * PV + e;
            if (idx < V) {
              if constexpr (DT == kBF16) {
                x[r][j * PV + e] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(rows[r])[idx] << 16);
              } else {
                x[r][j * PV + e] = reinterpret_cast<const float*>(rows[r])[idx];
              }
            }
          }
        }
      }
    }
  }
}

template <int DT, int NV, int R>
__device__ __forceinline__ void load_rows(const char* const (&rows)[R], int64_t vbeg, int64_t vend,
                                          const RowSplit& sp, int64_t V,
                                          float (&x)[R][NV * Elem<DT>::kPerVec]) {
  RawChunk<NV, R> raw;
  issue_rows<DT, NV, R>(raw, rows, vbeg, sp);
  unpack_rows<DT, NV, R>(raw, rows, vbeg, vend, sp, V, x);
}

// Scalar load of one logit.
template <int DT>
__device__ __forceinline__ float load_one(const void* row, int64_t idx) {
  if constexpr (DT == kBF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[idx] << 16);
  } else {
    return reinterpret_cast<const float*>(row)[idx];
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp partials.  A partial over a set of logits a_i, in base-2 units:
//   ref = m * log2(e) rounded once (m = max a_i; -inf for an empty set),
//   z   = sum_i 2^(a_i log2 e - ref),
//   y   = sum_i 2^(a_i log2 e - ref) * (a_i log2 e - ref)   (entropy moment).
// Then lse = (ref + log2 z) ln 2 and H = ln 2 (log2 z - y / z).
struct Lse {
  float ref, z, y;
};

__device__ __forceinline__ Lse lse_empty() { return Lse{kNegInf, 0.f, 0.f}; }

// Merge two partials.  NaN anywhere gives NaN; an empty partial (z = 0) is the
// identity.  Non-empty operands are put in a canonical order first, so the result
// does not depend on which side each came from (bitwise), whatever the compiler
// contracts into FMAs.
__device__ __forceinline__ Lse lse_merge(Lse a, Lse b) {
  if (a.z != a.z || b.z != b.z || a.ref != a.ref || b.ref != b.ref || a.y != a.y || b.y != b.y) {
    const float nan = __builtin_nanf("");
    return Lse{nan, nan, nan};
  }
  if (!(a.z > 0.f)) return (b.z > 0.f) ? b : lse_empty();
  if (!(b.z > 0.f)) return a;
  const bool swap = (b.ref > a.ref) || (b.ref == a.ref && (b.z > a.z || (b.z == a.z && b.y > a.y)));
  if (swap) { Lse t = a; a = b; b = t; }
  const float d = b.ref - a.ref;        // <= 0
  const float f = fast_exp2(d);
  const float z = a.z + b.z * f;
  const float y = a.y + (b.y + d * b.z) * f;
  return Lse{a.ref, z, y};
}

__device__ __forceinline__ float lse_log2(const Lse& s) { return s.ref + fast_log2(s.z); }

// ---------------------------------------------------------------------------
// Wave64 butterflies: every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ Lse wave_lse(Lse s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Lse t{__shfl_xor(s.ref, o, 64), __shfl_xor(s.z, o, 64), __shfl_xor(s.y, o, 64)};
    s = lse_merge(s, t);
  }
  return s;
}

// Block (256-thread) reductions through LDS; results identical in every thread.
// `scratch` holds at least kWaves * N floats.  Ends with a barrier-free read, so
// callers must not reuse `scratch` before the next __syncthreads().
template <int N>
__device__ __forceinline__ void block_sum(float (&v)[N], float* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) scratch[i * kWaves + wave] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float* s = scratch + i * kWaves;
    v[i] = (s[0] + s[1]) + (s[2] + s[3]);
  }
}

template <int N>
__device__ __forceinline__ void block_lse(Lse (&v)[N], float* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_lse(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      scratch[(i * kWaves + wave) * 3 + 0] = v[i].ref;
      scratch[(i * kWaves + wave) * 3 + 1] = v[i].z;
      scratch[(i * kWaves + wave) * 3 + 2] = v[i].y;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float* s = scratch + i * kWaves * 3;
    Lse w0{s[0], s[1], s[2]}, w1{s[3], s[4], s[5]}, w2{s[6], s[7], s[8]}, w3{s[9], s[10], s[11]};
    v[i] = lse_merge(lse_merge(w0, w1), lse_merge(w2, w3));
  }
}

// ---------------------------------------------------------------------------
// Cluster exchange.  Data shared between workgroups of one launch goes through
// device-coherent accesses (relaxed agent-scope atomics: sc1 loads and stores on
// gfx950), so no L2 writeback or invalidation is needed: a publisher writes its
// partials with coherent stores, waits for them to complete (s_waitcnt), then
// increments the cluster counter; a consumer polls the counter with coherent
// loads and then reads the partials with coherent loads.  Waits are bounded by the
// 100 MHz real-time counter (the limit is a kernel argument: 1 s by default) so
// that no wave can spin forever; a timeout sets `err` and the caller carries on
// with statistics it marks as NaN, so the affected rows are reported as failed.
constexpr uint64_t kDefaultWaitLimitTicks = 100000000ull;   // 1 s of the 100 MHz counter
constexpr uint32_t kErrSyncTimeout = 1u;

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coherent(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait for every outstanding vector memory operation of this wave and nothing else:
// s_waitcnt with vmcnt 0 and expcnt / lgkmcnt at their maxima (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait for this wave's outstanding memory operations (the coherent stores that
// precede an arrival) to complete.  The signal fences keep the compiler from
// moving memory operations across the wait.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Arrive on a counter after this thread's coherent stores; returns the old value.
__device__ __forceinline__ int arrive(int* counter) {
  wait_stores();
  const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return old;
}

// ---- self-announcing records ------------------------------------------------
// A record word is 64 bits written with one coherent atomic store, so a reader
// sees either zero (not yet written: the workspace starts zeroed) or the whole
// word.  Every encoding below is non-zero, so "non-zero" is the ready flag and a
// consumer gets the data with the poll itself: no separate counter, no ordering
// between a data store and a flag store.
__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
  return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}
__device__ __forceinline__ float unpack_lo(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ float unpack_hi(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }
constexpr uint32_t kSign = 0x80000000u;
// a non-negative float with its sign bit set as a marker (decode: clear the bit)
__device__ __forceinline__ float mark(float nonneg) { return __uint_as_float(__float_as_uint(nonneg) | kSign); }
__device__ __forceinline__ float unmark(float v) { return __uint_as_float(__float_as_uint(v) & ~kSign); }

__device__ __forceinline__ void put_word(uint64_t* p, uint64_t w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Zero n 64-bit record words with the whole block.
__device__ __forceinline__ void block_zero_words(uint64_t* p, int64_t n) {
  for (int64_t i = threadIdx.x; i < n; i += kBlock) put_word(p + i, 0ull);
}

__device__ __forceinline__ void reset_counter(int* counter) { st_coherent(counter, 0); }

// Zero n floats of workspace with the whole block (coherent stores).
__device__ __forceinline__ void block_zero(float* p, int64_t n) {
  for (int64_t i = threadIdx.x; i < n; i += kBlock) st_coherent(p + i, 0.f);
}

// ---------------------------------------------------------------------------
// Wave reductions as in-place DPP chains: each step is one fused VALU op
// v = op(v[source lane], v) over row_shr 1, 2, 4, 8, then row_bcast 15 (rows 1 and
// 3) and row_bcast 31 (rows 2 and 3), so lane 63 ends with the result.  A lane
// whose source is out of range or whose row is masked off is not written and keeps
// its own value (the identity of both operations).  N independent values run
// interleaved, so that their steps fill each other's DPP read delay (a VALU write
// must be two wait states ahead of a DPP read of the same register); s_nop covers
// what they do not, and the leading s_nop covers an EXEC write just before.  All
// lanes must be active.
#define MTP_DPP_STEP(OP, R, CTRL, MASK) "v_" OP "_f32_dpp " R ", " R ", " R " " CTRL " row_mask:" MASK " bank_mask:0xf\n\t"
#define MTP_DPP_CHAIN1(OP)                                                                                  \
  "s_nop 4\n\t" MTP_DPP_STEP(OP, "%0", "row_shr:1", "0xf") "s_nop 1\n\t" MTP_DPP_STEP(OP, "%0", "row_shr:2", "0xf") \
  "s_nop 1\n\t" MTP_DPP_STEP(OP, "%0", "row_shr:4", "0xf") "s_nop 1\n\t" MTP_DPP_STEP(OP, "%0", "row_shr:8", "0xf") \
  "s_nop 1\n\t" MTP_DPP_STEP(OP, "%0", "row_bcast:15", "0xa") "s_nop 1\n\t"                                     \
  MTP_DPP_STEP(OP, "%0", "row_bcast:31", "0xc") "s_nop 1"
#define MTP_DPP_PAIR(OP, CTRL, MASK) MTP_DPP_STEP(OP, "%0", CTRL, MASK) MTP_DPP_STEP(OP, "%1", CTRL, MASK)
#define MTP_DPP_CHAIN2(OP)                                                                              \
  "s_nop 4\n\t" MTP_DPP_PAIR(OP, "row_shr:1", "0xf") "s_nop 0\n\t" MTP_DPP_PAIR(OP, "row_shr:2", "0xf")   \
  "s_nop 0\n\t" MTP_DPP_PAIR(OP, "row_shr:4", "0xf") "s_nop 0\n\t" MTP_DPP_PAIR(OP, "row_shr:8", "0xf")   \
  "s_nop 0\n\t" MTP_DPP_PAIR(OP, "row_bcast:15", "0xa") "s_nop 0\n\t" MTP_DPP_PAIR(OP, "row_bcast:31", "0xc") \
  "s_nop 1"
#define MTP_DPP_TRIPLE(OP, CTRL, MASK) MTP_DPP_PAIR(OP, CTRL, MASK) MTP_DPP_STEP(OP, "%2", CTRL, MASK)
#define MTP_DPP_CHAIN3(OP)                                                                                    \
  "s_nop 4\n\t" MTP_DPP_TRIPLE(OP, "row_shr:1", "0xf") MTP_DPP_TRIPLE(OP, "row_shr:2", "0xf")                  \
  MTP_DPP_TRIPLE(OP, "row_shr:4", "0xf") MTP_DPP_TRIPLE(OP, "row_shr:8", "0xf")                               \
  MTP_DPP_TRIPLE(OP, "row_bcast:15", "0xa") MTP_DPP_TRIPLE(OP, "row_bcast:31", "0xc") "s_nop 1"

__device__ __forceinline__ float lane63(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }

// In place: v[i] becomes the wave's sum (kMax false) or maximum (kMax true) of
// v[i], in every lane's copy of the returned value.  The maximum ignores a NaN
// operand (v_max_f32); callers propagate NaNs through the sums instead.
template <bool kMax, int N>
__device__ __forceinline__ void wave_reduce(float (&v)[N]) {
  static_assert(N >= 1, "at least one value");
  if constexpr (N > 3) {   // groups of three
    float a[3] = {v[0], v[1], v[2]}, b[N - 3];
#pragma unroll
    for (int i = 3; i < N; ++i) b[i - 3] = v[i];
    wave_reduce<kMax, 3>(a);
    wave_reduce<kMax, N - 3>(b);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = i < 3 ? a[i] : b[i - 3];
    return;
  } else if constexpr (N == 1) {
    if constexpr (kMax) asm volatile(MTP_DPP_CHAIN1("max") : "+v"(v[0]));
    else asm volatile(MTP_DPP_CHAIN1("add") : "+v"(v[0]));
  } else if constexpr (N == 2) {
    if constexpr (kMax) asm volatile(MTP_DPP_CHAIN2("max") : "+v"(v[0]), "+v"(v[1]));
    else asm volatile(MTP_DPP_CHAIN2("add") : "+v"(v[0]), "+v"(v[1]));
  } else {
    if constexpr (kMax) asm volatile(MTP_DPP_CHAIN3("max") : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]));
    else asm volatile(MTP_DPP_CHAIN3("add") : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]));
  }
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = lane63(v[i]);
}

__device__ __forceinline__ float wave_total(float v) {
  float a[1] = {v};
  wave_reduce<false, 1>(a);
  return a[0];
}

// NaN-propagating maximum (IEEE maximum: no canonicalisation of the operands).
__device__ __forceinline__ float fmaximum(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float wave_maximum(float v) {
  float a[1] = {v};
  wave_reduce<true, 1>(a);
  return a[0];
}

// Wave minimum of unsigned integers with the same chain (v_min_u32), every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  asm volatile(
      "s_nop 4\n\t"
      "v_min_u32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_min_u32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_min_u32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_min_u32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_min_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\ts_nop 1\n\t"
      "v_min_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\ts_nop 1"
      : "+v"(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave maximum of unsigned integers with the same chain (v_max_u32), every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  asm volatile(
      "s_nop 4\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\ts_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\ts_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\ts_nop 1"
      : "+v"(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// A lane's value moved by a DPP control (gfx9 encodings: row_shr:n = 0x110 + n,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143); lanes without a source, or in rows
// outside ROW_MASK, read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the wave in lane order: within each row of 16 lanes by
// shifts of 1, 2, 4 and 8 lanes, then row 0's total into row 1 and row 2's into row
// 3, then the total of rows 0-1 into rows 2 and 3.  Lane 63 holds the wave total.
__device__ __forceinline__ float wave_incl_sum(float v) {
  v += dpp_or_zero<0x111>(v);
  v += dpp_or_zero<0x112>(v);
  v += dpp_or_zero<0x114>(v);
  v += dpp_or_zero<0x118>(v);
  v += dpp_or_zero<0x142, 0xa>(v);
  v += dpp_or_zero<0x143, 0xc>(v);
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ Lse lse_nan() {
  const float nan = __builtin_nanf("");
  return Lse{nan, nan, nan};
}

// Log-sum-exp partials of R rows over a wave, the rows interleaved so that their
// dependency chains overlap.  L converts logits to base-2 exponents: log2 e, or
// log2 e / T for temperature T.  For row r the wave's largest logit M is the
// reference (ref = M L rounded up), x[r] is overwritten with e = 2^(x L - ref) <= 1 and the sums of
// e, and for r < RY of e * (x L - ref) (the entropy moment), are taken over the
// wave.  A wave holding only -inf gives the empty partial (ref = -inf, z = 0, e = 0);
// a NaN gives z = NaN.  The entropy moment is
// accumulated without guarding 0 * (-inf); if that produced a NaN it is summed again
// from the e values alone (e log2 e over e > 0).
template <int NE, int R, int RY>
__device__ __forceinline__ void wave_pass1(float (&x)[R][NE], Lse (&out)[R], float L = kLog2e) {
  float M[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float m = x[r][0];
#pragma unroll
    for (int i = 1; i < NE; ++i) m = fmaximum(m, x[r][i]);
    M[r] = m;
  }
  wave_reduce<true, R>(M);
  float ref[R], z0[R], z1[R], y0[R], y1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ref[r] = M[r] > kNegInf ? ref_up(M[r], L) : 0.f;   // 0 keeps -inf - ref = -inf
    z0[r] = z1[r] = y0[r] = y1[r] = -0.f;   // -0 + x = x: the first additions fold away
  }
#pragma unroll
  for (int i = 0; i < NE; ++i) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float t = __builtin_fmaf(x[r][i], L, -ref[r]);
      const float e = fast_exp2(t);
      if (i & 1) z1[r] += e; else z0[r] += e;
      if (r < RY) {
        if (i & 1) y1[r] = __builtin_fmaf(e, t, y1[r]); else y0[r] = __builtin_fmaf(e, t, y0[r]);
      }
      x[r][i] = e;
    }
  }
  // the R + RY sums in one interleaved chain
  float zy[R + RY], Z[R], Y[R];
#pragma unroll
  for (int r = 0; r < R; ++r) zy[r] = z0[r] + z1[r];
#pragma unroll
  for (int r = 0; r < RY; ++r) zy[R + r] = y0[r] + y1[r];
  wave_reduce<false, R + RY>(zy);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    Z[r] = zy[r];
    Y[r] = r < RY ? zy[R + r] : 0.f;
  }
#pragma unroll
  for (int r = 0; r < RY; ++r) {
    if (Y[r] != Y[r] && Z[r] == Z[r]) {
      float y = 0.f;
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (x[r][i] > 0.f) y = __builtin_fmaf(x[r][i], fast_log2(x[r][i]), y);
      Y[r] = wave_total(y);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) out[r] = Lse{M[r] > kNegInf ? ref[r] : kNegInf, Z[r], Y[r]};   // ref -inf when empty
}

// Merge of per-lane partials of R rows into one per row, the same bits in every
// lane; rows r < RY merge the entropy moment too.  An empty partial is (ref = -inf,
// z = 0, y = 0) and weighs 2^(-inf) = 0; a row with only empty partials gives the
// empty partial; a NaN reference or sum propagates.
__device__ __forceinline__ float finite_ref(float R) { return R == kNegInf ? -__FLT_MAX__ : R; }

template <int R, int RY>
__device__ __forceinline__ void wave_merge(Lse (&s)[R]) {
  float Rm[R], zc[R], yc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) Rm[r] = s[r].ref;
  wave_reduce<true, R>(Rm);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float d = s[r].ref - finite_ref(Rm[r]);
    const float f = fast_exp2(d);
    zc[r] = s[r].z * f;
    yc[r] = r < RY ? __builtin_fmaf(fmaxf(d, -1e30f), s[r].z, s[r].y) * f : 0.f;
  }
  float zy[R + RY];
#pragma unroll
  for (int r = 0; r < R; ++r) zy[r] = zc[r];
#pragma unroll
  for (int r = 0; r < RY; ++r) zy[R + r] = yc[r];
  wave_reduce<false, R + RY>(zy);
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = Lse{Rm[r], zy[r], r < RY ? zy[R + r] : 0.f};
}

// Merge of N partials held in LDS (stride 3 floats), computed alike in every lane,
// with the same conventions as wave_merge.
template <int N, bool kY>
__device__ __forceinline__ Lse merge_lds(const float* p) {
  float ref[N], z[N], y[N];
  float R = kNegInf;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    ref[i] = p[3 * i]; z[i] = p[3 * i + 1]; y[i] = kY ? p[3 * i + 2] : 0.f;
    R = fmaximum(R, ref[i]);
  }
  const float Rf = finite_ref(R);
  float Z = 0.f, Y = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float d = ref[i] - Rf;
    const float f = fast_exp2(d);
    Z = __builtin_fmaf(z[i], f, Z);
    if constexpr (kY) Y = __builtin_fmaf(__builtin_fmaf(fmaxf(d, -1e30f), z[i], y[i]), f, Y);
  }
  return Lse{R, Z, Y};
}

// ---------------------------------------------------------------------------
// Wave-segment streaming.  A chunk is split into kWaves contiguous segments of
// NV*64 vectors, one per wave; lane l of a wave holds vectors s0 + j*64 + l
// (j < NV), so each load instruction reads 1 KB contiguous per wave.
// issue_seg() puts all loads in flight at once (addresses clamped into the row);
// unpack_seg() widens them: when `full` (wave-uniform) every vector lies inside the
// chunk and the row; otherwise vectors at or past `lim` read as -inf and the row's
// partial last vector (index `tail`, if tail < `cend`) is read element by element.
// Streaming loads: non-temporal (each logit is read once).
constexpr int kStreamCpol = 2;

// v0 = the wave's first vector + lane.  The descriptors start at the wave's first
// vector, so byte offsets stay within the segment for rows of any length (a row
// may exceed the 2^31 bytes one descriptor spans); a vector clamped below that
// start gives a negative offset, which the descriptor's bound turns into zeros.
template <int DT, int NV, int R>
__device__ __forceinline__ void issue_seg(RawChunk<NV, R>& raw, const char* const (&rows)[R], int v0, int last) {
  if (last >= 0) {
    const int vb = __builtin_amdgcn_readfirstlane(v0 - (int)(threadIdx.x & 63));
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int off = (min(v0 + j * 64, last) - vb) * 16;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        raw.v[r][j] = __builtin_amdgcn_raw_buffer_load_b128(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rows[r]) + (int64_t)vb * 16, 0, 0x7fffffff, 0x00020000),
            off, 0, kStreamCpol);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < NV; ++j) raw.v[r][j] = u32x4{0u, 0u, 0u, 0u};
  }
}

// The same loads with a fixed count: all R rows (pass the same row twice when
// there is only one), every row read through a buffer descriptor bounded by the
// row's `row_bytes` (a read past it returns zeros); when `live` is false, or the row
// has no full vector, every lane reads offset 0.  A load count that does not depend
// on the item lets the compiler wait for exactly the loads it needs.
template <int DT, int NV, int R>
__device__ __forceinline__ void issue_seg_fixed(RawChunk<NV, R>& raw, const char* const (&rows)[R], int v0,
                                                int last, bool live, int row_bytes) {
  const bool ok = live && last >= 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int off = ok ? min(v0 + j * 64, last) * 16 : 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      raw.v[r][j] = __builtin_amdgcn_raw_buffer_load_b128(
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rows[r]), 0, row_bytes, 0x00020000), off, 0, kStreamCpol);
  }
}

template <int DT, int NV, int R>
__device__ __forceinline__ void unpack_seg(const RawChunk<NV, R>& raw, const char* const (&rows)[R], int v0,
                                           bool full, int lim, int tail, int cend, int V,
                                           float (&x)[R][NV * Elem<DT>::kPerVec]) {
  constexpr int PV = Elem<DT>::kPerVec;
  constexpr uint32_t kMasked = DT == kBF16 ? 0xFF80FF80u : 0xFF800000u;
  auto put = [&](int r, int j, int w, uint32_t word) {
    if constexpr (DT == kBF16) {
      x[r][j * PV + 2 * w] = bf16_lo(word);
      x[r][j * PV + 2 * w + 1] = bf16_hi(word);
    } else {
      x[r][j * PV + w] = __uint_as_float(word);
    }
  };
  if (full) {   // wave-uniform: the whole segment lies inside the chunk and the row
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int w = 0; w < 4; ++w) put(r, j, w, raw.v[r][j][w]);
      }
    return;
  }
  // also covers a bad (no valid data) case: last < 0 has raw = 0 but every vector masked
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const bool ok = v0 + j * 64 < lim;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int w = 0; w < 4; ++w) put(r, j, w, ok ? raw.v[r][j][w] : kMasked);
    }
  }
  if (tail < cend) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (v0 + j * 64 == tail) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int e = 0; e < PV; ++e) {
            const int idx = tail * PV + e;
            if (idx < V) x[r][j * PV + e] = load_one<DT>(rows[r], idx);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cluster records through buffer instructions with an explicit cache policy:
// device scope (sc1), so that a load never hits a stale copy in the CU's L1 (a
// workgroup-scope load, sc0 alone, may) and a store is visible to every CU.
#ifndef MTP_REC_CPOL
#define MTP_REC_CPOL 16
#endif
constexpr int kRecCpol = MTP_REC_CPOL;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ uint64_t rec_load(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kRecCpol);
  return (uint64_t)v[0] | ((uint64_t)v[1] << 32);
}
__device__ __forceinline__ void rec_store(__amdgpu_buffer_rsrc_t r, int byte_off, uint64_t w) {
  const u32x2 v = {(uint32_t)w, (uint32_t)(w >> 32)};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, kRecCpol);
}

// Wait until word `word` of every record of a row is published (non-zero):
// `v` is this lane's word of record `lane`, loaded earlier, and lanes still seeing
// zero load again; records past the first 64 are loaded here.  `merge` folds each
// lane's words in record order (first record, then l + 64, ...).  Bounded by
// `limit` ticks of the 100 MHz counter: a timeout sets the error word and returns
// true (the same in every lane).  The first 64 words are tested before any load of
// this function is issued, so that test waits only for the caller's load and not
// for the (in-order) loads the caller issued after it.
template <typename Fold>
__device__ __forceinline__ bool poll_words(uint64_t v, __amdgpu_buffer_rsrc_t rs, int C, int st, int word,
                                           uint32_t* err, uint64_t limit, Fold fold) {
  const int lane = threadIdx.x & 63;
  uint64_t t0 = 0;
  bool timed_out = false;
  auto settle = [&](int c, uint64_t& w) {
    bool ready = !(c < C) || w != 0ull;
    while (!timed_out && __ballot(!ready) != 0ull) {
      if (t0 == 0) t0 = __builtin_amdgcn_s_memrealtime();
      __builtin_amdgcn_s_sleep(1);
      if (!ready) {
        w = rec_load(rs, c * st + word * 8);
        ready = w != 0ull;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > limit) {
        if (lane == 0) __hip_atomic_fetch_or(err, kErrSyncTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        timed_out = true;
      }
    }
  };
  settle(lane, v);
  if (lane < C) fold(true, v);
  for (int c0 = 64; c0 < C; c0 += 64) {
    const int c = c0 + lane;
    if (c < C) v = rec_load(rs, c * st + word * 8);
    settle(c, v);
    if (c < C) fold(false, v);
  }
  return timed_out;
}

// The row's merged log-sum-exp (no entropy moment) from word `word` of the records;
// NaN if the wait timed out.
__device__ __forceinline__ Lse poll_row(uint64_t v, __amdgpu_buffer_rsrc_t rs, int C, int st, int word,
                                        uint32_t* err, uint64_t limit) {
  Lse acc = lse_empty();
  const bool timed_out = poll_words(v, rs, C, st, word, err, limit, [&](bool first, uint64_t w) {
    const Lse r{unpack_lo(w), unmark(unpack_hi(w)), 0.f};
    acc = first ? r : lse_merge(acc, r);
  });
  Lse a[1] = {acc};
  wave_merge<1, 0>(a);
  return timed_out ? lse_nan() : a[0];
}

// ---------------------------------------------------------------------------
// Philox4x32-10: ten rounds of the Philox S-box on four 32-bit words with a
// two-word key advanced by the Weyl increments between rounds.
struct P4 { uint32_t x[4]; };

__device__ __forceinline__ P4 philox4x32_10(P4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    // each 32 x 32 -> 64-bit product is one v_mad_u64_u32, each three-way
    // exclusive or one v_bitop3_b32 (truth table 0x96: a ^ b ^ c)
    const uint64_t p0 = (uint64_t)M0 * c.x[0], p1 = (uint64_t)M1 * c.x[2];
    P4 n;
    n.x[0] = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.x[1], k0, 0x96);
    n.x[1] = (uint32_t)p1;
    n.x[2] = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.x[3], k1, 0x96);
    n.x[3] = (uint32_t)p0;
    c = n;
  }
  return c;
}

// The two verify uniforms of a row: counter = offset + position (64-bit, words 0-1),
// key = seed; u from word 0, u' from word 1, each (w >> 8) * 2^-24.
__device__ __forceinline__ void row_uniforms(uint64_t seed, uint64_t offset, uint64_t position,
                                             float* u, float* u_prime) {
  const uint64_t c = offset + position;
  P4 in{{(uint32_t)c, (uint32_t)(c >> 32), 0u, 0u}};
  P4 o = philox4x32_10(in, (uint32_t)seed, (uint32_t)(seed >> 32));
  *u = (float)(o.x[0] >> 8) * 0x1p-24f;
  *u_prime = (float)(o.x[1] >> 8) * 0x1p-24f;
}

// Exponential variates for four consecutive elements 4 v4 .. 4 v4 + 3 of a row, in
// base-2 units: E = -log2 U = -ln U / ln 2, U = (k + 1/2) 2^-24 with k = word >> 8
// of Philox at counter (c, 1 + v4, 0), key = seed.  The Gumbel noise is -ln(-ln U),
// so argmax_v (ln w_v + G_v) = argmax_v w_v / E_v = argmax_v (log2 w_v - log2 E_v)
// (the exponential race).  U has 25 significant bits above 1/2, so float32 rounds
// it (U_r); the rounding d = U - U_r comes back exactly from one fused multiply-add
// (k 2^-24 - U_r is a small multiple of 2^-25) and one addition, and
//   E = -log2 U_r - log2(1 + d / U_r) = -log2 U_r - d log2(e) + eps,
// |eps| <= |d| log2(e) (1 - U_r) / U_r + d^2 / U_r^2, below 1e-7 relative to E for
// every U (|d| <= 2^-25; E ~ (1 - U) log2(e) near 1).  The hardware base-2 log keeps
// about 1e-7 of relative accuracy down to U = 1 - 2^-24, where E is smallest and
// the likely winners are, so E is within a few 1e-7 relative of -log2 U throughout.
__device__ __forceinline__ float expo_of_word(uint32_t w) {
  const float kf = (float)(w >> 8);
  const float Ur = __builtin_fmaf(kf, 0x1p-24f, 0x1p-25f);          // U rounded once
  const float d = __builtin_fmaf(kf, 0x1p-24f, -Ur) + 0x1p-25f;       // U - U_r, exact
  return __builtin_fmaf(-d, kLog2e, -fast_log2(Ur));
}

__device__ __forceinline__ void expo4(uint64_t seed, uint64_t c, uint32_t v4, float (&E)[4]) {
  const P4 in{{(uint32_t)c, (uint32_t)(c >> 32), v4 + 1u, 0u}};
  const P4 o = philox4x32_10(in, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
  for (int j = 0; j < 4; ++j) E[j] = expo_of_word(o.x[j]);
}

}  // namespace mtp
