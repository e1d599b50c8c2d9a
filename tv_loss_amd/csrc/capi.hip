// C ABI of libmtp: argument validation, workspace layout, launch.
//
// Every argument check runs before the first HIP call, so a rejected call touches
// neither the device nor any output.  The only global state is a per-device cache
// of the compute-unit count and kernel occupancies, filled under a mutex.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>

#include "mtp.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

// Ticks of the 100 MHz counter after which a bounded wait gives up (process-wide).
std::atomic<uint64_t> g_wait_limit{mtp::kDefaultWaitLimitTicks};
// Vectors per chunk of the persistent kernels (0: each kernel's own chunk of
// kBlock x vectors-per-thread; process-wide, diagnostics only).
std::atomic<int32_t> g_chunk_vectors{0};

mtp_status fail(mtp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

mtp_status ok() {
  g_err[0] = 0;
  return MTP_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(mtp_dtype dt) { return dt == MTP_BF16 ? 2 : 4; }
int per_vec(mtp_dtype dt) { return dt == MTP_BF16 ? 8 : 4; }

constexpr int64_t kMaxVocab = int64_t(1) << 30;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int32_t kMaxTopK = 1 << 20;

mtp_status check_common(mtp_dtype dt, int32_t gamma, int32_t vocab) {
  if (dt != MTP_F32 && dt != MTP_BF16) return fail(MTP_ERR_DTYPE, "unknown dtype code %d", (int)dt);
  if (gamma < 1 || gamma > MTP_MAX_GAMMA)
    return fail(MTP_ERR_SHAPE, "gamma = %d outside [1, %d]", gamma, MTP_MAX_GAMMA);
  if (vocab < 1 || vocab > kMaxVocab) return fail(MTP_ERR_SHAPE, "vocab = %d outside [1, 2^30]", vocab);
  return MTP_OK;
}

mtp_status check_row_base(const void* p, int64_t stride_elems, mtp_dtype dt, const char* what) {
  if (!aligned16(p)) return fail(MTP_ERR_ALIGN, "%s pointer is not 16-byte aligned", what);
  if ((stride_elems * elem_bytes(dt)) % 16 != 0)
    return fail(MTP_ERR_ALIGN, "%s stride of %lld elements is not a multiple of 16 bytes", what,
                (long long)stride_elems);
  return MTP_OK;
}

// ---- per-device limits --------------------------------------------------------
struct DeviceInfo {
  int cus = 0;
  std::map<int, int> occ;   // kernel key -> workgroups per CU
};
std::mutex g_dev_mu;
std::map<int, DeviceInfo> g_dev;

// Workgroups of a persistent kernel the current device holds at once (all of a
// launch's workgroups must be resident together: a super-group waits on its
// members' records), from the kernel's occupancy, cached per device and key.
template <typename Occ>
mtp_status capacity(int key, Occ occupancy, int64_t* per_gpu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MTP_ERR_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& info = g_dev[dev];
  if (info.cus == 0) {
    if (hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(MTP_ERR_DEVICE, "cannot query the compute-unit count");
  }
  auto it = info.occ.find(key);
  if (it == info.occ.end()) {
    int n = 0;
    hipError_t e = occupancy(&n);
    if (e != hipSuccess || n < 1) return fail(MTP_ERR_DEVICE, "occupancy query failed");
    it = info.occ.emplace(key, n).first;
  }
  *per_gpu = (int64_t)it->second * info.cus;
  return MTP_OK;
}

// The compute units of the current device (known once a capacity query has run).
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  const int n = g_dev[dev].cus;
  return n > 0 ? n : 1;
}

// Measured on MI355X (four verify workgroups per compute unit): each later dispatch
// round takes about 6 % longer per item.
constexpr double kVerifyRoundCost = 0.06;
// ... and for the fused TV forward + backward (two workgroups per compute unit:
// 4.81 -> 4.70 ms on T = 8192; the single-read forward measured no faster with it)
constexpr double kTvRoundCost = 0.08;

// Item counts per dispatch round for S super-groups of C workgroups, W per round,
// N items, an item of round r costing 1 + cost r: the smallest end time T at which
// the super-groups can hold N items (each floor(T / (1 + cost r))), then the excess
// taken from the super-groups that would end last.  No split (W = 0: strided items)
// when some super-group would get fewer than four items or there are more rounds
// than kMaxRounds.
mtp::RoundSplit plan_round_split(int S, int C, int64_t N, int W, double cost) {
  mtp::RoundSplit rs{};
  if (S < 1 || C < 1 || W < 1 || N < 4 * (int64_t)S) return rs;
  const int R = (int)(((int64_t)S * C - 1) / W) + 1;
  if (R > mtp::kMaxRounds) return rs;
  int cnt[mtp::kMaxRounds];
  double t[mtp::kMaxRounds];
  auto first = [&](int r) { return (int)std::min<int64_t>(S, ((int64_t)r * W + C) / C - 1); };
  for (int r = 0; r < R; ++r) {
    cnt[r] = first(r + 1) - first(r);
    t[r] = 1.0 + cost * r;
  }
  auto per_sg = [&](double T, int r) { return (int64_t)(T / t[r] + 1e-9); };
  auto capacity_at = [&](double T) {
    int64_t n = 0;
    for (int r = 0; r < R; ++r) n += cnt[r] * per_sg(T, r);
    return n;
  };
  // T is some n t[r]: the smallest such with enough capacity
  double T = 0.0;
  {
    double lo = 0.0, hi = (double)N * t[R - 1];
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (capacity_at(mid) >= N) hi = mid; else lo = mid;
    }
    T = hi;
  }
  int64_t excess = capacity_at(T) - N;
  for (int r = 0; r < R; ++r) {
    rs.items[r] = (int)per_sg(T, r);
    rs.short_by[r] = 0;
  }
  // take the excess from the super-groups that end last (largest items * cost)
  while (excess > 0) {
    int best = -1;
    for (int r = 0; r < R; ++r)
      if (rs.short_by[r] < cnt[r] && (best < 0 || rs.items[r] * t[r] > rs.items[best] * t[best])) best = r;
    if (best < 0) break;
    const int64_t take = std::min<int64_t>(excess, cnt[best] - rs.short_by[best]);
    rs.short_by[best] += (int)take;
    excess -= take;
    // a round that gave one item from all its super-groups ends one item earlier
    if (rs.short_by[best] == cnt[best]) {
      rs.items[best] -= 1;
      rs.short_by[best] = 0;
    }
  }
  int64_t total = 0;
  for (int r = 0; r < R; ++r) {
    if (rs.items[r] - (rs.short_by[r] > 0) < 4) return mtp::RoundSplit{};
    total += (int64_t)cnt[r] * rs.items[r] - rs.short_by[r];
  }
  if (total != N) return mtp::RoundSplit{};   // the ranges must tile the items exactly
  rs.W = W;
  rs.rounds = R;
  return rs;
}

mtp_status verify_capacity(int dt, int mode, int64_t* per_gpu) {
  return capacity(dt * 4 + mode, [&](int* n) { return mtp::verify_occupancy(dt, mode, n); }, per_gpu);
}

mtp_status tv_pipe_capacity(int dt, int G, bool shared, int64_t* per_gpu) {
  return capacity(1000 + dt * 64 + G * 2 + (shared ? 1 : 0),
                  [&](int* n) { return mtp::tv_pipe_occupancy(dt, G, shared, n); }, per_gpu);
}

mtp_status tv_fused_capacity(int dt, int gdt, int G, bool shared, int64_t* per_gpu) {
  return capacity(2000 + dt * 256 + gdt * 128 + G * 2 + (shared ? 1 : 0),
                  [&](int* n) { return mtp::tv_fused_occupancy(dt, gdt, G, shared, n); }, per_gpu);
}

// ---- workspace layouts --------------------------------------------------------
// The chunking of a persistent kernel (verify, single-read and fused TV): whole
// chunks of kBlock * nv vectors, or fewer vectors per chunk under the diagnostic
// cap, the kernels' workgroups then covering the chunk in part (lanes past its end
// read nothing).
mtp::RowSplit persistent_split(int64_t V, int pv, int nv) {
  mtp::RowSplit sp = mtp::make_split(V, pv, nv, false);
  const int32_t cap = g_chunk_vectors.load(std::memory_order_relaxed);
  if (cap > 0 && cap < sp.vec_per_chunk) {
    sp.vec_per_chunk = cap;
    sp.nchunks = (int)((sp.nvec + cap - 1) / cap);
  }
  return sp;
}

struct VerifyLayout {
  size_t err, part1, part2, part3, gkeys, total;
  mtp::RowSplit sp;
  int64_t ngroups;
};

VerifyLayout verify_layout(int32_t B, int32_t G, int32_t V, mtp_dtype dt, int mode) {
  VerifyLayout L{};
  L.sp = persistent_split(V, per_vec(dt), mtp::verify_vec_per_thread(dt));
  L.ngroups = (int64_t)B * (G + 1);
  const int64_t C = L.sp.nchunks;
  size_t off = 0;
  L.err = off; off = align256(off + 4);
  L.part1 = off; off = align256(off + (size_t)L.ngroups * C * mtp::verify_record_words(mode) * 8);
  L.part2 = off; off = align256(off + (size_t)L.ngroups * C * mtp::kWaves * 8);
  L.part3 = off;
  if (mode == mtp::kVerifyTargetOnly) off = align256(off + (size_t)L.ngroups * C * mtp::kWaves * 4);
  L.gkeys = off;
  if (mode == mtp::kVerifyGumbel) off = align256(off + (size_t)L.ngroups * C * mtp::kWaves * 2 * 8);
  L.total = off;
  return L;
}

struct TvLayout {
  size_t err, part1, part2, pos, total;
  mtp::RowSplit sp;
};

// The forward's workspace: error word, part1 (two passes: (ref, z) float2 per
// [t][chunk][row]; single read: one record word per [t][chunk][row]), part2
// [t][chunk][2 gamma] floats, per-position losses [t].  `pipe` picks the single-read
// forward's chunking.
TvLayout tv_layout(int32_t T, int32_t G, int32_t V, mtp_dtype dt, bool shared, bool pipe) {
  TvLayout L{};
  L.sp = pipe ? persistent_split(V, per_vec(dt), mtp::tv_pipe_vec_per_thread(dt, G, shared))
              : mtp::make_split(V, per_vec(dt), mtp::tv_fwd_vec_per_thread(dt, G, shared), false);
  const int64_t C = L.sp.nchunks;
  size_t off = 0;
  L.err = off; off = align256(off + 4);
  L.part1 = off; off = align256(off + (size_t)T * C * mtp::tv_fwd_part1_words(G, shared) * 8);
  L.part2 = off; off = align256(off + (size_t)T * C * 2 * G * 4);
  L.pos = off; off = align256(off + (size_t)T * 4);
  L.total = off;
  return L;
}

// Bytes a forward call may need: the larger of the two layouts (which forward runs
// also depends on the device's co-residency).
size_t tv_workspace_bytes(int32_t T, int32_t G, int32_t V, mtp_dtype dt, bool shared) {
  size_t b = tv_layout(T, G, V, dt, shared, false).total;
  if (mtp::tv_pipe_vec_per_thread(dt, G, shared) > 0) {
    const size_t p = tv_layout(T, G, V, dt, shared, true).total;
    b = p > b ? p : b;
  }
  return b;
}

// The fused forward + backward: error word, normaliser records part1
// [t][chunk][rows], overlap / S records part3 [t][chunk][gamma], per-position
// losses [t]; the single-read forward's chunking.
struct FusedLayout {
  size_t err, part1, part3, pos, total;
  mtp::RowSplit sp;
};

FusedLayout fused_layout(int32_t T, int32_t G, int32_t V, mtp_dtype dt, bool shared) {
  FusedLayout L{};
  L.sp = persistent_split(V, per_vec(dt), mtp::tv_pipe_vec_per_thread(dt, G, shared));
  const int64_t C = L.sp.nchunks;
  size_t off = 0;
  L.err = off; off = align256(off + 4);
  L.part1 = off; off = align256(off + (size_t)T * C * mtp::tv_fwd_part1_words(G, shared) * 8);
  L.part3 = off; off = align256(off + (size_t)T * C * G * 8);
  L.pos = off; off = align256(off + (size_t)T * 4);
  L.total = off;
  return L;
}

bool fused_shape(int32_t G, bool shared) { return G <= mtp::kWaves && mtp::tv_pipe_vec_per_thread(MTP_BF16, G, shared) > 0; }

// Bytes a fused call may need: its own layout or, for the shapes it hands to the
// forward and backward calls, theirs.
size_t fused_workspace_bytes(int32_t T, int32_t G, int32_t V, mtp_dtype dt, bool shared) {
  size_t b = tv_workspace_bytes(T, G, V, dt, shared);
  if (fused_shape(G, shared)) {
    const size_t f = fused_layout(T, G, V, dt, shared).total;
    b = f > b ? f : b;
  }
  return b;
}

// top-K path: error word, draft log-sum-exp partials [t][chunk][gamma] as float2,
// per-position losses [t]
TvLayout topk_layout(int32_t T, int32_t G, int32_t V, mtp_dtype dt) {
  TvLayout L{};
  L.sp = mtp::make_split(V, per_vec(dt), mtp::tv_topk_fwd_vec_per_thread(dt, G), false);
  const int64_t C = L.sp.nchunks;
  size_t off = 0;
  L.err = off; off = align256(off + 4);
  L.part1 = off; off = align256(off + (size_t)T * C * G * 8);
  L.part2 = off;
  L.pos = off; off = align256(off + (size_t)T * 4);
  L.total = off;
  return L;
}

// Persistent super-groups of C workgroups, at most `cap` of them resident at once
// (the workgroups that share the work), L groups to process.  Returns the number
// of super-groups and of layers (groups per super-group), balanced.
void plan_layers(int64_t cap, int C, int64_t L, int* sgroups, int* layers) {
  int64_t smax = cap / C;
  if (smax < 1) smax = 1;
  const int64_t k = (L + smax - 1) / smax;
  const int64_t S = (L + k - 1) / k;
  *sgroups = (int)S;
  *layers = (int)k;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

mtp_status check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return MTP_OK;
  if (!ws) return fail(MTP_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (((uintptr_t)ws & 255u) != 0) return fail(MTP_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (have < need) return fail(MTP_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return MTP_OK;
}

}  // namespace

extern "C" {

const char* mtp_status_string(mtp_status s) {
  switch (s) {
    case MTP_OK: return "MTP_OK";
    case MTP_ERR_NULL: return "MTP_ERR_NULL";
    case MTP_ERR_SHAPE: return "MTP_ERR_SHAPE";
    case MTP_ERR_DTYPE: return "MTP_ERR_DTYPE";
    case MTP_ERR_ALIGN: return "MTP_ERR_ALIGN";
    case MTP_ERR_WORKSPACE: return "MTP_ERR_WORKSPACE";
    case MTP_ERR_DEVICE: return "MTP_ERR_DEVICE";
    case MTP_ERR_LAUNCH: return "MTP_ERR_LAUNCH";
  }
  return "MTP_ERR_UNKNOWN";
}

const char* mtp_last_error(void) { return g_err; }

const char* mtp_version(void) { return "libmtp 0.2 (gfx950)"; }

uint64_t mtp_set_wait_limit(uint64_t ticks) { return g_wait_limit.exchange(ticks); }

int32_t mtp_set_chunk_vectors(int32_t vectors) { return g_chunk_vectors.exchange(vectors > 0 ? vectors : 0); }

mtp_status mtp_verify_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                     size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_NULL, "bytes is NULL");
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (batch < 0) return fail(MTP_ERR_SHAPE, "batch = %d is negative", batch);
  *bytes = batch == 0 ? 0 : verify_layout(batch, gamma, vocab, dtype, mtp::kVerifyRejection).total;
  return ok();
}

mtp_status mtp_verify_target_only_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                                 size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_NULL, "bytes is NULL");
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (batch < 0) return fail(MTP_ERR_SHAPE, "batch = %d is negative", batch);
  *bytes = batch == 0 ? 0 : verify_layout(batch, gamma, vocab, dtype, mtp::kVerifyTargetOnly).total;
  return ok();
}

mtp_status mtp_verify_max_vocab(mtp_dtype dtype, int32_t* vocab) {
  if (!vocab) return fail(MTP_ERR_NULL, "vocab is NULL");
  if (dtype != MTP_F32 && dtype != MTP_BF16) return fail(MTP_ERR_DTYPE, "unknown dtype code %d", (int)dtype);
  int64_t cap = INT64_MAX;
  for (int mode : {mtp::kVerifyRejection, mtp::kVerifyTargetOnly, mtp::kVerifyGumbel}) {
    int64_t per_gpu = 0;
    mtp_status s = verify_capacity(dtype, mode, &per_gpu);
    if (s) return s;
    cap = per_gpu < cap ? per_gpu : cap;
  }
  // every chunk holds kBlock * vec_per_thread vectors (or the diagnostic cap); the
  // last may be partial
  const int32_t vcap = g_chunk_vectors.load(std::memory_order_relaxed);
  const int64_t nat = (int64_t)mtp::kBlock * mtp::verify_vec_per_thread(dtype);
  const int64_t per_chunk = (vcap > 0 && vcap < nat ? vcap : nat) * per_vec(dtype);
  const int64_t v = cap * per_chunk;
  *vocab = (int32_t)(v < kMaxVocab ? v : kMaxVocab);
  return ok();
}

mtp_status mtp_verify_gumbel_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                            size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_NULL, "bytes is NULL");
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (batch < 0) return fail(MTP_ERR_SHAPE, "batch = %d is negative", batch);
  *bytes = batch == 0 ? 0 : verify_layout(batch, gamma, vocab, dtype, mtp::kVerifyGumbel).total;
  return ok();
}

}  // extern "C"

namespace {

bool bad_temperature(float T) { return !(T > 0.f) || T == __builtin_inff(); }

// Host-side checks of a verify call's arguments (no HIP call).
mtp_status verify_check_args(int mode, float temperature, const void* target, int64_t target_row_stride,
                             const void* draft, int64_t draft_row_stride, mtp_dtype dtype, int32_t batch,
                             int32_t gamma, int32_t vocab, const int32_t* draft_tokens, const uint8_t* accept,
                             const int32_t* accepted_len, const int32_t* next_token, const int32_t* draft_token) {
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (batch < 0) return fail(MTP_ERR_SHAPE, "batch = %d is negative", batch);
  if (batch == 0) return MTP_OK;
  if (!target || !draft || !accept || !accepted_len || !next_token)
    return fail(MTP_ERR_NULL, "a required pointer (target, draft, accept, accepted_len, next_token) is NULL");
  const bool target_only = mode == mtp::kVerifyTargetOnly;
  if (!target_only && !draft_tokens) return fail(MTP_ERR_NULL, "draft_tokens is NULL");
  if (target_only && !draft_token) return fail(MTP_ERR_NULL, "draft_token is NULL");
  if (target_row_stride < vocab || draft_row_stride < vocab)
    return fail(MTP_ERR_SHAPE, "row strides (%lld, %lld) must be >= vocab (%d)", (long long)target_row_stride,
                (long long)draft_row_stride, vocab);
  if ((s = check_row_base(target, target_row_stride, dtype, "target"))) return s;
  if ((s = check_row_base(draft, draft_row_stride, dtype, "draft"))) return s;
  if (mode == mtp::kVerifyGumbel && bad_temperature(temperature))
    return fail(MTP_ERR_SHAPE, "temperature %g is not a positive finite number", (double)temperature);
  return MTP_OK;
}

// The verify entry points: rejection sampling (draft_tokens given), target-only
// (draft_token out) or rejection sampling at a temperature with Gumbel-max row
// samples.  Argument errors return before any HIP call.
mtp_status verify_impl(int mode, float temperature, const void* target, int64_t target_row_stride, const void* draft,
                       int64_t draft_row_stride, mtp_dtype dtype, int32_t batch, int32_t gamma, int32_t vocab,
                       const int32_t* draft_tokens, uint64_t seed, uint64_t offset, uint8_t* accept,
                       int32_t* accepted_len, int32_t* next_token, int32_t* draft_token, float* p_yhat,
                       uint8_t* rs_better, int32_t* row_token, float* overlap, float* tv, float* entropy,
                       int32_t* row_status, void* workspace, size_t workspace_bytes, void* stream) {
  mtp_status s = verify_check_args(mode, temperature, target, target_row_stride, draft, draft_row_stride, dtype,
                                   batch, gamma, vocab, draft_tokens, accept, accepted_len, next_token, draft_token);
  if (s) return s;
  if (batch == 0) return ok();
  const bool target_only = mode == mtp::kVerifyTargetOnly;
  const VerifyLayout L = verify_layout(batch, gamma, vocab, dtype, mode);
  if ((s = check_workspace(workspace, workspace_bytes, L.total))) return s;
  if (L.ngroups > 0x7fffffffLL / 8) return fail(MTP_ERR_SHAPE, "batch * (gamma + 1) is too large");

  // ---- device-dependent checks ---------------------------------------------
  int64_t per_gpu = 0;
  if ((s = verify_capacity(dtype, mode, &per_gpu))) return s;
  if ((int64_t)L.sp.nchunks > per_gpu)
    return fail(MTP_ERR_SHAPE, "vocab %d needs %d co-resident workgroups per row; the GPU holds %lld", vocab,
                L.sp.nchunks, (long long)per_gpu);
  int sgroups = 0, layers = 0;
  plan_layers(per_gpu, L.sp.nchunks, L.ngroups, &sgroups, &layers);

  mtp::VerifyArgs a{};
  a.target = target; a.t_stride = target_row_stride;
  a.draft = draft; a.d_stride = draft_row_stride;
  a.tokens = target_only ? nullptr : draft_tokens;
  a.B = batch; a.G = gamma; a.V = vocab;
  a.seed = seed; a.offset = offset;
  a.accept = accept; a.accepted_len = accepted_len; a.next_token = next_token;
  a.row_token = row_token; a.overlap = overlap; a.tv = tv; a.entropy = entropy; a.row_status = row_status;
  a.draft_token = draft_token; a.p_yhat = p_yhat; a.rs_better = rs_better;
  a.err = at<uint32_t>(workspace, L.err);
  a.part1 = at<uint64_t>(workspace, L.part1);
  a.part2 = at<uint64_t>(workspace, L.part2);
  a.part3 = target_only ? at<float>(workspace, L.part3) : nullptr;
  a.gkeys = mode == mtp::kVerifyGumbel ? at<uint64_t>(workspace, L.gkeys) : nullptr;
  a.inv_temp = mode == mtp::kVerifyGumbel ? 1.f / temperature : 1.f;
  a.wait_limit = g_wait_limit.load(std::memory_order_relaxed);
  a.sp = L.sp;
  a.ngroups = (int)L.ngroups;
  a.sgroups = sgroups;
  a.layers = layers;
  a.div_b = mtp::make_fastdiv((uint32_t)batch);
  a.div_g1 = mtp::make_fastdiv((uint32_t)(gamma + 1));
  // The split by dispatch round measured faster from about 16 items per super-group
  // (long tail, 160: 3 % less time; 20: 1 %); with fewer, the split by thirds, whose
  // last super-groups end early to host the finish (rollout, 10: 1.5 % less time).
  if (L.ngroups >= 16 * (int64_t)sgroups)
    a.split = plan_round_split(sgroups, L.sp.nchunks, L.ngroups, device_cus(), kVerifyRoundCost);
  if (a.split.W == 0 && sgroups >= 3 && L.ngroups >= 4 * (int64_t)sgroups) a.split.W = -1;
  hipError_t e = mtp::launch_verify(a, dtype, mode, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "verify launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

// ---- mtp_verify_noalloc: the verify workspace in a file-scope device array ----
// For callers that cannot allocate device memory.  Each GPU holds its own copy of
// `scratch` for the life of the process; host code never uses the array's name as
// an address: hipGetSymbolAddress gives each device's copy once, and that pointer
// is what the kernels get.  The verify kernels leave every word they use at zero
// when a call completes, so the array only needs zeroing once per device.
constexpr size_t kScratchBytes = MTP_VERIFY_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

__global__ void zero_scratch(uint64_t* p, size_t nwords) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;   // device -> address of that device's `scratch`

// This device's scratch address; on the first call on a device, looks it up and
// zeroes the array on `stream` (a zero-fill kernel, not a memset node).
mtp_status device_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MTP_ERR_DEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
      return fail(MTP_ERR_DEVICE, "cannot query the stream's capture status");
    if (cs != hipStreamCaptureStatusNone)
      return fail(MTP_ERR_DEVICE, "the first mtp_verify_noalloc call on a device zeroes its scratch array and "
                                  "must not be captured");
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MTP_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(zero_scratch, dim3(1024), dim3(256), 0, stream, reinterpret_cast<uint64_t*>(p),
                       kScratchBytes / 8);
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess) return fail(MTP_ERR_LAUNCH, "zeroing the scratch array failed: %s", hipGetErrorString(le));
    it = g_scratch.emplace(dev, p).first;
  }
  *out = it->second;
  return MTP_OK;
}

}  // namespace

extern "C" {

mtp_status mtp_verify(const void* target, int64_t target_row_stride, const void* draft,
                      int64_t draft_row_stride, mtp_dtype dtype, int32_t batch, int32_t gamma,
                      int32_t vocab, const int32_t* draft_tokens, uint64_t seed, uint64_t offset,
                      uint8_t* accept, int32_t* accepted_len, int32_t* next_token, int32_t* row_token,
                      float* overlap, float* tv, float* entropy, int32_t* row_status, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return verify_impl(mtp::kVerifyRejection, 1.f, target, target_row_stride, draft, draft_row_stride, dtype, batch, gamma, vocab,
                     draft_tokens, seed, offset, accept, accepted_len, next_token, nullptr, nullptr, nullptr,
                     row_token, overlap, tv, entropy, row_status, workspace, workspace_bytes, stream);
}

mtp_status mtp_verify_target_only(const void* target, int64_t target_row_stride, const void* draft,
                                  int64_t draft_row_stride, mtp_dtype dtype, int32_t batch, int32_t gamma,
                                  int32_t vocab, uint64_t seed, uint64_t offset, uint8_t* accept,
                                  int32_t* accepted_len, int32_t* next_token, int32_t* draft_token, float* p_yhat,
                                  uint8_t* rs_better, int32_t* row_token, float* overlap, float* tv,
                                  float* entropy, int32_t* row_status, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return verify_impl(mtp::kVerifyTargetOnly, 1.f, target, target_row_stride, draft, draft_row_stride, dtype, batch, gamma, vocab,
                     nullptr, seed, offset, accept, accepted_len, next_token, draft_token, p_yhat, rs_better,
                     row_token, overlap, tv, entropy, row_status, workspace, workspace_bytes, stream);
}

mtp_status mtp_verify_gumbel(const void* target, int64_t target_row_stride, const void* draft,
                             int64_t draft_row_stride, mtp_dtype dtype, int32_t batch, int32_t gamma,
                             int32_t vocab, const int32_t* draft_tokens, float temperature, uint64_t seed,
                             uint64_t offset, uint8_t* accept, int32_t* accepted_len, int32_t* next_token,
                             int32_t* row_token, float* overlap, float* tv, float* entropy, int32_t* row_status,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(mtp::kVerifyGumbel, temperature, target, target_row_stride, draft, draft_row_stride, dtype,
                     batch, gamma, vocab, draft_tokens, seed, offset, accept, accepted_len, next_token, nullptr,
                     nullptr, nullptr, row_token, overlap, tv, entropy, row_status, workspace, workspace_bytes,
                     stream);
}

mtp_status mtp_gumbel_sample_workspace_size(int32_t rows, int32_t vocab, mtp_dtype dtype, size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_NULL, "bytes is NULL");
  if (dtype != MTP_F32 && dtype != MTP_BF16) return fail(MTP_ERR_DTYPE, "unknown dtype code %d", (int)dtype);
  if (rows < 0) return fail(MTP_ERR_SHAPE, "rows = %d is negative", rows);
  if (vocab < 1 || vocab > kMaxVocab) return fail(MTP_ERR_SHAPE, "vocab = %d outside [1, 2^30]", vocab);
  *bytes = rows == 0 ? 0 : align256((size_t)rows * mtp::gumbel_sample_chunks_per_row(dtype, vocab) * 8);
  return ok();
}

mtp_status mtp_gumbel_sample(const void* logits, int64_t row_stride, mtp_dtype dtype, int32_t rows, int32_t vocab,
                             float temperature, uint64_t seed, uint64_t offset, int32_t* tokens, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (dtype != MTP_F32 && dtype != MTP_BF16) return fail(MTP_ERR_DTYPE, "unknown dtype code %d", (int)dtype);
  if (rows < 0) return fail(MTP_ERR_SHAPE, "rows = %d is negative", rows);
  if (vocab < 1 || vocab > kMaxVocab) return fail(MTP_ERR_SHAPE, "vocab = %d outside [1, 2^30]", vocab);
  if (bad_temperature(temperature))
    return fail(MTP_ERR_SHAPE, "temperature %g is not a positive finite number", (double)temperature);
  if (rows == 0) return ok();
  if (!logits || !tokens) return fail(MTP_ERR_NULL, "logits or tokens is NULL");
  if (row_stride < vocab)
    return fail(MTP_ERR_SHAPE, "row stride %lld must be >= vocab (%d)", (long long)row_stride, vocab);
  mtp_status s = check_row_base(logits, row_stride, dtype, "logits");
  if (s) return s;
  const int64_t nch = mtp::gumbel_sample_chunks_per_row(dtype, vocab);
  if ((int64_t)rows * nch * mtp::kBlock > 0xffffffffLL)
    return fail(MTP_ERR_SHAPE, "rows * vocab is too large for one launch");
  if ((s = check_workspace(workspace, workspace_bytes, align256((size_t)rows * nch * 8)))) return s;
  hipError_t e = mtp::launch_gumbel_sample(logits, row_stride, dtype, rows, vocab, kLog2e / temperature, seed,
                                           offset, tokens, reinterpret_cast<uint64_t*>(workspace),
                                           (hipStream_t)stream);
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "Gumbel sample launch failed: %s", hipGetErrorString(e));
  return ok();
}

mtp_status mtp_tv_loss_workspace_size(int32_t T, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                      int32_t shared_target, size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_NULL, "bytes is NULL");
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (T < 1) return fail(MTP_ERR_SHAPE, "T = %d must be >= 1", T);
  *bytes = tv_workspace_bytes(T, gamma, vocab, dtype, shared_target != 0);
  return ok();
}

static mtp_status check_tv_inputs(const void* target, int64_t tp, int64_t th, const void* draft, int64_t dp,
                                  int64_t dh, mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab) {
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (T < 1) return fail(MTP_ERR_SHAPE, "T = %d must be >= 1", T);
  if (!target || !draft) return fail(MTP_ERR_NULL, "target or draft is NULL");
  if (tp < 0 || th < 0 || dp < 0 || dh < 0) return fail(MTP_ERR_SHAPE, "negative stride");
  if ((s = check_row_base(target, tp, dtype, "target position"))) return s;
  if ((s = check_row_base(target, th, dtype, "target head"))) return s;
  if ((s = check_row_base(draft, dp, dtype, "draft position"))) return s;
  if ((s = check_row_base(draft, dh, dtype, "draft head"))) return s;
  return MTP_OK;
}

mtp_status mtp_tv_loss_fwd(const void* target, int64_t target_pos_stride, int64_t target_head_stride,
                           const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                           mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab, float* loss,
                           float* pos_loss, float* saved, void* workspace, size_t workspace_bytes,
                           void* stream) {
  mtp_status s = check_tv_inputs(target, target_pos_stride, target_head_stride, draft, draft_pos_stride,
                                 draft_head_stride, dtype, T, gamma, vocab);
  if (s) return s;
  if (!loss || !saved) return fail(MTP_ERR_NULL, "loss or saved is NULL");
  const bool shared = target_head_stride == 0;
  if ((s = check_workspace(workspace, workspace_bytes, tv_workspace_bytes(T, gamma, vocab, dtype, shared)))) return s;
  // the single-read forward when a position's rows fit it and every chunk of a row
  // can be resident at once; otherwise the two streaming passes
  bool pipe = false;
  int sgroups = 0, layers = 0;
  if (mtp::tv_pipe_vec_per_thread(dtype, gamma, shared) > 0) {
    int64_t per_gpu = 0;
    if ((s = tv_pipe_capacity(dtype, gamma, shared, &per_gpu))) return s;
    const TvLayout Lp = tv_layout(T, gamma, vocab, dtype, shared, true);
    if ((int64_t)Lp.sp.nchunks <= per_gpu) {
      pipe = true;
      plan_layers(per_gpu, Lp.sp.nchunks, T, &sgroups, &layers);
    }
  }
  const TvLayout L = tv_layout(T, gamma, vocab, dtype, shared, pipe);
  if ((int64_t)T * L.sp.nchunks > 0x7fffffffLL) return fail(MTP_ERR_SHAPE, "T * chunks is too large");
  mtp::TvArgs a{};
  a.target = target; a.t_pos = target_pos_stride; a.t_head = target_head_stride;
  a.draft = draft; a.d_pos = draft_pos_stride; a.d_head = draft_head_stride;
  a.T = T; a.G = gamma; a.V = vocab;
  a.loss = loss; a.pos_loss = pos_loss; a.saved = saved;
  a.err = at<uint32_t>(workspace, L.err);
  a.part1 = at<uint64_t>(workspace, L.part1);
  a.part2 = at<float>(workspace, L.part2);
  a.pos_ws = at<float>(workspace, L.pos);
  a.sp = L.sp;
  a.sgroups = sgroups;   // positions strided (a split by dispatch round measured no faster)
  a.wait_limit = g_wait_limit.load(std::memory_order_relaxed);
  hipError_t e = pipe ? mtp::launch_tv_pipe_fwd(a, dtype, shared, (hipStream_t)stream)
                      : mtp::launch_tv_fwd(a, dtype, shared, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "TV forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

static mtp_status check_topk_inputs(const int32_t* idx, const float* val, int64_t kp, int64_t kh, int32_t K,
                                    const void* draft, int64_t dp, int64_t dh, mtp_dtype dtype, int32_t T,
                                    int32_t gamma, int32_t vocab) {
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (T < 1) return fail(MTP_ERR_SHAPE, "T = %d must be >= 1", T);
  if (K < 1 || K > kMaxTopK) return fail(MTP_ERR_SHAPE, "K = %d outside [1, %d]", K, kMaxTopK);
  if (!idx || !val || !draft) return fail(MTP_ERR_NULL, "target_idx, target_val or draft is NULL");
  if (kp < 0 || kh < 0 || dp < 0 || dh < 0) return fail(MTP_ERR_SHAPE, "negative stride");
  if (((uintptr_t)idx & 3u) || ((uintptr_t)val & 3u))
    return fail(MTP_ERR_ALIGN, "target_idx or target_val is not 4-byte aligned");
  if ((s = check_row_base(draft, dp, dtype, "draft position"))) return s;
  if ((s = check_row_base(draft, dh, dtype, "draft head"))) return s;
  return MTP_OK;
}

mtp_status mtp_tv_topk_workspace_size(int32_t T, int32_t gamma, int32_t vocab, mtp_dtype dtype, size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_NULL, "bytes is NULL");
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (T < 1) return fail(MTP_ERR_SHAPE, "T = %d must be >= 1", T);
  *bytes = topk_layout(T, gamma, vocab, dtype).total;
  return ok();
}

mtp_status mtp_tv_topk_fwd(const int32_t* target_idx, const float* target_val, int64_t topk_pos_stride,
                           int64_t topk_head_stride, int32_t K, const void* draft, int64_t draft_pos_stride,
                           int64_t draft_head_stride, mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab,
                           float* loss, float* pos_loss, float* saved, void* workspace, size_t workspace_bytes,
                           void* stream) {
  mtp_status s = check_topk_inputs(target_idx, target_val, topk_pos_stride, topk_head_stride, K, draft,
                                   draft_pos_stride, draft_head_stride, dtype, T, gamma, vocab);
  if (s) return s;
  if (!loss || !saved) return fail(MTP_ERR_NULL, "loss or saved is NULL");
  const TvLayout L = topk_layout(T, gamma, vocab, dtype);
  if ((s = check_workspace(workspace, workspace_bytes, L.total))) return s;
  if ((int64_t)T * L.sp.nchunks > 0x7fffffffLL) return fail(MTP_ERR_SHAPE, "T * chunks is too large");
  mtp::TvArgs a{};
  a.idx = target_idx; a.val = target_val; a.k_pos = topk_pos_stride; a.k_head = topk_head_stride; a.K = K;
  a.draft = draft; a.d_pos = draft_pos_stride; a.d_head = draft_head_stride;
  a.T = T; a.G = gamma; a.V = vocab;
  a.loss = loss; a.pos_loss = pos_loss; a.saved = saved;
  a.err = at<uint32_t>(workspace, L.err);
  a.part1 = at<uint64_t>(workspace, L.part1);
  a.pos_ws = at<float>(workspace, L.pos);
  a.sp = L.sp;
  hipError_t e = mtp::launch_tv_topk_fwd(a, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "top-K TV forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

mtp_status mtp_tv_topk_bwd(const int32_t* target_idx, const float* target_val, int64_t topk_pos_stride,
                           int64_t topk_head_stride, int32_t K, const void* draft, int64_t draft_pos_stride,
                           int64_t draft_head_stride, mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab,
                           const float* saved, const float* grad_loss, void* grad, int64_t grad_pos_stride,
                           int64_t grad_head_stride, mtp_dtype grad_dtype, void* stream) {
  mtp_status s = check_topk_inputs(target_idx, target_val, topk_pos_stride, topk_head_stride, K, draft,
                                   draft_pos_stride, draft_head_stride, dtype, T, gamma, vocab);
  if (s) return s;
  if (grad_dtype != MTP_F32 && grad_dtype != MTP_BF16)
    return fail(MTP_ERR_DTYPE, "unknown grad dtype code %d", (int)grad_dtype);
  if (!saved || !grad_loss || !grad) return fail(MTP_ERR_NULL, "saved, grad_loss or grad is NULL");
  if (grad_pos_stride < 0 || grad_head_stride < 0) return fail(MTP_ERR_SHAPE, "negative grad stride");
  if ((s = check_row_base(grad, grad_pos_stride, grad_dtype, "grad position"))) return s;
  if ((s = check_row_base(grad, grad_head_stride, grad_dtype, "grad head"))) return s;
  mtp::TvArgs a{};
  a.idx = target_idx; a.val = target_val; a.k_pos = topk_pos_stride; a.k_head = topk_head_stride; a.K = K;
  a.draft = draft; a.d_pos = draft_pos_stride; a.d_head = draft_head_stride;
  a.T = T; a.G = gamma; a.V = vocab;
  a.saved_in = saved; a.grad_loss = grad_loss;
  a.grad = grad; a.g_pos = grad_pos_stride; a.g_head = grad_head_stride; a.grad_dt = grad_dtype;
  a.sp = mtp::make_split(vocab, per_vec(dtype), mtp::tv_bwd_vec_per_thread(dtype));
  if ((int64_t)T * a.sp.nchunks > 0x7fffffffLL) return fail(MTP_ERR_SHAPE, "T * chunks is too large");
  hipError_t e = mtp::launch_tv_topk_bwd(a, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "top-K TV backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

mtp_status mtp_tv_loss_bwd(const void* target, int64_t target_pos_stride, int64_t target_head_stride,
                           const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                           mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab, const float* saved,
                           const float* grad_loss, void* grad, int64_t grad_pos_stride,
                           int64_t grad_head_stride, mtp_dtype grad_dtype, void* stream) {
  mtp_status s = check_tv_inputs(target, target_pos_stride, target_head_stride, draft, draft_pos_stride,
                                 draft_head_stride, dtype, T, gamma, vocab);
  if (s) return s;
  if (grad_dtype != MTP_F32 && grad_dtype != MTP_BF16)
    return fail(MTP_ERR_DTYPE, "unknown grad dtype code %d", (int)grad_dtype);
  if (!saved || !grad_loss || !grad) return fail(MTP_ERR_NULL, "saved, grad_loss or grad is NULL");
  if (grad_pos_stride < 0 || grad_head_stride < 0) return fail(MTP_ERR_SHAPE, "negative grad stride");
  if ((s = check_row_base(grad, grad_pos_stride, grad_dtype, "grad position"))) return s;
  if ((s = check_row_base(grad, grad_head_stride, grad_dtype, "grad head"))) return s;
  const bool shared = target_head_stride == 0;
  mtp::TvArgs a{};
  a.target = target; a.t_pos = target_pos_stride; a.t_head = target_head_stride;
  a.draft = draft; a.d_pos = draft_pos_stride; a.d_head = draft_head_stride;
  a.T = T; a.G = gamma; a.V = vocab;
  a.saved_in = saved; a.grad_loss = grad_loss;
  a.grad = grad; a.g_pos = grad_pos_stride; a.g_head = grad_head_stride; a.grad_dt = grad_dtype;
  a.sp = mtp::make_split(vocab, per_vec(dtype), mtp::tv_bwd_full_vec_per_thread(dtype, gamma, shared));
  if ((int64_t)T * a.sp.nchunks > 0x7fffffffLL) return fail(MTP_ERR_SHAPE, "T * chunks is too large");
  hipError_t e = mtp::launch_tv_bwd(a, dtype, shared, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "TV backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

mtp_status mtp_verify_noalloc(const void* target, int64_t target_row_stride, const void* draft,
                              int64_t draft_row_stride, mtp_dtype dtype, int32_t batch, int32_t gamma,
                              int32_t vocab, const int32_t* draft_tokens, uint64_t seed, uint64_t offset,
                              uint8_t* accept, int32_t* accepted_len, int32_t* next_token, int32_t* row_token,
                              float* overlap, float* tv, float* entropy, int32_t* row_status, void* stream) {
  mtp_status s = verify_check_args(mtp::kVerifyRejection, 1.f, target, target_row_stride, draft, draft_row_stride,
                                   dtype, batch, gamma, vocab, draft_tokens, accept, accepted_len, next_token,
                                   nullptr);
  if (s) return s;
  if (batch == 0) return ok();
  const size_t need = verify_layout(batch, gamma, vocab, dtype, mtp::kVerifyRejection).total;
  if (need > kScratchBytes)
    return fail(MTP_ERR_WORKSPACE,
                "batch %d x (gamma %d + 1) rows of vocab %d need %zu bytes of scratch; mtp_verify_noalloc has %zu "
                "(use mtp_verify with a workspace)", batch, gamma, vocab, need, kScratchBytes);
  void* ws = nullptr;
  if ((s = device_scratch((hipStream_t)stream, &ws))) return s;
  return verify_impl(mtp::kVerifyRejection, 1.f, target, target_row_stride, draft, draft_row_stride, dtype, batch,
                     gamma, vocab, draft_tokens, seed, offset, accept, accepted_len, next_token, nullptr, nullptr,
                     nullptr, row_token, overlap, tv, entropy, row_status, ws, kScratchBytes, stream);
}

mtp_status mtp_tv_loss_fwd_bwd_workspace_size(int32_t T, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                              int32_t shared_target, size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_NULL, "bytes is NULL");
  mtp_status s = check_common(dtype, gamma, vocab);
  if (s) return s;
  if (T < 1) return fail(MTP_ERR_SHAPE, "T = %d must be >= 1", T);
  *bytes = fused_workspace_bytes(T, gamma, vocab, dtype, shared_target != 0);
  return ok();
}

mtp_status mtp_tv_loss_fwd_bwd(const void* target, int64_t target_pos_stride, int64_t target_head_stride,
                               const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                               mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab, const float* grad_loss,
                               float* loss, float* pos_loss, float* saved, void* grad, int64_t grad_pos_stride,
                               int64_t grad_head_stride, mtp_dtype grad_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  mtp_status s = check_tv_inputs(target, target_pos_stride, target_head_stride, draft, draft_pos_stride,
                                 draft_head_stride, dtype, T, gamma, vocab);
  if (s) return s;
  if (grad_dtype != MTP_F32 && grad_dtype != MTP_BF16)
    return fail(MTP_ERR_DTYPE, "unknown grad dtype code %d", (int)grad_dtype);
  if (!loss || !saved || !grad_loss || !grad) return fail(MTP_ERR_NULL, "loss, saved, grad_loss or grad is NULL");
  if (grad_pos_stride < 0 || grad_head_stride < 0) return fail(MTP_ERR_SHAPE, "negative grad stride");
  if ((s = check_row_base(grad, grad_pos_stride, grad_dtype, "grad position"))) return s;
  if ((s = check_row_base(grad, grad_head_stride, grad_dtype, "grad head"))) return s;
  const bool shared = target_head_stride == 0;
  if ((s = check_workspace(workspace, workspace_bytes, fused_workspace_bytes(T, gamma, vocab, dtype, shared)))) return s;
  // one sweep when the shape fits the fused kernel and every chunk of a row can be
  // resident at once; otherwise the forward call, then the backward call
  bool fused = false;
  int sgroups = 0, layers = 0;
  FusedLayout L{};
  // One head with bfloat16 logits and a bfloat16 gradient is the one shape where
  // the one-sweep kernel runs out of registers (it spills) and the two calls are
  // faster (0.63 against 0.81 ms at T = 2048, V = 151936): it takes the two calls.
  const bool spills = gamma == 1 && dtype == MTP_BF16 && grad_dtype == MTP_BF16;
  if (fused_shape(gamma, shared) && !spills) {
    int64_t per_gpu = 0;
    if ((s = tv_fused_capacity(dtype, grad_dtype, gamma, shared, &per_gpu))) return s;
    L = fused_layout(T, gamma, vocab, dtype, shared);
    if ((int64_t)L.sp.nchunks <= per_gpu && (int64_t)T * L.sp.nchunks <= 0x7fffffffLL) {
      fused = true;
      plan_layers(per_gpu, L.sp.nchunks, T, &sgroups, &layers);
    }
  }
  if (!fused) {
    if ((s = mtp_tv_loss_fwd(target, target_pos_stride, target_head_stride, draft, draft_pos_stride,
                             draft_head_stride, dtype, T, gamma, vocab, loss, pos_loss, saved, workspace,
                             workspace_bytes, stream)))
      return s;
    return mtp_tv_loss_bwd(target, target_pos_stride, target_head_stride, draft, draft_pos_stride,
                           draft_head_stride, dtype, T, gamma, vocab, saved, grad_loss, grad, grad_pos_stride,
                           grad_head_stride, grad_dtype, stream);
  }
  mtp::TvArgs a{};
  a.target = target; a.t_pos = target_pos_stride; a.t_head = target_head_stride;
  a.draft = draft; a.d_pos = draft_pos_stride; a.d_head = draft_head_stride;
  a.T = T; a.G = gamma; a.V = vocab;
  a.loss = loss; a.pos_loss = pos_loss; a.saved = saved;
  a.grad_loss = grad_loss;
  a.grad = grad; a.g_pos = grad_pos_stride; a.g_head = grad_head_stride; a.grad_dt = grad_dtype;
  a.err = at<uint32_t>(workspace, L.err);
  a.part1 = at<uint64_t>(workspace, L.part1);
  a.part3 = at<uint64_t>(workspace, L.part3);
  a.pos_ws = at<float>(workspace, L.pos);
  a.sp = L.sp;
  a.sgroups = sgroups;
  if (T >= 16 * (int64_t)sgroups)
    a.split = plan_round_split(sgroups, L.sp.nchunks, T, device_cus(), kTvRoundCost);
  a.wait_limit = g_wait_limit.load(std::memory_order_relaxed);
  hipError_t e = mtp::launch_tv_fused(a, dtype, shared, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "fused TV loss launch failed: %s", hipGetErrorString(e));
  return ok();
}

mtp_status mtp_workspace_error(const void* workspace, uint32_t* host_word, void* stream) {
  if (!workspace || !host_word) return fail(MTP_ERR_NULL, "workspace or host_word is NULL");
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(host_word, workspace, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(MTP_ERR_DEVICE, "cannot read the workspace error word");
  return ok();
}

}  // extern "C"
