// Host side of the C ABI declared in include/rkv.h: argument validation,
// workspace layout, the launch sequence, error reporting and launch timing.
//
// Every check happens before the first HIP call, so an invalid call leaves
// device memory and the stream untouched and can be tested without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rkv.h"
#include "rkv_launch.hpp"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the caller's workspace (or a size count when base is null).
struct Carve {
  char* base;
  size_t used = 0;
  template <typename X>
  X* take(size_t count) {
    X* p = base ? reinterpret_cast<X*>(base + used) : nullptr;
    used += align_up(count * sizeof(X));
    return p;
  }
};

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return (1 << s) == v ? s : -1;
}

// Query rows per GQA head in the importance kernels: 8, 16 or 32 (>= w).
int rows_per_group_shift(int w) { return w <= 8 ? 3 : (w <= 16 ? 4 : 5); }

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return an > 0 && bn > 0 && pa < pb + bn && pb < pa + an;
}

// ---- timing -----------------------------------------------------------------
struct TimingRec {
  const char* name;
  hipEvent_t start, stop;
};
struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t pool_used = 0;
  std::vector<TimingRec> recs;
};
TimingState& timing() {
  static TimingState t;
  return t;
}
constexpr size_t kMaxTimed = 65536;

}  // namespace

namespace rkv {

struct TimingSlot {
  size_t index;
};

TimingSlot* timing_begin(const char* name, hipStream_t st) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.on || t.recs.size() >= kMaxTimed) return nullptr;
  while (t.pool_used + 2 > t.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    t.pool.push_back(e);
  }
  TimingRec r{name, t.pool[t.pool_used], t.pool[t.pool_used + 1]};
  t.pool_used += 2;
  if (hipEventRecord(r.start, st) != hipSuccess) return nullptr;
  t.recs.push_back(r);
  return reinterpret_cast<TimingSlot*>(t.recs.size());   // 1-based index as a token
}

void timing_end(TimingSlot* slot, hipStream_t st) {
  if (slot == nullptr) return;
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  const size_t idx = reinterpret_cast<size_t>(slot) - 1;
  if (idx < t.recs.size()) (void)hipEventRecord(t.recs[idx].stop, st);
}

}  // namespace rkv

using rkv::bf16_bits;
using rkv::DenseProblem;
using rkv::PagedProblem;

// ---- dense --------------------------------------------------------------------
namespace {

struct DenseLayout {
  float* rinv;       // [units][N] 1/||k_t|| (0 for a zero key)
  float* z;          // [units][N] joint scores when the caller does not ask for them
  float* part;       // [units][chunks][NQB*32] per-chunk softmax (max, sum)
  float* fin;        // [units][NQB*32] per query row (max, 1/sum)
  int32_t* counters; // [8 + units] item claims per XCD, then blocks completed per unit
  float* zsum;       // [units / select_group][N] summed scores of head-shared selection
  size_t bytes;
};

int check_common(int head_dim, int gqa, int window, float lam, int dtype) {
  if (head_dim != 128) return fail(RKV_EINVAL, "head_dim must be 128 (got %d)", head_dim);
  if (gqa < 1) return fail(RKV_EINVAL, "gqa_group must be >= 1 (got %d)", gqa);
  if (window < 1) return fail(RKV_EINVAL, "window must be >= 1 (got %d)", window);
  if (window > 32) return fail(RKV_EUNSUPPORTED, "window above 32 is not supported (got %d)", window);
  if (!std::isfinite(lam)) return fail(RKV_EINVAL, "mix_lambda must be finite");
  if (dtype != RKV_F32 && dtype != RKV_BF16) return fail(RKV_EINVAL, "unknown dtype %d", dtype);
  const int rows = gqa << rows_per_group_shift(window);
  const int max_rows = dtype == RKV_BF16 ? 128 : 64;
  if (rows > max_rows)
    return fail(RKV_EUNSUPPORTED,
                "gqa_group * window rounded up to 8/16/32 per head must be <= %d (got %d)",
                max_rows, rows);
  const rkv::K2Lds plan = rkv::k2_lds_plan(dtype == RKV_BF16 ? 256 : 512, gqa * window, (rows + 31) / 32);
  if (plan.total > rkv::kLdsBytesPerCU)
    return fail(RKV_EUNSUPPORTED,
                "gqa_group * window = %d needs %d bytes of LDS for the %s kernels (limit %d)",
                gqa * window, plan.total, dtype == RKV_BF16 ? "bf16" : "fp32", rkv::kLdsBytesPerCU);
  return RKV_OK;
}

int check_dense_desc(const rkv_dense_desc* d) {
  if (d == nullptr) return fail(RKV_EINVAL, "desc is NULL");
  int rc = check_common(d->head_dim, d->gqa_group, d->window, d->mix_lambda, d->dtype);
  if (rc) return rc;
  if (d->num_heads < 0) return fail(RKV_EINVAL, "num_heads must be >= 0 (got %d)", d->num_heads);
  if (d->n_cand < 1) return fail(RKV_EINVAL, "n_cand must be >= 1 (got %d)", d->n_cand);
  if (d->budget <= d->window)
    return fail(RKV_EINVAL, "budget (%d) must exceed window (%d)", d->budget, d->window);
  if (d->kv_head_stride != 0 && d->kv_head_stride < (int64_t)d->n_cand * 128)
    return fail(RKV_EINVAL, "kv_head_stride %lld is below n_cand*128", (long long)d->kv_head_stride);
  if (d->out_head_stride != 0 && d->out_head_stride < (int64_t)d->budget * 128)
    return fail(RKV_EINVAL, "out_head_stride %lld is below budget*128", (long long)d->out_head_stride);
  if ((int64_t)d->num_heads * d->n_cand > (int64_t)1 << 40)
    return fail(RKV_EINVAL, "num_heads * n_cand too large");
  if ((int64_t)(d->num_heads + 7) / 8 * 8 * ((d->n_cand + rkv::kK2Rows - 1) / rkv::kK2Rows) > INT32_MAX)
    return fail(RKV_EINVAL, "num_heads * ceil(n_cand / 128) must stay below 2^31");
  if (d->variant & RKV_VARIANT_SHARED_HEADS)
    return fail(RKV_EINVAL, "RKV_VARIANT_SHARED_HEADS is for paged calls; dense calls take select_group");
  if (d->variant & ~rkv::kVariantMask)
    return fail(RKV_EINVAL, "unknown variant bits 0x%x", (unsigned)(d->variant & ~rkv::kVariantMask));
  if (d->select_group < 0) return fail(RKV_EINVAL, "select_group must be >= 0 (got %d)", d->select_group);
  if (d->select_group > 1 && d->num_heads % d->select_group != 0)
    return fail(RKV_EINVAL, "num_heads (%d) must be a multiple of select_group (%d)", d->num_heads,
                d->select_group);
  return RKV_OK;
}

int nqb_of(int gqa, int window);

DenseLayout dense_layout(const rkv_dense_desc* d, char* base) {
  Carve c{base};
  const size_t units = (size_t)d->num_heads, n = (size_t)d->n_cand;
  const size_t nqb = (size_t)nqb_of(d->gqa_group, d->window);
  const size_t chunks = (n + rkv::kK1Keys - 1) / rkv::kK1Keys;
  DenseLayout L;
  L.rinv = c.take<float>(units * n);
  L.z = c.take<float>(units * n);
  L.part = c.take<float>(units * chunks * nqb * 32 * 2);
  L.fin = c.take<float>(units * nqb * 32 * 2);
  L.counters = c.take<int32_t>(8 + units);
  L.zsum = d->select_group > 1 ? c.take<float>(units / (size_t)d->select_group * n) : nullptr;
  L.bytes = std::max<size_t>(c.used, kAlign);
  return L;
}

int nqb_of(int gqa, int window) {
  const int rows = gqa << rows_per_group_shift(window);
  return (rows + 31) / 32;
}

template <typename T>
int dense_run(const rkv_dense_desc* d, const void* K, const void* V, const void* Q,
              int32_t* kept, void* K_out, void* V_out, float* dbg_I, float* dbg_R, float* dbg_Z,
              const DenseLayout& L, hipStream_t st) {
  DenseProblem<T> p;
  p.K = static_cast<const T*>(K);
  p.V = static_cast<const T*>(V);
  p.Q = static_cast<const T*>(Q);
  p.kv_stride = d->kv_head_stride ? d->kv_head_stride : (int64_t)d->n_cand * 128;
  p.num_units = d->num_heads;
  p.N = d->n_cand;
  p.B = d->budget;
  p.G = d->gqa_group;
  p.W = d->window;
  p.k1_chunks = (d->n_cand + rkv::kK1Keys - 1) / rkv::kK1Keys;
  p.k2_blocks = (d->n_cand + rkv::kK2Rows - 1) / rkv::kK2Rows;
  p.variant = d->variant;
  const int64_t out_stride = d->out_head_stride ? d->out_head_stride : (int64_t)d->budget * 128;
  const int units = d->num_heads;
  const int nkeep = std::min(d->n_cand, d->budget);
  hipError_t e;
  if (d->n_cand > d->budget) {
    const int rpg_shift = rows_per_group_shift(d->window);
    const int nqb = nqb_of(d->gqa_group, d->window);
    // head-shared selection: units are scored alone, then each group selects
    // once on its summed scores and every unit gathers its own rows
    const int group = d->select_group > 1 ? d->select_group : 1;
    const bool shared = group > 1;
    float* z = dbg_Z ? dbg_Z : L.z;
    bool scored = false;
    if constexpr (sizeof(T) == 2) {
      if (rkv::k2_resident_fits(p, nqb)) {
        // every key read once, the first N-128 held in registers
        e = rkv::run_k2_resident(p, nqb, shared ? z : dbg_Z, dbg_R, dbg_I, d->mix_lambda,
                                 rpg_shift, kept, static_cast<T*>(K_out), static_cast<T*>(V_out),
                                 out_stride, shared ? 1 : 0, st);
        if (e != hipSuccess) return hip_fail(e, "compression launch");
        scored = true;
      } else if (rkv::k2_resident2_fits(p, rpg_shift)) {
        // up to 2048 + 128 candidates: keys held in registers in two passes
        e = rkv::run_k2_resident2(p, shared ? z : dbg_Z, dbg_R, dbg_I, d->mix_lambda, rpg_shift,
                                  kept, static_cast<T*>(K_out), static_cast<T*>(V_out), out_stride,
                                  shared ? 1 : 0, st);
        if (e != hipSuccess) return hip_fail(e, "compression launch");
        scored = true;
      } else if (rkv::fused_plan_choose(p.N, p.B, p.G * p.W, nqb).total > 0) {
        e = rkv::run_k2_fused(p, nqb, shared ? z : dbg_Z, dbg_R, dbg_I, d->mix_lambda, rpg_shift,
                              kept, static_cast<T*>(K_out), static_cast<T*>(V_out), out_stride,
                              shared ? 1 : 0, st);
        if (e != hipSuccess) return hip_fail(e, "compression launch");
        scored = true;
      }
    }
    if (!scored) {
      // units too long for one workgroup's LDS, and fp32: statistics pass first
      e = rkv::run_k1<T>(p, nqb, units * p.k1_chunks, units, L.part, L.fin, L.rinv, L.counters,
                         rpg_shift, st);
      if (e != hipSuccess) return hip_fail(e, "importance launch");
      if constexpr (sizeof(T) == 2) {
        // bf16: row blocks by the long-unit kernel, then selection and gather
        const int lb = rkv::long_block_rows(nqb, p.symmetric());
        p.long_shift = lb == 1024 ? 10 : 9;
        const int count = units * ((p.N + lb - 1) / lb);
        e = rkv::run_k2_long(p, nqb, count, L.rinv, L.fin, z, dbg_R, dbg_I, d->mix_lambda, rpg_shift,
                             st);
        if (e != hipSuccess) return hip_fail(e, "redundancy launch");
        if (!shared) {
          e = rkv::run_k4(p, units, z, kept, 1, st);
          if (e != hipSuccess) return hip_fail(e, "select launch");
          e = rkv::run_k5_dense<T>(p, kept, static_cast<T*>(K_out), static_cast<T*>(V_out),
                                   out_stride, nkeep, st);
          if (e != hipSuccess) return hip_fail(e, "gather launch");
        }
      } else {
        // fp32: XCD-local teams of workgroups per unit, the last one finishing it
        const int k2_items = 8 * ((units + 7) / 8) * p.k2_blocks;
        e = rkv::run_k2<T>(p, nqb, k2_items, L.rinv, L.fin, z, dbg_R, dbg_I, d->mix_lambda,
                           rpg_shift, L.counters, kept, static_cast<T*>(K_out),
                           static_cast<T*>(V_out), out_stride, shared ? 0 : 1, st);
        if (e != hipSuccess) return hip_fail(e, "compression launch");
      }
    }
    if (shared) {
      e = rkv::run_k4_group(p, group, z, L.zsum, kept, st);
      if (e != hipSuccess) return hip_fail(e, "shared selection launch");
      e = rkv::run_k5_dense<T>(p, kept, static_cast<T*>(K_out), static_cast<T*>(V_out), out_stride,
                               nkeep, st);
      if (e != hipSuccess) return hip_fail(e, "gather launch");
    }
    return RKV_OK;
  }
  e = rkv::run_k4(p, units, L.z, kept, 1, st);   // N <= B: identity selection and a plain copy
  if (e != hipSuccess) return hip_fail(e, "select launch");
  e = rkv::run_k5_dense<T>(p, kept, static_cast<T*>(K_out), static_cast<T*>(V_out), out_stride,
                           nkeep, st);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return RKV_OK;
}

}  // namespace

extern "C" size_t rkv_workspace_size(const rkv_dense_desc* desc) {
  if (check_dense_desc(desc) != RKV_OK) return 0;
  return dense_layout(desc, nullptr).bytes;
}

namespace {

// Checks of a dense call's buffers (the descriptor is valid and num_heads > 0).
int check_dense_buffers(const rkv_dense_desc* desc, const void* K, const void* V, const void* Q_win,
                        const int32_t* kept_idx, const void* K_out, const void* V_out) {
  if (!K || !V || !Q_win || !kept_idx || !K_out || !V_out)
    return fail(RKV_EINVAL, "K, V, Q_win, kept_idx, K_out and V_out must be non-NULL");
  const size_t es = desc->dtype == RKV_BF16 ? 2 : 4;
  const int64_t in_stride = desc->kv_head_stride ? desc->kv_head_stride : (int64_t)desc->n_cand * 128;
  const int64_t out_stride = desc->out_head_stride ? desc->out_head_stride : (int64_t)desc->budget * 128;
  const size_t in_bytes = ((size_t)(desc->num_heads - 1) * in_stride + (size_t)desc->n_cand * 128) * es;
  const size_t out_bytes = ((size_t)(desc->num_heads - 1) * out_stride +
                            (size_t)std::min(desc->n_cand, desc->budget) * 128) * es;
  if (ranges_overlap(K_out, out_bytes, K, in_bytes) || ranges_overlap(K_out, out_bytes, V, in_bytes) ||
      ranges_overlap(V_out, out_bytes, K, in_bytes) || ranges_overlap(V_out, out_bytes, V, in_bytes) ||
      ranges_overlap(K_out, out_bytes, V_out, out_bytes))
    return fail(RKV_EINVAL, "K_out and V_out must not overlap each other, K or V");
  return RKV_OK;
}

}  // namespace

extern "C" int rkv_compress(const rkv_dense_desc* desc, const void* K, const void* V,
                            const void* Q_win, int32_t* kept_idx, void* K_out, void* V_out,
                            float* dbg_I, float* dbg_R, float* dbg_Z, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int rc = check_dense_desc(desc);
  if (rc) return rc;
  const size_t need = dense_layout(desc, nullptr).bytes;
  if (desc->num_heads == 0) return RKV_OK;
  rc = check_dense_buffers(desc, K, V, Q_win, kept_idx, K_out, V_out);
  if (rc) return rc;
  if (!workspace || workspace_bytes < need)
    return fail(RKV_EWORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(RKV_EWORKSPACE, "workspace must be 256-byte aligned");
  const DenseLayout L = dense_layout(desc, static_cast<char*>(workspace));
  hipStream_t st = static_cast<hipStream_t>(stream);
  g_error.clear();
  if (desc->dtype == RKV_BF16)
    return dense_run<bf16_bits>(desc, K, V, Q_win, kept_idx, K_out, V_out, dbg_I, dbg_R, dbg_Z, L, st);
  return dense_run<float>(desc, K, V, Q_win, kept_idx, K_out, V_out, dbg_I, dbg_R, dbg_Z, L, st);
}

// ---- dense compression without allocation ---------------------------------------
// The workspace of rkv_compress_static: a device array of fixed size that
// every GPU the library runs on holds from load to process exit. In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is handed to kernels.
static __device__ __align__(256) char scratch[RKV_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RKV_EUNSUPPORTED, "device %d: at most %d devices are served", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % kAlign)
      return fail(RKV_EHIP, "device scratch of device %d is not 256-byte aligned", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RKV_OK;
}

}  // namespace

extern "C" int rkv_compress_static(const rkv_dense_desc* desc, const void* K, const void* V,
                                   const void* Q_win, int32_t* kept_idx, void* K_out, void* V_out,
                                   float* dbg_I, float* dbg_R, float* dbg_Z, void* stream) {
  int rc = check_dense_desc(desc);
  if (rc) return rc;
  const size_t need = dense_layout(desc, nullptr).bytes;
  if (desc->num_heads == 0) return RKV_OK;
  rc = check_dense_buffers(desc, K, V, Q_win, kept_idx, K_out, V_out);
  if (rc) return rc;
  if (need > RKV_STATIC_SCRATCH_BYTES)
    return fail(RKV_EWORKSPACE,
                "this call needs %zu bytes of workspace, above the %zu of the static scratch: "
                "split the units over several calls or use rkv_compress",
                need, (size_t)RKV_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  rc = device_scratch(&ws);
  if (rc) return rc;
  const DenseLayout L = dense_layout(desc, static_cast<char*>(ws));
  hipStream_t st = static_cast<hipStream_t>(stream);
  g_error.clear();
  if (desc->dtype == RKV_BF16)
    return dense_run<bf16_bits>(desc, K, V, Q_win, kept_idx, K_out, V_out, dbg_I, dbg_R, dbg_Z, L, st);
  return dense_run<float>(desc, K, V, Q_win, kept_idx, K_out, V_out, dbg_I, dbg_R, dbg_Z, L, st);
}

// ---- paged --------------------------------------------------------------------
namespace rkv {
// head-shared selection on pages (k4_shared.hip)
template <typename T>
hipError_t run_k4_paged_shared(const PagedProblem<T>& p, int num_seqs, const float* Z, float* zsum,
                               int32_t* kept, hipStream_t st);
}  // namespace rkv

namespace {

struct PagedPlan {
  // host-side metadata, uploaded in one copy
  std::vector<int32_t> seq_len, bud, free_off, unit_list;
  std::vector<int64_t> score_base, kept_base, k1_base, kc_base;
  std::vector<int2> k1_list, k2_list;
  std::vector<rkv::LongItem> long_list;
  int64_t total_scores = 0, total_kept = 0, total_chunks = 0;
  int64_t kc_elems = 0;   // contiguous key copy of the scored units (bf16, long-unit kernel)
  int32_t freed = 0;
  int nqb = 1;
  bool shared = false;   // head-shared selection: a sequence's heads keep one set
};

int check_paged(const rkv_paged_desc* d, const int32_t* seq_len, const int32_t* budget) {
  if (d == nullptr) return fail(RKV_EINVAL, "desc is NULL");
  int rc = check_common(d->head_dim, d->gqa_group, d->window, d->mix_lambda, d->dtype);
  if (rc) return rc;
  if (d->num_seqs < 0) return fail(RKV_EINVAL, "num_seqs must be >= 0");
  if (d->num_kv_heads < 1) return fail(RKV_EINVAL, "num_kv_heads must be >= 1");
  if (d->page_size < 1 || d->page_size > 4096 || log2_exact(d->page_size) < 0)
    return fail(RKV_EINVAL, "page_size must be a power of two in [1, 4096] (got %d)", d->page_size);
  if (d->max_pages_per_seq < 1) return fail(RKV_EINVAL, "max_pages_per_seq must be >= 1");
  if (d->num_pages < 1) return fail(RKV_EINVAL, "num_pages must be >= 1");
  if ((int64_t)d->num_seqs * d->num_kv_heads > (1 << 30)) return fail(RKV_EINVAL, "too many units");
  if (d->variant & ~(rkv::kVariantMask | RKV_VARIANT_SHARED_HEADS))
    return fail(RKV_EINVAL, "unknown variant bits 0x%x",
                (unsigned)(d->variant & ~(rkv::kVariantMask | RKV_VARIANT_SHARED_HEADS)));
  const int64_t slot = d->slot_stride ? d->slot_stride : 128;
  const int64_t head = d->head_stride ? d->head_stride : (int64_t)d->page_size * 128;
  const int64_t page = d->page_stride ? d->page_stride : (int64_t)d->num_kv_heads * d->page_size * 128;
  if (slot < 128 || head < 1 || page < 1)
    return fail(RKV_EINVAL, "page strides must be positive and slot_stride >= 128");
  if (d->num_seqs > 0 && (!seq_len || !budget))
    return fail(RKV_EINVAL, "seq_len_host and budget_host must be non-NULL");
  for (int s = 0; s < d->num_seqs; ++s) {
    const int n = seq_len[s], b = budget[s];
    if (n < 1) return fail(RKV_EINVAL, "seq_len[%d] = %d must be >= 1", s, n);
    if (b <= d->window) return fail(RKV_EINVAL, "budget[%d] = %d must exceed window %d", s, b, d->window);
    if (b % d->page_size) return fail(RKV_EINVAL, "budget[%d] = %d is not a multiple of page_size %d", s, b, d->page_size);
    if ((int64_t)(n + d->page_size - 1) / d->page_size > d->max_pages_per_seq)
      return fail(RKV_EINVAL, "seq_len[%d] = %d needs more than max_pages_per_seq pages", s, n);
  }
  return RKV_OK;
}

void paged_plan(const rkv_paged_desc* d, const int32_t* seq_len, const int32_t* budget, PagedPlan& P) {
  const int S = d->num_seqs, H = d->num_kv_heads, ps = d->page_size;
  P.nqb = nqb_of(d->gqa_group, d->window);
  P.shared = (d->variant & RKV_VARIANT_SHARED_HEADS) != 0;
  P.seq_len.assign(seq_len, seq_len + S);
  P.bud.assign(budget, budget + S);
  P.free_off.resize(S);
  P.score_base.resize(S);
  P.kept_base.resize(S);
  P.k1_base.assign((size_t)S * H, 0);
  P.kc_base.assign((size_t)S * H, 0);
  P.long_list.clear();
  P.kc_elems = 0;
  const bool bf16 = d->dtype == RKV_BF16;
  const bool sym = (d->variant & rkv::kVariantSymmetric) != 0;
  struct Costed { int64_t cost; rkv::LongItem it; };
  std::vector<Costed> litems;
  P.unit_list.clear();
  P.k1_list.clear();
  P.k2_list.clear();
  int64_t sc = 0, kp = 0, ch = 0;
  int32_t fr = 0;
  struct Item { int unit, blocks, n; };
  std::vector<Item> scored;
  for (int s = 0; s < S; ++s) {
    const int n = seq_len[s], b = budget[s];
    P.score_base[s] = sc;
    P.kept_base[s] = kp;
    P.free_off[s] = fr;
    sc += (int64_t)H * n;
    kp += (int64_t)H * std::min(n, b);
    if (n > b) {
      fr += (n + ps - 1) / ps - b / ps;
      const int nch = (n + rkv::kK1Keys - 1) / rkv::kK1Keys;
      for (int hk = 0; hk < H; ++hk) {
        const int u = s * H + hk;
        P.unit_list.push_back(u);
        P.k1_base[u] = ch;
        for (int c = 0; c < nch; ++c) P.k1_list.push_back(make_int2(u, c));
        ch += nch;
        scored.push_back({u, (n + rkv::kK2Rows - 1) / rkv::kK2Rows, n});
        if (bf16) {
          // long-unit kernel: contiguous copy of the unit's keys, items of
          // lb rows (tb tiles), costed by the tiles each streams
          P.kc_base[u] = P.kc_elems;
          const int lb = rkv::long_block_rows(P.nqb, sym), tb = lb / 128;
          const int nb = (n + 127) / 128, nbl = (n + lb - 1) / lb;
          for (int blk = 0; blk < nbl; ++blk) {
            rkv::LongItem it{u, blk, n, 0, P.kc_elems, sc - (int64_t)H * n + (int64_t)hk * n};
            const int own = std::min(tb, nb - tb * blk);
            const int64_t tiles = sym ? nb + own - 1 : (int64_t)tb * blk + own;
            litems.push_back({tiles, it});
          }
          P.kc_elems += (int64_t)n * 128;
        }
      }
    }
  }
  // Redundancy items: units longest first, dealt to the 8 XCDs round-robin;
  // each unit's row blocks stay on one XCD (longest block first) so its keys
  // are shared through that XCD's L2.
  std::stable_sort(scored.begin(), scored.end(), [](const Item& a, const Item& b) { return a.n > b.n; });
  std::vector<std::vector<int2>> q(8);
  for (size_t i = 0; i < scored.size(); ++i)
    for (int blk = scored[i].blocks - 1; blk >= 0; --blk) q[i % 8].push_back(make_int2(scored[i].unit, blk));
  size_t longest = 0;
  for (auto& v : q) longest = std::max(longest, v.size());
  for (size_t k = 0; k < longest; ++k)
    for (int x = 0; x < 8; ++x) P.k2_list.push_back(k < q[x].size() ? q[x][k] : make_int2(-1, 0));
  // long-unit items in order of decreasing work (ties: unit, then block)
  std::stable_sort(litems.begin(), litems.end(),
                   [](const Costed& a, const Costed& b) { return a.cost > b.cost; });
  for (const Costed& c : litems) P.long_list.push_back(c.it);
  P.total_scores = sc;
  P.total_kept = kp;
  P.total_chunks = ch;
  P.freed = fr;
}

struct PagedLayout {
  int32_t* seq_len;
  int32_t* bud;
  int32_t* free_off;
  int32_t* unit_list;
  int64_t* score_base;
  int64_t* kept_base;
  int64_t* k1_base;
  int2* k1_list;
  int2* k2_list;
  int64_t* kc_base;
  rkv::LongItem* long_list;
  void* kc;            // contiguous key copy (not uploaded)
  float* rinv;
  float* z;
  float* part;
  float* fin;
  float* zsum;         // head-shared selection: per-sequence sums of Z (else null)
  size_t meta_bytes;   // the uploaded prefix
  size_t bytes;
};

PagedLayout paged_layout(const rkv_paged_desc* d, const PagedPlan& P, char* base) {
  Carve c{base};
  const size_t S = (size_t)d->num_seqs, U = (size_t)d->num_seqs * d->num_kv_heads;
  PagedLayout L;
  L.seq_len = c.take<int32_t>(S);
  L.bud = c.take<int32_t>(S);
  L.free_off = c.take<int32_t>(S);
  L.unit_list = c.take<int32_t>(P.unit_list.size());
  L.score_base = c.take<int64_t>(S);
  L.kept_base = c.take<int64_t>(S);
  L.k1_base = c.take<int64_t>(U);
  L.k1_list = c.take<int2>(P.k1_list.size());
  L.k2_list = c.take<int2>(P.k2_list.size());
  L.kc_base = c.take<int64_t>(U);
  L.long_list = c.take<rkv::LongItem>(P.long_list.size());
  L.meta_bytes = c.used;
  L.kc = c.take<uint16_t>((size_t)P.kc_elems);
  L.rinv = c.take<float>(P.total_scores);
  L.z = c.take<float>(P.total_scores);
  L.part = c.take<float>((size_t)P.total_chunks * P.nqb * 32 * 2);
  L.fin = c.take<float>(U * P.nqb * 32 * 2);
  L.zsum = P.shared ? c.take<float>((size_t)(P.total_scores / std::max(1, d->num_kv_heads))) : nullptr;
  L.bytes = std::max<size_t>(c.used, kAlign);
  return L;
}

// Host image of the metadata prefix, laid out exactly as paged_layout places it.
void pack_meta(const PagedPlan& P, const PagedLayout& L, const char* base, std::vector<char>& img) {
  img.assign(L.meta_bytes, 0);
  auto put = [&](const void* dst, const void* src, size_t bytes) {
    if (bytes) std::memcpy(img.data() + (static_cast<const char*>(dst) - base), src, bytes);
  };
  put(L.seq_len, P.seq_len.data(), P.seq_len.size() * 4);
  put(L.bud, P.bud.data(), P.bud.size() * 4);
  put(L.free_off, P.free_off.data(), P.free_off.size() * 4);
  put(L.unit_list, P.unit_list.data(), P.unit_list.size() * 4);
  put(L.score_base, P.score_base.data(), P.score_base.size() * 8);
  put(L.kept_base, P.kept_base.data(), P.kept_base.size() * 8);
  put(L.k1_base, P.k1_base.data(), P.k1_base.size() * 8);
  put(L.k1_list, P.k1_list.data(), P.k1_list.size() * sizeof(int2));
  put(L.k2_list, P.k2_list.data(), P.k2_list.size() * sizeof(int2));
  put(L.kc_base, P.kc_base.data(), P.kc_base.size() * 8);
  put(L.long_list, P.long_list.data(), P.long_list.size() * sizeof(rkv::LongItem));
}

template <typename T>
int paged_run(const rkv_paged_desc* d, void* Kp, void* Vp, int32_t* page_table, const void* Q,
              int32_t* kept, int32_t* free_list, int32_t free_start, float* dbg_Z,
              const PagedPlan& P, const PagedLayout& L, hipStream_t st) {
  PagedProblem<T> p;
  p.Kp = static_cast<const T*>(Kp);
  p.Vp = static_cast<const T*>(Vp);
  p.Q = static_cast<const T*>(Q);
  p.page_table = page_table;
  p.slot_stride = d->slot_stride ? d->slot_stride : 128;
  p.head_stride = d->head_stride ? d->head_stride : (int64_t)d->page_size * 128;
  p.page_stride = d->page_stride ? d->page_stride : (int64_t)d->num_kv_heads * d->page_size * 128;
  p.maxp = d->max_pages_per_seq;
  p.num_pages = d->num_pages;
  p.ps_shift = log2_exact(d->page_size);
  p.H = d->num_kv_heads;
  p.G = d->gqa_group;
  p.W = d->window;
  p.seq_len = L.seq_len;
  p.bud = L.bud;
  p.score_base = L.score_base;
  p.kept_base = L.kept_base;
  p.k1_base = L.k1_base;
  p.k1_list = L.k1_list;
  p.k1_count = (int)P.k1_list.size();
  p.k2_list = L.k2_list;
  p.k2_count = (int)P.k2_list.size();
  p.unit_list = L.unit_list;
  p.unit_count = (int)P.unit_list.size();
  p.all_units = d->num_seqs * d->num_kv_heads;
  p.variant = d->variant & rkv::kVariantMask;   // the scoring readings
  float* z = dbg_Z ? dbg_Z : L.z;
  hipError_t e;
  if (p.unit_count > 0) {
    const int rpg_shift = rows_per_group_shift(d->window);
    if constexpr (sizeof(T) == 2) {   // the statistics pass also copies the keys
      p.Kc = static_cast<T*>(L.kc);
      p.kc_base = L.kc_base;
      p.long_list = L.long_list;
      p.long_cnt = (int)P.long_list.size();
    }
    e = rkv::run_k1<T>(p, P.nqb, p.k1_count, p.all_units, L.part, L.fin, L.rinv, nullptr,
                       rpg_shift, st);
    if (e != hipSuccess) return hip_fail(e, "importance launch");
    if constexpr (sizeof(T) == 2)
      e = rkv::run_k2_long(p, P.nqb, p.long_cnt, L.rinv, L.fin, z, nullptr, nullptr, d->mix_lambda,
                           rpg_shift, st);
    else
      e = rkv::run_k2<T>(p, P.nqb, p.k2_count, L.rinv, L.fin, z, nullptr, nullptr, d->mix_lambda,
                         rpg_shift, nullptr, nullptr, nullptr, nullptr, 0, 0, st);
    if (e != hipSuccess) return hip_fail(e, "redundancy launch");
  }
  if (P.shared)
    e = rkv::run_k4_paged_shared<T>(p, d->num_seqs, z, L.zsum, kept, st);
  else
    e = rkv::run_k4(p, p.all_units, z, kept, 0, st);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  if (p.unit_count > 0) {
    e = rkv::run_k5_paged<T>(p, static_cast<T*>(Kp), static_cast<T*>(Vp), kept, st);
    if (e != hipSuccess) return hip_fail(e, "compaction launch");
    e = rkv::run_free_pages(page_table, p.maxp, L.seq_len, L.bud, L.free_off, p.ps_shift,
                            d->num_seqs, free_list, free_start, st);
    if (e != hipSuccess) return hip_fail(e, "page return launch");
  }
  return RKV_OK;
}

thread_local std::vector<char> t_meta_image;

}  // namespace

extern "C" size_t rkv_paged_workspace_size(const rkv_paged_desc* desc, const int32_t* seq_len_host,
                                           const int32_t* budget_host) {
  if (check_paged(desc, seq_len_host, budget_host) != RKV_OK) return 0;
  PagedPlan P;
  paged_plan(desc, seq_len_host, budget_host, P);
  return paged_layout(desc, P, nullptr).bytes;
}

extern "C" int rkv_compress_paged(const rkv_paged_desc* desc, void* K_pages, void* V_pages,
                                  int32_t* page_table, const int32_t* seq_len_host,
                                  const int32_t* budget_host, const void* Q_win, int32_t* kept_idx,
                                  int32_t* free_list, int32_t free_capacity,
                                  int32_t* free_count_host, float* dbg_Z, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int rc = check_paged(desc, seq_len_host, budget_host);
  if (rc) return rc;
  if (desc->num_seqs == 0) return RKV_OK;
  if (!K_pages || !V_pages || !page_table || !Q_win || !kept_idx || !free_count_host)
    return fail(RKV_EINVAL, "K_pages, V_pages, page_table, Q_win, kept_idx and free_count_host must be non-NULL");
  if (K_pages == V_pages) return fail(RKV_EINVAL, "K_pages and V_pages must differ");
  PagedPlan P;
  paged_plan(desc, seq_len_host, budget_host, P);
  const int32_t count = *free_count_host;
  if (count < 0 || free_capacity < 0 || count > free_capacity)
    return fail(RKV_EINVAL, "free_count (%d) must lie in [0, free_capacity = %d]", count, free_capacity);
  if ((int64_t)count + P.freed > free_capacity)
    return fail(RKV_EFREELIST, "%d freed pages do not fit: %d of %d entries in use", P.freed, count,
                free_capacity);
  if (P.freed > 0 && free_list == nullptr) return fail(RKV_EINVAL, "free_list is NULL");
  const size_t need = paged_layout(desc, P, nullptr).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(RKV_EWORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(RKV_EWORKSPACE, "workspace must be 256-byte aligned");
  char* base = static_cast<char*>(workspace);
  const PagedLayout L = paged_layout(desc, P, base);
  pack_meta(P, L, base, t_meta_image);
  hipStream_t st = static_cast<hipStream_t>(stream);
  g_error.clear();
  hipError_t e = hipMemcpyAsync(base, t_meta_image.data(), L.meta_bytes, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "metadata upload");
  if (desc->dtype == RKV_BF16)
    rc = paged_run<bf16_bits>(desc, K_pages, V_pages, page_table, Q_win, kept_idx, free_list, count,
                              dbg_Z, P, L, st);
  else
    rc = paged_run<float>(desc, K_pages, V_pages, page_table, Q_win, kept_idx, free_list, count,
                          dbg_Z, P, L, st);
  if (rc == RKV_OK) *free_count_host = count + P.freed;
  return rc;
}

// ---- page accounting for admission ---------------------------------------------
extern "C" int rkv_paged_plan(int32_t num_seqs, const int32_t* seq_len_host,
                              const int32_t* budget_host, int32_t page_size, int32_t divide_length,
                              rkv_page_plan* plan_host, int64_t* totals_host) {
  if (num_seqs < 0) return fail(RKV_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (page_size < 1 || page_size > 4096 || log2_exact(page_size) < 0)
    return fail(RKV_EINVAL, "page_size must be a power of two in [1, 4096] (got %d)", page_size);
  if (divide_length < 0) return fail(RKV_EINVAL, "divide_length must be >= 0 (got %d)", divide_length);
  if (num_seqs > 0 && (!seq_len_host || !budget_host))
    return fail(RKV_EINVAL, "seq_len_host and budget_host must be non-NULL");
  for (int s = 0; s < num_seqs; ++s) {
    const int32_t n = seq_len_host[s], b = budget_host[s];
    if (n < 0) return fail(RKV_EINVAL, "seq_len[%d] = %d must be >= 0", s, n);
    if (b < 0 || b % page_size)
      return fail(RKV_EINVAL, "budget[%d] = %d must be 0 or a positive multiple of page_size %d", s,
                  b, page_size);
    if ((int64_t)b + divide_length > INT32_MAX)
      return fail(RKV_EINVAL, "budget[%d] + divide_length overflows", s);
  }
  int64_t tot[4] = {0, 0, 0, 0};
  auto pages = [&](int64_t tokens) { return (int32_t)((tokens + page_size - 1) / page_size); };
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t n = seq_len_host[s], b = budget_host[s];
    rkv_page_plan pl;
    pl.pages_now = pages(n);
    if (b == 0 || divide_length == 0) {   // compression off for this sequence
      pl.pages_peak = -1;
      pl.pages_after = pl.pages_now;
      pl.pages_freed = 0;
      pl.steps_to_event = -1;
    } else {
      const int64_t cap = b + divide_length;   // length at which the append compresses
      pl.pages_peak = pages(std::max(n, cap));
      pl.pages_after = (int32_t)(b / page_size);
      pl.pages_freed = pl.pages_peak - pl.pages_after;
      pl.steps_to_event = n >= cap ? 0 : (int32_t)(cap - n);
      tot[0] += pl.pages_now;
      tot[1] += pl.pages_peak;
      tot[2] += pl.pages_after;
      tot[3] += pl.pages_freed;
    }
    if (plan_host) plan_host[s] = pl;
  }
  if (totals_host)
    for (int i = 0; i < 4; ++i) totals_host[i] = tot[i];
  return RKV_OK;
}

// ---- errors and timing --------------------------------------------------------
extern "C" const char* rkv_last_error(void) { return g_error.c_str(); }

extern "C" int rkv_timing_enable(int enable) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.recs.clear();
  t.pool_used = 0;
  t.on = enable != 0;
  return RKV_OK;
}

extern "C" int rkv_timing_read(const char** names, int32_t* launches, double* total_ms,
                               int32_t max_kernels) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  std::vector<const char*> order;
  std::vector<int32_t> cnt;
  std::vector<double> ms;
  for (const TimingRec& r : t.recs) {
    float el = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&el, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "timing read");
    size_t k = 0;
    while (k < order.size() && std::strcmp(order[k], r.name) != 0) ++k;
    if (k == order.size()) {
      order.push_back(r.name);
      cnt.push_back(0);
      ms.push_back(0.0);
    }
    cnt[k] += 1;
    ms[k] += el;
  }
  for (size_t k = 0; k < order.size() && (int32_t)k < max_kernels; ++k) {
    if (names) names[k] = order[k];
    if (launches) launches[k] = cnt[k];
    if (total_ms) total_ms[k] = ms[k];
  }
  return (int)order.size();
}
