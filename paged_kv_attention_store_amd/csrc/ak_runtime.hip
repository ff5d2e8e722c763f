// C ABI of libak: argument validation, the plan's device workspace and upload,
// kernel sequencing for ak_run, diagnostics.  Declarations and contracts are
// in include/ak.h.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <sstream>
#include <string>
#include <vector>

#include "ak_launch.h"

namespace ak {

namespace {

thread_local std::string g_err;

ak_status fail(ak_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

ak_status hip_fail(hipError_t e, const char* where) {
  std::ostringstream os;
  os << where << ": " << hipGetErrorString(e);
  g_err = os.str();
  return AK_ERR_HIP;
}

int esize(int dt) {
  switch (dt) {
    case AK_F32: return 4;
    case AK_BF16: return 2;
    case AK_FP8_E4M3: return 1;
    case AK_I32: return 4;
    case AK_I64: return 8;
    default: return 0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- profiling

enum { kKinds = 5 };
struct Profiler {
  std::mutex mu;
  int32_t mask = 0;   // kernel kinds timed (bit k = kind k)
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  int64_t launches[kKinds] = {};
  double ms[kKinds] = {};

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler g_prof;

struct ProfScope {
  int kind;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(int k, hipStream_t st) : kind(k), s(st) {
    if (!(g_prof.mask & (1 << k))) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    a = g_prof.get();
    b = g_prof.get();
    if (a) (void)hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!a || !b) return;
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.pending.push_back({kind, a, b});
  }
};

int g_cus_cached[64] = {};

int device_cus(int dev) {
  if (dev >= 0 && dev < 64 && g_cus_cached[dev] > 0) return g_cus_cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev >= 0 && dev < 64) g_cus_cached[dev] = cus;
  return cus;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

void set_error(const std::string& msg) { g_err = msg; }

}  // namespace ak

using namespace ak;

// ------------------------------------------------------------------- store

extern "C" ak_status ak_store_kv(const ak_tensor* k, const ak_tensor* v,
                                 const ak_tensor* slot_mapping, ak_tensor* k_cache,
                                 ak_tensor* v_cache, void* stream) {
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(AK_ERR_INVALID_ARG, "ak_store_kv: null tensor descriptor");
  if (k->ndim != 3 || v->ndim != 3 || slot_mapping->ndim != 1 || k_cache->ndim != 4 ||
      v_cache->ndim != 4)
    return fail(AK_ERR_INVALID_ARG, "ak_store_kv: expected k/v [N,Hkv,D], slots [N], caches [P,B,Hkv,D]");
  const int64_t N = k->shape[0], Hkv = k->shape[1], D = k->shape[2];
  for (int i = 0; i < 3; ++i)
    if (v->shape[i] != k->shape[i])
      return fail(AK_ERR_SHAPE_MISMATCH, "ak_store_kv: k and v shapes differ");
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i])
      return fail(AK_ERR_SHAPE_MISMATCH, "ak_store_kv: k_cache and v_cache shapes differ");
  if (slot_mapping->shape[0] != N)
    return fail(AK_ERR_SHAPE_MISMATCH, "ak_store_kv: slot_mapping length differs from N");
  if (k_cache->shape[2] != Hkv || k_cache->shape[3] != D)
    return fail(AK_ERR_SHAPE_MISMATCH, "ak_store_kv: cache heads/head_dim differ from k/v");
  if (slot_mapping->dtype != AK_I64)
    return fail(AK_ERR_UNSUPPORTED, "ak_store_kv: slot_mapping must be int64");
  if (k->dtype != v->dtype || k_cache->dtype != v_cache->dtype)
    return fail(AK_ERR_UNSUPPORTED, "ak_store_kv: k/v (or the two caches) differ in dtype");
  const int sd = k->dtype, dd = k_cache->dtype;
  const bool ok_pair = (sd == AK_F32 && (dd == AK_F32 || dd == AK_BF16 || dd == AK_FP8_E4M3)) ||
                       (sd == AK_BF16 && (dd == AK_BF16 || dd == AK_FP8_E4M3));
  if (!ok_pair) return fail(AK_ERR_UNSUPPORTED, "ak_store_kv: unsupported dtype conversion");
  if (N < 0 || Hkv <= 0 || D <= 0 || (D % 8) != 0 || k_cache->shape[1] <= 0)
    return fail(AK_ERR_INVALID_ARG, "ak_store_kv: bad sizes (head_dim must be a multiple of 8)");
  if (N == 0) return AK_OK;
  if (!k->data || !v->data || !slot_mapping->data || !k_cache->data || !v_cache->data)
    return fail(AK_ERR_INVALID_ARG, "ak_store_kv: null data pointer");
  if (k->stride[2] != 1 || v->stride[2] != 1 || k_cache->stride[3] != 1 || v_cache->stride[3] != 1 ||
      slot_mapping->stride[0] != 1)
    return fail(AK_ERR_UNSUPPORTED, "ak_store_kv: head_dim (and slot_mapping) must be contiguous");
  const ak_tensor* src[2] = {k, v};
  const ak_tensor* dst[2] = {k_cache, v_cache};
  for (int i = 0; i < 2; ++i) {
    const int64_t sb = esize(sd), db = esize(dd);
    if (!aligned16(src[i]->data) || !aligned16(dst[i]->data) || (src[i]->stride[0] * sb) % 16 ||
        (src[i]->stride[1] * sb) % 16 || (dst[i]->stride[0] * db) % 8 || (dst[i]->stride[1] * db) % 8 ||
        (dst[i]->stride[2] * db) % 8)
      return fail(AK_ERR_UNSUPPORTED, "ak_store_kv: rows must be 16-byte (source) / 8-byte (cache) aligned");
    if (dd == AK_FP8_E4M3 && !(dst[i]->scale > 0.f && std::isfinite(dst[i]->scale)))
      return fail(AK_ERR_INVALID_ARG, "ak_store_kv: fp8 cache needs a positive finite scale");
  }
  if (Hkv * (D / 8) > INT32_MAX / 2 || N > INT32_MAX / 2)
    return fail(AK_ERR_UNSUPPORTED, "ak_store_kv: too many rows");
  StoreArgs a{};
  for (int i = 0; i < 2; ++i) {
    a.src[i] = src[i]->data;
    a.dst[i] = dst[i]->data;
    a.s_st[i] = src[i]->stride[0];
    a.s_sh[i] = src[i]->stride[1];
    a.d_sp[i] = dst[i]->stride[0];
    a.d_sb[i] = dst[i]->stride[1];
    a.d_sh[i] = dst[i]->stride[2];
    a.scale[i] = dst[i]->scale;
  }
  a.slots = static_cast<const int64_t*>(slot_mapping->data);
  a.num_slots = k_cache->shape[0] * k_cache->shape[1];
  a.N = (int32_t)N;
  a.Hkv = (int32_t)Hkv;
  a.D = (int32_t)D;
  a.B = (int32_t)k_cache->shape[1];
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope ps(0, s);
    e = launch_store_kv(a, sd, dd, s);
  }
  if (e != hipSuccess) return hip_fail(e, "ak_store_kv launch");
  return AK_OK;
}

// -------------------------------------------------------------------- plan

// Plan workspaces (device buffer + pinned host staging for the upload) are
// recycled through a small per-process pool: a plan is built once per step, and
// a fresh hipMalloc / hipFree per step would cost milliseconds and synchronise
// the device.  A workspace returns to the pool with an event recorded after the
// last work that used it (its upload and every ak_run); it is handed out again
// only once that event has completed, so reuse never races in-flight kernels.
namespace ak {
namespace {

struct Workspace {
  void* dev = nullptr;
  size_t dev_bytes = 0;
  void* host = nullptr;     // pinned
  size_t host_bytes = 0;
  hipEvent_t done = nullptr;
  int device = 0;
};

constexpr size_t kPoolMax = 16;
std::mutex g_pool_mu;
std::vector<Workspace> g_pool;   // oldest first

void release_ws(Workspace& w) {
  if (w.dev) (void)hipFree(w.dev);
  if (w.host) (void)hipHostFree(w.host);
  if (w.done) (void)hipEventDestroy(w.done);
  w = Workspace{};
}

// (Re)allocate the buffers of `w` to at least the requested sizes.  `w` must be
// idle (its event completed).
ak_status size_ws(Workspace& w, size_t dev_bytes, size_t host_bytes) {
  if (w.dev_bytes < dev_bytes) {
    if (w.dev) (void)hipFree(w.dev);
    w.dev = nullptr;
    // round up so later, slightly larger batches fit
    w.dev_bytes = std::max<size_t>(align256(dev_bytes + dev_bytes / 4), 1 << 16);
    hipError_t e = hipMalloc(&w.dev, w.dev_bytes);
    if (e != hipSuccess) {
      w.dev_bytes = 0;
      return e == hipErrorOutOfMemory ? fail(AK_ERR_OOM, "ak_plan: device workspace")
                                      : hip_fail(e, "ak_plan: hipMalloc");
    }
  }
  if (w.host_bytes < host_bytes) {
    if (w.host) (void)hipHostFree(w.host);
    w.host = nullptr;
    w.host_bytes = std::max<size_t>(align256(host_bytes + host_bytes / 4), 1 << 16);
    hipError_t e = hipHostMalloc(&w.host, w.host_bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      w.host_bytes = 0;
      return hip_fail(e, "ak_plan: pinned staging");
    }
  }
  if (!w.done) {
    hipError_t e = hipEventCreateWithFlags(&w.done, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "ak_plan: event");
  }
  return AK_OK;
}

// A workspace of at least the requested sizes on `device`.  Idle pooled
// workspaces are preferred; with none idle and the pool full, the oldest one is
// waited for (the host is then more than kPoolMax plans ahead of the device) and
// reused, so steady-state planning allocates nothing.
ak_status acquire_ws(int device, size_t dev_bytes, size_t host_bytes, Workspace* out) {
  Workspace w;
  bool found = false;
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    // the smallest idle workspace that fits (so plans of different sizes keep
    // finding theirs, and no reallocation -- whose hipFree synchronises the
    // device -- is needed in steady state); else the largest idle one, grown
    int idle_fit = -1, idle_any = -1, oldest = -1;
    for (size_t i = 0; i < g_pool.size(); ++i) {
      Workspace& c = g_pool[i];
      if (c.device != device) continue;
      if (oldest < 0) oldest = (int)i;
      if (c.done && hipEventQuery(c.done) != hipSuccess) continue;
      if (c.dev_bytes >= dev_bytes && c.host_bytes >= host_bytes) {
        if (idle_fit < 0 || c.dev_bytes < g_pool[idle_fit].dev_bytes) idle_fit = (int)i;
      } else if (idle_any < 0 || c.dev_bytes > g_pool[idle_any].dev_bytes) {
        idle_any = (int)i;
      }
    }
    int pick = idle_fit >= 0 ? idle_fit : idle_any;
    if (pick < 0 && g_pool.size() >= kPoolMax) pick = oldest;
    if (pick >= 0) {
      w = g_pool[pick];
      g_pool.erase(g_pool.begin() + pick);
      found = true;
    }
  }
  if (found && w.done) (void)hipEventSynchronize(w.done);   // immediate unless host is far ahead
  w.device = device;
  ak_status st = size_ws(w, dev_bytes, host_bytes);
  if (st != AK_OK) {
    release_ws(w);
    return st;
  }
  *out = w;
  return AK_OK;
}

void return_ws(Workspace& w) {
  if (!w.dev && !w.host) return;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  g_pool.push_back(w);
  w = Workspace{};
}

}  // namespace
}  // namespace ak

struct ak_plan_private : ak_plan_t {
  ak::Workspace ws;
  ak_plan_opts fixed_opts{};   // planner options of a fixed plan, reused by every update
};

namespace ak {
namespace {

// Destroyed plan objects are kept (their vectors keep their capacity), so the
// host side of a new plan reuses warm memory instead of faulting in fresh pages.
constexpr size_t kPlanCacheMax = 16;
std::mutex g_plan_mu;
std::vector<ak_plan_private*> g_plan_cache;

ak_plan_private* new_plan() {
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    if (!g_plan_cache.empty()) {
      ak_plan_private* p = g_plan_cache.back();
      g_plan_cache.pop_back();
      return p;
    }
  }
  return new (std::nothrow) ak_plan_private();
}

void recycle_plan(ak_plan_private* p) {
  // reset every field to its default but keep the vectors' storage
  std::vector<int32_t> kv_lens = std::move(p->kv_lens);
  std::vector<Req> reqs = std::move(p->reqs);
  std::vector<Item> small = std::move(p->small_items), large = std::move(p->large_items);
  std::vector<MergeJob> merges = std::move(p->merges);
  kv_lens.clear();
  reqs.clear();
  small.clear();
  large.clear();
  merges.clear();
  *p = ak_plan_private();
  p->kv_lens = std::move(kv_lens);
  p->reqs = std::move(reqs);
  p->small_items = std::move(small);
  p->large_items = std::move(large);
  p->merges = std::move(merges);
  std::lock_guard<std::mutex> lk(g_plan_mu);
  if (g_plan_cache.size() < kPlanCacheMax) {
    g_plan_cache.push_back(p);
    return;
  }
  delete p;
}

}  // namespace
}  // namespace ak

extern "C" ak_status ak_plan(const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* last_page_len,
                             int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t causal, int32_t window,
                             const ak_plan_opts* opts, ak_plan_t** plan) {
  if (!plan) return fail(AK_ERR_INVALID_ARG, "ak_plan: null output pointer");
  *plan = nullptr;
  const bool host_only = opts && (opts->flags & AK_PLAN_HOST_ONLY);
  auto* p = new_plan();
  if (!p) return fail(AK_ERR_OOM, "ak_plan: out of host memory");
  int dev = 0;
  int cus = opts && opts->num_cus > 0 ? opts->num_cus : 0;
  if (!host_only) {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
      recycle_plan(p);
      return hip_fail(e, "ak_plan: hipGetDevice");
    }
    if (cus == 0) cus = device_cus(dev);
  }
  if (cus == 0) cus = 256;
  p->xcds = kXcds;
  ak_status st;
  try {
    st = build_plan_host(qo_indptr, kv_indptr, last_page_len, batch_size, num_qo_heads,
                         num_kv_heads, head_dim, page_size, causal, window, opts, cus, p);
  } catch (const std::bad_alloc&) {
    st = fail(AK_ERR_OOM, "ak_plan: out of host memory");
  }
  if (st != AK_OK) {
    recycle_plan(p);
    return st;
  }
  p->host_only = host_only;
  p->device = dev;
  p->kv_indices = kv_indices;
  if (!host_only && p->num_kv_pages > 0 && !kv_indices) {
    recycle_plan(p);
    return fail(AK_ERR_INVALID_ARG, "ak_plan: null kv_indices with a non-empty page table");
  }
  if (!host_only) {
    const size_t b_req = align256(p->reqs.size() * sizeof(Req));
    const size_t b_small = align256(p->small_items.size() * sizeof(Item));
    const size_t b_large = align256(p->large_items.size() * sizeof(Item));
    const size_t b_merge = align256(p->merges.size() * sizeof(MergeJob));
    // arrival counters of split small units, uploaded as zeros (each run leaves
    // them at zero again)
    const size_t b_cnt = align256((size_t)p->small_merges * sizeof(int32_t));
    const size_t b_wg = align256(p->wg_first.size() * sizeof(int32_t));
    const size_t b_po = align256((size_t)p->partial_rows * p->D * sizeof(float));
    const size_t b_pl = align256((size_t)p->partial_rows * sizeof(float));
    const size_t meta = b_req + b_small + b_large + b_merge + b_cnt + b_wg;
    p->d_bytes = meta + b_po + b_pl;
    if (p->d_bytes > 0) {
      st = acquire_ws(dev, p->d_bytes, meta, &p->ws);
      if (st != AK_OK) {
        recycle_plan(p);
        return st;
      }
      p->d_buf = p->ws.dev;
      unsigned char* base = static_cast<unsigned char*>(p->d_buf);
      p->d_reqs = reinterpret_cast<Req*>(base);
      p->d_small = reinterpret_cast<Item*>(base + b_req);
      p->d_large = reinterpret_cast<Item*>(base + b_req + b_small);
      p->d_merges = reinterpret_cast<MergeJob*>(base + b_req + b_small + b_large);
      p->d_merges_large = p->d_merges + p->small_merges;
      p->d_counters = reinterpret_cast<int32_t*>(base + b_req + b_small + b_large + b_merge);
      p->d_wg_first = b_wg ? reinterpret_cast<int32_t*>(base + b_req + b_small + b_large + b_merge + b_cnt)
                           : nullptr;
      p->d_part_o = reinterpret_cast<float*>(base + meta);
      p->d_part_lse = reinterpret_cast<float*>(base + meta + b_po);
      unsigned char* h = static_cast<unsigned char*>(p->ws.host);
      if (!p->reqs.empty()) std::memcpy(h, p->reqs.data(), p->reqs.size() * sizeof(Req));
      if (!p->small_items.empty())
        std::memcpy(h + b_req, p->small_items.data(), p->small_items.size() * sizeof(Item));
      if (!p->large_items.empty())
        std::memcpy(h + b_req + b_small, p->large_items.data(), p->large_items.size() * sizeof(Item));
      if (!p->merges.empty())
        std::memcpy(h + b_req + b_small + b_large, p->merges.data(),
                    p->merges.size() * sizeof(MergeJob));
      if (b_cnt) std::memset(h + b_req + b_small + b_large + b_merge, 0, b_cnt);
      if (b_wg)
        std::memcpy(h + b_req + b_small + b_large + b_merge + b_cnt, p->wg_first.data(),
                    p->wg_first.size() * sizeof(int32_t));
      hipStream_t s = opts ? static_cast<hipStream_t>(opts->stream) : nullptr;
      hipError_t e = hipSuccess;
      if (meta > 0) e = hipMemcpyAsync(p->d_buf, h, meta, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipEventRecord(p->ws.done, s);
      if (e != hipSuccess) {
        (void)hipStreamSynchronize(s);
        return_ws(p->ws);
        recycle_plan(p);
        return hip_fail(e, "ak_plan: upload");
      }
    }
  }
  *plan = p;
  return AK_OK;
}

extern "C" void ak_plan_destroy(ak_plan_t* plan) {
  if (!plan) return;
  auto* pp = static_cast<ak_plan_private*>(plan);
  if (pp->fixed) {
    // a fixed plan owns its workspace; hipFree waits for work still using it
    if (pp->ws.done) (void)hipEventSynchronize(pp->ws.done);
    release_ws(pp->ws);
  } else {
    return_ws(pp->ws);   // the workspace's event covers its last use
  }
  recycle_plan(pp);
}

// ------------------------------------------------------------- fixed plans

namespace ak {
namespace {

struct FixedLayout {
  size_t req, small, large, merge, merge_large, cnt, meta, po, pl, total;
};

// plan creation and updates synchronise and copy from the host: never inside a
// stream capture
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

FixedLayout fixed_layout(const FixedCaps& c, int D) {
  FixedLayout l{};
  l.req = 0;
  l.small = l.req + align256((size_t)c.batch * sizeof(Req));
  l.large = l.small + align256((size_t)c.small * sizeof(Item));
  l.merge = l.large + align256((size_t)c.large * sizeof(Item));
  // the two merge lists are adjacent (one launch covers both on the fp32 path)
  l.merge_large = l.merge + (size_t)c.merges_small * sizeof(MergeJob);
  l.cnt = l.merge + align256((size_t)(c.merges_small + c.merges_large) * sizeof(MergeJob));
  l.meta = l.cnt + align256((size_t)c.merges_small * sizeof(int32_t));
  l.po = l.meta;
  l.pl = l.po + align256((size_t)c.partial_rows * D * sizeof(float));
  l.total = l.pl + align256((size_t)c.partial_rows * sizeof(float));
  return l;
}

}  // namespace
}  // namespace ak

extern "C" ak_status ak_plan_fixed(int32_t max_batch, int64_t max_tokens, int64_t max_query_len,
                                   int64_t max_pages, const int32_t* kv_indices, int32_t num_qo_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                   int32_t causal, int32_t window, const ak_plan_opts* opts,
                                   ak_plan_t** plan) {
  if (!plan) return fail(AK_ERR_INVALID_ARG, "ak_plan_fixed: null output pointer");
  *plan = nullptr;
  if (max_batch < 0 || max_tokens < 0 || max_pages < 0 || max_query_len < 0)
    return fail(AK_ERR_INVALID_ARG, "ak_plan_fixed: negative capacity");
  if (max_tokens > INT32_MAX / 64 || max_pages > INT32_MAX)
    return fail(AK_ERR_UNSUPPORTED, "ak_plan_fixed: capacity too large");
  const bool host_only = opts && (opts->flags & AK_PLAN_HOST_ONLY);
  if (opts && (opts->flags & AK_PLAN_STREAM_K))
    return fail(AK_ERR_UNSUPPORTED, "ak_plan_fixed: stream-K plans are not fixed-capacity");
  auto* p = new_plan();
  if (!p) return fail(AK_ERR_OOM, "ak_plan_fixed: out of host memory");
  int dev = 0;
  int cus = opts && opts->num_cus > 0 ? opts->num_cus : 0;
  if (!host_only) {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
      recycle_plan(p);
      return hip_fail(e, "ak_plan_fixed: hipGetDevice");
    }
    if (cus == 0) cus = device_cus(dev);
  }
  if (cus == 0) cus = 256;
  // the geometry is validated by planning an empty batch
  ak_status st = build_plan_host(nullptr, nullptr, nullptr, 0, num_qo_heads, num_kv_heads, head_dim,
                                 page_size, causal, window, opts, cus, p);
  if (st != AK_OK) {
    recycle_plan(p);
    return st;
  }
  if (!host_only && max_pages > 0 && !kv_indices) {
    recycle_plan(p);
    return fail(AK_ERR_INVALID_ARG, "ak_plan_fixed: null kv_indices buffer");
  }
  p->fixed = true;
  p->host_only = host_only;
  p->device = dev;
  p->kv_indices = kv_indices;
  if (opts) p->fixed_opts = *opts;
  p->fixed_opts.stream = nullptr;
  p->fixed_opts.num_cus = cus;
  p->caps.batch = max_batch;
  p->caps.tokens = max_tokens;
  p->caps.qlen = max_query_len > 0 ? std::min<int64_t>(max_query_len, max_tokens) : max_tokens;
  p->caps.pages = max_pages;
  fixed_capacities(p->Hkv, p->G, p->B, cus, &p->fixed_opts, &p->caps);
  if (p->caps.partial_rows > INT32_MAX / 2 ||
      p->caps.merges_small + p->caps.merges_large > INT32_MAX / 2) {
    recycle_plan(p);
    return fail(AK_ERR_UNSUPPORTED, "ak_plan_fixed: split workspace too large");
  }
  if (!host_only) {
    const FixedLayout l = fixed_layout(p->caps, p->D);
    hipStream_t s = opts ? static_cast<hipStream_t>(opts->stream) : nullptr;
    if (capturing(s)) {
      recycle_plan(p);
      return fail(AK_ERR_INVALID_ARG, "ak_plan_fixed: the stream is being captured");
    }
    Workspace& w = p->ws;
    w.device = dev;
    hipError_t e = hipSuccess;
    if (l.total > 0) e = hipMalloc(&w.dev, l.total);
    if (e == hipSuccess && l.meta > 0) e = hipHostMalloc(&w.host, l.meta, hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&w.done, hipEventDisableTiming);
    // every item and merge job starts as padding (zero rows, zero parts), every
    // arrival counter at zero
    if (e == hipSuccess && l.meta > 0) e = hipMemsetAsync(w.dev, 0, l.meta, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      release_ws(w);
      recycle_plan(p);
      return e == hipErrorOutOfMemory ? fail(AK_ERR_OOM, "ak_plan_fixed: workspace")
                                      : hip_fail(e, "ak_plan_fixed: workspace");
    }
    w.dev_bytes = l.total;
    w.host_bytes = l.meta;
    unsigned char* base = static_cast<unsigned char*>(w.dev);
    p->d_buf = w.dev;
    p->d_bytes = l.total;
    p->d_reqs = reinterpret_cast<Req*>(base + l.req);
    p->d_small = reinterpret_cast<Item*>(base + l.small);
    p->d_large = reinterpret_cast<Item*>(base + l.large);
    p->d_merges = reinterpret_cast<MergeJob*>(base + l.merge);
    p->d_merges_large = reinterpret_cast<MergeJob*>(base + l.merge_large);
    p->d_counters = reinterpret_cast<int32_t*>(base + l.cnt);
    p->d_part_o = reinterpret_cast<float*>(base + l.po);
    p->d_part_lse = reinterpret_cast<float*>(base + l.pl);
  }
  *plan = p;
  return AK_OK;
}

extern "C" ak_status ak_plan_update(ak_plan_t* plan, const int32_t* qo_indptr,
                                    const int32_t* kv_indptr, const int32_t* last_page_len,
                                    int32_t batch_size, void* stream) {
  if (!plan) return fail(AK_ERR_INVALID_ARG, "ak_plan_update: null plan");
  auto* p = static_cast<ak_plan_private*>(plan);
  if (!p->fixed) return fail(AK_ERR_INVALID_ARG, "ak_plan_update: not a fixed plan");
  if (batch_size > p->caps.batch) {
    std::ostringstream os;
    os << "ak_plan_update: batch_size " << batch_size << " exceeds the plan's " << p->caps.batch;
    return fail(AK_ERR_SHAPE_MISMATCH, os.str());
  }
  ak_plan_private* t = new_plan();
  if (!t) return fail(AK_ERR_OOM, "ak_plan_update: out of host memory");
  ak_status st;
  try {
    st = build_plan_host(qo_indptr, kv_indptr, last_page_len, batch_size, p->Hq, p->Hkv, p->D, p->B,
                         p->causal, p->window, &p->fixed_opts, p->num_cus, t);
  } catch (const std::bad_alloc&) {
    st = fail(AK_ERR_OOM, "ak_plan_update: out of host memory");
  }
  if (st == AK_OK) {
    for (int32_t r = 0; r < t->R; ++r)
      if (t->reqs[r].n > p->caps.qlen) {
        std::ostringstream os;
        os << "ak_plan_update: request " << r << " has " << t->reqs[r].n
           << " query tokens, more than the plan's max_query_len " << p->caps.qlen;
        st = fail(AK_ERR_SHAPE_MISMATCH, os.str());
        break;
      }
  }
  if (st == AK_OK && (t->T > p->caps.tokens || t->num_kv_pages > p->caps.pages)) {
    std::ostringstream os;
    os << "ak_plan_update: " << t->T << " query tokens and " << t->num_kv_pages
       << " pages exceed the plan's " << p->caps.tokens << " and " << p->caps.pages;
    st = fail(AK_ERR_SHAPE_MISMATCH, os.str());
  }
  if (st == AK_OK && ((int64_t)t->small_items.size() > p->caps.small ||
                      (int64_t)t->large_items.size() > p->caps.large ||
                      t->small_merges > p->caps.merges_small ||
                      (int64_t)t->merges.size() - t->small_merges > p->caps.merges_large ||
                      t->partial_rows > p->caps.partial_rows))
    st = fail(AK_ERR_UNSUPPORTED, "ak_plan_update: the batch's work list exceeds the fixed workspace "
                                  "(KV lengths outside the guaranteed range)");
  if (st != AK_OK) {
    recycle_plan(t);
    return st;
  }
  if (!p->host_only && capturing(static_cast<hipStream_t>(stream))) {
    recycle_plan(t);
    return fail(AK_ERR_INVALID_ARG, "ak_plan_update: the stream is being captured");
  }
  if (!p->host_only) {
    const FixedLayout l = fixed_layout(p->caps, p->D);
    Workspace& w = p->ws;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipEventSynchronize(w.done);   // the previous upload has left the staging buffer
    unsigned char* h = static_cast<unsigned char*>(w.host);
    unsigned char* d = static_cast<unsigned char*>(w.dev);
    // live entries, then padding over what the previous update left behind
    auto stage = [&](size_t off, const void* src, int64_t n, int64_t hw, size_t esz) {
      const int64_t m = std::max(n, hw);
      if (e != hipSuccess || m == 0) return;
      if (n > 0) std::memcpy(h + off, src, (size_t)n * esz);
      if (hw > n) std::memset(h + off + (size_t)n * esz, 0, (size_t)(hw - n) * esz);
      e = hipMemcpyAsync(d + off, h + off, (size_t)m * esz, hipMemcpyHostToDevice, s);
    };
    stage(l.req, t->reqs.data(), (int64_t)t->reqs.size(), 0, sizeof(Req));
    stage(l.small, t->small_items.data(), (int64_t)t->small_items.size(), p->hw_small, sizeof(Item));
    stage(l.large, t->large_items.data(), (int64_t)t->large_items.size(), p->hw_large, sizeof(Item));
    const int64_t ms = t->small_merges, ml = (int64_t)t->merges.size() - ms;
    stage(l.merge, t->merges.data(), ms, p->hw_msmall, sizeof(MergeJob));
    stage(l.merge_large, t->merges.data() + ms, ml, p->hw_mlarge, sizeof(MergeJob));
    if (e == hipSuccess) e = hipEventRecord(w.done, s);
    if (e != hipSuccess) {
      recycle_plan(t);
      return hip_fail(e, "ak_plan_update: upload");
    }
    p->hw_small = (int64_t)t->small_items.size();
    p->hw_large = (int64_t)t->large_items.size();
    p->hw_msmall = ms;
    p->hw_mlarge = ml;
  }
  p->R = t->R;
  p->T = t->T;
  p->num_kv_pages = t->num_kv_pages;
  p->partial_rows = t->partial_rows;
  p->split_units = t->split_units;
  p->small_merges = t->small_merges;
  std::swap(p->kv_lens, t->kv_lens);
  std::swap(p->reqs, t->reqs);
  std::swap(p->small_items, t->small_items);
  std::swap(p->large_items, t->large_items);
  std::swap(p->merges, t->merges);
  recycle_plan(t);
  return AK_OK;
}

// --------------------------------------------------------------------- run

extern "C" ak_status ak_run(const ak_plan_t* p, const ak_tensor* q, const ak_tensor* k_cache,
                            const ak_tensor* v_cache, ak_tensor* out, ak_tensor* lse,
                            void* stream) {
  if (!p || !q || !k_cache || !v_cache || !out)
    return fail(AK_ERR_INVALID_ARG, "ak_run: null plan or tensor descriptor");
  if (p->host_only) return fail(AK_ERR_INVALID_ARG, "ak_run: plan was built host-only");
  if (q->ndim != 3 || out->ndim != 3 || k_cache->ndim != 4 || v_cache->ndim != 4 ||
      (lse && lse->ndim != 2))
    return fail(AK_ERR_INVALID_ARG, "ak_run: expected q/out [T,Hq,D], caches [P,B,Hkv,D], lse [T,Hq]");
  // a fixed plan runs on its token capacity (rows past the live ones are untouched)
  const int64_t T_run = p->fixed ? p->caps.tokens : p->T;
  if (q->shape[0] != T_run || q->shape[1] != p->Hq || q->shape[2] != p->D) {
    std::ostringstream os;
    os << "ak_run: q is [" << q->shape[0] << "," << q->shape[1] << "," << q->shape[2]
       << "] but the plan expects [" << T_run << "," << p->Hq << "," << p->D << "]";
    return fail(AK_ERR_SHAPE_MISMATCH, os.str());
  }
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(AK_ERR_SHAPE_MISMATCH, "ak_run: out shape differs from q");
  for (int i = 0; i < 4; ++i)
    if (k_cache->shape[i] != v_cache->shape[i])
      return fail(AK_ERR_SHAPE_MISMATCH, "ak_run: k_cache and v_cache shapes differ");
  if (k_cache->shape[1] != p->B || k_cache->shape[2] != p->Hkv || k_cache->shape[3] != p->D)
    return fail(AK_ERR_SHAPE_MISMATCH, "ak_run: cache page size, KV heads or head_dim differ from the plan");
  if (lse && (lse->shape[0] != T_run || lse->shape[1] != p->Hq))
    return fail(AK_ERR_SHAPE_MISMATCH, "ak_run: lse shape differs from [T, Hq]");
  if (lse && lse->dtype != AK_F32) return fail(AK_ERR_UNSUPPORTED, "ak_run: lse must be float32");
  if (out->dtype != q->dtype) return fail(AK_ERR_UNSUPPORTED, "ak_run: out dtype must equal q dtype");
  if (k_cache->dtype != v_cache->dtype)
    return fail(AK_ERR_UNSUPPORTED, "ak_run: k_cache and v_cache dtypes differ");
  const int qd = q->dtype, kd = k_cache->dtype;
  const bool ok = (qd == AK_F32 && kd == AK_F32) ||
                  (qd == AK_BF16 && (kd == AK_BF16 || kd == AK_FP8_E4M3));
  if (!ok) return fail(AK_ERR_UNSUPPORTED, "ak_run: supported q/cache dtypes are f32/f32, bf16/bf16, bf16/fp8");
  // a fixed plan launches over its whole capacity, whatever the live batch, so
  // that a captured graph stays valid for every later update
  const int ns = p->fixed ? (int)p->caps.small : (int)p->small_items.size();
  const int nl = p->fixed ? (int)p->caps.large : (int)p->large_items.size();
  // the merge kernel finishes split large jobs, and split small units too unless
  // the plan merges those inside the small-tile kernel (bf16 / fp8 q only)
  const int64_t n_ms = p->fixed ? p->caps.merges_small : p->small_merges;
  const int64_t n_ml = p->fixed ? p->caps.merges_large : (int64_t)p->merges.size() - p->small_merges;
  const bool all_merges = qd == AK_F32 || !p->merge_in_kernel;
  const int nm = (int)(all_merges ? n_ms + n_ml : n_ml);
  if (T_run == 0 || (ns == 0 && nl == 0)) return AK_OK;
  if (!q->data || !out->data || !k_cache->data || !v_cache->data)
    return fail(AK_ERR_INVALID_ARG, "ak_run: null data pointer");
  if (q->stride[2] != 1 || out->stride[2] != 1 || k_cache->stride[3] != 1 || v_cache->stride[3] != 1)
    return fail(AK_ERR_UNSUPPORTED, "ak_run: head_dim must be contiguous");
  const int qb = esize(qd), cb = esize(kd);
  if (!aligned16(q->data) || !aligned16(out->data) || !aligned16(k_cache->data) ||
      !aligned16(v_cache->data) || (q->stride[0] * qb) % 16 || (q->stride[1] * qb) % 16 ||
      (out->stride[0] * qb) % 16 || (out->stride[1] * qb) % 16)
    return fail(AK_ERR_UNSUPPORTED, "ak_run: q/out rows must be 16-byte aligned");
  for (const ak_tensor* c : {k_cache, v_cache})
    for (int i = 0; i < 3; ++i) {
      if ((c->stride[i] * cb) % 16) return fail(AK_ERR_UNSUPPORTED, "ak_run: cache rows must be 16-byte aligned");
      // page, slot and head offsets are formed in 32-bit byte units per page
      if (c->stride[i] < 0 || c->stride[i] * cb >= (int64_t(1) << 31) / (i == 1 ? 256 : 1))
        return fail(AK_ERR_UNSUPPORTED, "ak_run: cache strides must be non-negative and below 2 GiB");
    }
  if (kd == AK_FP8_E4M3 && !(k_cache->scale > 0.f && v_cache->scale > 0.f &&
                             std::isfinite(k_cache->scale) && std::isfinite(v_cache->scale)))
    return fail(AK_ERR_INVALID_ARG, "ak_run: fp8 caches need positive finite scales");

  AttnArgs a{};
  a.reqs = p->d_reqs;
  a.kv_indices = p->kv_indices;
  a.q = q->data;
  a.k_cache = k_cache->data;
  a.v_cache = v_cache->data;
  a.out = out->data;
  a.lse = lse ? static_cast<float*>(lse->data) : nullptr;
  a.part_o = p->d_part_o;
  a.merges = p->d_merges;
  a.counters = p->d_counters;
  a.wg_first = p->stream_k ? p->d_wg_first : nullptr;
  a.part_lse = p->d_part_lse;
  a.q_st = q->stride[0];
  a.q_sh = q->stride[1];
  a.o_st = out->stride[0];
  a.o_sh = out->stride[1];
  a.l_st = lse ? lse->stride[0] : 0;
  a.l_sh = lse ? lse->stride[1] : 0;
  a.k_sp = k_cache->stride[0];
  a.k_sb = k_cache->stride[1];
  a.k_sh = k_cache->stride[2];
  a.v_sp = v_cache->stride[0];
  a.v_sb = v_cache->stride[1];
  a.v_sh = v_cache->stride[2];
  a.num_pages = k_cache->shape[0];
  a.G = p->G;
  a.log2B = p->log2B;
  a.causal = p->causal;
  a.window = p->window;
  const float kscale = kd == AK_FP8_E4M3 ? k_cache->scale : 1.f;
  a.score_scale = p->sm_scale * kLog2e * kscale;
  a.v_scale = kd == AK_FP8_E4M3 ? v_cache->scale : 1.f;
  if (a.num_pages <= 0) return fail(AK_ERR_SHAPE_MISMATCH, "ak_run: empty KV pool");

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (qd == AK_F32) {
    a.items = p->d_small;
    {
      ProfScope ps(4, s);
      e = launch_attn_f32(a, ns, p->D, s);
    }
    if (e != hipSuccess) return hip_fail(e, "ak_run: fp32 attention (small items)");
    a.items = p->d_large;
    {
      ProfScope ps(4, s);
      e = launch_attn_f32(a, nl, p->D, s);
    }
    if (e != hipSuccess) return hip_fail(e, "ak_run: fp32 attention (large items)");
  } else {
    if (nl > 0) {
      a.items = p->d_large;
      ProfScope ps(2, s);
      e = launch_attn_large(a, nl, p->D, kd, s);
    }
    if (e != hipSuccess) return hip_fail(e, "ak_run: large-tile attention");
    if (ns > 0) {
      a.items = p->d_small;
      ProfScope ps(1, s);
      e = launch_attn_small(a, ns, p->D, kd, p->shared_pages,
                            p->stream_k ? (int)p->wg_first.size() - 1 : 0, s);
    }
    if (e != hipSuccess) return hip_fail(e, "ak_run: small-tile attention");
  }
  if (nm > 0) {
    MergeArgs m{};
    m.jobs = all_merges ? p->d_merges : p->d_merges_large;
    m.part_o = p->d_part_o;
    m.part_lse = p->d_part_lse;
    m.out = out->data;
    m.lse = a.lse;
    m.o_st = a.o_st;
    m.o_sh = a.o_sh;
    m.l_st = a.l_st;
    m.l_sh = a.l_sh;
    m.n_jobs = nm;
    {
      ProfScope ps(3, s);
      e = launch_merge(m, p->D, qd, s);
    }
    if (e != hipSuccess) return hip_fail(e, "ak_run: merge");
  }
  // the plan's workspace may be recycled only after this run has finished
  const auto* pp = static_cast<const ak_plan_private*>(p);
  if (pp->ws.done && !p->fixed) {
    e = hipEventRecord(pp->ws.done, s);
    if (e != hipSuccess) return hip_fail(e, "ak_run: event record");
  }
  return AK_OK;
}

extern "C" ak_status ak_merge_states(const ak_tensor* o_a, const ak_tensor* lse_a,
                                     const ak_tensor* o_b, const ak_tensor* lse_b, ak_tensor* out,
                                     ak_tensor* lse_out, void* stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !out)
    return fail(AK_ERR_INVALID_ARG, "ak_merge_states: null tensor descriptor");
  for (const ak_tensor* t : {o_a, o_b, static_cast<const ak_tensor*>(out)})
    if (t->ndim != 3) return fail(AK_ERR_INVALID_ARG, "ak_merge_states: states must be [T, H, D]");
  for (const ak_tensor* t : {lse_a, lse_b})
    if (t->ndim != 2) return fail(AK_ERR_INVALID_ARG, "ak_merge_states: lse must be [T, H]");
  if (lse_out && lse_out->ndim != 2) return fail(AK_ERR_INVALID_ARG, "ak_merge_states: lse must be [T, H]");
  const int64_t T = out->shape[0], H = out->shape[1], D = out->shape[2];
  for (const ak_tensor* t : {o_a, o_b})
    if (t->shape[0] != T || t->shape[1] != H || t->shape[2] != D)
      return fail(AK_ERR_SHAPE_MISMATCH, "ak_merge_states: o_a, o_b and out shapes differ");
  for (const ak_tensor* t : {lse_a, lse_b, static_cast<const ak_tensor*>(lse_out)})
    if (t && (t->shape[0] != T || t->shape[1] != H))
      return fail(AK_ERR_SHAPE_MISMATCH, "ak_merge_states: lse shape differs from [T, H]");
  const int32_t dt = out->dtype;
  if ((dt != AK_F32 && dt != AK_BF16) || o_a->dtype != dt || o_b->dtype != dt)
    return fail(AK_ERR_UNSUPPORTED, "ak_merge_states: states must all be F32 or all BF16");
  for (const ak_tensor* t : {lse_a, lse_b, static_cast<const ak_tensor*>(lse_out)})
    if (t && t->dtype != AK_F32) return fail(AK_ERR_UNSUPPORTED, "ak_merge_states: lse must be F32");
  if (D != 64 && D != 128) return fail(AK_ERR_UNSUPPORTED, "ak_merge_states: head_dim must be 64 or 128");
  if (T == 0 || H == 0) return AK_OK;
  if (T > INT32_MAX || H > INT32_MAX) return fail(AK_ERR_UNSUPPORTED, "ak_merge_states: too many rows");
  for (const ak_tensor* t : {o_a, o_b, static_cast<const ak_tensor*>(out), lse_a, lse_b,
                             static_cast<const ak_tensor*>(lse_out)})
    if (t && !t->data) return fail(AK_ERR_INVALID_ARG, "ak_merge_states: null data pointer");
  const int eb = dt == AK_F32 ? 4 : 2;
  for (const ak_tensor* t : {o_a, o_b, static_cast<const ak_tensor*>(out)})
    if (t->stride[2] != 1 || !aligned16(t->data) || (t->stride[0] * eb) % 16 || (t->stride[1] * eb) % 16)
      return fail(AK_ERR_UNSUPPORTED, "ak_merge_states: rows must be contiguous and 16-byte aligned");
  Merge2Args m{};
  m.oa = o_a->data;
  m.ob = o_b->data;
  m.la = static_cast<const float*>(lse_a->data);
  m.lb = static_cast<const float*>(lse_b->data);
  m.out = out->data;
  m.lse = lse_out ? static_cast<float*>(lse_out->data) : nullptr;
  m.a_st = o_a->stride[0];
  m.a_sh = o_a->stride[1];
  m.b_st = o_b->stride[0];
  m.b_sh = o_b->stride[1];
  m.o_st = out->stride[0];
  m.o_sh = out->stride[1];
  m.la_st = lse_a->stride[0];
  m.la_sh = lse_a->stride[1];
  m.lb_st = lse_b->stride[0];
  m.lb_sh = lse_b->stride[1];
  m.l_st = lse_out ? lse_out->stride[0] : 0;
  m.l_sh = lse_out ? lse_out->stride[1] : 0;
  m.T = (int32_t)T;
  m.H = (int32_t)H;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope ps(3, s);
    e = launch_merge2(m, (int)D, dt, s);
  }
  if (e != hipSuccess) return hip_fail(e, "ak_merge_states: launch");
  return AK_OK;
}

// ------------------------------------------------- allocation-free variant

// The device memory behind ak_run_noalloc: one plan's work list, merge list,
// arrival counters and split partials, in a fixed array each device holds for
// the life of the process.  Host code never passes `scratch` itself to a kernel
// or a copy (in host code the name is only a stand-in); it uses the address
// hipGetSymbolAddress returns on each device.
namespace ak {
constexpr size_t kScratchBytes = size_t(64) << 20;
}
static __device__ __align__(256) unsigned char scratch[ak::kScratchBytes];

namespace ak {
namespace {

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on `dev` (the current device), looked up
// once per device.
ak_status scratch_address(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(AK_ERR_UNSUPPORTED, "ak_run_noalloc: device index out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "ak_run_noalloc: hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(AK_ERR_HIP, "ak_run_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return AK_OK;
}

thread_local std::vector<unsigned char> t_staging;   // host copy of the uploaded metadata

}  // namespace
}  // namespace ak

extern "C" ak_status ak_run_noalloc(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                    const int32_t* kv_indices, const int32_t* last_page_len,
                                    int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t page_size, int32_t causal,
                                    int32_t window, const ak_plan_opts* opts, const ak_tensor* q,
                                    const ak_tensor* k_cache, const ak_tensor* v_cache,
                                    ak_tensor* out, ak_tensor* lse, void* stream) {
  if (opts && (opts->flags & AK_PLAN_HOST_ONLY))
    return fail(AK_ERR_INVALID_ARG, "ak_run_noalloc: a host-only plan cannot run");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "ak_run_noalloc: hipGetDevice");
  unsigned char* base = nullptr;
  ak_status st = scratch_address(dev, &base);
  if (st != AK_OK) return st;
  auto* p = new_plan();
  if (!p) return fail(AK_ERR_OOM, "ak_run_noalloc: out of host memory");
  const int cus = opts && opts->num_cus > 0 ? opts->num_cus : device_cus(dev);
  p->xcds = kXcds;
  try {
    st = build_plan_host(qo_indptr, kv_indptr, last_page_len, batch_size, num_qo_heads,
                         num_kv_heads, head_dim, page_size, causal, window, opts, cus, p);
  } catch (const std::bad_alloc&) {
    st = fail(AK_ERR_OOM, "ak_run_noalloc: out of host memory");
  }
  if (st == AK_OK && p->num_kv_pages > 0 && !kv_indices)
    st = fail(AK_ERR_INVALID_ARG, "ak_run_noalloc: null kv_indices with a non-empty page table");
  // the same regions as ak_plan's workspace, laid out from the start of scratch
  const size_t b_req = align256(p->reqs.size() * sizeof(Req));
  const size_t b_small = align256(p->small_items.size() * sizeof(Item));
  const size_t b_large = align256(p->large_items.size() * sizeof(Item));
  const size_t b_merge = align256(p->merges.size() * sizeof(MergeJob));
  const size_t b_cnt = align256((size_t)p->small_merges * sizeof(int32_t));
  const size_t b_wg = align256(p->wg_first.size() * sizeof(int32_t));
  const size_t b_po = align256((size_t)p->partial_rows * p->D * sizeof(float));
  const size_t b_pl = align256((size_t)p->partial_rows * sizeof(float));
  const size_t meta = b_req + b_small + b_large + b_merge + b_cnt + b_wg;
  if (st == AK_OK && meta + b_po + b_pl > kScratchBytes) {
    std::ostringstream os;
    os << "ak_run_noalloc: the batch's work list and split partials need " << meta + b_po + b_pl
       << " bytes, more than the " << kScratchBytes << "-byte scratch array (use ak_plan + ak_run)";
    st = fail(AK_ERR_UNSUPPORTED, os.str());
  }
  if (st != AK_OK) {
    recycle_plan(p);
    return st;
  }
  p->device = dev;
  p->kv_indices = kv_indices;
  p->d_buf = base;
  p->d_bytes = meta + b_po + b_pl;
  p->d_reqs = reinterpret_cast<Req*>(base);
  p->d_small = reinterpret_cast<Item*>(base + b_req);
  p->d_large = reinterpret_cast<Item*>(base + b_req + b_small);
  p->d_merges = reinterpret_cast<MergeJob*>(base + b_req + b_small + b_large);
  p->d_merges_large = p->d_merges + p->small_merges;
  p->d_counters = reinterpret_cast<int32_t*>(base + b_req + b_small + b_large + b_merge);
  p->d_wg_first = b_wg ? reinterpret_cast<int32_t*>(base + b_req + b_small + b_large + b_merge + b_cnt)
                       : nullptr;
  p->d_part_o = reinterpret_cast<float*>(base + meta);
  p->d_part_lse = reinterpret_cast<float*>(base + meta + b_po);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (meta > 0 && p->T > 0) {
    // one copy of the metadata, arrival counters as zeros (whatever the last
    // call on this device left in the array)
    std::vector<unsigned char>& h = t_staging;
    try {
      if (h.size() < meta) h.resize(meta);
    } catch (const std::bad_alloc&) {
      recycle_plan(p);
      return fail(AK_ERR_OOM, "ak_run_noalloc: out of host memory");
    }
    unsigned char* hp = h.data();
    std::memset(hp, 0, meta);
    if (!p->reqs.empty()) std::memcpy(hp, p->reqs.data(), p->reqs.size() * sizeof(Req));
    if (!p->small_items.empty())
      std::memcpy(hp + b_req, p->small_items.data(), p->small_items.size() * sizeof(Item));
    if (!p->large_items.empty())
      std::memcpy(hp + b_req + b_small, p->large_items.data(), p->large_items.size() * sizeof(Item));
    if (!p->merges.empty())
      std::memcpy(hp + b_req + b_small + b_large, p->merges.data(), p->merges.size() * sizeof(MergeJob));
    if (b_wg)
      std::memcpy(hp + b_req + b_small + b_large + b_merge + b_cnt, p->wg_first.data(),
                  p->wg_first.size() * sizeof(int32_t));
    // from pageable memory: the host buffer is free for reuse once the call returns
    e = hipMemcpyAsync(base, hp, meta, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      recycle_plan(p);
      return hip_fail(e, "ak_run_noalloc: metadata upload");
    }
  }
  st = ak_run(p, q, k_cache, v_cache, out, lse, stream);
  recycle_plan(p);
  return st;
}

// ------------------------------------------------------------- diagnostics

extern "C" const char* ak_last_error(void) { return g_err.c_str(); }

extern "C" ak_status ak_plan_info(const ak_plan_t* p, int64_t* info, int32_t n) {
  if (!p || !info || n < 0) return fail(AK_ERR_INVALID_ARG, "ak_plan_info: null argument");
  const int64_t v[13] = {p->R,
                        p->T,
                        (int64_t)(p->small_items.size() + p->large_items.size()),
                        (int64_t)p->small_items.size(),
                        (int64_t)p->large_items.size(),
                        p->split_units,
                        (int64_t)p->merges.size(),
                        p->partial_rows,
                        p->caps.small,
                        p->caps.large,
                        p->caps.merges_small + p->caps.merges_large,
                        p->caps.partial_rows,
                        p->stream_k ? (int64_t)p->wg_first.size() - 1 : 0};
  for (int i = 0; i < n && i < 13; ++i) info[i] = v[i];
  return AK_OK;
}

extern "C" ak_status ak_plan_export(const ak_plan_t* p, int32_t* items, int64_t capacity,
                                    int64_t* count, int32_t* kv_lens) {
  if (!p || !count) return fail(AK_ERR_INVALID_ARG, "ak_plan_export: null argument");
  const int64_t n = (int64_t)(p->small_items.size() + p->large_items.size());
  *count = n;
  if (kv_lens && p->R > 0) std::memcpy(kv_lens, p->kv_lens.data(), p->R * sizeof(int32_t));
  if (n > capacity || (n > 0 && !items))
    return fail(AK_ERR_INVALID_ARG, "ak_plan_export: item buffer too small");
  int32_t* o = items;
  for (const auto* v : {&p->small_items, &p->large_items})
    for (const Item& it : *v) {
      std::memcpy(o, &it, 8 * sizeof(int32_t));   // the eight public fields
      o += 8;
    }
  return AK_OK;
}

extern "C" ak_status ak_plan_workgroups(const ak_plan_t* p, int32_t* wg_first, int64_t capacity,
                                        int64_t* count) {
  if (!p || !count) return fail(AK_ERR_INVALID_ARG, "ak_plan_workgroups: null argument");
  const int64_t n = (int64_t)p->wg_first.size();
  *count = n;
  if (n > capacity || (n > 0 && !wg_first))
    return fail(AK_ERR_INVALID_ARG, "ak_plan_workgroups: buffer too small");
  if (n > 0) std::memcpy(wg_first, p->wg_first.data(), (size_t)n * sizeof(int32_t));
  return AK_OK;
}

extern "C" ak_status ak_gather_slots(const ak_plan_t* p, int32_t addressing, int64_t* slots,
                                     void* stream) {
  if (!p || !slots) return fail(AK_ERR_INVALID_ARG, "ak_gather_slots: null argument");
  if (addressing < 0 || addressing > 2)
    return fail(AK_ERR_INVALID_ARG,
                "ak_gather_slots: addressing must be 0 (decode), 1 (prefill) or 2 (prefill, 32-bit)");
  if (p->host_only) return fail(AK_ERR_INVALID_ARG, "ak_gather_slots: plan was built host-only");
  if (p->R == 0) return AK_OK;
  std::vector<int64_t> off(p->R, 0);
  int64_t acc = 0;
  for (int r = 0; r < p->R; ++r) {
    off[r] = acc;
    acc += p->kv_lens[r];
  }
  if (acc == 0) return AK_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t* d_off = nullptr;
  hipError_t e = hipMalloc(&d_off, off.size() * sizeof(int64_t));
  if (e != hipSuccess) return hip_fail(e, "ak_gather_slots: hipMalloc");
  e = hipMemcpyAsync(d_off, off.data(), off.size() * sizeof(int64_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = launch_gather_slots(p->d_reqs, d_off, p->kv_indices, p->R, p->log2B,
                            addressing == 2 ? (int64_t(1) << 24) : INT32_MAX, addressing, slots, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(d_off);
  if (e != hipSuccess) return hip_fail(e, "ak_gather_slots");
  return AK_OK;
}

extern "C" ak_status ak_csr_from_block_table(const int32_t* block_table, int64_t max_blocks,
                                             const int32_t* seq_lens, int32_t batch_size,
                                             int32_t page_size, int32_t block_ratio, int32_t* kv_indptr,
                                             int32_t* kv_indices, int64_t capacity,
                                             int32_t* last_page_len, void* stream) {
  if (batch_size < 0 || page_size < 1 || max_blocks < 0 || capacity < 0 || block_ratio < 1)
    return fail(AK_ERR_INVALID_ARG,
                "ak_csr_from_block_table: negative size, page_size < 1 or block_ratio < 1");
  if ((int64_t)page_size * block_ratio > (1 << 20) || max_blocks * block_ratio > INT32_MAX)
    return fail(AK_ERR_UNSUPPORTED, "ak_csr_from_block_table: block too large");
  if (!kv_indptr || (batch_size > 0 && (!block_table || !seq_lens || !last_page_len)) ||
      (capacity > 0 && !kv_indices))
    return fail(AK_ERR_INVALID_ARG, "ak_csr_from_block_table: null pointer");
  hipError_t e = launch_csr_from_block_table(block_table, max_blocks, seq_lens, batch_size, page_size,
                                             block_ratio, kv_indptr, kv_indices, capacity, last_page_len,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ak_csr_from_block_table");
  return AK_OK;
}

extern "C" ak_status ak_slot_mapping(const int32_t* block_table, int64_t max_pages,
                                     const int32_t* qo_indptr, const int32_t* seq_lens,
                                     int32_t batch_size, int32_t page_size, int64_t* slot_mapping,
                                     int64_t num_tokens, void* stream) {
  if (batch_size < 0 || page_size < 1 || max_pages < 0 || num_tokens < 0)
    return fail(AK_ERR_INVALID_ARG, "ak_slot_mapping: negative size or page_size < 1");
  if (num_tokens == 0) return AK_OK;
  if (!qo_indptr || !slot_mapping || (batch_size > 0 && (!block_table || !seq_lens)))
    return fail(AK_ERR_INVALID_ARG, "ak_slot_mapping: null pointer");
  hipError_t e = launch_slot_mapping(block_table, max_pages, qo_indptr, seq_lens, batch_size,
                                     page_size, slot_mapping, num_tokens,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ak_slot_mapping");
  return AK_OK;
}

extern "C" ak_status ak_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, void* stream) {
  if (n < 0 || (n % 8) != 0) return fail(AK_ERR_INVALID_ARG, "ak_fp8_to_bf16: n must be a multiple of 8");
  if (n == 0) return AK_OK;
  if (!codes || !out || ((uintptr_t)codes & 7u) || ((uintptr_t)out & 15u))
    return fail(AK_ERR_INVALID_ARG, "ak_fp8_to_bf16: null or misaligned pointer");
  hipError_t e = launch_fp8_to_bf16(codes, out, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ak_fp8_to_bf16");
  return AK_OK;
}

extern "C" ak_status ak_profile_enable(int32_t kinds) {
  if (kinds < 0) return fail(AK_ERR_INVALID_ARG, "ak_profile_enable: negative kind mask");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.mask = kinds;
  return AK_OK;
}

extern "C" ak_status ak_profile_read(int64_t* launches, double* total_ms, int32_t n) {
  std::vector<Profiler::Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    recs.swap(g_prof.pending);
  }
  for (auto& r : recs) {
    float ms = 0.f;
    (void)hipEventSynchronize(r.b);
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      g_prof.launches[r.kind] += 1;
      g_prof.ms[r.kind] += ms;
    }
  }
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (auto& r : recs) {
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  for (int i = 0; i < n && i < kKinds; ++i) {
    if (launches) launches[i] = g_prof.launches[i];
    if (total_ms) total_ms[i] = g_prof.ms[i];
  }
  for (int i = 0; i < kKinds; ++i) {
    g_prof.launches[i] = 0;
    g_prof.ms[i] = 0.0;
  }
  return AK_OK;
}

extern "C" const char* ak_version(void) { return "ak 0.1 (gfx950)"; }
