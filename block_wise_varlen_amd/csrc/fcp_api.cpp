// C ABI of the block-level varlen attention library: argument checks, planning, the
// upload of work lists into the caller's workspace, and kernel launches. No call here
// blocks on the stream; no exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <exception>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "fcp.h"
#include "fcp_comm.h"
#include "fcp_kernels.h"
#include "fcp_pipeline.h"
#include "fcp_plan.h"

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_err(hipError_t e, const char* what) {
  return set_err(FCP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Pinned host buffers used to upload work lists. A buffer is reused once the copy that
// last read it has completed (its event has fired). The pool holds at most
// kMaxStaging buffers: when every buffer is too small or still being read, an idle one is
// replaced by a larger one, and when all of them are still being read the call waits
// for the copy issued longest ago (only with more than kMaxStaging uploads in flight).
struct Staging {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t ev = nullptr;
  bool busy = false;      // a thread is between taking the buffer and recording its event
  uint64_t last_use = 0;  // order of the last upload that read it
};
constexpr size_t kMaxStaging = 8;
std::mutex g_pool_mu;
std::vector<std::unique_ptr<Staging>> g_pool;
uint64_t g_uploads = 0;

// Under g_pool_mu: a buffer of at least n bytes whose last copy has completed, making room
// or waiting as described above; null with *err set on a HIP failure.
Staging* take_staging(size_t n, int* err) {
  Staging* idle_small = nullptr;
  Staging* oldest = nullptr;
  for (auto& b : g_pool) {
    if (b->busy) continue;
    const bool idle = hipEventQuery(b->ev) == hipSuccess;
    if (idle && b->bytes >= n) return b.get();
    if (idle && (!idle_small || b->bytes < idle_small->bytes)) idle_small = b.get();
    if (!oldest || b->last_use < oldest->last_use) oldest = b.get();
  }
  Staging* st = nullptr;
  if (g_pool.size() < kMaxStaging) {
    g_pool.push_back(std::make_unique<Staging>());
    st = g_pool.back().get();
    hipError_t e = hipEventCreateWithFlags(&st->ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      g_pool.pop_back();
      *err = hip_err(e, "hipEventCreate(staging)");
      return nullptr;
    }
  } else {
    st = idle_small ? idle_small : oldest;
    if (!st) {
      *err = set_err(FCP_ERR_INTERNAL, "every staging buffer is in use by another thread");
      return nullptr;
    }
    hipError_t e = hipEventSynchronize(st->ev);
    if (e != hipSuccess) {
      *err = hip_err(e, "staging event");
      return nullptr;
    }
    if (st->bytes >= n) return st;
    e = hipHostFree(st->ptr);
    st->ptr = nullptr;
    st->bytes = 0;
    if (e != hipSuccess) {
      *err = hip_err(e, "hipHostFree(staging)");
      return nullptr;
    }
  }
  const size_t bytes = n < (1u << 20) ? (1u << 20) : n;
  hipError_t e = hipHostMalloc(&st->ptr, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    st->ptr = nullptr;
    *err = hip_err(e, "hipHostMalloc(staging)");
    return nullptr;
  }
  st->bytes = bytes;
  return st;
}

int upload(const std::vector<uint8_t>& blob, void* ws, hipStream_t stream) {
  const size_t n = blob.size();
  if (n == 0) return FCP_OK;
  Staging* st = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    int err = FCP_OK;
    st = take_staging(n, &err);
    if (!st) return err;
    st->busy = true;
    st->last_use = ++g_uploads;
  }
  std::memcpy(st->ptr, blob.data(), n);
  hipError_t e = hipMemcpyAsync(ws, st->ptr, n, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipEventRecord(st->ev, stream);
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    st->busy = false;
  }
  if (e != hipSuccess) return hip_err(e, "work-list upload");
  return FCP_OK;
}

// Events that order the pipeline's two streams. An event goes back to the pool once the
// work it marks has completed, so a later call never re-records one that a pending wait
// may still refer to.
std::mutex g_ev_mu;
std::vector<hipEvent_t> g_ev_pool;

int take_sync_events(size_t n, std::vector<hipEvent_t>* out) {
  std::lock_guard<std::mutex> lk(g_ev_mu);
  for (size_t i = 0; i < g_ev_pool.size() && out->size() < n;) {
    if (hipEventQuery(g_ev_pool[i]) == hipSuccess) {
      out->push_back(g_ev_pool[i]);
      g_ev_pool[i] = g_ev_pool.back();
      g_ev_pool.pop_back();
    } else {
      ++i;
    }
  }
  while (out->size() < n) {
    hipEvent_t e = nullptr;
    const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) {
      g_ev_pool.insert(g_ev_pool.end(), out->begin(), out->end());
      out->clear();
      return hip_err(r, "hipEventCreate(pipeline)");
    }
    out->push_back(e);
  }
  return FCP_OK;
}

void give_back_events(const std::vector<hipEvent_t>& evs) {
  std::lock_guard<std::mutex> lk(g_ev_mu);
  g_ev_pool.insert(g_ev_pool.end(), evs.begin(), evs.end());
}

// The kernels are written for gfx950 only.
int check_device() {
  static std::mutex mu;
  static std::vector<int> ok;  // per device: 0 unknown, 1 yes, 2 no
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_err(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(mu);
  if ((int)ok.size() <= dev) ok.resize(dev + 1, 0);
  if (ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_err(e, "hipGetDeviceProperties");
    ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  if (ok[dev] != 1) return set_err(FCP_ERR_UNSUPPORTED, "device is not gfx950");
  return FCP_OK;
}

// Optional per-kernel timing: event pairs recorded around launches while enabled.
struct TimedLaunch {
  int id;
  hipEvent_t begin, end;
};
std::mutex g_time_mu;
bool g_time_on = false;
std::vector<TimedLaunch> g_time_pending;
std::vector<hipEvent_t> g_time_free;

hipEvent_t take_event() {
  if (!g_time_free.empty()) {
    hipEvent_t e = g_time_free.back();
    g_time_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (which enqueues one kernel on `stream`), bracketed by events if timing
// is on.
template <class F>
hipError_t timed(int id, hipStream_t stream, F&& launch) {
  hipEvent_t b = nullptr, e = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    if (g_time_on) {
      b = take_event();
      e = take_event();
    }
  }
  if (b && e) (void)hipEventRecord(b, stream);
  const hipError_t err = launch();
  if (b && e) {
    (void)hipEventRecord(e, stream);
    std::lock_guard<std::mutex> lk(g_time_mu);
    g_time_pending.push_back(TimedLaunch{id, b, e});
  }
  return err;
}

unsigned long long* clock_base();

// Clock-sample slot of kernel `id` while timing is on (null otherwise).
unsigned long long* clock_slot(int id) {
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    if (!g_time_on) return nullptr;
  }
  unsigned long long* base = clock_base();
  return base ? base + 2 * id : nullptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int need_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    if (!p) return set_err(FCP_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (!aligned16(p)) return set_err(FCP_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  }
  return FCP_OK;
}

// Common front half of every entry point: plan, check workspace and device, upload.
int prepare(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n, int op,
            std::initializer_list<const void*> ptrs, void* ws, size_t ws_bytes,
            hipStream_t stream, fcp::Plan* P) {
  std::string msg;
  int st = fcp::make_plan(dims, pairs, n, op, P, &msg);
  if (st != FCP_OK) return set_err(st, msg);
  if (n == 0) return FCP_OK;
  st = need_ptrs(ptrs);
  if (st != FCP_OK) return st;
  if (!ws || ws_bytes < P->ws_bytes || !aligned16(ws))
    return set_err(FCP_ERR_WORKSPACE, "workspace missing, misaligned or smaller than " +
                                          std::to_string(P->ws_bytes) + " bytes");
  st = check_device();
  if (st != FCP_OK) return st;
  return upload(P->blob, ws, stream);
}

template <class T>
const T* at(void* ws, size_t off) {
  return reinterpret_cast<const T*>(static_cast<char*>(ws) + off);
}

// Work lists of fcp_block_attn_fwd_fused_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends. Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): each device's address of
// its copy is looked up once, with that device current, and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_err(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return set_err(FCP_ERR_UNSUPPORTED, "device id above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_err(e, "hipGetSymbolAddress(scratch)");
    if (!p) return set_err(FCP_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FCP_OK;
}

// Shader-clock samples of timed launches (ClockStamp in the kernels): per kernel id, the
// summed shader-clock and 100 MHz reference ticks of its workgroups, in a file-scope
// device array whose per-device address is looked up like scratch's.
__device__ __align__(256) unsigned long long clock_ticks[FCP_KERNEL_COUNT][2];
void* g_clock_ptr[kMaxDevices] = {};

// Address of this device's clock_ticks (zeroed when first looked up), or null.
unsigned long long* clock_base() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_clock_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(clock_ticks)) != hipSuccess || !p) return nullptr;
    if (hipMemset(p, 0, sizeof(clock_ticks)) != hipSuccess) return nullptr;
    g_clock_ptr[dev] = p;
  }
  return static_cast<unsigned long long*>(g_clock_ptr[dev]);
}

template <class F>
int guarded(F&& f) {
  try {
    g_err.clear();
    return f();
  } catch (const std::exception& e) {
    return set_err(FCP_ERR_INTERNAL, std::string("internal error: ") + e.what());
  } catch (...) {
    return set_err(FCP_ERR_INTERNAL, "internal error");
  }
}

}  // namespace

extern "C" {

int fcp_abi_version(void) { return FCP_ABI_VERSION; }

const char* fcp_status_string(int status) {
  switch (status) {
    case FCP_OK: return "ok";
    case FCP_ERR_INVALID_ARG: return "invalid argument";
    case FCP_ERR_UNSUPPORTED: return "unsupported";
    case FCP_ERR_WORKSPACE: return "workspace too small";
    case FCP_ERR_HIP: return "HIP runtime error";
    case FCP_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* fcp_last_error(void) { return g_err.c_str(); }

int fcp_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_time_mu);
  g_time_on = on != 0;
  return FCP_OK;
}

int fcp_timing_read(double* total_ms, int32_t* launches, int32_t n) {
  return fcp_timing_read_clock(total_ms, launches, nullptr, n);
}

int fcp_timing_read_clock(double* total_ms, int32_t* launches, double* sclk_mhz, int32_t n) {
  return guarded([&] {
    std::vector<TimedLaunch> recs;
    {
      std::lock_guard<std::mutex> lk(g_time_mu);
      recs.swap(g_time_pending);
    }
    for (int32_t i = 0; i < n; ++i) {
      if (total_ms) total_ms[i] = 0.0;
      if (launches) launches[i] = 0;
    }
    int st = FCP_OK;
    for (const TimedLaunch& r : recs) {
      float ms = 0.f;
      hipError_t e = hipEventSynchronize(r.end);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.begin, r.end);
      if (e != hipSuccess) {
        st = hip_err(e, "timing event");
      } else if (r.id < n) {
        if (total_ms) total_ms[r.id] += ms;
        if (launches) launches[r.id] += 1;
      }
    }
    {
      std::lock_guard<std::mutex> lk(g_time_mu);
      for (const TimedLaunch& r : recs) {
        g_time_free.push_back(r.begin);
        g_time_free.push_back(r.end);
      }
    }
    // Clock samples of this device's timed launches, all complete after the event waits.
    for (int32_t i = 0; sclk_mhz && i < n; ++i) sclk_mhz[i] = 0.0;
    int dev = 0;
    void* cb = nullptr;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
      std::lock_guard<std::mutex> lk(g_scratch_mu);
      cb = g_clock_ptr[dev];
    }
    if (cb) {
      unsigned long long ticks[FCP_KERNEL_COUNT][2];
      hipError_t e = hipMemcpy(ticks, cb, sizeof ticks, hipMemcpyDeviceToHost);
      if (e == hipSuccess) e = hipMemset(cb, 0, sizeof ticks);
      if (e != hipSuccess) return hip_err(e, "clock samples");
      for (int32_t i = 0; sclk_mhz && i < n && i < FCP_KERNEL_COUNT; ++i)
        if (ticks[i][1] > 0) sclk_mhz[i] = 100.0 * (double)ticks[i][0] / (double)ticks[i][1];
    }
    return st;
  });
}

const char* fcp_kernel_name(int id) {
  static const char* names[FCP_KERNEL_COUNT] = {"fwd_partial", "fwd_fused", "merge",
                                                "bwd_delta",   "bwd_dq",    "bwd_dkdv",
                                                "bwd_dkdv_reduce", "pipe_copy"};
  return (id >= 0 && id < FCP_KERNEL_COUNT) ? names[id] : "";
}

int fcp_validate(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op) {
  return guarded([&] {
    std::string msg;
    const int st = fcp::validate(dims, pairs, n_pairs, op, &msg);
    return st == FCP_OK ? st : set_err(st, msg);
  });
}

int fcp_plan_info(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op,
                  int64_t* out, int32_t n_out) {
  return guarded([&] {
    if (n_out < 0 || (n_out > 0 && !out)) return set_err(FCP_ERR_INVALID_ARG, "bad output array");
    fcp::Plan P;
    std::string msg;
    const int st = fcp::make_plan(dims, pairs, n_pairs, op, &P, &msg);
    if (st != FCP_OK) return set_err(st, msg);
    int64_t v[FCP_PLAN_INFO_COUNT] = {};
    v[FCP_PLAN_QITEMS] = P.n_qitems;
    v[FCP_PLAN_KVITEMS] = P.n_kvitems;
    v[FCP_PLAN_SPLIT_TILES] = P.n_reduce;
    v[FCP_PLAN_SLOTS] = P.n_slots;
    v[FCP_PLAN_WS_BYTES] = (int64_t)P.ws_bytes;
    // Placement: launched workgroups, empty ones, and the most KV heads any XCD meets.
    auto placement = [&](size_t off, int n, bool q_side, int64_t* most_heads) {
      const fcp::WgMap* m = reinterpret_cast<const fcp::WgMap*>(P.blob.data() + off);
      std::vector<std::vector<int>> heads(fcp::kXcds);
      for (int b = 0; b < n; ++b) {
        if (m[b].item < 0) {
          ++v[FCP_PLAN_EMPTY_WORKGROUPS];
          continue;
        }
        const int kvh = q_side ? m[b].head * P.shape.hpw / P.shape.group : m[b].head;
        heads[b % fcp::kXcds].push_back(kvh);
      }
      for (auto& h : heads) {
        std::sort(h.begin(), h.end());
        *most_heads = std::max<int64_t>(*most_heads, std::unique(h.begin(), h.end()) - h.begin());
      }
    };
    v[FCP_PLAN_Q_WORKGROUPS] = P.n_qwg;
    v[FCP_PLAN_KV_WORKGROUPS] = P.n_kvwg;
    if (P.n_qwg > 0) placement(P.off_qmap, P.n_qwg, true, &v[FCP_PLAN_Q_KVHEADS_PER_XCD]);
    if (P.n_kvwg > 0) placement(P.off_kvmap, P.n_kvwg, false, &v[FCP_PLAN_KV_KVHEADS_PER_XCD]);
    if (P.n_kvitems > 0) {
      const fcp::KvItem* it = reinterpret_cast<const fcp::KvItem*>(P.blob.data() + P.off_kvitems);
      for (int i = 0; i < P.n_kvitems; ++i) {
        if (it[i].slot < 0) continue;
        const int first = it[i].heads & 0xffff, count = it[i].heads >> 16;
        if (count > 1) ++v[FCP_PLAN_MULTIHEAD_PARTS];
        if (count > 1 && first > 0) ++v[FCP_PLAN_MULTIHEAD_OFFSET_PARTS];
      }
    }
    for (int32_t i = 0; i < n_out; ++i) out[i] = i < FCP_PLAN_INFO_COUNT ? v[i] : 0;
    return FCP_OK;
  });
}

size_t fcp_workspace_bytes(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs,
                           int op) {
  size_t out = 0;
  guarded([&] {
    fcp::Plan P;
    std::string msg;
    const int st = fcp::make_plan(dims, pairs, n_pairs, op, &P, &msg);
    if (st != FCP_OK) return set_err(st, msg);
    out = P.ws_bytes;
    return FCP_OK;
  });
  return out;
}

int fcp_block_attn_fwd(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                       const fcp_pair_t* pairs, int32_t n_pairs, float* o_part,
                       float* lse_part, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fcp_block_attn_fwd_ex(dims, q, k, v, pairs, n_pairs, o_part, lse_part, FCP_PART_F32,
                               ws, ws_bytes, stream);
}

int fcp_block_attn_fwd_ex(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                          const fcp_pair_t* pairs, int32_t n_pairs, void* o_part,
                          float* lse_part, int32_t part_format, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  return guarded([&] {
    if (part_format != FCP_PART_F32 && part_format != FCP_PART_BF16)
      return set_err(FCP_ERR_INVALID_ARG, "unknown partial format");
    fcp::Plan P;
    int st = prepare(dims, pairs, n_pairs, FCP_OP_FWD, {q, k, v, o_part, lse_part}, ws,
                     ws_bytes, stream, &P);
    if (st != FCP_OK || n_pairs == 0) return st;
    const fcp::Shape& s = P.shape;
    fcp::FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.items = at<fcp::QItem>(ws, P.off_qitems);
    a.wg = at<fcp::WgMap>(ws, P.off_qmap);
    a.n_wg = P.n_qwg;
    a.segs = at<fcp::KvSeg>(ws, P.off_segs);
    a.seg_out = at<int32_t>(ws, P.off_segout);
    a.n_items = P.n_qitems;
    a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
    a.scale_log2 = s.scale * 1.4426950408889634f;
    if (part_format == FCP_PART_BF16)
      a.o_part16 = static_cast<uint16_t*>(o_part);
    else
      a.o_part = static_cast<float*>(o_part);
    a.lse_part = lse_part;
    a.clk = clock_slot(FCP_KERNEL_FWD);
    const hipError_t e =
        timed(FCP_KERNEL_FWD, stream, [&] { return fcp::launch_fwd(a, s.d, false, stream); });
    return e == hipSuccess ? FCP_OK : hip_err(e, "forward launch");
  });
}

int fcp_block_attn_fwd_fused(const fcp_dims_t* dims, const void* q, const void* k,
                             const void* v, const fcp_pair_t* pairs, int32_t n_pairs, void* o,
                             float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return guarded([&] {
    fcp::Plan P;
    int st = prepare(dims, pairs, n_pairs, FCP_OP_FWD_FUSED, {q, k, v, o, lse}, ws, ws_bytes,
                     stream, &P);
    if (st != FCP_OK || n_pairs == 0) return st;
    const fcp::Shape& s = P.shape;
    fcp::FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.items = at<fcp::QItem>(ws, P.off_qitems);
    a.wg = at<fcp::WgMap>(ws, P.off_qmap);
    a.n_wg = P.n_qwg;
    a.segs = at<fcp::KvSeg>(ws, P.off_segs);
    a.n_items = P.n_qitems;
    a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
    a.scale_log2 = s.scale * 1.4426950408889634f;
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.clk = clock_slot(FCP_KERNEL_FWD_FUSED);
    const hipError_t e = timed(FCP_KERNEL_FWD_FUSED, stream,
                                [&] { return fcp::launch_fwd(a, s.d, true, stream); });
    return e == hipSuccess ? FCP_OK : hip_err(e, "fused forward launch");
  });
}

int fcp_block_attn_fwd_fused_noalloc(const fcp_dims_t* dims, const void* q, const void* k,
                                     const void* v, const fcp_pair_t* pairs, int32_t n_pairs,
                                     void* o, float* lse, hipStream_t stream) {
  return guarded([&] {
    fcp::Plan P;
    std::string msg;
    int st = fcp::make_plan(dims, pairs, n_pairs, FCP_OP_FWD_FUSED, &P, &msg);
    if (st != FCP_OK) return set_err(st, msg);
    if (n_pairs == 0) return FCP_OK;
    st = need_ptrs({q, k, v, o, lse});
    if (st != FCP_OK) return st;
    // Checked before any HIP call: an oversized table never reaches the device.
    if (P.ws_bytes > kScratchBytes)
      return set_err(FCP_ERR_WORKSPACE,
                     "work lists need " + std::to_string(P.ws_bytes) +
                         " bytes, above the " + std::to_string(kScratchBytes) +
                         "-byte static scratch of fcp_block_attn_fwd_fused_noalloc; use "
                         "fcp_block_attn_fwd_fused with a workspace");
    st = check_device();
    if (st != FCP_OK) return st;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != FCP_OK) return st;
    // From pageable host memory: the runtime has taken the bytes when the call returns,
    // and the copy is ordered on `stream` after earlier work that reads the array.
    hipError_t e = hipMemcpyAsync(ws, P.blob.data(), P.blob.size(), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_err(e, "work-list upload (static scratch)");
    const fcp::Shape& s = P.shape;
    fcp::FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.items = at<fcp::QItem>(ws, P.off_qitems);
    a.wg = at<fcp::WgMap>(ws, P.off_qmap);
    a.n_wg = P.n_qwg;
    a.segs = at<fcp::KvSeg>(ws, P.off_segs);
    a.n_items = P.n_qitems;
    a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
    a.scale_log2 = s.scale * 1.4426950408889634f;
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    e = fcp::launch_fwd(a, s.d, true, stream);
    return e == hipSuccess ? FCP_OK : hip_err(e, "fused forward launch (static scratch)");
  });
}

int fcp_merge_partials(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs,
                       const float* o_part, const float* lse_part, void* o, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return fcp_merge_partials_ex(dims, pairs, n_pairs, o_part, lse_part, FCP_PART_F32, o, lse, ws,
                               ws_bytes, stream);
}

int fcp_merge_partials_ex(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs,
                          const void* o_part, const float* lse_part, int32_t part_format,
                          void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return guarded([&] {
    if (part_format != FCP_PART_F32 && part_format != FCP_PART_BF16)
      return set_err(FCP_ERR_INVALID_ARG, "unknown partial format");
    fcp::Plan P;
    int st = prepare(dims, pairs, n_pairs, FCP_OP_MERGE, {o_part, lse_part, o, lse}, ws,
                     ws_bytes, stream, &P);
    if (st != FCP_OK || n_pairs == 0) return st;
    fcp::MergeArgs a{};
    if (part_format == FCP_PART_BF16)
      a.o_part16 = static_cast<const uint16_t*>(o_part);
    else
      a.o_part = static_cast<const float*>(o_part);
    a.lse_part = lse_part;
    a.rows = at<fcp::RowItem>(ws, P.off_rows);
    a.parts = at<int32_t>(ws, P.off_parts);
    a.n_rows = P.n_rows;
    a.hq = P.shape.hq;
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    const hipError_t e =
        timed(FCP_KERNEL_MERGE, stream, [&] { return fcp::launch_merge(a, P.shape.d, stream); });
    return e == hipSuccess ? FCP_OK : hip_err(e, "merge launch");
  });
}

int fcp_block_attn_bwd(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout,
                       const fcp_pair_t* pairs, int32_t n_pairs, float* dq, float* dk,
                       float* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fcp_block_attn_bwd_ex(dims, q, k, v, o, lse, dout, pairs, n_pairs, dq, dk, dv, 0, ws,
                               ws_bytes, stream);
}

int fcp_block_attn_bwd_ex(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout,
                          const fcp_pair_t* pairs, int32_t n_pairs, float* dq, float* dk,
                          float* dv, int32_t flags, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  return guarded([&] {
    if (flags & ~FCP_BWD_OVERWRITE) return set_err(FCP_ERR_INVALID_ARG, "unknown flag bits");
    fcp::Plan P;
    int st = prepare(dims, pairs, n_pairs, FCP_OP_BWD, {q, k, v, o, lse, dout, dq, dk, dv}, ws,
                     ws_bytes, stream, &P);
    if (st != FCP_OK || n_pairs == 0) return st;
    const fcp::Shape& s = P.shape;
    fcp::BwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.dout = static_cast<const uint16_t*>(dout);
    a.o = static_cast<const uint16_t*>(o);
    a.lse = lse;
    a.stats = reinterpret_cast<float*>(static_cast<char*>(ws) + P.off_stats);
    a.q_rows = dims->q_rows;
    a.qitems = at<fcp::QItem>(ws, P.off_qitems);
    a.segs = at<fcp::KvSeg>(ws, P.off_segs);
    a.kvitems = at<fcp::KvItem>(ws, P.off_kvitems);
    a.qsegs = at<fcp::QSeg>(ws, P.off_qsegs);
    a.qwg = at<fcp::WgMap>(ws, P.off_qmap);
    a.kvwg = at<fcp::WgMap>(ws, P.off_kvmap);
    a.n_qwg = P.n_qwg;
    a.n_kvwg = P.n_kvwg;
    a.n_qitems = P.n_qitems;
    a.n_kvitems = P.n_kvitems;
    a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
    a.scale = s.scale;
    a.scale_log2 = s.scale * 1.4426950408889634f;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.accumulate = (flags & FCP_BWD_OVERWRITE) ? 0 : 1;
    const size_t part_floats = (size_t)P.n_slots * s.hkv * fcp::kKvTileBwd * s.d;
    a.part_dk = reinterpret_cast<float*>(static_cast<char*>(ws) + P.off_partial);
    a.part_dv = a.part_dk + part_floats;
    a.reduce = at<fcp::ReduceItem>(ws, P.off_reduce);
    a.n_reduce = P.n_reduce;
    a.clk = clock_slot(FCP_KERNEL_DQ);
    hipError_t e =
        timed(FCP_KERNEL_DQ, stream, [&] { return fcp::launch_bwd_dq(a, s.d, stream); });
    if (e != hipSuccess) return hip_err(e, "dQ launch");
    a.clk = clock_slot(FCP_KERNEL_DKDV);
    e = timed(FCP_KERNEL_DKDV, stream, [&] { return fcp::launch_bwd_dkdv(a, s.d, stream); });
    if (e != hipSuccess) return hip_err(e, "dK/dV launch");
    if (P.n_reduce > 0) {
      e = timed(FCP_KERNEL_DKDV_REDUCE, stream,
                [&] { return fcp::launch_bwd_reduce(a, s.d, stream); });
      if (e != hipSuccess) return hip_err(e, "dK/dV reduce launch");
    }
    return FCP_OK;
  });
}

size_t fcp_pipeline_workspace_bytes(const fcp_dims_t* dims, const fcp_stage_t* stages,
                                    int32_t n_stages, const fcp_copy_t* copies,
                                    const fcp_pair_t* pairs, int32_t depth, int64_t src_rows) {
  size_t out = 0;
  guarded([&] {
    fcp::PipelinePlan P;
    std::string msg;
    const int st = fcp::make_pipeline_plan(dims, stages, n_stages, copies, pairs, depth,
                                           src_rows, &P, &msg);
    if (st != FCP_OK) return set_err(st, msg);
    out = P.ws_bytes;
    return FCP_OK;
  });
  return out;
}

int fcp_pipeline_fwd(const fcp_dims_t* dims, const void* q, void* k, void* v,
                     const void* k_src, const void* v_src, int64_t src_rows,
                     const fcp_stage_t* stages, int32_t n_stages, const fcp_copy_t* copies,
                     const fcp_pair_t* pairs, int32_t depth, float* o_part, float* lse_part,
                     void* o, float* lse, int32_t flags, void* ws, size_t ws_bytes,
                     hipStream_t stream, hipStream_t copy_stream) {
  return guarded([&] {
    if (flags & ~(FCP_PIPE_COPY_SHADER | FCP_PIPE_PART_BF16))
      return set_err(FCP_ERR_INVALID_ARG, "unknown flag bits");
    const bool part16 = flags & FCP_PIPE_PART_BF16;
    fcp::PipelinePlan P;
    std::string msg;
    int st = fcp::make_pipeline_plan(dims, stages, n_stages, copies, pairs, depth, src_rows,
                                     &P, &msg);
    if (st != FCP_OK) return set_err(st, msg);
    if (P.n_pairs == 0 && P.n_copies == 0) return FCP_OK;
    st = need_ptrs({k, v});
    if (st == FCP_OK && P.n_copies > 0) st = need_ptrs({k_src, v_src});
    if (st == FCP_OK && P.n_pairs > 0) st = need_ptrs({q, o_part, lse_part, o, lse});
    if (st != FCP_OK) return st;
    if (P.n_pairs > 0 && (!ws || ws_bytes < P.ws_bytes || !aligned16(ws)))
      return set_err(FCP_ERR_WORKSPACE, "workspace missing, misaligned or smaller than " +
                                            std::to_string(P.ws_bytes) + " bytes");
    st = check_device();
    if (st != FCP_OK) return st;
    st = upload(P.blob, ws, stream);
    if (st != FCP_OK) return st;

    const fcp::Shape& s = P.shape;
    const size_t row_bytes = (size_t)s.hkv * s.d * sizeof(uint16_t);
    const hipMemcpyKind kind =
        (flags & FCP_PIPE_COPY_SHADER) ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToDeviceNoCU;
    const bool overlap = copy_stream != stream;
    // Events: [0] start on stream, then per stage "copied" (on copy_stream) and
    // "computed" (on stream).
    std::vector<hipEvent_t> ev;
    if (overlap) {
      st = take_sync_events(1 + 2 * (size_t)n_stages, &ev);
      if (st != FCP_OK) return st;
    }
    auto copied = [&](int32_t t) { return ev[1 + 2 * t]; };
    auto computed = [&](int32_t t) { return ev[2 + 2 * t]; };
    hipError_t e = hipSuccess;
    if (overlap) {
      e = hipEventRecord(ev[0], stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(copy_stream, ev[0], 0);
    }
    for (int32_t t = 0; t < n_stages && e == hipSuccess; ++t) {
      const int32_t c0 = P.first_copy[t], c1 = P.first_copy[t + 1];
      if (c1 > c0) {
        hipStream_t cs = overlap ? copy_stream : stream;
        if (overlap && t >= depth) e = hipStreamWaitEvent(cs, computed(t - depth), 0);
        if (e != hipSuccess) break;
        e = timed(FCP_KERNEL_PIPE_COPY, cs, [&] {
          hipError_t r = hipSuccess;
          for (int32_t i = c0; i < c1 && r == hipSuccess; ++i) {
            const fcp_copy_t& c = copies[i];
            const size_t dst = (size_t)c.dst_row * row_bytes, src = (size_t)c.src_row * row_bytes;
            const size_t n = (size_t)c.n_rows * row_bytes;
            r = hipMemcpyAsync(static_cast<char*>(k) + dst,
                               static_cast<const char*>(k_src) + src, n, kind, cs);
            if (r == hipSuccess)
              r = hipMemcpyAsync(static_cast<char*>(v) + dst,
                                 static_cast<const char*>(v_src) + src, n, kind, cs);
          }
          return r;
        });
        if (e != hipSuccess) break;
        if (overlap) {
          e = hipEventRecord(copied(t), cs);
          if (e == hipSuccess) e = hipStreamWaitEvent(stream, copied(t), 0);
          if (e != hipSuccess) break;
        }
      }
      const fcp::Plan& sp = P.stage[t];
      if (sp.n_qitems > 0) {
        void* base = static_cast<char*>(ws) + P.stage_off[t];
        fcp::FwdArgs a{};
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        a.items = at<fcp::QItem>(base, sp.off_qitems);
        a.wg = at<fcp::WgMap>(base, sp.off_qmap);
        a.n_wg = sp.n_qwg;
        a.segs = at<fcp::KvSeg>(base, sp.off_segs);
        a.seg_out = at<int32_t>(base, sp.off_segout);
        a.n_items = sp.n_qitems;
        a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
        a.scale_log2 = s.scale * 1.4426950408889634f;
        if (part16)
          a.o_part16 = reinterpret_cast<uint16_t*>(o_part);
        else
          a.o_part = o_part;
        a.lse_part = lse_part;
        a.clk = clock_slot(FCP_KERNEL_FWD);
        e = timed(FCP_KERNEL_FWD, stream, [&] { return fcp::launch_fwd(a, s.d, false, stream); });
        if (e != hipSuccess) break;
      }
      if (overlap) e = hipEventRecord(computed(t), stream);
    }
    if (e == hipSuccess && P.n_pairs > 0) {
      void* base = static_cast<char*>(ws) + P.merge_off;
      fcp::MergeArgs a{};
      if (part16)
        a.o_part16 = reinterpret_cast<const uint16_t*>(o_part);
      else
        a.o_part = o_part;
      a.lse_part = lse_part;
      a.rows = at<fcp::RowItem>(base, P.merge.off_rows);
      a.parts = at<int32_t>(base, P.merge.off_parts);
      a.n_rows = P.merge.n_rows;
      a.hq = s.hq;
      a.o = static_cast<uint16_t*>(o);
      a.lse = lse;
      e = timed(FCP_KERNEL_MERGE, stream, [&] { return fcp::launch_merge(a, s.d, stream); });
    }
    if (overlap) give_back_events(ev);
    return e == hipSuccess ? FCP_OK : hip_err(e, "pipelined forward");
  });
}

int fcp_comm_plan(int32_t n_workers, int32_t n_edges, const int32_t* src, const int32_t* dst,
                  int32_t* stage, int32_t* n_stages) {
  return guarded([&] {
    std::string msg;
    const int st = fcp::comm_plan(n_workers, n_edges, src, dst, stage, n_stages, &msg);
    return st == FCP_OK ? st : set_err(st, msg);
  });
}

}  // extern "C"
