// C ABI of the block-level varlen attention library: argument checks, planning, the
// upload of work lists into the caller's workspace, and kernel launches. No call here
// blocks on the stream; no exception crosses the ABI.
#include <hip/hip_runtime.h>

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
// last read it has completed (its event has fired).
struct Staging {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t ev = nullptr;
  bool busy = false;
};
std::mutex g_pool_mu;
std::vector<std::unique_ptr<Staging>> g_pool;

int upload(const fcp::Plan& P, void* ws, hipStream_t stream) {
  const size_t n = P.blob.size();
  if (n == 0) return FCP_OK;
  Staging* st = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    for (auto& b : g_pool) {
      if (b->busy || b->bytes < n) continue;
      if (hipEventQuery(b->ev) != hipSuccess) continue;
      st = b.get();
      break;
    }
    if (!st) {
      auto b = std::make_unique<Staging>();
      b->bytes = n < (1u << 20) ? (1u << 20) : n;
      hipError_t e = hipHostMalloc(&b->ptr, b->bytes, hipHostMallocDefault);
      if (e != hipSuccess) return hip_err(e, "hipHostMalloc(staging)");
      e = hipEventCreateWithFlags(&b->ev, hipEventDisableTiming);
      if (e != hipSuccess) return hip_err(e, "hipEventCreate(staging)");
      st = b.get();
      g_pool.push_back(std::move(b));
    }
    st->busy = true;
  }
  std::memcpy(st->ptr, P.blob.data(), n);
  hipError_t e = hipMemcpyAsync(ws, st->ptr, n, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipEventRecord(st->ev, stream);
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    st->busy = false;
  }
  if (e != hipSuccess) return hip_err(e, "work-list upload");
  return FCP_OK;
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
  return upload(*P, ws, stream);
}

template <class T>
const T* at(void* ws, size_t off) {
  return reinterpret_cast<const T*>(static_cast<char*>(ws) + off);
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
    std::lock_guard<std::mutex> lk(g_time_mu);
    for (const TimedLaunch& r : recs) {
      g_time_free.push_back(r.begin);
      g_time_free.push_back(r.end);
    }
    return st;
  });
}

const char* fcp_kernel_name(int id) {
  static const char* names[FCP_KERNEL_COUNT] = {"fwd_partial", "fwd_fused", "merge",
                                                "bwd_delta",   "bwd_dq",    "bwd_dkdv",
                                                "bwd_dkdv_reduce"};
  return (id >= 0 && id < FCP_KERNEL_COUNT) ? names[id] : "";
}

int fcp_validate(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op) {
  return guarded([&] {
    std::string msg;
    const int st = fcp::validate(dims, pairs, n_pairs, op, &msg);
    return st == FCP_OK ? st : set_err(st, msg);
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
  return guarded([&] {
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
    a.segs = at<fcp::KvSeg>(ws, P.off_segs);
    a.n_items = P.n_qitems;
    a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
    a.scale_log2 = s.scale * 1.4426950408889634f;
    a.o_part = o_part;
    a.lse_part = lse_part;
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
    a.segs = at<fcp::KvSeg>(ws, P.off_segs);
    a.n_items = P.n_qitems;
    a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
    a.scale_log2 = s.scale * 1.4426950408889634f;
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    const hipError_t e = timed(FCP_KERNEL_FWD_FUSED, stream,
                                [&] { return fcp::launch_fwd(a, s.d, true, stream); });
    return e == hipSuccess ? FCP_OK : hip_err(e, "fused forward launch");
  });
}

int fcp_merge_partials(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs,
                       const float* o_part, const float* lse_part, void* o, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return guarded([&] {
    fcp::Plan P;
    int st = prepare(dims, pairs, n_pairs, FCP_OP_MERGE, {o_part, lse_part, o, lse}, ws,
                     ws_bytes, stream, &P);
    if (st != FCP_OK || n_pairs == 0) return st;
    fcp::MergeArgs a{};
    a.o_part = o_part;
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
  return guarded([&] {
    fcp::Plan P;
    int st = prepare(dims, pairs, n_pairs, FCP_OP_BWD, {q, k, v, o, lse, dout, dq, dk, dv}, ws,
                     ws_bytes, stream, &P);
    if (st != FCP_OK || n_pairs == 0) return st;
    const fcp::Shape& s = P.shape;
    float* stats = reinterpret_cast<float*>(static_cast<char*>(ws) + P.off_delta);
    fcp::DeltaArgs da{};
    da.o = static_cast<const uint16_t*>(o);
    da.dout = static_cast<const uint16_t*>(dout);
    da.lse = lse;
    da.rows = at<fcp::RowItem>(ws, P.off_rows);
    da.n_rows = P.n_rows;
    da.hq = s.hq;
    da.stats = stats;
    da.q_rows = dims->q_rows;
    hipError_t e =
        timed(FCP_KERNEL_DELTA, stream, [&] { return fcp::launch_delta(da, s.d, stream); });
    if (e != hipSuccess) return hip_err(e, "delta launch");
    fcp::BwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.dout = static_cast<const uint16_t*>(dout);
    a.stats = stats;
    a.q_rows = dims->q_rows;
    a.qitems = at<fcp::QItem>(ws, P.off_qitems);
    a.segs = at<fcp::KvSeg>(ws, P.off_segs);
    a.kvitems = at<fcp::KvItem>(ws, P.off_kvitems);
    a.qsegs = at<fcp::QSeg>(ws, P.off_qsegs);
    a.n_qitems = P.n_qitems;
    a.n_kvitems = P.n_kvitems;
    a.hq = s.hq, a.hkv = s.hkv, a.group = s.group, a.hpw = s.hpw, a.n_hgroups = s.n_hgroups;
    a.scale = s.scale;
    a.scale_log2 = s.scale * 1.4426950408889634f;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    const size_t part_floats = (size_t)P.n_slots * s.hkv * fcp::kKvTileBwd * s.d;
    a.part_dk = reinterpret_cast<float*>(static_cast<char*>(ws) + P.off_partial);
    a.part_dv = a.part_dk + part_floats;
    a.reduce = at<fcp::ReduceItem>(ws, P.off_reduce);
    a.n_reduce = P.n_reduce;
    e = timed(FCP_KERNEL_DQ, stream, [&] { return fcp::launch_bwd_dq(a, s.d, stream); });
    if (e != hipSuccess) return hip_err(e, "dQ launch");
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

int fcp_comm_plan(int32_t n_workers, int32_t n_edges, const int32_t* src, const int32_t* dst,
                  int32_t* stage, int32_t* n_stages) {
  return guarded([&] {
    std::string msg;
    const int st = fcp::comm_plan(n_workers, n_edges, src, dst, stage, n_stages, &msg);
    return st == FCP_OK ? st : set_err(st, msg);
  });
}

}  // extern "C"
