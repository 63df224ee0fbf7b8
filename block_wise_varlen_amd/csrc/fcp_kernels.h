// Kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fcp_types.h"

namespace fcp {

struct FwdArgs {
  const uint16_t* q;   // bf16 [q_rows, hq, D]
  const uint16_t* k;   // bf16 [kv_rows, hkv, D]
  const uint16_t* v;   // bf16 [kv_rows, hkv, D]
  const QItem* items;  // n_items
  const WgMap* wg;     // launch order: workgroup -> (item, query-head group)
  int n_wg;
  const KvSeg* segs;
  const int32_t* seg_out;  // per-pair mode: partial row of each KvSeg's first query
  int n_items;
  int hq, hkv, group, hpw, n_hgroups;
  float scale_log2;  // softmax scale * log2(e)
  float* o_part;     // fp32 [part_rows, hq, D]   (per-pair mode)
  uint16_t* o_part16;  // bf16 [part_rows, hq, D]  (per-pair mode, bf16 partials; else null)
  float* lse_part;   // fp32 [part_rows, hq]
  uint16_t* o;       // bf16 [q_rows, hq, D]      (final mode)
  float* lse;        // fp32 [q_rows, hq]
  unsigned long long* clk;  // optional clock sampling (ClockStamp), or null
};

struct MergeArgs {
  const float* o_part;      // fp32 partials, or
  const uint16_t* o_part16;  // bf16 partials (non-null selects them)
  const float* lse_part;
  const RowItem* rows;
  const int32_t* parts;  // out_row of each partial, grouped per Q range
  int n_rows;
  int hq;
  uint16_t* o;  // bf16 [q_rows, hq, D]
  float* lse;   // fp32 [q_rows, hq]
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const uint16_t* o;   // bf16 merged output
  const float* lse;    // fp32 [q_rows, hq] merged LSE, natural log
  float* stats;        // fp32 [hq, q_rows, 2]: written by the dQ kernel, read by dK/dV
  int64_t q_rows;
  const QItem* qitems;
  const KvSeg* segs;
  const KvItem* kvitems;
  const QSeg* qsegs;
  const WgMap* qwg;   // dQ launch order: workgroup -> (item, query-head group)
  const WgMap* kvwg;  // dK/dV launch order: workgroup -> (item, KV head)
  int n_qwg, n_kvwg;
  int n_qitems, n_kvitems;
  int hq, hkv, group, hpw, n_hgroups;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  float* dq;         // fp32 [q_rows, hq, D]   (+= when accumulate, else =)
  float* dk;         // fp32 [kv_rows, hkv, D] (+= when accumulate, else =)
  float* dv;         // fp32 [kv_rows, hkv, D] (+= when accumulate, else =)
  int accumulate;    // 1: add into dq / dk / dv; 0: write them (each row has one writer)
  float* part_dk;    // fp32 [slots, hkv, kKvTileBwd, D] partials of split items
  float* part_dv;
  const ReduceItem* reduce;
  int n_reduce;
  unsigned long long* clk;  // optional clock sampling of the launched kernel, or null
};

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool final_out, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_bwd_reduce(const BwdArgs& a, int head_dim, hipStream_t stream);

}  // namespace fcp
