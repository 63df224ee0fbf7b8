// Walk over the KV tiles a forward / dQ work item visits: its KV segments in order and,
// within each, the KT-key tiles that any of its queries can see (causal ranges stop at
// the diagonal of the item's last query).
#pragma once

#include "fcp_common.h"
#include "fcp_types.h"

namespace fcp {

// Number of KT-key tiles of segment `s` visible to queries [q_off, q_off + rows).
template <int KT>
__device__ __forceinline__ int visible_kv_tiles(const KvSeg& s, int q_off, int rows) {
  int last = s.kv_len - 1;
  if (s.flags & 1) last = min(last, q_off + rows - 1 + s.mask_offset);
  return last < 0 ? 0 : last / KT + 1;
}

// Position (segment s, tile t of nt) in the flattened tile sequence of one work item.
template <int KT>
struct KvTileCursor {
  KvSeg sg;
  int s, t, nt;
  bool valid;
  __device__ static KvTileCursor first(const KvSeg* segs, int s0, int s_end, int q_off,
                                       int rows) {
    KvTileCursor c{};
    c.valid = false;
    for (c.s = s0; c.s < s_end; ++c.s) {
      c.sg = load_uniform(segs, c.s);
      c.nt = visible_kv_tiles<KT>(c.sg, q_off, rows);
      if (c.nt > 0) {
        c.valid = true;
        c.t = 0;
        break;
      }
    }
    return c;
  }
  __device__ KvTileCursor next(const KvSeg* segs, int s_end, int q_off, int rows) const {
    if (!valid) return *this;
    if (t + 1 < nt) {
      KvTileCursor c = *this;
      c.t = t + 1;
      return c;
    }
    return first(segs, s + 1, s_end, q_off, rows);
  }
  // First key of the tile within its KV range, and the keys left from there.
  __device__ int j0() const { return t * KT; }
};

}  // namespace fcp
