// Host-side validation and work-list planning for the block-level varlen attention
// library (the varlen tile scheduler). Pure C++: no HIP calls, so it runs and is tested
// without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "fcp.h"
#include "fcp_types.h"

namespace fcp {

// Launch shape derived from fcp_dims_t.
struct Shape {
  int hq = 0, hkv = 0, d = 0;
  int group = 0;      // query heads per KV head
  int hpw = 0;        // query heads per forward / dQ workgroup (one KV head's)
  int n_hgroups = 0;  // hq / hpw: workgroups per forward / dQ item
  int tile_tokens = 0;  // query tokens per forward / dQ item (32 * 8 / hpw)
  float scale = 0.f;  // softmax scale (already resolved from 0)
};

// Byte offsets of the tables inside the caller's workspace.
struct Plan {
  Shape shape;
  std::vector<uint8_t> blob;  // host image of everything uploaded (prefix of ws)
  size_t ws_bytes = 0;        // blob + device-only regions
  size_t off_qitems = 0, off_segs = 0, off_rows = 0, off_parts = 0, off_segout = 0;
  size_t off_kvitems = 0, off_qsegs = 0, off_stats = 0, off_reduce = 0, off_partial = 0;
  size_t off_qmap = 0, off_kvmap = 0;  // launch orders (WgMap) of the Q- and KV-side kernels
  int n_qitems = 0, n_rows = 0, n_kvitems = 0, n_reduce = 0, n_slots = 0;
  int n_qwg = 0, n_kvwg = 0;           // workgroups (grid size) of those launches
};

// Validates dims and pairs for `op`; on failure returns the status and sets *err.
int validate(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op,
             std::string* err);

// Validates, then builds the work lists and workspace layout for `op`.
int make_plan(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op,
              Plan* plan, std::string* err);

}  // namespace fcp
