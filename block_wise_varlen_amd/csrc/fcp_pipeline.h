// Host-side validation and planning of a block-level pipelined forward: stages that each
// bring KV blocks into the local KV buffer and compute the block pairs that read them.
// Pure C++: no HIP calls, so it runs and is tested without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "fcp.h"
#include "fcp_plan.h"

namespace fcp {

struct PipelinePlan {
  Shape shape;
  std::vector<Plan> stage;        // forward plan per stage (n_qitems == 0: no pairs)
  std::vector<size_t> stage_off;  // byte offset of each stage's tables in the workspace
  std::vector<int32_t> first_copy, first_pair;  // prefix sums over the stage table
  Plan merge;                     // merge of every pair's partial
  size_t merge_off = 0;
  std::vector<uint8_t> blob;      // upload image: every plan's tables at its offset
  size_t ws_bytes = 0;
  int32_t n_copies = 0, n_pairs = 0;
};

// Validates the stage table, the copies and the pairs; builds one forward plan per stage
// and the merge plan, laid out back to back in one workspace.
int make_pipeline_plan(const fcp_dims_t* dims, const fcp_stage_t* stages, int32_t n_stages,
                       const fcp_copy_t* copies, const fcp_pair_t* pairs, int32_t depth,
                       int64_t src_rows, PipelinePlan* plan, std::string* err);

}  // namespace fcp
