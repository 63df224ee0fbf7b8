// Planning of the block-level pipelined forward (FCP paper Sec. 4.2, "Block-level
// pipelining", Figure 7): a worker's computation is split into block-grained stages;
// while stage s computes, the blocks of stage s+1 are brought in, so communication
// overlaps computation. Here a stage's "pull" is a device copy of KV rows from a source
// buffer into the worker's KV buffer. The caller rotates through `depth` KV regions: the
// copies of stage s wait for stage s-depth's computation, so they may overwrite rows that
// stages up to s-depth read, never rows of stages s-depth+1 .. s-1, which may still run.
#include "fcp_pipeline.h"

#include <algorithm>
#include <cstring>

namespace fcp {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

struct Range {
  int64_t a, b;  // [a, b)
};

// True when some range of `xs` intersects some range of `ys`.
bool intersects(std::vector<Range> xs, std::vector<Range> ys) {
  auto by_start = [](const Range& l, const Range& r) { return l.a < r.a; };
  std::sort(xs.begin(), xs.end(), by_start);
  std::sort(ys.begin(), ys.end(), by_start);
  size_t i = 0, j = 0;
  while (i < xs.size() && j < ys.size()) {
    if (xs[i].a < ys[j].b && ys[j].a < xs[i].b) return true;
    if (xs[i].b <= ys[j].b) ++i;
    else ++j;
  }
  return false;
}

}  // namespace

int make_pipeline_plan(const fcp_dims_t* dims, const fcp_stage_t* stages, int32_t n_stages,
                       const fcp_copy_t* copies, const fcp_pair_t* pairs, int32_t depth,
                       int64_t src_rows, PipelinePlan* P, std::string* err) {
  if (!dims) return fail(err, FCP_ERR_INVALID_ARG, "dims is NULL");
  if (depth < 1) return fail(err, FCP_ERR_INVALID_ARG, "depth must be >= 1");
  if (n_stages < 0) return fail(err, FCP_ERR_INVALID_ARG, "n_stages must be >= 0");
  if (n_stages > 0 && !stages) return fail(err, FCP_ERR_INVALID_ARG, "stages is NULL");
  if (src_rows < 0) return fail(err, FCP_ERR_INVALID_ARG, "src_rows must be >= 0");
  P->first_copy.assign(n_stages + 1, 0);
  P->first_pair.assign(n_stages + 1, 0);
  int64_t nc = 0, np = 0;
  for (int32_t s = 0; s < n_stages; ++s) {
    if (stages[s].n_copies < 0 || stages[s].n_pairs < 0)
      return fail(err, FCP_ERR_INVALID_ARG,
                  "stage " + std::to_string(s) + " has a negative count");
    nc += stages[s].n_copies;
    np += stages[s].n_pairs;
    if (nc > INT32_MAX || np > INT32_MAX)
      return fail(err, FCP_ERR_INVALID_ARG, "more than INT32_MAX copies or pairs");
    P->first_copy[s + 1] = (int32_t)nc;
    P->first_pair[s + 1] = (int32_t)np;
  }
  P->n_copies = (int32_t)nc;
  P->n_pairs = (int32_t)np;
  if (nc > 0 && !copies) return fail(err, FCP_ERR_INVALID_ARG, "copies is NULL");
  if (np > 0 && !pairs) return fail(err, FCP_ERR_INVALID_ARG, "pairs is NULL");

  // Whole-table checks: partial rows disjoint (forward) and Q ranges identical or
  // disjoint (merge).
  int st = validate(dims, pairs, P->n_pairs, FCP_OP_FWD, err);
  if (st != FCP_OK) return st;
  st = validate(dims, pairs, P->n_pairs, FCP_OP_MERGE, err);
  if (st != FCP_OK) return st;

  for (int32_t i = 0; i < P->n_copies; ++i) {
    const fcp_copy_t& c = copies[i];
    if (c.n_rows < 1 || c.src_row < 0 || c.dst_row < 0 || c.src_row > src_rows - c.n_rows ||
        c.dst_row > dims->kv_rows - c.n_rows)
      return fail(err, FCP_ERR_INVALID_ARG,
                  "copy " + std::to_string(i) + " {src " + std::to_string(c.src_row) +
                      ", dst " + std::to_string(c.dst_row) + ", rows " +
                      std::to_string(c.n_rows) + "} is empty or out of range");
  }
  // Stage s's copies may run while stages s-depth+1 .. s-1 compute.
  for (int32_t s = 1; s < n_stages; ++s) {
    std::vector<Range> w, r;
    for (int32_t i = P->first_copy[s]; i < P->first_copy[s + 1]; ++i)
      w.push_back({copies[i].dst_row, copies[i].dst_row + copies[i].n_rows});
    if (w.empty()) continue;
    const int32_t s0 = std::max(0, s - depth + 1);
    for (int32_t i = P->first_pair[s0]; i < P->first_pair[s]; ++i)
      r.push_back({pairs[i].kv_start, (int64_t)pairs[i].kv_start + pairs[i].kv_len});
    if (intersects(std::move(w), std::move(r)))
      return fail(err, FCP_ERR_INVALID_ARG,
                  "stage " + std::to_string(s) + " copies into KV rows that the pairs of one of "
                      "the previous depth-1 stages read");
  }

  // One forward plan per stage, then the merge plan, each at an aligned offset.
  P->stage.assign(n_stages, Plan{});
  P->stage_off.assign(n_stages, 0);
  size_t off = 0;
  for (int32_t s = 0; s < n_stages; ++s) {
    const int32_t n = stages[s].n_pairs;
    if (n == 0) continue;
    st = make_plan(dims, pairs + P->first_pair[s], n, FCP_OP_FWD, &P->stage[s], err);
    if (st != FCP_OK) return st;
    P->stage_off[s] = off;
    off = align_up(off + P->stage[s].ws_bytes);
  }
  st = make_plan(dims, pairs, P->n_pairs, FCP_OP_MERGE, &P->merge, err);
  if (st != FCP_OK) return st;
  P->shape = P->merge.shape;
  P->merge_off = off;
  P->ws_bytes = align_up(off + P->merge.ws_bytes);
  const size_t image = P->n_pairs ? P->merge_off + P->merge.blob.size() : 0;
  P->blob.assign(image, 0);
  for (int32_t s = 0; s < n_stages; ++s)
    if (!P->stage[s].blob.empty())
      std::memcpy(P->blob.data() + P->stage_off[s], P->stage[s].blob.data(),
                  P->stage[s].blob.size());
  if (!P->merge.blob.empty())
    std::memcpy(P->blob.data() + P->merge_off, P->merge.blob.data(), P->merge.blob.size());
  if (P->n_pairs == 0) P->ws_bytes = 0;
  return FCP_OK;
}

}  // namespace fcp
