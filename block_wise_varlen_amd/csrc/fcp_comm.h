// Congestion-free communication planner (host only): the block transfers among the
// workers of a context-parallel group, as a bipartite multigraph from send nodes to
// receive nodes, are split into the minimum number of sub-stages in which every worker
// sends at most one block and receives at most one block.
#pragma once

#include <stdint.h>

#include <string>

namespace fcp {

// Edge e moves one block from worker src[e] to worker dst[e]. Writes stage[e] in
// [0, *n_stages) so that every stage is a matching, with *n_stages the maximal degree
// Delta of the graph (the optimum). Returns an FCP status and sets *err on failure.
int comm_plan(int32_t n_workers, int32_t n_edges, const int32_t* src, const int32_t* dst,
              int32_t* stage, int32_t* n_stages, std::string* err);

}  // namespace fcp
