// Congestion-free communication planner (FCP paper Sec. 4.2, "Congestion-free solver"):
// the data flow among N workers is a bipartite multigraph with N send nodes and N
// receive nodes and one edge per block transfer; a sub-stage in which every worker
// sends and receives at most one block is a matching of that graph (Lemma 1), so at
// least Delta sub-stages are needed, Delta the maximal degree (Lemma 2), and Delta
// suffice: the edges split into Delta disjoint matchings. The pages leave the
// construction to an appendix that is not reproduced; the one here is the classic proof
// of that fact for bipartite multigraphs, made efficient:
//  1. pad the graph to a Delta-regular one with dummy edges between send and receive
//     nodes that lack degree (both sides lack N*Delta - |E| in total);
//  2. split recursively: a regular graph of even degree splits into two halves of equal
//     degree by walking closed trails and giving their edges alternately to each half
//     (bipartite closed trails have even length, so every vertex keeps half its edges on
//     each side); one of odd degree first gives up a perfect matching, found with the
//     Hopcroft-Karp algorithm the pages name (a regular bipartite graph always has one);
//  3. a 1-regular graph is a perfect matching: one stage; dummy edges are dropped.
// Cost O(|E| sqrt(N) log Delta) on the padded graph.
#include "fcp_comm.h"

#include <algorithm>
#include <deque>
#include <stdexcept>
#include <vector>

#include "fcp.h"

namespace fcp {
namespace {

struct Graph {
  int n = 0;                 // vertices per side
  std::vector<int32_t> u, v; // edge endpoints: send node u, receive node v
};

// Perfect matching of a regular bipartite multigraph restricted to `edges`
// (Hopcroft-Karp). Returns the matched edge ids (one per send node).
std::vector<int32_t> perfect_matching(const Graph& g, const std::vector<int32_t>& edges) {
  const int n = g.n;
  std::vector<std::vector<int32_t>> adj(n);  // edge ids by send node
  for (int32_t e : edges) adj[g.u[e]].push_back(e);
  std::vector<int32_t> match_l(n, -1), match_r(n, -1);  // edge ids
  std::vector<int32_t> dist(n), it(n);
  const int32_t INF = 1 << 30;
  for (;;) {
    // BFS from the free send nodes over alternating paths.
    std::deque<int32_t> q;
    for (int x = 0; x < n; ++x) {
      dist[x] = match_l[x] < 0 ? 0 : INF;
      if (match_l[x] < 0) q.push_back(x);
    }
    bool found = false;
    while (!q.empty()) {
      const int32_t x = q.front();
      q.pop_front();
      for (int32_t e : adj[x]) {
        const int32_t y = g.v[e];
        const int32_t m = match_r[y];
        if (m < 0) {
          found = true;
        } else {
          const int32_t x2 = g.u[m];
          if (dist[x2] == INF) {
            dist[x2] = dist[x] + 1;
            q.push_back(x2);
          }
        }
      }
    }
    if (!found) break;
    // DFS along the layers (iterative, with per-node edge cursors).
    std::fill(it.begin(), it.end(), 0);
    for (int s = 0; s < n; ++s) {
      if (match_l[s] >= 0) continue;
      std::vector<int32_t> path;  // edges tried, one per layer
      std::vector<int32_t> nodes{s};
      while (!nodes.empty()) {
        const int32_t x = nodes.back();
        bool advanced = false;
        while (it[x] < (int32_t)adj[x].size()) {
          const int32_t e = adj[x][it[x]++];
          const int32_t y = g.v[e];
          const int32_t m = match_r[y];
          if (m < 0) {
            // Augment along nodes/path + e.
            path.push_back(e);
            for (int32_t pe : path) {
              match_l[g.u[pe]] = pe;
              match_r[g.v[pe]] = pe;
            }
            nodes.clear();
            advanced = true;
            break;
          }
          const int32_t x2 = g.u[m];
          if (dist[x2] == dist[x] + 1) {
            path.push_back(e);
            nodes.push_back(x2);
            advanced = true;
            break;
          }
        }
        if (!advanced) {  // dead end: drop x from this phase
          dist[x] = INF;
          nodes.pop_back();
          if (!path.empty()) path.pop_back();
        }
      }
    }
  }
  std::vector<int32_t> out;
  out.reserve(n);
  for (int x = 0; x < n; ++x)
    if (match_l[x] >= 0) out.push_back(match_l[x]);
  return out;
}

// Splits a regular bipartite multigraph of even degree into two halves of equal degree.
void euler_split(const Graph& g, const std::vector<int32_t>& edges, std::vector<int32_t>* a,
                 std::vector<int32_t>* b) {
  const int n = g.n;
  // Vertices 0..n-1 send side, n..2n-1 receive side.
  std::vector<std::vector<int32_t>> adj(2 * n);
  for (int32_t e : edges) {
    adj[g.u[e]].push_back(e);
    adj[n + g.v[e]].push_back(e);
  }
  std::vector<int32_t> cur(2 * n, 0);
  std::vector<char> used(g.u.size(), 0);
  for (int start = 0; start < 2 * n; ++start) {
    for (;;) {
      // Next unused edge at `start`; if none, this vertex is exhausted.
      while (cur[start] < (int32_t)adj[start].size() && used[adj[start][cur[start]]]) ++cur[start];
      if (cur[start] == (int32_t)adj[start].size()) break;
      // Walk a closed trail from `start`, alternating halves.
      int x = start;
      bool half = false;
      for (;;) {
        while (cur[x] < (int32_t)adj[x].size() && used[adj[x][cur[x]]]) ++cur[x];
        if (cur[x] == (int32_t)adj[x].size()) break;  // back at the start, trail closed
        const int32_t e = adj[x][cur[x]++];
        used[e] = 1;
        (half ? b : a)->push_back(e);
        half = !half;
        x = x < n ? n + g.v[e] : g.u[e];
      }
    }
  }
}

void color(const Graph& g, std::vector<int32_t> edges, int deg, int base,
           std::vector<int32_t>* col) {
  while (deg > 0) {
    if (deg == 1) {
      for (int32_t e : edges) (*col)[e] = base;
      return;
    }
    if (deg & 1) {
      const std::vector<int32_t> m = perfect_matching(g, edges);
      if ((int)m.size() != g.n) throw std::runtime_error("no perfect matching in a regular graph");
      std::vector<char> in(g.u.size(), 0);
      for (int32_t e : m) {
        (*col)[e] = base;
        in[e] = 1;
      }
      std::vector<int32_t> rest;
      rest.reserve(edges.size() - m.size());
      for (int32_t e : edges)
        if (!in[e]) rest.push_back(e);
      edges.swap(rest);
      ++base;
      --deg;
      continue;
    }
    std::vector<int32_t> a, b;
    a.reserve(edges.size() / 2);
    b.reserve(edges.size() / 2);
    euler_split(g, edges, &a, &b);
    color(g, std::move(a), deg / 2, base, col);
    edges.swap(b);
    base += deg / 2;
    deg /= 2;
  }
}

}  // namespace

int comm_plan(int32_t n_workers, int32_t n_edges, const int32_t* src, const int32_t* dst,
              int32_t* stage, int32_t* n_stages, std::string* err) {
  if (n_workers <= 0 || n_edges < 0 || n_stages == nullptr ||
      (n_edges > 0 && (src == nullptr || dst == nullptr || stage == nullptr))) {
    *err = "n_workers must be positive, n_edges non-negative, and the arrays non-null";
    return FCP_ERR_INVALID_ARG;
  }
  std::vector<int32_t> ds(n_workers, 0), dr(n_workers, 0);
  for (int32_t e = 0; e < n_edges; ++e) {
    if (src[e] < 0 || src[e] >= n_workers || dst[e] < 0 || dst[e] >= n_workers) {
      *err = "edge " + std::to_string(e) + " names a worker outside [0, n_workers)";
      return FCP_ERR_INVALID_ARG;
    }
    ++ds[src[e]];
    ++dr[dst[e]];
  }
  int32_t delta = 0;
  for (int i = 0; i < n_workers; ++i) delta = std::max({delta, ds[i], dr[i]});
  *n_stages = delta;
  if (n_edges == 0) return FCP_OK;
  Graph g;
  g.n = n_workers;
  g.u.assign(src, src + n_edges);
  g.v.assign(dst, dst + n_edges);
  // Pad to a delta-regular multigraph.
  for (int x = 0, y = 0; x < n_workers; ++x) {
    while (ds[x] < delta) {
      while (dr[y] == delta) ++y;
      const int32_t k = std::min(delta - ds[x], delta - dr[y]);
      for (int32_t t = 0; t < k; ++t) {
        g.u.push_back(x);
        g.v.push_back(y);
      }
      ds[x] += k;
      dr[y] += k;
    }
  }
  std::vector<int32_t> edges(g.u.size());
  for (size_t e = 0; e < edges.size(); ++e) edges[e] = (int32_t)e;
  std::vector<int32_t> col(g.u.size(), -1);
  color(g, std::move(edges), delta, 0, &col);
  for (int32_t e = 0; e < n_edges; ++e) stage[e] = col[e];
  return FCP_OK;
}

}  // namespace fcp
