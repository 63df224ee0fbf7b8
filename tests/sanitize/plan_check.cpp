// Host-side driver for a sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer,
// g++ on the CPU) of the library's pure C++ planners: the varlen tile scheduler
// (validate / make_plan), the congestion-free communication planner (comm_plan) and the
// pipeline stage planner (make_pipeline_plan). It feeds them randomized tables -- valid
// and invalid, with extreme offsets -- and checks what every accepted plan promises:
// tables inside the workspace, per-op item counts, and that every stage of a
// communication plan is a matching with exactly max-degree stages.
//
// Usage: plan_check <seed> <cases>     (exit status 0 when every check passed)
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "fcp.h"
#include "fcp_comm.h"
#include "fcp_pipeline.h"
#include "fcp_plan.h"

namespace {

int g_fail = 0;
int g_accepted[6] = {};  // accepted plans per op + 1 (op -1 .. 4)
int g_comm_ok = 0, g_pipe_ok = 0;

void check(bool ok, const char* what, long long a = 0, long long b = 0) {
  if (!ok) {
    std::fprintf(stderr, "check failed: %s (%lld, %lld)\n", what, a, b);
    ++g_fail;
  }
}

struct Rng {
  std::mt19937_64 g;
  explicit Rng(uint64_t s) : g(s) {}
  int64_t in(int64_t lo, int64_t hi) {  // inclusive
    return std::uniform_int_distribution<int64_t>(lo, hi)(g);
  }
  bool p(double x) { return std::uniform_real_distribution<double>(0, 1)(g) < x; }
};

fcp_dims_t random_dims(Rng& r) {
  static const int hkv_opts[] = {1, 2, 4, 8};
  static const int g_opts[] = {1, 2, 4, 8, 16, 3};
  fcp_dims_t d{};
  d.num_kv_heads = hkv_opts[r.in(0, 3)];
  d.num_q_heads = d.num_kv_heads * g_opts[r.in(0, r.p(0.9) ? 4 : 5)];
  d.head_dim = r.p(0.95) ? (r.p(0.5) ? 64 : 128) : 96;
  d.softmax_scale = r.p(0.8) ? 0.f : (r.p(0.9) ? 0.125f : -1.f);
  d.q_rows = r.in(1, 5000);
  d.kv_rows = r.in(1, 5000);
  d.part_rows = r.in(0, 20000);
  return d;
}

std::vector<fcp_pair_t> random_pairs(Rng& r, const fcp_dims_t& d, int n) {
  std::vector<fcp_pair_t> v;
  int64_t out = 0;
  for (int i = 0; i < n; ++i) {
    fcp_pair_t p{};
    p.seq_id = (int32_t)r.in(0, 5);
    const bool wild = r.p(0.03);  // may fall outside the row extents
    p.q_len = (int32_t)r.in(r.p(0.02) ? -3 : 1, std::min<int64_t>(700, d.q_rows));
    p.q_start = (int32_t)r.in(r.p(0.02) ? -5 : 0,
                              std::max<int64_t>(0, (wild ? d.q_rows : d.q_rows - p.q_len)));
    p.kv_len = (int32_t)r.in(r.p(0.02) ? 0 : 1, std::min<int64_t>(900, d.kv_rows));
    p.kv_start = (int32_t)r.in(0, std::max<int64_t>(0, (wild ? d.kv_rows : d.kv_rows - p.kv_len)));
    const int kind = (int)r.in(0, 9);
    p.mask_offset = kind == 0 ? INT32_MIN : kind == 1 ? INT32_MAX
                                          : (int32_t)r.in(-2000, 2000);
    p.out_row = (int32_t)out;
    out += p.q_len > 0 ? p.q_len : 1;
    if (r.p(0.03)) p.out_row = (int32_t)r.in(0, 3000);  // may overlap
    if (!wild && r.p(0.7) && !v.empty()) {  // share the Q range of an earlier pair
      const fcp_pair_t& o = v[r.in(0, (int64_t)v.size() - 1)];
      p.q_start = o.q_start;
      p.q_len = o.q_len;
    }
    p.flags = r.p(0.98) ? (int32_t)r.in(0, 1) : 2;
    v.push_back(p);
  }
  return v;
}

void check_plan(const fcp::Plan& P, int op, int n_pairs) {
  const size_t blob = P.blob.size();
  check(blob <= P.ws_bytes, "blob inside workspace", (long long)blob, (long long)P.ws_bytes);
  auto inside = [&](size_t off, size_t n, size_t rec) {
    check(n == 0 || off + n * rec <= blob, "table inside blob", (long long)off,
          (long long)(n * rec));
  };
  if (op == FCP_OP_FWD || op == FCP_OP_FWD_FUSED) {
    inside(P.off_qitems, P.n_qitems, sizeof(fcp::QItem));
    check(n_pairs == 0 || P.n_qitems > 0, "forward has items");
  }
  // launch maps: every (item, head) exactly once, empty workgroups only as padding
  auto check_map = [&](size_t off, int n_wg, int n_items, int n_heads) {
    inside(off, n_wg, sizeof(fcp::WgMap));
    if (n_wg == 0 || off + (size_t)n_wg * sizeof(fcp::WgMap) > blob) return;
    const fcp::WgMap* m = reinterpret_cast<const fcp::WgMap*>(P.blob.data() + off);
    std::vector<int> seen((size_t)n_items * n_heads, 0);
    for (int b = 0; b < n_wg; ++b) {
      if (m[b].item < 0) continue;
      const bool ok = m[b].item < n_items && m[b].head >= 0 && m[b].head < n_heads;
      check(ok, "map entry in range", m[b].item, m[b].head);
      if (ok) ++seen[(size_t)m[b].item * n_heads + m[b].head];
    }
    for (size_t u = 0; u < seen.size(); ++u) check(seen[u] == 1, "unit launched once", (long long)u, seen[u]);
    check(m[n_wg - 1].item >= 0, "no trailing empty workgroup");
  };
  if (op == FCP_OP_FWD || op == FCP_OP_FWD_FUSED || op == FCP_OP_BWD)
    check_map(P.off_qmap, P.n_qwg, P.n_qitems, P.shape.n_hgroups);
  if (op == FCP_OP_BWD) check_map(P.off_kvmap, P.n_kvwg, P.n_kvitems, P.shape.hkv);
  if (op == FCP_OP_MERGE) inside(P.off_rows, P.n_rows, sizeof(fcp::RowItem));
  if (op == FCP_OP_BWD) {
    inside(P.off_kvitems, P.n_kvitems, sizeof(fcp::KvItem));
    inside(P.off_reduce, P.n_reduce, sizeof(fcp::ReduceItem));
    check(P.off_stats >= blob && P.off_partial >= P.off_stats && P.off_partial <= P.ws_bytes,
          "backward regions ordered");
    const fcp::KvItem* it =
        reinterpret_cast<const fcp::KvItem*>(P.blob.data() + P.off_kvitems);
    for (int i = 0; i < P.n_kvitems; ++i) {
      check(it[i].kv_rows >= 1 && it[i].kv_rows <= fcp::kKvTileBwd, "kv item rows",
            it[i].kv_rows);
      const int first = it[i].heads & 0xffff, count = it[i].heads >> 16;
      check(count >= 1 && first + count <= P.shape.group, "kv item heads", first, count);
      check(it[i].slot < P.n_slots, "kv item slot", it[i].slot, P.n_slots);
    }
  }
}

void scheduler_cases(Rng& r, int cases) {
  for (int c = 0; c < cases; ++c) {
    const fcp_dims_t d0 = random_dims(r);
    const int n = (int)r.in(0, 40);
    fcp_dims_t d = d0;
    const std::vector<fcp_pair_t> pairs = random_pairs(r, d, n);
    int64_t need = 0;
    for (const fcp_pair_t& p : pairs) need = std::max<int64_t>(need, (int64_t)p.out_row + p.q_len);
    if (r.p(0.9)) d.part_rows = need;  // partial rows fit, unless the draw says otherwise
    for (int op = -1; op <= 4; ++op) {
      std::string err;
      const int st = fcp::validate(&d, pairs.data(), n, op, &err);
      fcp::Plan P;
      const int st2 = fcp::make_plan(&d, pairs.data(), n, op, &P, &err);
      check(st == st2, "make_plan status equals validate's", st, st2);
      if (st2 == FCP_OK) {
        ++g_accepted[op + 1];
        check_plan(P, op, n);
      }
      else check(!err.empty(), "an error carries a message");
    }
  }
}

void comm_cases(Rng& r, int cases) {
  for (int c = 0; c < cases; ++c) {
    const int32_t w = (int32_t)r.in(1, 40);
    const int32_t n = (int32_t)r.in(0, 300);
    std::vector<int32_t> src(n), dst(n), stage(n, -1);
    for (int32_t e = 0; e < n; ++e) {
      src[e] = (int32_t)r.in(0, w - 1);
      dst[e] = (int32_t)r.in(0, w - 1);
    }
    const bool bad = r.p(0.05) && n > 0;
    if (bad) src[r.in(0, n - 1)] = r.p(0.5) ? w : -1;
    int32_t k = -1;
    std::string err;
    const int st = fcp::comm_plan(w, n, src.data(), dst.data(), stage.data(), &k, &err);
    if (bad) {
      check(st == FCP_ERR_INVALID_ARG, "bad worker id rejected", st);
      continue;
    }
    check(st == FCP_OK, "comm plan accepted", st);
    if (st != FCP_OK) continue;
    ++g_comm_ok;
    std::vector<int32_t> dout(w, 0), din(w, 0);
    for (int32_t e = 0; e < n; ++e) ++dout[src[e]], ++din[dst[e]];
    int32_t delta = 0;
    for (int32_t i = 0; i < w; ++i) delta = std::max(delta, std::max(dout[i], din[i]));
    check(k == delta, "stages == max degree", k, delta);
    std::vector<std::vector<int>> sent(k, std::vector<int>(w, 0)), recv = sent;
    for (int32_t e = 0; e < n; ++e) {
      check(stage[e] >= 0 && stage[e] < k, "stage in range", stage[e], k);
      if (stage[e] < 0 || stage[e] >= k) continue;
      check(++sent[stage[e]][src[e]] == 1, "one send per stage", stage[e], src[e]);
      check(++recv[stage[e]][dst[e]] == 1, "one receive per stage", stage[e], dst[e]);
    }
  }
}

void pipeline_cases(Rng& r, int cases) {
  for (int c = 0; c < cases; ++c) {
    fcp_dims_t d = random_dims(r);
    const int32_t n_stages = (int32_t)r.in(0, 8);
    std::vector<fcp_stage_t> stages(n_stages);
    std::vector<fcp_copy_t> copies;
    std::vector<fcp_pair_t> pairs;
    int64_t src_rows = r.in(0, 4000);
    for (auto& s : stages) {
      s.n_copies = (int32_t)r.in(r.p(0.02) ? -1 : 0, 3);
      s.n_pairs = (int32_t)r.in(0, 4);
      for (int i = 0; i < std::max(0, s.n_copies); ++i)
        copies.push_back(fcp_copy_t{r.in(0, std::max<int64_t>(0, src_rows - 1)),
                                    r.in(0, std::max<int64_t>(0, d.kv_rows - 1)),
                                    r.in(r.p(0.02) ? 0 : 1, 600)});
      auto more = random_pairs(r, d, s.n_pairs);
      pairs.insert(pairs.end(), more.begin(), more.end());
    }
    int64_t out = 0;
    for (auto& p : pairs) {  // disjoint partial rows, as the forward requires
      p.out_row = (int32_t)out;
      out += std::max(1, p.q_len);
    }
    d.part_rows = out;
    fcp::PipelinePlan P;
    std::string err;
    const int depth = (int)r.in(r.p(0.02) ? 0 : 1, 4);
    const int st = fcp::make_pipeline_plan(&d, stages.data(), n_stages, copies.data(),
                                           pairs.data(), depth, src_rows, &P, &err);
    if (st != FCP_OK) {
      check(!err.empty(), "pipeline error carries a message");
      continue;
    }
    ++g_pipe_ok;
    check(P.blob.size() <= P.ws_bytes || P.n_pairs == 0, "pipeline blob inside workspace");
    check((int)P.stage.size() == n_stages, "a plan per stage", (long long)P.stage.size());
    for (int32_t s = 0; s < n_stages; ++s)
      if (P.stage[s].n_qitems > 0)
        check(P.stage_off[s] + P.stage[s].blob.size() <= P.blob.size(), "stage tables inside");
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: plan_check <seed> <cases>\n");
    return 2;
  }
  const uint64_t seed = std::strtoull(argv[1], nullptr, 10);
  const int cases = std::atoi(argv[2]);
  Rng r(seed);
  scheduler_cases(r, cases);
  comm_cases(r, cases);
  pipeline_cases(r, cases);
  std::printf("plan_check seed %llu: %d cases each; accepted plans fwd %d merge %d bwd %d "
              "fused %d (unknown ops %d), comm %d, pipeline %d; %d failed checks\n",
              (unsigned long long)seed, cases, g_accepted[1], g_accepted[2], g_accepted[3],
              g_accepted[4], g_accepted[0] + g_accepted[5], g_comm_ok, g_pipe_ok, g_fail);
  return g_fail == 0 ? 0 : 1;
}
