// Validation of block-pair tables and the varlen tile scheduler.
//
// Pairs follow the FCP per-worker model (FCP paper Sec. 4.1 and Sec. 4.2): a worker's Q
// blocks, cut into per-sequence segments, meet local or pulled KV ranges. The scheduler
// expands pairs into workgroup-sized tiles, weights each tile by the KV (or Q) tiles the
// mask leaves visible, and orders the list heaviest first so the longest tiles start
// first on the 256 compute units (the greedy longest-processing-time rule that FCP
// applies across workers, Sec. 4.1, applied here across CUs).
#include "fcp_plan.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <numeric>

namespace fcp {
namespace {

constexpr size_t kAlign = 256;
// Compute units of the target GPU, for load-balancing decisions only.
constexpr int64_t kTargetCUs = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

std::string pair_str(int i, const fcp_pair_t& p) {
  char buf[256];
  snprintf(buf, sizeof buf,
           "pair %d {seq %d, q %d+%d, kv %d+%d, mask_offset %d, out_row %d, flags %d}", i,
           p.seq_id, p.q_start, p.q_len, p.kv_start, p.kv_len, p.mask_offset, p.out_row,
           p.flags);
  return buf;
}

int shape_of(const fcp_dims_t* dims, Shape* s, std::string* err) {
  if (!dims) return fail(err, FCP_ERR_INVALID_ARG, "dims is NULL");
  if (dims->num_q_heads < 1 || dims->num_kv_heads < 1)
    return fail(err, FCP_ERR_INVALID_ARG, "head counts must be >= 1");
  if (dims->num_q_heads > 4096)
    return fail(err, FCP_ERR_UNSUPPORTED, "num_q_heads above 4096");
  if (dims->num_q_heads % dims->num_kv_heads != 0)
    return fail(err, FCP_ERR_UNSUPPORTED, "num_q_heads is not a multiple of num_kv_heads");
  const int g = dims->num_q_heads / dims->num_kv_heads;
  if (!(g == 1 || g == 2 || g == 4 || g % 8 == 0))
    return fail(err, FCP_ERR_UNSUPPORTED, "head group size must be 1, 2, 4 or a multiple of 8");
  if (dims->head_dim != 64 && dims->head_dim != 128)
    return fail(err, FCP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const float sc = dims->softmax_scale;
  if (!(sc == 0.f || (std::isfinite(sc) && sc > 0.f)))
    return fail(err, FCP_ERR_INVALID_ARG, "softmax_scale must be 0 or finite and > 0");
  if (dims->q_rows < 0 || dims->kv_rows < 0 || dims->part_rows < 0)
    return fail(err, FCP_ERR_INVALID_ARG, "row extents must be >= 0");
  if (dims->q_rows > INT32_MAX || dims->kv_rows > INT32_MAX || dims->part_rows > INT32_MAX)
    return fail(err, FCP_ERR_INVALID_ARG, "row extents must fit in int32");
  s->hq = dims->num_q_heads;
  s->hkv = dims->num_kv_heads;
  s->d = dims->head_dim;
  s->group = g;
  s->hpw = g < 8 ? g : 8;
  s->n_hgroups = s->hq / s->hpw;
  s->tile_tokens = kColBlock * (kColBlocksPerWG / s->hpw);
  s->scale = sc == 0.f ? 1.0f / std::sqrt((float)dims->head_dim) : sc;
  return FCP_OK;
}

// Rejects overlapping [start, start + len) intervals unless `allow_identical` and the two
// intervals are equal.
int check_overlap(std::vector<std::pair<int64_t, int64_t>> iv, bool allow_identical,
                  const char* what, std::string* err) {
  std::sort(iv.begin(), iv.end());
  for (size_t i = 1; i < iv.size(); ++i) {
    const auto& a = iv[i - 1];
    const auto& b = iv[i];
    if (allow_identical && a == b) continue;
    if (a.first + a.second > b.first) {
      char buf[200];
      snprintf(buf, sizeof buf, "%s ranges [%lld, %lld) and [%lld, %lld) overlap", what,
               (long long)a.first, (long long)(a.first + a.second), (long long)b.first,
               (long long)(b.first + b.second));
      return fail(err, FCP_ERR_INVALID_ARG, buf);
    }
  }
  return FCP_OK;
}

// Pairs with identical Q range, ordered by q_start.
struct Group {
  int32_t q_start, q_len;
  std::vector<int> pairs;
};

std::vector<Group> group_by_q(const fcp_pair_t* pairs, int n) {
  std::vector<int> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
    if (pairs[a].q_start != pairs[b].q_start) return pairs[a].q_start < pairs[b].q_start;
    return pairs[a].q_len < pairs[b].q_len;
  });
  std::vector<Group> out;
  for (int i : idx) {
    if (out.empty() || out.back().q_start != pairs[i].q_start ||
        out.back().q_len != pairs[i].q_len)
      out.push_back(Group{pairs[i].q_start, pairs[i].q_len, {}});
    out.back().pairs.push_back(i);
  }
  return out;
}

// The causal offset of a pair clamped to [-q_len, kv_len]: every offset at or above
// kv_len - 1 lets each query see every key, every offset at or below -q_len lets none see
// any, so the clamp keeps the mask and keeps the kernels' int arithmetic on it in range.
int32_t mask_of(const fcp_pair_t& p) {
  if (!(p.flags & FCP_PAIR_CAUSAL)) return 0;
  return std::max(-p.q_len, std::min(p.mask_offset, p.kv_len));
}

// KV tiles of `kv_len` keys that queries [q_off, q_off + rows) can see.
int32_t visible_kv_tiles(const KvSeg& s, int32_t q_off, int32_t rows) {
  int64_t last = s.kv_len - 1;
  if (s.flags & FCP_PAIR_CAUSAL)
    last = std::min<int64_t>(last, (int64_t)q_off + rows - 1 + s.mask_offset);
  return last < 0 ? 0 : (int32_t)(last / kKvTile + 1);
}

// Q tiles of `q_len` queries that see any of keys [key_off, key_off + rows).
int32_t visible_q_tiles(const QSeg& s, int32_t key_off) {
  int64_t first = 0;
  if (s.flags & FCP_PAIR_CAUSAL) first = std::max<int64_t>(0, (int64_t)key_off - s.mask_offset);
  if (first >= s.q_len) return 0;
  return (int32_t)((s.q_len - first + kQTileBwd - 1) / kQTileBwd);
}

template <class T>
size_t put(std::vector<uint8_t>* blob, const std::vector<T>& v) {
  const size_t off = align_up(blob->size());
  blob->resize(off + v.size() * sizeof(T));
  if (!v.empty()) std::memcpy(blob->data() + off, v.data(), v.size() * sizeof(T));
  return off;
}

// One workgroup of a launch before placement: a work item with a head (query-head group
// or KV head), its cost and the KV head whose K/V (forward, dQ) or Q tiles (dK/dV) it
// reads.
struct Unit {
  int32_t item, head;
  int64_t cost;
  int32_t kv_head;
};

// Launch order that keeps the work of one KV head on its own XCDs, whose L2 then serves
// the repeated reads of that head's K/V tiles (forward, dQ) or Q/dO tiles (dK/dV) (FCP
// paper Sec. 3.1 ties the efficiency of small blocks to how often each loaded element is
// reused). KV head h may use XCD x iff x % hkv == h % hkv when hkv divides kXcds (one
// XCD per head at 8 heads, 8 / hkv XCDs per head below that), else x % kXcds ==
// h % kXcds when kXcds divides hkv, else any XCD. Units go heaviest first, each to the
// least-loaded XCD (by cost) it may use; the launch takes the XCDs' queues row by row,
// one unit per XCD (workgroup b runs on XCD b % kXcds), with empty workgroups where a
// queue runs out before the others. Measured: the earlier alternative of cutting each
// head's Q ranges into contiguous per-XCD runs lost 15-21% at 2 and 1 KV heads (its XCDs
// received unequal mixes of heavy and light items), and the order here keeps the
// heaviest-first start that the 256 CUs need.
std::vector<WgMap> xcd_order(std::vector<Unit> units, int hkv) {
  std::stable_sort(units.begin(), units.end(),
                   [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
  std::vector<std::vector<Unit>> queue(kXcds);
  int64_t load[kXcds] = {};
  for (const Unit& u : units) {
    int best = -1;
    for (int x = 0; x < kXcds; ++x) {
      const bool ok = (kXcds % hkv == 0)   ? x % hkv == u.kv_head % hkv
                      : (hkv % kXcds == 0) ? x == u.kv_head % kXcds
                                           : true;
      if (ok && (best < 0 || load[x] < load[best])) best = x;
    }
    queue[best].push_back(u);
    load[best] += std::max<int64_t>(1, u.cost);
  }
  size_t rows = 0;
  for (const auto& q : queue) rows = std::max(rows, q.size());
  std::vector<WgMap> out;
  out.reserve(rows * kXcds);
  for (size_t j = 0; j < rows; ++j)
    for (int x = 0; x < kXcds; ++x)
      out.push_back(j < queue[x].size() ? WgMap{queue[x][j].item, queue[x][j].head}
                                        : WgMap{-1, -1});
  while (!out.empty() && out.back().item < 0) out.pop_back();
  return out;
}

// Forward / dQ workgroups: every item for every query-head group.
std::vector<WgMap> q_order(const std::vector<QItem>& items, const Shape& s) {
  std::vector<Unit> units;
  units.reserve(items.size() * s.n_hgroups);
  for (int32_t i = 0; i < (int32_t)items.size(); ++i)
    for (int32_t hg = 0; hg < s.n_hgroups; ++hg)
      units.push_back(Unit{i, hg, items[i].cost, hg * s.hpw / s.group});
  return xcd_order(std::move(units), s.hkv);
}

void sort_heaviest_first(std::vector<QItem>* items) {
  std::stable_sort(items->begin(), items->end(),
                   [](const QItem& a, const QItem& b) { return a.cost > b.cost; });
}

// Q-stationary items over groups of identical Q range (both forwards and dQ). With
// seg_out, also records each segment's pair's first partial-output row.
void group_items(const fcp_pair_t* pairs, const std::vector<Group>& groups, const Shape& s,
                 std::vector<QItem>* items, std::vector<KvSeg>* segs,
                 std::vector<int32_t>* seg_out = nullptr) {
  for (const Group& g : groups) {
    const int32_t sb = (int32_t)segs->size();
    for (int p : g.pairs) {
      segs->push_back(KvSeg{pairs[p].kv_start, pairs[p].kv_len, mask_of(pairs[p]),
                            pairs[p].flags});
      if (seg_out) seg_out->push_back(pairs[p].out_row);
    }
    for (int32_t t = 0; t < g.q_len; t += s.tile_tokens) {
      QItem it{};
      it.q_row0 = g.q_start + t;
      it.q_rows = std::min(s.tile_tokens, g.q_len - t);
      it.q_off = t;
      it.out_row0 = it.q_row0;
      it.seg_begin = sb;
      it.seg_count = (int32_t)g.pairs.size();
      for (int32_t j = 0; j < it.seg_count; ++j)
        it.cost += visible_kv_tiles((*segs)[sb + j], t, it.q_rows);
      items->push_back(it);
    }
  }
  sort_heaviest_first(items);
}

}  // namespace

int validate(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op,
             std::string* err) {
  Shape s;
  int st = shape_of(dims, &s, err);
  if (st != FCP_OK) return st;
  if (op < FCP_OP_FWD || op > FCP_OP_FWD_FUSED)
    return fail(err, FCP_ERR_INVALID_ARG, "unknown op");
  if (n_pairs < 0) return fail(err, FCP_ERR_INVALID_ARG, "n_pairs < 0");
  if (n_pairs > 0 && !pairs) return fail(err, FCP_ERR_INVALID_ARG, "pairs is NULL");
  const bool uses_parts = (op == FCP_OP_FWD || op == FCP_OP_MERGE);
  std::vector<std::pair<int64_t, int64_t>> qr, outr;
  qr.reserve(n_pairs);
  for (int i = 0; i < n_pairs; ++i) {
    const fcp_pair_t& p = pairs[i];
    if (p.q_len < 1 || p.kv_len < 1)
      return fail(err, FCP_ERR_INVALID_ARG, pair_str(i, p) + ": q_len and kv_len must be >= 1");
    if (p.q_start < 0 || (int64_t)p.q_start + p.q_len > dims->q_rows)
      return fail(err, FCP_ERR_INVALID_ARG, pair_str(i, p) + ": Q range outside q_rows");
    if (op != FCP_OP_MERGE && (p.kv_start < 0 || (int64_t)p.kv_start + p.kv_len > dims->kv_rows))
      return fail(err, FCP_ERR_INVALID_ARG, pair_str(i, p) + ": KV range outside kv_rows");
    if (p.flags & ~FCP_PAIR_CAUSAL)
      return fail(err, FCP_ERR_INVALID_ARG, pair_str(i, p) + ": unknown flag bits");
    if (uses_parts && (p.out_row < 0 || (int64_t)p.out_row + p.q_len > dims->part_rows))
      return fail(err, FCP_ERR_INVALID_ARG, pair_str(i, p) + ": partial rows outside part_rows");
    qr.emplace_back(p.q_start, p.q_len);
    if (uses_parts) outr.emplace_back(p.out_row, p.q_len);
  }
  if (uses_parts) {
    st = check_overlap(outr, false, "partial-output", err);
    if (st != FCP_OK) return st;
  }
  if (op != FCP_OP_FWD) {
    st = check_overlap(qr, true, "Q", err);
    if (st != FCP_OK) return st;
  }
  return FCP_OK;
}

int make_plan(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op,
              Plan* plan, std::string* err) {
  int st = validate(dims, pairs, n_pairs, op, err);
  if (st != FCP_OK) return st;
  Plan& P = *plan;
  P = Plan{};
  shape_of(dims, &P.shape, err);
  const Shape& s = P.shape;
  if (n_pairs == 0) return FCP_OK;

  if (op == FCP_OP_FWD) {
    // One item per tile of a Q range walks every pair of that range, as the fused
    // forward does, and writes each pair's partial where the pair ends.
    std::vector<QItem> items;
    std::vector<KvSeg> segs;
    std::vector<int32_t> seg_out;
    group_items(pairs, group_by_q(pairs, n_pairs), s, &items, &segs, &seg_out);
    const std::vector<WgMap> qmap = q_order(items, s);
    P.off_qitems = put(&P.blob, items);
    P.off_segs = put(&P.blob, segs);
    P.off_segout = put(&P.blob, seg_out);
    P.off_qmap = put(&P.blob, qmap);
    P.n_qitems = (int)items.size();
    P.n_qwg = (int)qmap.size();
  } else if (op == FCP_OP_FWD_FUSED) {
    std::vector<QItem> items;
    std::vector<KvSeg> segs;
    group_items(pairs, group_by_q(pairs, n_pairs), s, &items, &segs);
    const std::vector<WgMap> qmap = q_order(items, s);
    P.off_qitems = put(&P.blob, items);
    P.off_segs = put(&P.blob, segs);
    P.off_qmap = put(&P.blob, qmap);
    P.n_qitems = (int)items.size();
    P.n_qwg = (int)qmap.size();
  } else if (op == FCP_OP_MERGE) {
    std::vector<RowItem> rows;
    std::vector<int32_t> parts;
    for (const Group& g : group_by_q(pairs, n_pairs)) {
      const int32_t pb = (int32_t)parts.size();
      for (int p : g.pairs) parts.push_back(pairs[p].out_row);
      for (int32_t r = 0; r < g.q_len; ++r)
        rows.push_back(RowItem{g.q_start + r, r, pb, (int32_t)g.pairs.size()});
    }
    P.off_rows = put(&P.blob, rows);
    P.off_parts = put(&P.blob, parts);
    P.n_rows = (int)rows.size();
  } else {  // FCP_OP_BWD
    const std::vector<Group> groups = group_by_q(pairs, n_pairs);
    std::vector<QItem> items;
    std::vector<KvSeg> segs;
    group_items(pairs, groups, s, &items, &segs);
    // Elementary KV intervals: cut every KV range at every pair boundary, so each key
    // row belongs to one interval and one dK/dV work item owns it.
    std::vector<int64_t> cuts;
    cuts.reserve(2 * n_pairs);
    for (int i = 0; i < n_pairs; ++i) {
      cuts.push_back(pairs[i].kv_start);
      cuts.push_back((int64_t)pairs[i].kv_start + pairs[i].kv_len);
    }
    std::sort(cuts.begin(), cuts.end());
    cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
    std::vector<int> by_start(n_pairs);
    std::iota(by_start.begin(), by_start.end(), 0);
    std::sort(by_start.begin(), by_start.end(),
              [&](int a, int b) { return pairs[a].kv_start < pairs[b].kv_start; });
    std::vector<KvItem> kvitems;
    std::vector<QSeg> qsegs;
    std::vector<int> active;
    size_t next = 0;
    for (size_t c = 0; c + 1 < cuts.size(); ++c) {
      const int64_t a = cuts[c], b = cuts[c + 1];
      while (next < by_start.size() && pairs[by_start[next]].kv_start <= a)
        active.push_back(by_start[next++]);
      active.erase(std::remove_if(active.begin(), active.end(),
                                  [&](int p) {
                                    return (int64_t)pairs[p].kv_start + pairs[p].kv_len <= a;
                                  }),
                   active.end());
      if (active.empty()) continue;
      std::vector<int> cov(active);
      std::sort(cov.begin(), cov.end());
      const int32_t sb = (int32_t)qsegs.size();
      for (int p : cov)
        qsegs.push_back(QSeg{pairs[p].q_start, pairs[p].q_len,
                             (int32_t)(mask_of(pairs[p]) - (a - pairs[p].kv_start)),
                             pairs[p].flags});
      for (int64_t t = 0; t < b - a; t += kKvTileBwd) {
        KvItem it{};
        it.kv_row0 = (int32_t)(a + t);
        it.kv_rows = (int32_t)std::min<int64_t>(kKvTileBwd, b - a - t);
        it.key_off = (int32_t)t;
        it.seg_begin = sb;
        it.seg_count = (int32_t)cov.size();
        for (int32_t j = 0; j < it.seg_count; ++j)
          it.cost += visible_q_tiles(qsegs[sb + j], it.key_off);
        kvitems.push_back(it);
      }
    }
    // Each item streams (Q tile, query head) steps. An item far above the average load
    // per CU would set the makespan on its own, so heavy items are split by query-head
    // subsets (contributions of different heads add); their parts write fp32 partials
    // that a reduction adds into dk/dv in a fixed order.
    int64_t total = 0;
    for (KvItem& it : kvitems) {
      it.cost *= s.group;
      total += (int64_t)it.cost * s.hkv;
    }
    const int64_t target = std::max<int64_t>(1, total / (2 * kTargetCUs));
    std::vector<KvItem> split;
    std::vector<ReduceItem> reduce;
    int32_t n_slots = 0;
    for (const KvItem& it : kvitems) {
      const int parts = (int)std::min<int64_t>(s.group, (it.cost + target - 1) / target);
      if (parts <= 1) {
        KvItem one = it;
        one.heads = 0 | (s.group << 16);
        one.slot = -1;
        split.push_back(one);
        continue;
      }
      reduce.push_back(ReduceItem{it.kv_row0, it.kv_rows, n_slots, parts});
      for (int k = 0; k < parts; ++k) {
        const int h0 = k * s.group / parts, h1 = (k + 1) * s.group / parts;
        KvItem part = it;
        part.heads = h0 | ((h1 - h0) << 16);
        part.cost = it.cost / s.group * (h1 - h0);
        part.slot = n_slots + k;
        split.push_back(part);
      }
      n_slots += parts;
    }
    kvitems.swap(split);
    std::stable_sort(kvitems.begin(), kvitems.end(),
                     [](const KvItem& x, const KvItem& y) { return x.cost > y.cost; });
    // dK/dV workgroups: every item for every KV head.
    std::vector<Unit> kunits;
    kunits.reserve(kvitems.size() * s.hkv);
    for (int32_t i = 0; i < (int32_t)kvitems.size(); ++i)
      for (int32_t h = 0; h < s.hkv; ++h) kunits.push_back(Unit{i, h, kvitems[i].cost, h});
    const std::vector<WgMap> kvmap = xcd_order(std::move(kunits), s.hkv);
    const std::vector<WgMap> qmap = q_order(items, s);
    P.off_qitems = put(&P.blob, items);
    P.off_segs = put(&P.blob, segs);
    P.off_kvitems = put(&P.blob, kvitems);
    P.off_qsegs = put(&P.blob, qsegs);
    P.off_reduce = put(&P.blob, reduce);
    P.off_qmap = put(&P.blob, qmap);
    P.off_kvmap = put(&P.blob, kvmap);
    P.n_qwg = (int)qmap.size();
    P.n_kvwg = (int)kvmap.size();
    P.n_qitems = (int)items.size();
    P.n_kvitems = (int)kvitems.size();
    P.n_reduce = (int)reduce.size();
    P.n_slots = n_slots;
    P.off_stats = align_up(P.blob.size());
    P.off_partial = P.off_stats + align_up((size_t)dims->q_rows * s.hq * 2 * sizeof(float));
    // Partial slots: dK then dV, each [slot][kv head][kKvTileBwd][D] fp32.
    P.ws_bytes = P.off_partial +
                 align_up(2 * (size_t)n_slots * s.hkv * kKvTileBwd * s.d * sizeof(float));
    return FCP_OK;
  }
  P.ws_bytes = align_up(P.blob.size());
  return FCP_OK;
}

}  // namespace fcp
