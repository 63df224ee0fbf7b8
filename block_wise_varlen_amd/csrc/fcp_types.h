// Work-list records shared by the host planner and the gfx950 kernels.
//
// The planner turns the caller's block-pair table into flat lists of these records and
// uploads them into the caller's workspace; every kernel reads only these lists plus the
// tensors. All fields are int32; every record is 16 or 32 bytes.
#pragma once

#include <stdint.h>

namespace fcp {

// Tokens per column block of a forward / dQ tile (one MFMA 32x32 column block).
constexpr int kColBlock = 32;
// Column blocks per forward / dQ workgroup: 8 waves x 1 column block (two waves per SIMD).
constexpr int kColBlocksPerWG = 8;
// Granularity (keys) of the host's cost estimate that orders forward and dQ work items
// heaviest first (the kernels themselves stream 128-key tiles).
constexpr int kKvTile = 64;
// Keys per workgroup tile of the dK/dV kernel (4 SIMD pairs of waves x 32 keys).
constexpr int kKvTileBwd = 128;
// Query rows per Q tile streamed by the dK/dV kernel.
constexpr int kQTileBwd = 32;

// One forward / dQ work item: a tile of up to `q_rows` consecutive query rows of one
// Q range, for one group of query heads (the head group comes from the grid), against
// the KV segments seg[seg_begin .. seg_begin + seg_count).
struct QItem {
  int32_t q_row0;     // first Q row (absolute row in q / dout / o / lse / dq)
  int32_t q_rows;     // valid rows in this tile (<= tile tokens)
  int32_t q_off;      // offset of q_row0 within its Q range (query index i base)
  int32_t out_row0;   // first output row: o_part row (per-pair fwd) or q row
  int32_t seg_begin;  // first KvSeg of this item
  int32_t seg_count;  // number of KvSegs folded by this item
  int32_t cost;       // visible KV tiles (scheduling weight)
  int32_t pad;
};

// XCDs of the target GPU. Workgroups of a launch are handed to the XCDs round robin in
// workgroup-id order (workgroup b runs on XCD b % kXcds), so the launch order below
// decides which XCD (and which of their separate L2 caches) a work item meets; only
// locality, never correctness, depends on it.
constexpr int kXcds = 8;

// Workgroup b of a forward / dQ / dK/dV launch runs work item `item` for query-head group
// (forward, dQ) or KV head (dK/dV) `head`; item < 0 marks an empty workgroup that exits
// at once (padding that keeps the XCD assignment of the workgroups after it).
struct WgMap {
  int32_t item;
  int32_t head;
};

// KV side of one pair as seen from its Q range.
struct KvSeg {
  int32_t kv_start;     // first KV row
  int32_t kv_len;       // keys in the range
  int32_t mask_offset;  // causal: key j visible to query i iff j - i <= mask_offset
  int32_t flags;        // bit 0 causal
};

// One merge / Delta row: row `q_row`, which is row `row_in_group` of its Q range, and
// the partial rows part_rows[part_begin + p] + row_in_group for p < n_parts.
struct RowItem {
  int32_t q_row;
  int32_t row_in_group;
  int32_t part_begin;
  int32_t n_parts;
};

// One dK/dV work item: keys [kv_row0, kv_row0 + kv_rows) of an elementary KV interval
// (a run of keys covered by the same set of pairs), for one KV head (from the grid),
// against the Q sides qseg[seg_begin .. seg_begin + seg_count).
struct KvItem {
  int32_t kv_row0;     // first key row (absolute)
  int32_t kv_rows;     // valid keys (<= kKvTileBwd)
  int32_t key_off;     // offset of kv_row0 within its interval (key index j base)
  int32_t seg_begin;
  int32_t seg_count;
  int32_t cost;        // streamed (Q tile, head) steps
  int32_t heads;       // query heads of the group this item streams: first | count << 16
  int32_t slot;        // -1: add into dk/dv; else partial slot (reduced afterwards)
};

// Sum of the partial slots slot_begin .. slot_begin + n_slots - 1 of one KV tile, added
// into dk/dv rows kv_row0 .. kv_row0 + kv_rows - 1 (one KV head per workgroup).
struct ReduceItem {
  int32_t kv_row0;
  int32_t kv_rows;
  int32_t slot_begin;
  int32_t n_slots;
};

// Q side of one pair as seen from an elementary KV interval. Key index j counts from
// the interval start: key j visible to query i iff j - i <= mask_offset (causal).
struct QSeg {
  int32_t q_start;
  int32_t q_len;
  int32_t mask_offset;
  int32_t flags;
};

}  // namespace fcp
