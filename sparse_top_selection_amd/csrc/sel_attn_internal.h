// Internal declarations shared by the HIP sources of libselattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sel_attn.h"

namespace selattn {

struct UnionArgs {
  const int32_t* sel;
  const int32_t* sel_len;
  const int32_t* page_table;
  int32_t* union_cells;
  uint8_t* union_mask;
  int32_t* union_rows;   // pool row of each union cell for KV head 0, -1 if not resident
  int32_t* union_len;
  uint32_t* status;
  int32_t n_ctx;
  int32_t n_q;
  int32_t sel_cap;
  int32_t n_kv;
  int32_t n_pages;
};

struct PrefillArgs {
  const float* q;
  const int8_t* k_pool;
  const int8_t* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* union_rows;
  const uint8_t* union_mask;
  const int32_t* union_len;
  float* out;
  uint32_t* status;
  float score_scale;   // softmax_scale * log2(e): scores go straight into exp2
  int32_t n_ctx;
  int32_t n_q;
  int32_t n_kv;
  int32_t n_pages;
  uint32_t row_limit;  // union rows r with r + 64 (n_kv - 1) inside the pools: r < row_limit
  int32_t sel_cap;
  int32_t n_groups;
  int32_t per_xcd;     // workgroups each XCD walks through (grid = 8 * per_xcd)
  int32_t n_splits;    // work-groups per (group, KV head): 1 writes out directly,
                       // more write PrefillPartial records that a merge combines
  struct PrefillPartial* part;   // [n_groups * n_kv][n_splits] when n_splits > 1
};

// One split of a (group, KV head)'s union: for each of the 96 rows, the running
// maximum (log2 domain), the probability sum and O (2^6 times sum p v, the V
// offset removed), unnormalised.
struct PrefillPartial {
  float m[96];
  float l[96];
  float o[96][128];
};

// Work-groups per (group, KV head) that sel_attn_prefill_split uses for a grid
// of n_items = groups * KV heads whose unions hold at most max_cells cells
// (min(8 sel_cap, n_ctx)): enough to give the GPU kPrefillSplitTarget
// work-groups when the grid alone is smaller, at most 16, and no more than
// leave each split kPrefillMinSplitChunks chunks of the longest possible union.
// A split work-group's fixed cost (three dependent memory round trips before
// its first chunk, its record written and flushed, its share of the merge) is
// about the time of 8 to 12 chunks, so shorter shares gain nothing.
constexpr int kPrefillSplitTarget = 512;
constexpr int kPrefillMaxSplits = 16;
constexpr int kPrefillMinSplitChunks = 12;
inline int prefill_split_count(int64_t n_items, int64_t max_cells) {
  if (n_items <= 0 || n_items >= kPrefillSplitTarget) return 1;
  int64_t s = (kPrefillSplitTarget + n_items - 1) / n_items;
  if (s > kPrefillMaxSplits) s = kPrefillMaxSplits;
  const int64_t by_len = ((max_cells > 0 ? max_cells : 0) + 31) / 32 / kPrefillMinSplitChunks;
  if (s > by_len) s = by_len;
  return s > 1 ? (int)s : 1;
}

struct SelectArgs {
  const float* scores;   // [n_q][n_blocks]
  int32_t* sel;          // [n_q][sel_cap]
  int32_t* sel_len;      // [n_q]
  int32_t n_q;
  int32_t first_pos;     // position of query index 0
  int32_t n_blocks;      // ceil(n_ctx / 64): the score row stride
  int32_t sel_cap;
};

struct PositionsArgs {
  const float* q;
  const int8_t* k_pool;
  const int8_t* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* page_table;
  const int32_t* sel;
  const int32_t* sel_len;
  float* out;
  uint32_t* status;
  float score_scale;   // softmax_scale * log2(e)
  int32_t n_ctx;
  int32_t n_q;
  int32_t n_kv;
  int32_t n_pages;
  int32_t sel_cap;
  int32_t per_xcd;     // positions each XCD walks through (grid = 8 * per_xcd)
  int32_t n_splits;    // decode: splits of each position's list (of kDecodeSplit cells)
};

// Decode: cells per split, and one split's unnormalised state for one
// (position, KV head): running maximum (log2 domain), probability sum and
// O (2^6 times sum p v, the V bias removed) of the 12 query rows.
constexpr int kDecodeSplit = 64;   // at most 40 splits (sel_cap <= 2560)
struct DecodePartial {
  float m[16];
  float l[16];
  float o[12][128];
};

hipError_t launch_select_blocks(const SelectArgs& a, hipStream_t stream);
hipError_t launch_prefill_positions(const PositionsArgs& a, hipStream_t stream);
hipError_t launch_decode(const PositionsArgs& a, DecodePartial* part, hipStream_t stream);
hipError_t launch_union_build(const UnionArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_split(const PrefillArgs& a, hipStream_t stream);   // n_splits > 1

}  // namespace selattn
