// Work-list records shared by the host planner (plan.cpp) and the HIP kernels
// (kernels.hip).  Plain int32 records so the planner needs no HIP headers and the
// kernels read them with scalar loads.
#pragma once
#include <stdint.h>

#include "varlen_attn.h"

namespace va {

// One split-KV work item = one wavefront.  It reads kv positions [k0, k1) of request
// `req`'s block table for KV head `kvh` and scores them against up to 16 query columns
// (up to 32 in bf16 and fp8 plans, run by the two-block kernels) cols[col0 .. col0+ncols).  Each column's partial result goes to workspace slot
// cols[c].pbase + slot, or, with kItemDirect (the item covers its columns' whole kv range),
// straight to the output rows.
struct SplitItem {
  int32_t req, kvh, col0, ncols;
  int32_t k0, k1, slot, flags;  // flags: kItemMasked if some column's limit < k1 - 1; kItemDirect
};
enum { kItemMasked = 1, kItemDirect = 2 };

// A query column: flat Q row, query head, last visible kv position (S0 + i), and the
// first workspace slot of this (row, head) output.
struct Column {
  int32_t q_row, q_head, limit, pbase;
};

// One (row, head) output assembled from nparts partial results.
struct CombineRow {
  int32_t q_row, q_head, pbase, nparts;
};

// One MFMA prefill tile: query columns c0 .. c0+ncols of request `req` under KV head
// `kvh`, where column c is new row i = c / g with query head kvh*g + c % g, scored
// against keys [kbeg, kv_end) (row i sees keys up to S0 + i).  pbase < 0: the tile holds
// all of its columns' keys and writes normalised output rows; else it is one key chunk of
// a cut tile and tile column col writes its partial (m, l, acc) to workspace slot
// pbase + col * pstride for the combine pass.
// With kTileColumnList in flags the tile's columns are cols[c0 .. c0+ncols) (rows of one
// or several requests, each with its own causal limit), its keys [kbeg, kv_end) of request
// req's block table, and column col's partial goes to slot cols[c0+col].pbase + q0: a
// shared-prefix group tile (keys of the pages the group shares) or the tile of a group
// member's own keys after them.
struct PrefillTile {
  int32_t req, kvh, c0, ncols;
  int32_t q0, S0, kv_end, kbeg;
  int32_t pbase, pstride, flags, group;   // group: a shared-prefix group tile (counters only)
};
constexpr int32_t kTileColumnList = 1;

constexpr int kSplitCols = 16;       // query columns per split-KV item (MFMA N)
constexpr int kSplitWaves = 4;       // items (wavefronts) per split-KV workgroup
constexpr int kPrefillWaves = 4;     // wavefronts per prefill workgroup (32 columns each)
constexpr int kPrefillCols = 32 * kPrefillWaves;   // query columns per prefill tile
constexpr int kStepKeys = 64;        // kv positions per split-KV loop step
constexpr int kPrefillWgPerCu = 2;   // prefill workgroups resident per CU (LDS-bound)
constexpr int kCusPerXcd = 32;       // compute units of one XCD on gfx950

}  // namespace va

// Plan object (host side).  Defined here so kernels.hip can read the device pointers.
#ifdef __cplusplus
#include <mutex>
#include <string>
#include <vector>

struct va_plan {
  va_params p;
  int32_t num_reqs = 0;
  int32_t g = 1;
  int32_t split_len = 0;
  std::vector<int32_t> q_start, q_end, kv_len;
  std::vector<int32_t> block_table;          // host copy [num_reqs][max_pages_per_req]
  std::vector<int64_t> kv_offset;            // prefix sum of kv_len (gather output rows)
  std::vector<va::SplitItem> items;          // items of more than 16 columns first
  int32_t items_wide = 0;                    // how many items have more than 16 columns
  std::vector<va::Column> cols;
  std::vector<va::CombineRow> combine;
  std::vector<va::PrefillTile> tiles;         // in launch order
  int32_t tiles_whole = 0;                    // the first tiles_whole run on the whole-tile kernel
                                              // (all, or none when there are chunk or
                                              // column-list tiles)
  std::vector<va::PrefillTile> gtiles;        // copies of the column-list tiles in `tiles` (export)
  std::vector<char> is_split;               // per request: rows run as split-KV items
  int64_t pos_bytes = 0;                     // K+V bytes of one position over all KV heads
  mutable va_plan_stats stats{};             // page-level counters filled on first query
  mutable std::once_flag page_counters_once;
  // device copies (one allocation)
  void* dev = nullptr;
  size_t dev_bytes = 0;
  const va::SplitItem* d_items = nullptr;
  const va::Column* d_cols = nullptr;
  const va::CombineRow* d_combine = nullptr;
  const va::PrefillTile* d_tiles = nullptr;
  const int64_t* d_kv_offset = nullptr;
  int device = -1;
  size_t ws_ml_off = 0, ws_acc_off = 0, ws_bytes = 0;
};

namespace va {
void set_error(const std::string& msg);
va_status fail(va_status s, const std::string& msg);
// Device side of plan creation / destruction (kernels.hip).
va_status upload_plan(va_plan* plan);
// Compute units of the current device (256 on an MI355X; fewer in a partition mode), or 0
// when they cannot be queried.
int device_compute_units();
void free_plan_device(va_plan* plan);
bool prefill_kernel_available(const va_params& p);
}  // namespace va
#endif
