// Internal declarations shared by the split-KV kernel, the finish kernel and
// the host entry points of libwise.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "wise.h"

namespace wise {

constexpr int kBlock = WISE_BLOCK;     // tokens per tile / selection block
constexpr int kWavesPerGroup = 4;      // waves per split workgroup (one work item each)
constexpr int kMaxTilesPerItem = 16;   // tiles per work item (long items of large calls: kLongTiles)
constexpr int kMaxCtx = 65536;         // tokens; 2048 blocks, 64 support words
constexpr int kMaxBlocks = kMaxCtx / kBlock;
constexpr int kMaxWords = kMaxBlocks / 32;
constexpr int kMaxItemsPerUnit = 512;  // kMaxBlocks / smallest tiles-per-item (4)
constexpr int kRowError = 0xF;         // row code: bad device data for the row
constexpr int kItemBits = 9;           // item list entry: unit << 9 | item (kMaxItemsPerUnit = 2^9)

// Row code written by the static split kernel (wave of head 0, item 0) or
// the plan kernel and read by the listed split and the finish kernels:
// effective mode in bits 0..3 (kRowError for a bad row), requested mode in
// bits 4..7.
__host__ __device__ inline int encode_row(int eff, int req) { return (eff & 0xF) | ((req & 0xF) << 4); }

// Work decomposition: unit = (row, head); a unit's attended tiles (all causal
// tiles, or the support's tiles in ascending order) are cut into work items of
// tiles_per_item consecutive list entries.  One wave per item slot.
int tiles_per_item(int max_blocks, int64_t units);
constexpr int64_t kSmallLaunchItems = 1024;  // below this many 8-tile items a launch cuts items shorter
constexpr int kMaxFusedItems = 16;            // items (waves) of one fused split + finish workgroup
constexpr int kMaxFusedBlocks = 64;           // blocks of a short fused unit (one per lane in its selection)
constexpr int kWideFusedBlocks = 256;         // blocks of a long fused unit (four per lane in its selection)

// Large launches run longer items: every item leaves a partial (m, l, acc)
// in HBM, and those writes, interleaved with the K/V stream, cost far more
// than their bytes (about 5% of a 4K-8K launch at eight tiles per item).
// Calls with no sparse rows take the length on the host from the causal
// tiles of max_ctx; calls with sparse rows take it in the plan kernel from
// the tiles they really attend, by the same rule.  Launches below the
// threshold keep eight tiles, as the split design prescribes, so that a
// dense row among sparse ones does not set the launch latency.
constexpr int kLongTiles = 32;                 // longest item (stats and list entries stay one per lane)
constexpr int64_t kLongItemMinWaves = 4096;    // waves a launch keeps when its items grow

struct Layout {
  int rows, heads, head_dim, max_ctx, max_blocks, tiles_per_item, items_per_unit;
  size_t off_row_code, off_row_done, off_unit_items, off_n_items, off_item_list, off_part_ml, off_part_acc,
      off_stats, total;
};
// Returns false if the sizes are outside the supported range.
bool make_layout(int rows, int heads, int head_dim, int max_ctx, Layout *L);
// Tiles per item of a static call with no sparse rows (kLongTiles, 16 or
// the layout's own).
int long_tiles_per_item(const Layout &L);

struct SplitParams {
  const void *q, *k, *v;
  int64_t stride_page_b, stride_head_b, stride_token_b;  // bytes
  const int32_t *block_table;
  int64_t bt_stride;
  const int32_t *ctx_len;
  int32_t rows, heads, max_ctx, max_blocks, num_pages, page_shift;
  float qk_scale_log2;  // softmax scale * log2(e)
  int32_t tiles_per_item, items_per_unit, chunk_groups;
  int32_t fused_waves;  // fused split + finish: waves per workgroup (one workgroup per unit)
  int32_t long_items;  // listed calls: the plan kernel may lengthen items to 16 or 32 tiles
  // requested modes
  const uint8_t *row_mode;  // NULL: every row uniform_mode
  int32_t uniform_mode;
  // support state (unused when every row is DENSE); written only by the
  // fused split + finish kernel
  uint32_t *support;
  int32_t slots, layers, layer, words, required;
  const int32_t *slot_of_row;
  wise_tag *tags;
  const int64_t *row_request, *row_position;
  unsigned long long *counters;
  // fused split + finish only: the output, the selection target, and the
  // external LSE of the LSE route ([rows * heads], natural log)
  float *out;
  float eta;
  const float *lse;
  // workspace and optional export
  int32_t *row_code, *unit_items;
  unsigned long long *row_done;
  int32_t *n_items;      // [0] live items in item_list, [1] their tiles per item (calls with sparse rows)
  uint32_t *item_list;   // unit << kItemBits | item
  float2 *part_ml;
  float *part_acc;
  float2 *stats;
  float2 *stats_export;
};

struct FinishParams {
  int32_t rows, heads, head_dim, max_blocks, items_per_unit;
  const int32_t *ctx_len;
  float *out;
  const int32_t *row_code, *unit_items;
  // per row, one atomic word for rows spanning several finish workgroups:
  // workgroups finished (bits 0..15), heads with an error (bits 16..31),
  // blocks newly selected by the row's heads (32..63)
  unsigned long long *row_done;
  const float2 *part_ml;
  const float *part_acc;
  const float2 *stats;
  // support state; support == NULL after a dense-only call
  uint32_t *support;
  int32_t slots, layers, layer, words;
  const int32_t *slot_of_row;
  wise_tag *tags;
  const int64_t *row_request, *row_position;
  float eta;
  unsigned long long *counters;
  // [rows * heads] natural-log LSE of an external dense kernel, or NULL.
  // When set, the finish selects from mass = l_b exp(m_b - lse) and writes
  // no output (the preceding split read K only).
  const float *lse;
};

// Head-union page compaction of one reuse depth (see wise_pages.hip).
struct PageParams {
  int32_t rows, heads, max_ctx, page_shift, num_pages;
  const int32_t *block_table;
  int32_t bt_stride;
  const int32_t *ctx_len;
  const uint8_t *row_mode;  // NULL = every row SPARSE
  const uint32_t *support;
  int32_t slots, layers, layer, words, required;
  const int32_t *slot_of_row;
  const wise_tag *tags;
  const int64_t *row_request, *row_position;
  unsigned long long *counters;
  int32_t *bt_out;
  int32_t bt_out_stride;
  int32_t *ctx_out;
};

// Snapshot (support, tags of listed slots -> records) or restore (records ->
// slots); see wise_state.hip for the record layout.
struct StateParams {
  uint32_t *support;
  wise_tag *tags;
  int32_t slots, layers, heads, words;
  const int32_t *slots_list;  // [count] slot of each record
  int32_t count;
  void *records;
  size_t record_bytes, tags_offset;
  unsigned long long *counters;
};
void state_record_layout(int layers, int heads, int words, size_t *tags_offset, size_t *record_bytes);

// listed = plan kernel + persistent split over the compact item list (calls
// with sparse rows); otherwise the static one-wave-per-item-slot grid.
// k_only = read K only and keep tile stats (static grid, discovery modes).
// fused = static grid of one workgroup per unit that also runs the unit's
// finish (merge, selection, support, row bookkeeping).
// cus = compute units of the current device (sizes the persistent grid);
// ev_begin / ev_end (optional) are stamped with the split kernel's start and stop.
hipError_t launch_split(const SplitParams &p, int dtype, int head_dim, bool listed, bool k_only, bool fused,
                        int cus, hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream);

// The finish is fused into the split kernel, one workgroup per unit whose
// waves split the unit's tiles evenly and leave their partials in LDS, when
// a row's heads fit the 8-bit arrival count kept in the tag's reserved word
// and either
//  * a unit has at most 64 blocks and its items at the layout's length fit
//    the workgroup: up to 4 items at eight tiles each, or up to 16 (8 for
//    fp32 at head_dim 128, whose waves need more than 128 registers) when a
//    small launch cut its items shorter -- the workgroup has as many waves
//    as the unit has items; or
//  * a unit has at most 256 blocks (contexts up to 8K): 8 waves share its
//    tiles when the launch has at least 512 units, 16 in smaller launches
//    (fp32 at head_dim 128: 8) -- except a small call with no support state
//    (plain dense decode), which keeps the static grid: its four-wave
//    workgroups of eight-tile items fill every wave slot of the chip in one
//    round, where 16-wave workgroups (one per CU at this kernel's register
//    count) would take two.
// Returns the waves per workgroup, 0 when the call is not fused.  Decode and
// finish calls take the same decision from the same sizes and from whether
// they were given a support state.
constexpr int64_t kWideFusedMinUnits = 512;
inline int fused_max_items(const Layout &L, int dtype) {
  if (L.tiles_per_item >= 8) return kWavesPerGroup;
  return (dtype == WISE_F32 && L.head_dim == 128) ? 8 : kMaxFusedItems;
}
inline int fused_waves(const Layout &L, int heads, int dtype, bool stateful) {
  if (heads > 255) return 0;
  if (L.max_blocks <= kMaxFusedBlocks && L.items_per_unit <= fused_max_items(L, dtype))
    return L.items_per_unit <= 4 ? 4 : L.items_per_unit <= 8 ? 8 : 16;
  if (L.max_blocks > kWideFusedBlocks) return 0;
  const bool large = static_cast<int64_t>(L.rows) * heads >= kWideFusedMinUnits;
  if (!large && !stateful) return 0;
  return (large || (dtype == WISE_F32 && L.head_dim == 128)) ? 8 : 16;
}
hipError_t launch_finish(const FinishParams &p, hipStream_t stream);
hipError_t launch_compact_pages(const PageParams &p, hipStream_t stream);
hipError_t launch_state_copy(const StateParams &p, bool restore, hipStream_t stream);

}  // namespace wise
