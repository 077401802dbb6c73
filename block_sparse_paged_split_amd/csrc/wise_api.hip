// Host entry points of libwise: argument validation, workspace layout, and
// the launches of the split-KV kernel and the finish kernel on the caller's
// stream.  Nothing is allocated, nothing is synchronised.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "wise_internal.h"

namespace wise {

int tiles_per_item(int max_blocks, int64_t units) {
  // About eight tiles per program, as the split design prescribes.  A launch
  // with few items (a small batch of short rows) cuts them shorter, so that
  // more waves run at once, while a unit stays within one fused workgroup of
  // at most kMaxFusedItems items.
  const int64_t items8 = units * ((max_blocks + 7) / 8);
  if (items8 >= kSmallLaunchItems || max_blocks > kMaxFusedBlocks) return 8;
  int t = 1;
  while (t < 8 && (max_blocks + t - 1) / t > kMaxFusedItems) t <<= 1;
  return t;
}

int long_tiles_per_item(const Layout &L) {
  if (L.tiles_per_item != 8) return L.tiles_per_item;  // a small launch keeps its cut
  const int64_t units = static_cast<int64_t>(L.rows) * L.heads;
  for (int t = kLongTiles; t > 8; t >>= 1)
    if (units * ((L.max_blocks + t - 1) / t) >= kLongItemMinWaves) return t;
  return 8;
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool make_layout(int rows, int heads, int head_dim, int max_ctx, Layout *L) {
  if (rows < 1 || heads < 1 || (head_dim != 64 && head_dim != 128)) return false;
  if (max_ctx < 1 || max_ctx > kMaxCtx) return false;
  if (static_cast<int64_t>(rows) * heads > (int64_t{1} << 22)) return false;
  if (heads > 0x7FFF) return false;  // per-row arrival counts are packed in 16 bits
  L->rows = rows;
  L->heads = heads;
  L->head_dim = head_dim;
  L->max_ctx = max_ctx;
  L->max_blocks = (max_ctx + kBlock - 1) / kBlock;
  L->tiles_per_item = tiles_per_item(L->max_blocks, static_cast<int64_t>(rows) * heads);
  L->items_per_unit = (L->max_blocks + L->tiles_per_item - 1) / L->tiles_per_item;
  if (L->items_per_unit > kMaxItemsPerUnit || L->tiles_per_item > kMaxTilesPerItem) return false;
  const size_t units = static_cast<size_t>(rows) * heads;
  const size_t slots = units * L->items_per_unit;
  size_t off = 0;
  L->off_row_code = off;
  off += align256(sizeof(int32_t) * rows);
  L->off_row_done = off;
  off += align256(sizeof(unsigned long long) * rows);
  L->off_unit_items = off;
  off += align256(sizeof(int32_t) * units);
  L->off_n_items = off;
  off += 256;
  L->off_item_list = off;
  off += align256(sizeof(uint32_t) * slots);
  L->off_part_ml = off;
  off += align256(sizeof(float2) * slots);
  L->off_part_acc = off;
  off += align256(sizeof(float) * slots * head_dim);
  L->off_stats = off;
  off += align256(sizeof(float2) * units * L->max_blocks);
  L->total = off;
  // the split grid (units x item groups) must fit one launch dimension
  const int64_t groups = (L->items_per_unit + kWavesPerGroup - 1) / kWavesPerGroup;
  if (static_cast<int64_t>(units) * groups > INT32_MAX) return false;
  return true;
}

}  // namespace wise

using namespace wise;

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// k_only: the call reads q and K only (LSE route); v_cache and out may be NULL.
wise_status check_attn(const wise_attn *a, Layout *L, bool k_only = false) {
  if (!a) return WISE_E_ARG;
  if (a->dtype != WISE_BF16 && a->dtype != WISE_F32) return WISE_E_UNSUPPORTED;
  if (a->head_dim != 64 && a->head_dim != 128) return WISE_E_UNSUPPORTED;
  if (a->rows < 1 || a->heads < 1 || a->max_ctx < 1 || a->num_pages < 1) return WISE_E_ARG;
  if (!is_pow2(a->page_size) || a->page_size < 8 || a->page_size > 4096) return WISE_E_UNSUPPORTED;
  if (a->max_ctx > kMaxCtx) return WISE_E_UNSUPPORTED;
  if (!a->q || !a->k_cache || !a->block_table || !a->ctx_len) return WISE_E_ARG;
  if (!k_only && (!a->v_cache || !a->out)) return WISE_E_ARG;
  if (!aligned(a->q, 16) || !aligned(a->k_cache, 16) || (a->v_cache && !aligned(a->v_cache, 16)) ||
      (a->out && !aligned(a->out, 16)))
    return WISE_E_ARG;
  if (a->tile_stats && !aligned(a->tile_stats, 8)) return WISE_E_ARG;
  const int64_t e = a->dtype == WISE_BF16 ? 2 : 4;
  if (a->stride_page <= 0 || a->stride_head <= 0 || a->stride_token <= 0) return WISE_E_ARG;
  if ((a->stride_page * e) % 16 || (a->stride_head * e) % 16 || (a->stride_token * e) % 16) return WISE_E_ARG;
  if (a->stride_token * e * 8 > INT32_MAX / 2) return WISE_E_UNSUPPORTED;
  if (a->stride_token < a->head_dim) return WISE_E_ARG;
  const int64_t need_bt = (static_cast<int64_t>(a->max_ctx) + a->page_size - 1) / a->page_size;
  if (a->bt_stride < need_bt) return WISE_E_ARG;
  if (!std::isfinite(a->scale) || a->scale < 0.0f) return WISE_E_ARG;
  if ((a->ev_split_begin == nullptr) != (a->ev_split_end == nullptr)) return WISE_E_ARG;
  if (!make_layout(a->rows, a->heads, a->head_dim, a->max_ctx, L)) return WISE_E_UNSUPPORTED;
  return WISE_OK;
}

wise_status check_support(const wise_attn *a, const wise_support *s, const Layout &L) {
  if (!s) return WISE_E_ARG;
  if (!s->support || !s->tags || !s->row_request || !s->row_position) return WISE_E_ARG;
  if (s->slots < 1 || s->layers < 1 || s->layer < 0 || s->layer >= s->layers) return WISE_E_ARG;
  if (s->words < (L.max_blocks + 31) / 32) return WISE_E_ARG;
  if (s->discoveries_required < 1) return WISE_E_ARG;
  if (!(s->eta > 0.0f && s->eta <= 1.0f)) return WISE_E_ARG;
  if (!aligned(s->support, 4) || !aligned(s->tags, 8) || (s->counters && !aligned(s->counters, 8)))
    return WISE_E_ARG;
  (void)a;
  return WISE_OK;
}

wise_status check_ws(void *ws, size_t ws_bytes, const Layout &L) {
  if (!ws || !aligned(ws, 256)) return WISE_E_WORKSPACE;
  if (ws_bytes < L.total) return WISE_E_WORKSPACE;
  return WISE_OK;
}

float qk_scale_log2(const wise_attn *a) {
  const double sc = a->scale > 0.0f ? static_cast<double>(a->scale) : 1.0 / std::sqrt(static_cast<double>(a->head_dim));
  return static_cast<float>(sc * 1.4426950408889634074);  // log2(e)
}

// Compute units of the current device (cached per device; the only state
// the library keeps).
int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    cache[dev] = n;
  }
  return cache[dev];
}

int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

wise_status decode(const wise_attn *a, const wise_support *s, int uniform_mode, const uint8_t *row_mode,
                   void *ws, size_t ws_bytes, void *stream, const float *lse = nullptr) {
  const bool k_only = lse != nullptr;  // the LSE route reads K only
  Layout L;
  wise_status st = check_attn(a, &L, k_only);
  if (st != WISE_OK) return st;
  const bool stateful = uniform_mode != WISE_DENSE || row_mode != nullptr;
  if (stateful) {
    st = check_support(a, s, L);
    if (st != WISE_OK) return st;
  }
  st = check_ws(ws, ws_bytes, L);
  if (st != WISE_OK) return st;

  const int64_t e = a->dtype == WISE_BF16 ? 2 : 4;
  char *w = static_cast<char *>(ws);
  SplitParams p{};
  p.q = a->q;
  p.k = a->k_cache;
  p.v = a->v_cache;
  p.stride_page_b = a->stride_page * e;
  p.stride_head_b = a->stride_head * e;
  p.stride_token_b = a->stride_token * e;
  p.block_table = a->block_table;
  p.bt_stride = a->bt_stride;
  p.ctx_len = a->ctx_len;
  p.rows = a->rows;
  p.heads = a->heads;
  p.max_ctx = a->max_ctx;
  p.max_blocks = L.max_blocks;
  p.num_pages = a->num_pages;
  p.page_shift = log2i(a->page_size);
  p.qk_scale_log2 = qk_scale_log2(a);
  p.tiles_per_item = L.tiles_per_item;
  p.items_per_unit = L.items_per_unit;
  p.chunk_groups = (L.items_per_unit + kWavesPerGroup - 1) / kWavesPerGroup;
  p.row_mode = row_mode;
  p.uniform_mode = uniform_mode;
  if (stateful) {
    p.support = s->support;
    p.slots = s->slots;
    p.layers = s->layers;
    p.layer = s->layer;
    p.words = s->words;
    p.required = s->discoveries_required;
    p.slot_of_row = s->slot_of_row;
    p.tags = s->tags;
    p.row_request = s->row_request;
    p.row_position = s->row_position;
    p.counters = reinterpret_cast<unsigned long long *>(s->counters);
    p.eta = s->eta;
  }
  p.out = a->out;
  p.row_code = reinterpret_cast<int32_t *>(w + L.off_row_code);
  p.row_done = reinterpret_cast<unsigned long long *>(w + L.off_row_done);
  p.unit_items = reinterpret_cast<int32_t *>(w + L.off_unit_items);
  p.n_items = reinterpret_cast<int32_t *>(w + L.off_n_items);
  p.item_list = reinterpret_cast<uint32_t *>(w + L.off_item_list);
  p.part_ml = reinterpret_cast<float2 *>(w + L.off_part_ml);
  p.part_acc = reinterpret_cast<float *>(w + L.off_part_acc);
  p.stats = reinterpret_cast<float2 *>(w + L.off_stats);
  p.stats_export = reinterpret_cast<float2 *>(a->tile_stats);

  hipStream_t strm = static_cast<hipStream_t>(stream);
  // Rows that may be sparse make item counts data-dependent.  When a unit
  // spans several split workgroups, plan first and run the persistent split
  // over the compact item list; otherwise the static grid has one workgroup
  // per unit and no empty slots worth removing.
  // units that fit one split workgroup are also finished by it (the paired
  // wise_finish_select then has nothing left to do)
  p.fused_waves = fused_waves(L, a->heads, a->dtype, stateful);
  const bool fused = p.fused_waves > 0;
  p.lse = lse;
  const bool listed = !fused && (row_mode != nullptr || uniform_mode == WISE_SPARSE) && p.chunk_groups > 1;
  // a static call with no sparse rows: longer items for large launches (the
  // finish merges unit_items[u] partials at the workspace's slot stride)
  if (!fused && !listed && row_mode == nullptr && uniform_mode != WISE_SPARSE) {
    p.tiles_per_item = long_tiles_per_item(L);
    const int items = (L.max_blocks + p.tiles_per_item - 1) / p.tiles_per_item;
    p.chunk_groups = (items + kWavesPerGroup - 1) / kWavesPerGroup;
  }
  // a listed call's plan kernel may lengthen the items by the same rule,
  // from the tiles the call really attends
  p.long_items = listed && L.tiles_per_item == 8;
  const int cus = listed ? compute_units() : 0;
  if (listed && cus <= 0) return WISE_E_HIP;
  if (launch_split(p, a->dtype, a->head_dim, listed, k_only, fused, cus,
                   static_cast<hipEvent_t>(a->ev_split_begin), static_cast<hipEvent_t>(a->ev_split_end),
                   strm) != hipSuccess)
    return WISE_E_HIP;
  return WISE_OK;
}

wise_status finish(const wise_attn *a, const wise_support *s, const float *lse, void *ws, size_t ws_bytes,
                   void *stream) {
  Layout L;
  wise_status st = check_attn(a, &L, lse != nullptr);
  if (st != WISE_OK) return st;
  if (s) {
    st = check_support(a, s, L);
    if (st != WISE_OK) return st;
  }
  st = check_ws(ws, ws_bytes, L);
  if (st != WISE_OK) return st;
  // the decode call already finished these units (see decode())
  if (fused_waves(L, a->heads, a->dtype, s != nullptr) > 0) return WISE_OK;
  char *w = static_cast<char *>(ws);
  FinishParams p{};
  p.rows = a->rows;
  p.heads = a->heads;
  p.head_dim = a->head_dim;
  p.max_blocks = L.max_blocks;
  p.items_per_unit = L.items_per_unit;
  p.ctx_len = a->ctx_len;
  p.out = a->out;
  p.row_code = reinterpret_cast<const int32_t *>(w + L.off_row_code);
  p.row_done = reinterpret_cast<unsigned long long *>(w + L.off_row_done);
  p.unit_items = reinterpret_cast<const int32_t *>(w + L.off_unit_items);
  p.part_ml = reinterpret_cast<const float2 *>(w + L.off_part_ml);
  p.part_acc = reinterpret_cast<const float *>(w + L.off_part_acc);
  p.stats = reinterpret_cast<const float2 *>(w + L.off_stats);
  if (s) {
    p.support = s->support;
    p.slots = s->slots;
    p.layers = s->layers;
    p.layer = s->layer;
    p.words = s->words;
    p.slot_of_row = s->slot_of_row;
    p.tags = s->tags;
    p.row_request = s->row_request;
    p.row_position = s->row_position;
    p.eta = s->eta;
    p.counters = reinterpret_cast<unsigned long long *>(s->counters);
  }
  p.lse = lse;
  if (launch_finish(p, static_cast<hipStream_t>(stream)) != hipSuccess) return WISE_E_HIP;
  return WISE_OK;
}

// ---------------------------------------------------------------------------
// The library's own workspace, for callers that cannot allocate one.
// ---------------------------------------------------------------------------

// One copy per GPU, reserved when the library's code is loaded on that GPU
// and held until the process ends.  In host code this name is only a
// stand-in for the symbol, never a device address: the address of the
// current device's copy comes from hipGetSymbolAddress (once per device) and
// is the only one host code hands to kernels.  Nothing in it needs to start
// at zero: every call's kernels write what they later read.
__device__ __align__(256) unsigned char scratch[WISE_SCRATCH_BYTES];

std::mutex scratch_mutex;
void *scratch_address[64] = {nullptr};

// Device address of the current device's scratch copy, looked up on the
// first call on each device; NULL if the lookup fails.
void *device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_address[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_address[dev] = ptr;
  }
  return scratch_address[dev];
}

}  // namespace

extern "C" {

size_t wise_workspace_size(int32_t rows, int32_t heads, int32_t head_dim, int32_t max_ctx) {
  Layout L;
  return make_layout(rows, heads, head_dim, max_ctx, &L) ? L.total : 0;
}

int32_t wise_fused_waves(int32_t rows, int32_t heads, int32_t head_dim, int32_t max_ctx, int32_t dtype,
                         int32_t stateful) {
  Layout L;
  if ((dtype != WISE_BF16 && dtype != WISE_F32) || !make_layout(rows, heads, head_dim, max_ctx, &L)) return -1;
  return fused_waves(L, heads, dtype, stateful != 0);
}

wise_status wise_decode_dense(const wise_attn *a, void *ws, size_t ws_bytes, void *stream) {
  return decode(a, nullptr, WISE_DENSE, nullptr, ws, ws_bytes, stream);
}

wise_status wise_decode_discover(const wise_attn *a, const wise_support *s, int32_t union_with_previous,
                                 void *ws, size_t ws_bytes, void *stream) {
  return decode(a, s, union_with_previous ? WISE_DISCOVER_UNION : WISE_DISCOVER, nullptr, ws, ws_bytes,
                stream);
}

wise_status wise_decode_sparse(const wise_attn *a, const wise_support *s, const uint8_t *row_mode, void *ws,
                               size_t ws_bytes, void *stream) {
  return decode(a, s, WISE_SPARSE, row_mode, ws, ws_bytes, stream);
}

wise_status wise_finish_select(const wise_attn *a, const wise_support *s, void *ws, size_t ws_bytes,
                               void *stream) {
  return finish(a, s, nullptr, ws, ws_bytes, stream);
}

wise_status wise_discover_lse(const wise_attn *a, const wise_support *s, int32_t union_with_previous,
                              const float *lse, void *ws, size_t ws_bytes, void *stream) {
  if (!s || !lse || !aligned(lse, 4)) return WISE_E_ARG;
  // validate everything before the first launch, so an error enqueues nothing
  Layout L;
  wise_status st = check_attn(a, &L, true);
  if (st == WISE_OK) st = check_support(a, s, L);
  if (st == WISE_OK) st = check_ws(ws, ws_bytes, L);
  if (st != WISE_OK) return st;
  st = decode(a, s, union_with_previous ? WISE_DISCOVER_UNION : WISE_DISCOVER, nullptr, ws, ws_bytes, stream,
              lse);
  if (st != WISE_OK) return st;
  return finish(a, s, lse, ws, ws_bytes, stream);
}

wise_status wise_compact_pages(const wise_attn *a, const wise_support *s, const uint8_t *row_mode,
                               int32_t *bt_out, int32_t bt_out_stride, int32_t *ctx_out, void *stream) {
  Layout L;
  wise_status st = check_attn(a, &L, true);
  if (st != WISE_OK) return st;
  st = check_support(a, s, L);
  if (st != WISE_OK) return st;
  if (!bt_out || !ctx_out || !aligned(bt_out, 4) || !aligned(ctx_out, 4)) return WISE_E_ARG;
  if (bt_out == a->block_table || ctx_out == a->ctx_len) return WISE_E_ARG;  // not in place
  const int64_t need = (static_cast<int64_t>(a->max_ctx) + a->page_size - 1) / a->page_size;
  if (bt_out_stride < need) return WISE_E_ARG;
  PageParams p{};
  p.rows = a->rows;
  p.heads = a->heads;
  p.max_ctx = a->max_ctx;
  p.page_shift = log2i(a->page_size);
  p.num_pages = a->num_pages;
  p.block_table = a->block_table;
  p.bt_stride = a->bt_stride;
  p.ctx_len = a->ctx_len;
  p.row_mode = row_mode;
  p.support = s->support;
  p.slots = s->slots;
  p.layers = s->layers;
  p.layer = s->layer;
  p.words = s->words;
  p.required = s->discoveries_required;
  p.slot_of_row = s->slot_of_row;
  p.tags = s->tags;
  p.row_request = s->row_request;
  p.row_position = s->row_position;
  p.counters = reinterpret_cast<unsigned long long *>(s->counters);
  p.bt_out = bt_out;
  p.bt_out_stride = bt_out_stride;
  p.ctx_out = ctx_out;
  if (launch_compact_pages(p, static_cast<hipStream_t>(stream)) != hipSuccess) return WISE_E_HIP;
  return WISE_OK;
}

wise_status wise_decode_sparse_noalloc(const wise_attn *a, const wise_support *s, const uint8_t *row_mode,
                                       void *stream) {
  // every host check, the size limit included, before the device is touched
  Layout L;
  wise_status st = check_attn(a, &L);
  if (st == WISE_OK) st = check_support(a, s, L);
  if (st != WISE_OK) return st;
  if (L.total > static_cast<size_t>(WISE_SCRATCH_BYTES)) return WISE_E_WORKSPACE;
  void *ws = device_scratch();
  if (ws == nullptr) return WISE_E_HIP;
  st = decode(a, s, WISE_SPARSE, row_mode, ws, L.total, stream);
  if (st != WISE_OK) return st;
  return finish(a, s, nullptr, ws, L.total, stream);
}

size_t wise_snapshot_bytes(int32_t layers, int32_t heads, int32_t words) {
  if (layers < 1 || heads < 1 || words < 1) return 0;
  size_t off = 0, bytes = 0;
  state_record_layout(layers, heads, words, &off, &bytes);
  return bytes;
}

static wise_status state_copy(const wise_support *s, int32_t heads, const int32_t *slots, int32_t count,
                              void *records, size_t bytes, bool restore, void *stream) {
  if (!s || !s->support || !s->tags || !slots || !records) return WISE_E_ARG;
  if (s->slots < 1 || s->layers < 1 || s->words < 1 || heads < 1 || count < 0) return WISE_E_ARG;
  if (!aligned(s->support, 4) || !aligned(s->tags, 8) || !aligned(slots, 4) || !aligned(records, 8) ||
      (s->counters && !aligned(s->counters, 8)))
    return WISE_E_ARG;
  StateParams p{};
  state_record_layout(s->layers, heads, s->words, &p.tags_offset, &p.record_bytes);
  if (bytes < p.record_bytes * static_cast<size_t>(count)) return WISE_E_ARG;
  if (count == 0) return WISE_OK;
  p.support = s->support;
  p.tags = s->tags;
  p.slots = s->slots;
  p.layers = s->layers;
  p.heads = heads;
  p.words = s->words;
  p.slots_list = slots;
  p.count = count;
  p.records = records;
  p.counters = reinterpret_cast<unsigned long long *>(s->counters);
  if (launch_state_copy(p, restore, static_cast<hipStream_t>(stream)) != hipSuccess) return WISE_E_HIP;
  return WISE_OK;
}

wise_status wise_support_snapshot(const wise_support *s, int32_t heads, const int32_t *slots, int32_t count,
                                  void *dst, size_t dst_bytes, void *stream) {
  return state_copy(s, heads, slots, count, dst, dst_bytes, false, stream);
}

wise_status wise_support_restore(const wise_support *s, int32_t heads, const int32_t *slots, int32_t count,
                                 const void *src, size_t src_bytes, void *stream) {
  return state_copy(s, heads, slots, count, const_cast<void *>(src), src_bytes, true, stream);
}

const char *wise_status_string(wise_status st) {
  switch (st) {
    case WISE_OK: return "ok";
    case WISE_E_ARG: return "invalid argument";
    case WISE_E_UNSUPPORTED: return "unsupported size, dtype or layout";
    case WISE_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case WISE_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

}  // extern "C"
