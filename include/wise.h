/*
 * wise.h -- C ABI of working-set (WISE) paged decode attention for
 * recurrent-depth models, on AMD Instinct MI355X (gfx950).
 *
 * Method (WISE pull request page, InferMatrixLab/vllm-rlt pull 143,
 * "Summary" and "What changes"): the early recurrent depths run dense
 * split-KV decode attention over a paged KV cache and record, for every
 * 32-token tile, the softmax max and sum; a finish step merges the splits
 * and, for discovery rows, selects per (row, layer, head) the support: the
 * fewest tiles, heaviest first, whose softmax mass reaches eta (0.95 by
 * default), ORed across discovery depths.  Later depths attend only the
 * selected tiles, with Q/K/V and the softmax weights inside the support
 * recomputed.  Support lives in a [slot, layer, head, block] bitmask that
 * is tagged with the (request, position) it was discovered for; a row whose
 * discovery is missing or incomplete attends densely and is counted as a
 * fallback.
 *
 * Call sequence per (depth, layer):
 *     wise_decode_dense | wise_decode_discover | wise_decode_sparse
 *     wise_finish_select            (same workspace, same stream, next)
 * The decode call runs the split-KV kernel (one launch, every row mode);
 * the finish call merges the splits into `out`, runs the eta selection for
 * discovery rows, updates the bitmask, the tags and the counters.  For
 * contexts up to 8K (wise_fused_waves() > 0) the decode call's one kernel
 * already does all of that, and the finish call only validates.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller; they are
 *     borrowed until the enqueued work completes.  Scalars are host values.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is only
 *     enqueued; nothing is synchronised, nothing is allocated, no host
 *     state is kept, so calls are re-entrant and capturable in HIP graphs.
 *   - Host-checkable arguments are validated before anything is enqueued;
 *     on any error nothing is enqueued and the status says why.
 *   - Device data that cannot be checked without a sync (a context length
 *     outside [1, max_ctx], a page id outside [0, num_pages), a slot id
 *     outside [0, slots), a row mode outside the enum, an empty support)
 *     makes the affected (row, head) output NaN; wise_finish_select adds
 *     one to counters[WISE_CTR_ERRORS] per such (row, head).
 *   - Two calls that share a workspace must be ordered (same stream).
 *     Rows of one call must map to distinct slots.
 */
#ifndef WISE_H
#define WISE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tokens per tile and per selection block (the method's B = 32). */
#define WISE_BLOCK 32

typedef enum wise_status {
  WISE_OK = 0,
  WISE_E_ARG = 1,          /* a null required pointer or an out-of-range scalar */
  WISE_E_UNSUPPORTED = 2,  /* head_dim, dtype, page_size or a size limit not supported */
  WISE_E_WORKSPACE = 3,    /* ws is NULL/misaligned or ws_bytes < wise_workspace_size() */
  WISE_E_HIP = 4           /* a HIP launch or event call failed */
} wise_status;

/* Requested per-row mode (a uint8 per row in wise_decode_sparse's row_mode). */
typedef enum wise_mode {
  WISE_DENSE = 0,           /* plain paged decode attention, no state touched */
  WISE_DISCOVER = 1,        /* dense + tile stats; selection replaces the support */
  WISE_DISCOVER_UNION = 2,  /* dense + tile stats; selection is ORed into the support */
  WISE_SPARSE = 3           /* attend only the support's tiles */
} wise_mode;

typedef enum wise_dtype { WISE_BF16 = 0, WISE_F32 = 1 } wise_dtype;

/* Indices into the counters array (uint64 each, accumulated, never reset). */
enum {
  WISE_CTR_FALLBACKS = 0,   /* rows that requested UNION/SPARSE and ran dense */
  WISE_CTR_SELECTED = 1,    /* union blocks: DISCOVER adds K, UNION adds newly set bits */
  WISE_CTR_CAUSAL = 2,      /* causal blocks of DISCOVER units */
  WISE_CTR_ERRORS = 3,      /* (row, head) units whose output was set to NaN */
  WISE_NUM_COUNTERS = 4
};

/*
 * Support tag of one (slot, layer): the discovery window the support words
 * of that (slot, layer) hold.  discoveries = 0 means released / invalid.
 * A DISCOVER row sets {request, position, 1}; a DISCOVER_UNION row needs
 * {request, position} to match with discoveries >= 1 and adds one; a
 * SPARSE row needs them to match with discoveries >= discoveries_required.
 * A DISCOVER_UNION row whose window is broken runs dense and sets
 * discoveries = 0, so the rest of that token runs dense too.
 * reserved: a per-call arrival count of the library; it must be 0 whenever
 * no call is in flight (zero-initialise the tags), and every call leaves it
 * at 0.
 */
typedef struct wise_tag {
  int64_t request;
  int64_t position;
  int32_t discoveries;
  int32_t reserved;
} wise_tag; /* 24 bytes */

/*
 * Attention operands of one (depth, layer) call.
 *   q         [rows, heads, head_dim], contiguous, dtype.
 *   k_cache,  element (page, head, slot, dim) at
 *   v_cache     page*stride_page + head*stride_head + slot*stride_token + dim
 *             (element strides; dim is contiguous).  [pages, heads, P, d] has
 *             strides (heads*P*d, P*d, d); [pages, P, heads, d] has
 *             (P*heads*d, d, heads*d).  Pointers and every stride in bytes
 *             must be multiples of 16.
 *   block_table [rows, bt_stride] int32: logical page j of row r is physical
 *             page block_table[r*bt_stride + j]; bt_stride >= ceil(max_ctx/P).
 *             Only entries below ceil(ctx_len[r]/P) are read.
 *   ctx_len   [rows] int32, tokens attended (including the current one).
 *   max_ctx   host bound on ctx_len, sizes the grid and the workspace.
 *   scale     softmax scale; 0 selects 1/sqrt(head_dim).
 *   out       [rows, heads, head_dim] fp32, written by wise_finish_select.
 *   tile_stats optional [rows, heads, ceil(max_ctx/32), 2] fp32: for every
 *             tile a row attends, (max scaled score, sum exp(score - max))
 *             in natural-log units; other entries are left untouched.
 *   ev_split_begin/end optional hipEvent_t (timing hook), or NULL: stamped
 *             with the split-KV kernel's own start and stop by the launch
 *             (hipExtLaunchKernel), so their elapsed time is the kernel's
 *             duration.  Both or neither.
 * Supported: head_dim 64 or 128; page_size a power of two in [8, 4096];
 * max_ctx <= 65536; rows*heads <= 2^22.
 */
typedef struct wise_attn {
  int32_t rows, heads, head_dim, dtype;
  const void *q;
  const void *k_cache, *v_cache;
  int64_t stride_page, stride_head, stride_token;
  int32_t num_pages, page_size;
  const int32_t *block_table;
  int32_t bt_stride;
  const int32_t *ctx_len;
  int32_t max_ctx;
  float scale;
  float *out;
  float *tile_stats;
  void *ev_split_begin, *ev_split_end;
} wise_attn;

/*
 * Support state (the pages' WiseState) and the per-call selection inputs.
 *   support   [slots, layers, heads, words] uint32; bit b of a (slot, layer,
 *             head) is bit (b % 32) of word (b / 32).
 *             words >= ceil(ceil(max_ctx/32)/32).
 *   layer     the layer of this call, in [0, layers).
 *   slot_of_row [rows] int32 or NULL (row r uses slot r).
 *   tags      [slots, layers] wise_tag.
 *   row_request, row_position [rows] int64: the token each row decodes.
 *   discoveries_required  discovery depths a SPARSE row needs (>= 1).
 *   eta       cumulative-mass target in (0, 1].
 *   counters  [WISE_NUM_COUNTERS] uint64 or NULL.
 */
typedef struct wise_support {
  uint32_t *support;
  int32_t slots, layers, words, layer;
  const int32_t *slot_of_row;
  wise_tag *tags;
  const int64_t *row_request, *row_position;
  int32_t discoveries_required;
  float eta;
  uint64_t *counters;
} wise_support;

/* Bytes of workspace a call with these sizes needs (0 if unsupported).
 * The workspace holds the split partials and tile statistics the finish
 * step merges ("What changes", first bullet: the split kernel's partials
 * and a finish step over them). */
size_t wise_workspace_size(int32_t rows, int32_t heads, int32_t head_dim, int32_t max_ctx);

/* How a call of these sizes is launched ("What changes", first bullet: the
 * split kernel and the finish step over its partials).  Returns the waves per
 * workgroup of the one-launch kernel, which gives each (row, head) one
 * workgroup whose waves split the unit's attended tiles evenly and then run
 * the merge, the selection and the bookkeeping themselves (wise_finish_select
 * then only validates); 0 when the call runs the split grid followed by the
 * finish kernel; -1 for sizes or a dtype the library does not support.
 * stateful != 0 for calls given a support state (every call except a
 * wise_decode_dense without one).  A host-side query: it enqueues nothing
 * and touches no device. */
int32_t wise_fused_waves(int32_t rows, int32_t heads, int32_t head_dim, int32_t max_ctx, int32_t dtype,
                         int32_t stateful);

/* Every row DENSE ("What changes", first bullet: the dense row mode of the
 * split-KV paged decode).  No support state is read or written.  Follow
 * with wise_finish_select(a, NULL, ...). */
wise_status wise_decode_dense(const wise_attn *a, void *ws, size_t ws_bytes, void *stream);

/* Every row DISCOVER (union_with_previous == 0) or DISCOVER_UNION (!= 0)
 * ("What changes", first bullet: the discover row mode; "Summary": the
 * discovery depths; review thread and the author's reply: the second
 * discovery depth ORs into the first): dense attention that also records
 * every tile's (max, sum).  Follow with wise_finish_select(a, s, ...), which
 * selects and updates the state. */
wise_status wise_decode_discover(const wise_attn *a, const wise_support *s,
                                 int32_t union_with_previous, void *ws, size_t ws_bytes,
                                 void *stream);

/* Every row SPARSE (row_mode == NULL), or per-row modes from the device
 * array row_mode [rows] uint8 (one launch mixes dense, discover, union and
 * sparse rows) ("What changes", first bullet: the sparse row mode over a
 * compacted tile list, and one launch of rows in different modes; third
 * bullet: a row without a complete discovery for its token runs dense and
 * is counted).  Sparse rows walk only the tiles of their support, whose
 * list is compacted before the loop.  Follow with wise_finish_select(a, s). */
wise_status wise_decode_sparse(const wise_attn *a, const wise_support *s,
                               const uint8_t *row_mode, void *ws, size_t ws_bytes,
                               void *stream);

/* Merge the splits of the preceding decode call into a->out; for discovery
 * rows run the eta selection, write/OR the support, update the tags and
 * the counters ("What changes", first bullet: the finish kernel; "Summary":
 * B = 32 blocks and the eta = 0.95 rule; the author's reply on density: the
 * selected and causal block counts).  `a` and `s` must describe the same call as the decode
 * call (s == NULL after wise_decode_dense).  When the decode call gives each
 * (row, head) one workgroup, it has already done all of this in the same
 * kernel, and this call only validates its arguments (wise_fused_waves()
 * > 0): with heads <= 255, every call with max_ctx <= 8192, except plain
 * dense calls (s == NULL) of fewer than 512 (row, head) pairs with max_ctx >
 * 1024 (or > 2048 for small launches of short rows).  It is still required:
 * which shapes finish inside the decode kernel is the library's choice and
 * may change. */
wise_status wise_finish_select(const wise_attn *a, const wise_support *s, void *ws,
                               size_t ws_bytes, void *stream);

/*
 * Discovery after an external dense decode (WISE pull request page, "What
 * changes", second bullet: the FlashAttention route rereads K once to
 * rebuild block mass from the kernel's LSE).  Every row DISCOVER
 * (union_with_previous == 0) or DISCOVER_UNION (!= 0), with the tag rules
 * of wise_decode_discover.  One call does both steps: a split-KV pass that
 * reads q and K only and records every tile's (max, sum), then the
 * selection, with block mass m_b -> l_b * exp(m_b - lse) instead of the
 * merged (M, L); support, tags and counters are updated as by
 * wise_finish_select (one kernel when the finish fuses into the split, see
 * wise_finish_select; two otherwise).  No attention output is written: a->v_cache and
 * a->out are not read and may be NULL; a->tile_stats is honoured.
 *   lse  [rows, heads] fp32 device array: log(sum_t exp(scale * q.k_t))
 *        over the row's ctx_len tokens, natural log (what FlashAttention's
 *        decode reports as softmax LSE).  A non-finite entry is a data
 *        error of its (row, head): counted in counters[WISE_CTR_ERRORS], the
 *        row's discovery window is broken (tag discoveries = 0).
 * Errors as for the other calls; lse == NULL or s == NULL is WISE_E_ARG.
 * Uses the workspace like a decode + finish pair.
 */
wise_status wise_discover_lse(const wise_attn *a, const wise_support *s,
                              int32_t union_with_previous, const float *lse, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * Head-union, page-granular support through a compacted page table (WISE
 * pull request page, "What changes", second bullet: on the FlashAttention
 * route a sparse row attends the per-layer head union of its support at
 * page granularity through a compacted page table).  For every row:
 *   SPARSE (row_mode == NULL, or row_mode[r] == WISE_SPARSE) whose tag admits
 *     reuse (as wise_decode_sparse): page j of the row is kept when one of
 *     its valid tokens lies in a block set for ANY head of the (slot, layer)
 *     support; bt_out[r] lists the kept pages' physical ids in logical order
 *     and ctx_out[r] the tokens they hold ((kept - 1) * page_size + the
 *     valid tokens of the last kept page);
 *   SPARSE whose tag does not admit reuse: every page (a dense fallback,
 *     counted in counters[WISE_CTR_FALLBACKS]);
 *   DENSE: every page.
 * Every head of a row then attends the same tokens: run any paged dense
 * decode over (bt_out, ctx_out), e.g. wise_decode_dense with a copy of `a`
 * whose block_table, bt_stride and ctx_len are bt_out, bt_out_stride and
 * ctx_out, followed by wise_finish_select(copy, NULL).
 *   bt_out   [rows, bt_out_stride] int32 device array, bt_out_stride >=
 *            ceil(max_ctx / page_size); entries past a row's compacted
 *            pages are left untouched.  Must not be a->block_table.
 *   ctx_out  [rows] int32 device array; must not be a->ctx_len.
 * Data errors -- another row mode, a context outside [1, max_ctx], a slot
 * out of range, an empty head union, a kept page id outside
 * [0, num_pages) -- give ctx_out = 0 (the attention call then writes NaN
 * for the row) and add heads to counters[WISE_CTR_ERRORS].  `a` describes
 * the attention call (q, k_cache, block_table, ctx_len, num_pages, sizes);
 * v_cache and out are not read.
 * Enqueues one kernel; no workspace.
 */
wise_status wise_compact_pages(const wise_attn *a, const wise_support *s,
                               const uint8_t *row_mode, int32_t *bt_out,
                               int32_t bt_out_stride, int32_t *ctx_out, void *stream);

/*
 * Support/tag snapshot and restore across a KV offload (WISE pull request
 * page, review finding "Preserve WISE state across KV offload": freeing a
 * request for offload after its discovery depths loses its support and
 * tags; the finding asks to snapshot and restore them with the recurrent
 * state).  A record holds one slot's support words of every layer and head
 * and its tag of every layer; a restored tag names the same (request,
 * position), so a request resumed at the same token continues its sparse
 * reuse instead of falling back to dense.
 *
 * wise_snapshot_bytes: bytes of one record (0 if an argument is < 1).
 *   Layout: [layers][heads][words] uint32 support words, padded to a
 *   multiple of 8 bytes, then [layers] wise_tag.
 * wise_support_snapshot: record i <- slot slots[i] (i < count).  A slot
 *   outside [0, s->slots) yields an all-zero record (restoring it makes the
 *   slot's reuse fall back).
 * wise_support_restore: slot slots[i] <- record i.  A slot outside
 *   [0, s->slots) is skipped and counted in s->counters[WISE_CTR_ERRORS].
 *   Destination slots must be distinct and must not be read or written by
 *   other work in flight.
 *   s         support state: support, tags, slots, layers, words, counters
 *             (the other fields are not read).
 *   heads     heads per (slot, layer) of the support array.
 *   slots     [count] int32 device array; count >= 0 (0 enqueues nothing).
 *   dst/src   device (or device-accessible pinned host) buffer of
 *             dst_bytes/src_bytes >= count * wise_snapshot_bytes(...),
 *             8-byte aligned, caller-owned.
 * WISE_E_ARG for a null or misaligned pointer, sizes < 1, or a buffer too
 * small.  One kernel launch each; nothing allocated, nothing synchronised.
 */
size_t wise_snapshot_bytes(int32_t layers, int32_t heads, int32_t words);
wise_status wise_support_snapshot(const wise_support *s, int32_t heads, const int32_t *slots,
                                  int32_t count, void *dst, size_t dst_bytes, void *stream);
wise_status wise_support_restore(const wise_support *s, int32_t heads, const int32_t *slots,
                                 int32_t count, const void *src, size_t src_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): one whole
 * (depth, layer) call -- exactly wise_decode_sparse(a, s, row_mode, ...)
 * followed by wise_finish_select(a, s, ...), same kernels, same results --
 * whose workspace is the library's own device buffer of
 * WISE_SCRATCH_BYTES instead of a caller workspace.  Nothing is allocated:
 * each GPU the library is loaded on holds one such buffer until the process
 * ends.  Every call on a GPU uses that GPU's buffer, which keeps the last
 * call's contents; calls that overlap on one GPU (other streams, other host
 * threads) race on it and must be ordered by the caller.  Calls whose
 * wise_workspace_size(rows, heads, head_dim, max_ctx) exceeds
 * WISE_SCRATCH_BYTES return WISE_E_WORKSPACE before anything is enqueued
 * (e.g. 64 rows x 16 heads x 8K tokens at head_dim 128 fit; 128 rows x 16
 * heads x 32K do not).  Other errors as for the two calls it replaces.
 */
#define WISE_SCRATCH_BYTES ((size_t)32 << 20)
wise_status wise_decode_sparse_noalloc(const wise_attn *a, const wise_support *s,
                                       const uint8_t *row_mode, void *stream);

/* Static, human-readable name of a status. */
const char *wise_status_string(wise_status st);

#ifdef __cplusplus
}
#endif

#endif /* WISE_H */
