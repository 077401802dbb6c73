// Head-union, page-granular support through a compacted page table.
//
// Method: WISE pull request page (vllm-rlt pull 143), "What changes", second
// bullet (the FlashAttention route: each sparse row reads the whole KV pages
// that hold a block any head of the layer picked, through a shortened page
// table) and "Limits" (with pages of 256 tokens or more, that union leaves
// almost nothing out).
//
// One wave64 per row:
//  * plan as a SPARSE row (tag of the (slot, layer): same request and
//    position, enough discovery depths), else every page (dense fallback,
//    counted); DENSE rows keep every page;
//  * OR the support words of all heads of the (slot, layer) into LDS;
//  * page j is kept when its valid tokens [jP, min(n, jP+P)) meet a set
//    block; kept pages are compacted with ballot + mbcnt, 64 pages per step,
//    so the output table lists their physical ids in logical order (loads
//    are batched so that a row waits on memory a few times, not per head
//    or per step);
//  * the compacted context is (kept - 1) * P + the valid tokens of the last
//    kept page: only the context's last page can be partial, and it can
//    only be the last one kept.
// Rows with bad data (another mode, a context outside [1, max_ctx], a slot
// out of range, an empty union, a kept page id out of range) get context 0
// and count one error per head here.  The attention itself is any paged
// dense decode over (bt_out, ctx_out).
#include "wise_internal.h"

namespace wise {

namespace {

constexpr int kPageWaves = 4;
constexpr int kHeadBatch = 16;  // support loads in flight per lane
constexpr int kChunkBatch = 8;  // block-table loads in flight per lane (512 pages)

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// Any bit set in [lo, hi] (block indices, lo <= hi) of the union words.
__device__ __forceinline__ bool any_bit(const uint32_t *su, int lo, int hi) {
  const int wlo = lo >> 5, whi = hi >> 5;
  for (int w = wlo; w <= whi; ++w) {
    uint32_t m = su[w];
    if (w == wlo) m &= ~0u << (lo & 31);
    if (w == whi && (hi & 31) != 31) m &= (1u << ((hi & 31) + 1)) - 1u;
    if (m) return true;
  }
  return false;
}

__global__ __launch_bounds__(64 * kPageWaves) void compact_pages_kernel(const PageParams p) {
  __shared__ uint32_t s_union[kPageWaves][kMaxWords];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int r = blockIdx.x * kPageWaves + wave;
  if (r >= p.rows) return;
  // independent per-row loads, issued together
  const int n = p.ctx_len[r];
  const int req = p.row_mode ? static_cast<int>(p.row_mode[r]) : WISE_SPARSE;
  const int slot_in = p.slot_of_row ? p.slot_of_row[r] : r;
  int32_t *dst = p.bt_out + static_cast<int64_t>(r) * p.bt_out_stride;
  const int32_t *src = p.block_table + static_cast<int64_t>(r) * p.bt_stride;
  // a row with bad data gets context 0 (the attention call writes NaN for
  // it) and one error per head
  auto row_error = [&]() {
    if (lane == 0) {
      p.ctx_out[r] = 0;
      if (p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, static_cast<unsigned long long>(p.heads));
    }
  };
  if ((req != WISE_DENSE && req != WISE_SPARSE) || n < 1 || n > p.max_ctx) {
    row_error();
    return;
  }
  const int P = 1 << p.page_shift;
  const int npg = (n + P - 1) >> p.page_shift;
  const int slot = req == WISE_SPARSE ? slot_in : r;
  if (req == WISE_SPARSE && (slot < 0 || slot >= p.slots)) {
    row_error();
    return;
  }
  // Issued together, before anything waits: the first kChunkBatch steps of
  // the block table, the tag, and the support words of every head (lane w
  // holds word w; a row has at most kMaxWords = 64 of them).
  int32_t ids[kChunkBatch];
#pragma unroll
  for (int t = 0; t < kChunkBatch; ++t) {
    const int j = 64 * t + lane;
    ids[t] = j < npg ? src[j] : -1;
  }
  const int nb = (n + kBlock - 1) / kBlock;
  const int nw = req == WISE_SPARSE ? (nb + 31) >> 5 : 0;
  uint32_t u = 0u;
  bool full = true;
  if (req == WISE_SPARSE) {
    const wise_tag *t = p.tags + static_cast<int64_t>(slot) * p.layers + p.layer;
    const uint32_t *sw = p.support + (static_cast<int64_t>(slot) * p.layers + p.layer) * p.heads * p.words;
    if (lane < nw) {
      for (int h0 = 0; h0 < p.heads; h0 += kHeadBatch) {
        uint32_t x[kHeadBatch];
#pragma unroll
        for (int k = 0; k < kHeadBatch; ++k)
          x[k] = h0 + k < p.heads ? sw[static_cast<int64_t>(h0 + k) * p.words + lane] : 0u;
#pragma unroll
        for (int k = 0; k < kHeadBatch; ++k) u |= x[k];
      }
    }
    const bool same = t->request == p.row_request[r] && t->position == p.row_position[r];
    full = !(same && t->discoveries >= p.required);
    if (full && lane == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_FALLBACKS, 1ull);
  }
  // head union of the (slot, layer) support, bits past the context cleared
  uint32_t *su = s_union[wave];
  if (!full) {
    if (lane < nw) {
      const int valid = nb - 32 * lane;
      su[lane] = valid < 32 ? u & ((1u << valid) - 1u) : u;
    }
    wave_lds_sync();
  }

  // keep test (every page for DENSE rows and fallbacks) and compaction, 64
  // pages per step; the table entries of kChunkBatch steps are loaded before
  // the first of them is compacted
  int count = 0, last = -1;
  bool bad_page = false;
  for (int c0 = 0; c0 < npg; c0 += 64 * kChunkBatch) {
    if (c0 > 0) {
#pragma unroll
      for (int t = 0; t < kChunkBatch; ++t) {
        const int j = c0 + 64 * t + lane;
        ids[t] = j < npg ? src[j] : -1;
      }
    }
#pragma unroll
    for (int t = 0; t < kChunkBatch; ++t) {
      const int j0 = c0 + 64 * t;
      if (j0 >= npg) break;
      const int j = j0 + lane;
      bool keep = false;
      if (j < npg) {
        const int lo = (j << p.page_shift) / kBlock;
        const int hi = (min(n, (j + 1) << p.page_shift) - 1) / kBlock;
        keep = full || any_bit(su, lo, hi);
      }
      const unsigned long long bm = __builtin_amdgcn_ballot_w64(keep);
      const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0));
      if (keep) dst[count + rank] = ids[t];
      bad_page |= keep && static_cast<unsigned>(ids[t]) >= static_cast<unsigned>(p.num_pages);
      if (bm) last = j0 + 63 - __builtin_clzll(bm);
      count += __popcll(bm);
    }
  }
  // an empty union and a kept page id out of range are data errors;
  // keeping every page gives back n
  if (count == 0 || __builtin_amdgcn_ballot_w64(bad_page) != 0ull) {
    row_error();
    return;
  }
  if (lane == 0) p.ctx_out[r] = (count - 1) * P + min(P, n - last * P);
}

}  // namespace

hipError_t launch_compact_pages(const PageParams &p, hipStream_t stream) {
  const unsigned groups = static_cast<unsigned>((p.rows + kPageWaves - 1) / kPageWaves);
  hipLaunchKernelGGL(compact_pages_kernel, dim3(groups), dim3(64 * kPageWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wise
