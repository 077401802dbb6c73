// Split-KV paged decode attention with per-row modes (dense / discover /
// discover-union / sparse) for gfx950.
//
// Method: WISE pull request page (vllm-rlt pull 143), "What changes", first
// bullet (the split kernel's row modes, its finish step and the size of its
// programs).  Restated: a discovery row is attended in full and leaves, per
// 32-token tile, the max and the exp-sum of its scores; a sparse row visits
// only the tiles of its support, whose indices are gathered into a dense
// list before the tile loop so that the loop body has no per-tile test; and
// work items stay near eight tiles, so that in a launch mixing long dense
// rows with short sparse ones the longest row does not decide when the
// launch ends.
//
// MI355X design:
//  * One wave64 per work item (<= tiles_per_item consecutive entries of a
//    (row, head)'s tile list); each wave plans its own item (tag check,
//    fallback, tile count, compacted tile list), so that a call needs no
//    host readback.  Three launch shapes share the per-item body: the fused
//    kernel (one workgroup per (row, head) unit of up to 256 blocks, i.e.
//    contexts up to 8K, whose 4-16 waves split the unit's tiles evenly and
//    then finish the unit in the same kernel), and, for longer contexts,
//    the static grid (four independent waves per workgroup over every
//    (unit, item) slot, finished by the finish kernel) and the listed grid
//    (persistent waves over the compact item list a one-workgroup plan
//    kernel builds, for calls with sparse rows).  In those two grids items
//    keep about eight tiles unless the launch is large enough to outlast
//    any one item many times over; then they grow to 16 or 32 tiles
//    (decided on the host for calls with no sparse rows, in the plan kernel
//    from the attended tiles otherwise), since each item's partial
//    (m, l, acc) written to HBM amid the K/V stream costs far more than its
//    bytes.
//  * A 32-token K (or V) tile is read with 16-byte loads in which each load
//    instruction covers TPI whole tokens contiguously (1 KB per wave for
//    bf16 d=128): lane = (token subgroup g, 16-byte dim chunk c).  Every K
//    and V load of a tile is issued before any arithmetic.
//  * q.k uses v_dot2 (bf16 pairs, fp32 accumulate) or fp32 FMA, reduced
//    across the LPT lanes of a token with DPP row rotations; lanes 16 and 32
//    apart exchange through v_permlane16_swap / v_permlane32_swap (register
//    swaps, no LDS round trip).  Online softmax runs in base 2 on scores
//    pre-scaled by scale*log2(e).  Every reduction is a fixed butterfly, so
//    all lanes hold bitwise-identical statistics and a row's result does not
//    depend on the other rows of the launch.
#include <hip/hip_ext.h>

#include <algorithm>

#include "wise_internal.h"
#include "wise_select.h"

namespace wise {

namespace {

constexpr float kLn2 = 0.693147180559945309417f;

template <bool kBf16, int D>
struct Geo {
  static constexpr int E = kBf16 ? 2 : 4;       // bytes per element
  static constexpr int BPT = D * E;             // bytes per token row
  static constexpr int LPT = BPT / 16;          // lanes per token (16 B each)
  static constexpr int TPI = 64 / LPT;          // tokens per load instruction
  static constexpr int NI = kBlock / TPI;       // load instructions per tile
  static constexpr int EPL = 16 / E;            // elements per lane per load
  // waves per SIMD the persistent split kernel is compiled for (VGPR budget)
  static constexpr int kListedWavesPerEU = NI * 8 <= 64 ? 4 : 2;
  static_assert(LPT >= 8 && LPT <= 32, "unsupported head_dim/dtype");
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Lanes l and l ^ 16 (or l ^ 32) exchanged in registers: v_permlane16_swap
// (v_permlane32_swap) with both operands x leaves x of the lower partner in
// the first result and x of the upper partner in the second, in both lanes,
// so a combine of the pair gives bitwise the same value in both.
__device__ __forceinline__ float2 pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum16(float x) { const float2 q = pair16(x); return q.x + q.y; }
__device__ __forceinline__ float sum32(float x) { const float2 q = pair32(x); return q.x + q.y; }
__device__ __forceinline__ float max16(float x) { const float2 q = pair16(x); return fmaxf(q.x, q.y); }
__device__ __forceinline__ float max32(float x) { const float2 q = pair32(x); return fmaxf(q.x, q.y); }

// Sum over aligned groups of LPT consecutive lanes; every lane of a group
// gets the bitwise-same total.
template <int LPT>
__device__ __forceinline__ float lane_group_sum(float x) {
  if constexpr (LPT == 8) {
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  } else {
    x += dpp<0x128>(x);  // row_ror:8
    x += dpp<0x124>(x);  // row_ror:4
    x += dpp<0x122>(x);  // row_ror:2
    x += dpp<0x121>(x);  // row_ror:1
    if constexpr (LPT == 32) x = sum16(x);
  }
  return x;
}

// Combine across the TPI token subgroups (lanes l, l ^ LPT, l ^ 2 LPT, ...).
template <int LPT>
__device__ __forceinline__ float subgroup_max(float x) {
  if constexpr (LPT <= 8) x = fmaxf(x, dpp<0x128>(x));  // partner lane l ^ 8 within the row
  if constexpr (LPT <= 16) x = max16(x);
  return max32(x);
}
template <int LPT>
__device__ __forceinline__ float subgroup_sum(float x) {
  if constexpr (LPT <= 8) x += dpp<0x128>(x);
  if constexpr (LPT <= 16) x = sum16(x);
  return sum32(x);
}

// Inclusive prefix sum over lanes 0..lane: a shift scan within each 16-lane
// row (DPP row_shr; lanes shifted in from outside the row read 0), then the
// totals of the lower rows, read from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
            t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

// Dot product of one lane's 16 bytes of K with the same 16 bytes of q.
// (Whole-vector bit casts: casting a single swizzled element of an
// ext_vector into a bf16 vector is miscompiled by this toolchain.)
template <bool kBf16>
__device__ __forceinline__ float dot16(u32x4 k, u32x4 q) {
  if constexpr (kBf16) {
    const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, k);
    const bf16x8_t qb = __builtin_bit_cast(bf16x8_t, q);
    float a = __builtin_amdgcn_fdot2_f32_bf16(kb.s01, qb.s01, 0.0f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(kb.s23, qb.s23, a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(kb.s45, qb.s45, a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(kb.s67, qb.s67, a, false);
    return a;
  } else {
    float a = __uint_as_float(k[0]) * __uint_as_float(q[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) a = fmaf(__uint_as_float(k[i]), __uint_as_float(q[i]), a);
    return a;
  }
}

// acc[0..EPL) += w * v (the lane's EPL elements of one token's V row);
// bf16 element 2i is the low half of word i, element 2i+1 the high half.
template <bool kBf16>
__device__ __forceinline__ void axpy16(float *acc, float w, u32x4 v) {
  if constexpr (kBf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = v[i];
      acc[2 * i] = fmaf(w, bf16_lo(x), acc[2 * i]);
      acc[2 * i + 1] = fmaf(w, bf16_hi(x), acc[2 * i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, __uint_as_float(v[i]), acc[i]);
  }
}

__device__ __forceinline__ u32x4 load16(const char *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// ---------------------------------------------------------------------------
// Planning of one row: effective mode from the support tags, dense fallback.
// ---------------------------------------------------------------------------
struct RowPlan {
  int row, n, req, eff, slot;
  bool bad, fallback;
  uint32_t word;  // this lane's support word of (slot, head), when requested and the row asks for SPARSE
};

__device__ __forceinline__ const uint32_t *support_words(const SplitParams &p, int slot, int h);

// Effective mode of row r.  With h >= 0, a row that requests SPARSE also
// gets lane's support word of (slot, h).  Every load the plan may need is
// issued before any of them is used: when rows map to slots one to one (no
// slot_of_row), the slot is known without a load, so the tag, the row's
// (request, position) and the support word are issued first, whatever the
// mode turns out to be, and the context length and the mode after them;
// with slot_of_row the state follows that one load.  The tag is compared
// field by field without short-circuiting, so its words arrive in one round
// trip.
__device__ __forceinline__ RowPlan plan_row(const SplitParams &p, int r, int h = -1, int lane = 0) {
  RowPlan rp;
  rp.row = r;
  const bool ident = p.slot_of_row == nullptr;
  int64_t t_req = 0, t_pos = 0, r_req = 0, r_pos = 0;
  int t_disc = 0;
  uint32_t word = 0u;
  auto load_state = [&](int sl) {
    const wise_tag *t = p.tags + static_cast<int64_t>(sl) * p.layers + p.layer;
    t_req = t->request;
    t_pos = t->position;
    t_disc = t->discoveries;
    r_req = p.row_request[r];
    r_pos = p.row_position[r];
    if (h >= 0 && lane < p.words) word = support_words(p, sl, h)[lane];
  };
  if (p.tags != nullptr && ident && r < p.slots) load_state(r);
  rp.n = p.ctx_len[r];
  rp.req = p.row_mode ? static_cast<int>(p.row_mode[r]) : p.uniform_mode;
  rp.bad = rp.n < 1 || rp.n > p.max_ctx || rp.req < WISE_DENSE || rp.req > WISE_SPARSE;
  rp.eff = rp.req;
  rp.slot = r;
  rp.fallback = false;
  rp.word = 0u;
  if (!rp.bad && rp.req != WISE_DENSE) {
    int slot = r;
    if (!ident) {
      slot = p.slot_of_row[r];
      if (slot >= 0 && slot < p.slots) load_state(slot);
    }
    rp.slot = slot;
    if (slot < 0 || slot >= p.slots) {
      rp.bad = true;
    } else if (rp.req == WISE_DISCOVER_UNION || rp.req == WISE_SPARSE) {
      const bool same = (t_req == r_req) & (t_pos == r_pos);
      const int need = rp.req == WISE_SPARSE ? p.required : 1;
      if (!(same & (t_disc >= need))) {
        rp.eff = WISE_DENSE;
        rp.fallback = true;
      }
      // a sparse row attends the word's blocks; a union row ORs its selection into it
      if (rp.req == WISE_SPARSE || rp.req == WISE_DISCOVER_UNION) rp.word = word;
    }
  }
  return rp;
}

__device__ __forceinline__ const uint32_t *support_words(const SplitParams &p, int slot, int h) {
  return p.support + ((static_cast<int64_t>(slot) * p.layers + p.layer) * p.heads + h) * p.words;
}

// One wave: lane l < ceil(nb/32) holds support word l (raw, as loaded; bits
// past nb are cleared here); incl = inclusive prefix of the words'
// popcounts; returns the set-bit count.
__device__ __forceinline__ int support_scan(uint32_t raw, int nb, int lane, uint32_t &word, int &incl) {
  const int nw = (nb + 31) >> 5;
  word = 0u;
  if (lane < nw) {
    word = raw;
    const int valid = nb - 32 * lane;
    if (valid < 32) word &= (1u << valid) - 1u;
  }
  incl = wave_inclusive_scan(__popc(word), lane);
  return __builtin_amdgcn_readlane(incl, 63);
}

// ---------------------------------------------------------------------------
// One work item: list entries [first, first + ntiles) of unit (r, h) --
// either tiles first.. (all causal tiles) or the support's set bits of those
// ranks, compacted into a per-wave list before the loop.  Writes the
// item's partial (m, l, acc) and the tile stats.  kKOnly: K is read and the
// scores' tile stats and (m, l) are kept, V and the accumulator are not
// (discovery after an external dense kernel).
// ---------------------------------------------------------------------------
// Where one item's results go when the finish is fused into the split
// kernel: LDS of the unit's workgroup instead of the workspace.
struct UnitLds {
  float *acc;       // [items][D] partial accumulators
  float2 *ml;       // [items] partial (m, l); l < 0 marks a bad page
  float2 *stats;    // [blocks] tile stats by block index (non-sparse items)
};

// stream_partials: the accumulator partial goes out as a nontemporal store,
// which disturbs the K/V stream less behind long items (1-2% at 8K and on
// ragged batches, static and listed grids alike) but costs the listed
// grid's eight-tile items about as much (mixed 4K launch).
template <bool kBf16, int D, bool kKOnly>
__device__ __forceinline__ void run_item(const SplitParams &p, int u, int r, int h, int k, int n, bool sparse,
                                         int count, uint32_t word, int incl, int lane, int *tiles, int T,
                                         const UnitLds *lds = nullptr, bool stream_partials = false) {
  using G = Geo<kBf16, D>;
  const int first = k * T;
  const int ntiles = min(T, count - first);

  if (sparse) {
    // the previous item of this wave may still be reading the list
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const int excl = incl - __popc(word);
    const unsigned long long past = __builtin_amdgcn_ballot_w64(incl > first);
    int w = __builtin_amdgcn_readfirstlane(__builtin_ctzll(past));
    int got = 0;
    while (got < ntiles) {
      const uint32_t wv = __builtin_amdgcn_readlane(word, w);
      const int base = __builtin_amdgcn_readlane(excl, w);
      const bool set = lane < 32 && ((wv >> (lane & 31)) & 1u);
      const unsigned long long bm = __builtin_amdgcn_ballot_w64(set);
      const int rank = base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0));
      if (set && rank >= first && rank < first + ntiles) tiles[rank - first] = 32 * w + lane;
      got = min(ntiles, base + __popcll(bm) - first);
      ++w;
    }
    // the list is read back by every lane of this wave below
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }

  // ---- per-lane constants ----
  const int c = lane % G::LPT;  // 16-byte dim chunk: elements [c*EPL, c*EPL+EPL)
  const int g = lane / G::LPT;  // token subgroup: token j*TPI + g of load j
  const uint32_t lane_off = static_cast<uint32_t>(g * p.stride_token_b + c * 16);
  const u32x4 qv = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.q) +
                                                    (static_cast<int64_t>(u) * D + c * G::EPL) * G::E);
  const char *kh = static_cast<const char *>(p.k) + h * p.stride_head_b;  // wave-uniform
  const char *vh = kKOnly ? nullptr : static_cast<const char *>(p.v) + h * p.stride_head_b;
  const int32_t *bt = p.block_table + r * p.bt_stride;
  const int pmask = (1 << p.page_shift) - 1;

  float m_run = -INFINITY, l_run = 0.0f;
  float acc[G::EPL];
#pragma unroll
  for (int e = 0; e < G::EPL; ++e) acc[e] = 0.0f;
  float st_m = 0.0f, st_l = 0.0f;  // tile stats of list entry `lane`
  bool page_err = false;

  // Physical page of load instruction j of tile (list entry) i: lane j of a
  // page vector fetched one tile ahead.  A load instruction whose tokens are
  // all past the context reuses the page of the row's last token with the
  // slot offset it would have had, which stays inside that page; its lanes
  // are masked below.
  auto tile_of = [&](int i) -> int { return sparse ? __builtin_amdgcn_readfirstlane(tiles[i]) : first + i; };
  auto fetch_pages = [&](int b) -> int {
    const int tj = b * kBlock + min(lane, G::NI - 1) * G::TPI;
    return bt[min(tj, n - 1) >> p.page_shift];
  };
  int pages_next = fetch_pages(tile_of(0));

  for (int i = 0; i < ntiles; ++i) {
    const int b = tile_of(i);
    const int t0 = b * kBlock;
    const int nv = min(kBlock, n - t0);  // valid tokens in this tile (>= 1)
    const int pages = pages_next;
    if (i + 1 < ntiles) pages_next = fetch_pages(tile_of(i + 1));

    // issue every K and V load of the tile before any arithmetic
    u32x4 kr[G::NI], vr[G::NI];
#pragma unroll
    for (int j = 0; j < G::NI; ++j) {
      int page = __builtin_amdgcn_readlane(pages, j);
      const bool pbad = static_cast<unsigned>(page) >= static_cast<unsigned>(p.num_pages);
      page_err |= pbad;
      page = pbad ? 0 : page;
      const int64_t off = page * p.stride_page_b + ((t0 + j * G::TPI) & pmask) * p.stride_token_b;
      kr[j] = load16(kh + off + lane_off);
      if constexpr (!kKOnly) vr[j] = load16(vh + off + lane_off);
    }
    // keep all 2*NI loads in flight together: no arithmetic moves above here
    __builtin_amdgcn_sched_barrier(0);

    // scores of this lane's NI tokens (base-2 units)
    float s[G::NI];
#pragma unroll
    for (int j = 0; j < G::NI; ++j) {
      const float d = lane_group_sum<G::LPT>(dot16<kBf16>(kr[j], qv));
      s[j] = (j * G::TPI + g < nv) ? d * p.qk_scale_log2 : -INFINITY;
    }
    float mb = s[0];
#pragma unroll
    for (int j = 1; j < G::NI; ++j) mb = fmaxf(mb, s[j]);
    mb = subgroup_max<G::LPT>(mb);
    float pj[G::NI], ls = 0.0f;
#pragma unroll
    for (int j = 0; j < G::NI; ++j) {
      pj[j] = __builtin_amdgcn_exp2f(s[j] - mb);
      ls += pj[j];
    }
    const float lb = subgroup_sum<G::LPT>(ls);
    if (lane == i) {
      st_m = mb;
      st_l = lb;
    }

    // online-softmax update of this item's running (m, l, acc)
    const float m_new = fmaxf(m_run, mb);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float beta = __builtin_amdgcn_exp2f(mb - m_new);
    l_run = l_run * alpha + lb * beta;
    if constexpr (!kKOnly) {
#pragma unroll
      for (int e = 0; e < G::EPL; ++e) acc[e] *= alpha;
#pragma unroll
      for (int j = 0; j < G::NI; ++j) {
        const bool valid = j * G::TPI + g < nv;
        const u32x4 v = valid ? vr[j] : u32x4{0u, 0u, 0u, 0u};
        axpy16<kBf16>(acc, pj[j] * beta, v);
      }
    }
    m_run = m_new;
  }

  // ---- partial (m, l, acc) of this item, and the tile stats ----
  const int64_t slot_idx = static_cast<int64_t>(u) * p.items_per_unit + k;
  if constexpr (!kKOnly) {
#pragma unroll
    for (int e = 0; e < G::EPL; ++e) acc[e] = subgroup_sum<G::LPT>(acc[e]);
  }
  const float2 ml = page_err ? make_float2(0.0f, -1.0f) : make_float2(m_run, l_run);
  if (lds) {
    if (!kKOnly && g == 0) {
      float4 *dst = reinterpret_cast<float4 *>(lds->acc + k * D + c * G::EPL);
#pragma unroll
      for (int e = 0; e < G::EPL; e += 4) dst[e / 4] = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    }
    if (lane == 0) lds->ml[k] = ml;
  } else {
    if (!kKOnly && g == 0) {
      f32x4 *dst = reinterpret_cast<f32x4 *>(p.part_acc + slot_idx * D + c * G::EPL);
#pragma unroll
      for (int e = 0; e < G::EPL; e += 4) {
        const f32x4 v = {acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
        if (stream_partials)
          __builtin_nontemporal_store(v, dst + e / 4);
        else
          dst[e / 4] = v;
      }
    }
    if (lane == 0) p.part_ml[slot_idx] = ml;
  }
  if (lane < ntiles) {
    const int b = sparse ? tiles[lane] : first + lane;
    const int64_t si = static_cast<int64_t>(u) * p.max_blocks + b;
    if (lds) {
      if (!sparse) lds->stats[b] = make_float2(st_m, st_l);
    } else {
      p.stats[si] = make_float2(st_m, st_l);
    }
    if (p.stats_export) p.stats_export[si] = make_float2(st_m * kLn2, st_l);
  }
}

// ---------------------------------------------------------------------------
// Static grid: one wave per (unit, item slot); every wave plans its own item.
// Used for calls the fused kernel does not cover that have no sparse rows
// (every unit's item count then follows from its context length, so nearly
// every slot holds work; such calls may run longer items, tiles_per_item up
// to kLongTiles), and for sparse calls whose units fit one workgroup but do
// not fuse.
// ---------------------------------------------------------------------------
template <bool kBf16, int D, bool kKOnly>
__global__ __launch_bounds__(64 * kWavesPerGroup) void split_static_kernel(const SplitParams p) {
  __shared__ int s_tiles[kWavesPerGroup][kMaxTilesPerItem];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroup i runs on XCD i % 8.  Group-major order (i = group * units +
  // unit) keeps every unit on XCD unit % 8 for all its groups, so each row's
  // heads spread over all XCDs however short the row is (unit-major order
  // would pile the only non-empty group of short rows onto one XCD).
  const int units = p.rows * p.heads;
  const int grp = blockIdx.x / units;
  const int u = blockIdx.x - grp * units;           // unit = (row, head)
  const int k = grp * kWavesPerGroup + wave;        // item slot
  if (k >= p.items_per_unit) return;
  const int r = u / p.heads;
  const int h = u - r * p.heads;
  if (k > 0) {
    // No mode gives a row more tiles than its causal blocks: slots past them
    // leave after one load (rows far shorter than max_ctx leave most slots empty).
    const int n0 = p.ctx_len[r];
    const int nb0 = (n0 >= 1 && n0 <= p.max_ctx) ? (n0 + kBlock - 1) / kBlock : 0;
    if (k >= (nb0 + p.tiles_per_item - 1) / p.tiles_per_item) return;
  }
  const RowPlan rp = plan_row(p, r, h, lane);
  const int nb = rp.bad ? 0 : (rp.n + kBlock - 1) / kBlock;
  const bool sparse = !rp.bad && rp.eff == WISE_SPARSE;
  uint32_t word = 0u;
  int incl = 0;
  // K-only calls have nothing to do for a row whose discovery window broke
  const int count = (kKOnly && rp.eff == WISE_DENSE) ? 0
                    : sparse                         ? support_scan(rp.word, nb, lane, word, incl)
                                                     : nb;
  const int items = (count + p.tiles_per_item - 1) / p.tiles_per_item;
  if (k == 0 && lane == 0) {
    p.unit_items[u] = items;
    if (h == 0) {
      p.row_code[r] = encode_row(rp.bad ? kRowError : rp.eff, rp.req);
      p.row_done[r] = 0ull;  // the finish kernel's per-row arrival word
      if (rp.fallback && p.counters) atomicAdd(p.counters + WISE_CTR_FALLBACKS, 1ull);
    }
  }
  if (k >= items) return;
  run_item<kBf16, D, kKOnly>(p, u, r, h, k, rp.n, sparse, count, word, incl, lane, s_tiles[wave], p.tiles_per_item,
                             nullptr, true);
}

// ---------------------------------------------------------------------------
// Fused split + finish, for calls whose units fit one workgroup each (see
// fused_waves()): the waves leave their partials and tile stats in LDS, and
// two waves then finish the unit side by side.  Wave 1 runs the eta
// selection and writes or ORs the support; wave 0 merges the partials into
// the output exactly as the finish kernel would (the same merge in the same
// order, so the output bits do not depend on which kernel ran it).  A
// discovery row's tag and density counters are updated by the last of its
// heads to arrive, counted in the tag's reserved word.  For short units of
// calls that read V, wave 0 sends the arrival (arrivals | error heads << 8)
// before its output stores and each head's selection wave adds its newly
// selected blocks to the density counter itself, so the arrival does not
// wait for the selection.  Otherwise -- long units, and the LSE route, whose
// short K-only launch would end with a burst of same-address counter
// atomics -- the selection wave carries the arrival with the row's selected
// blocks (<< 16 in the same word).
// Both waves compute the unit's (M, L) by the same operations, so they agree
// bit for bit.  The last arrival returns the word to zero.  Every unit of
// the row planned from the tag before any head arrives, so the update
// cannot race with a plan.
// ---------------------------------------------------------------------------
// (M, L) of a unit from its items' partials in LDS: M = max m_i, L = sum
// l_i 2^(m_i - M) (or M = the external LSE in base-2 units and L = 1 on the
// LSE route); err = no items, a bad page in one, or a non-finite LSE.  With
// s_w, the item weights 2^(m_i - M) are left there for the merge.
template <bool kKOnly>
__device__ __forceinline__ void unit_norm(const SplitParams &p, int u, int items, const float2 *s_ml, float *s_w,
                                          int lane, float &M, float &L, bool &err) {
  const float2 ml = lane < items ? s_ml[lane] : make_float2(-INFINITY, 0.0f);
  M = sel::wave_max(ml.x);
  err = items == 0 || __builtin_amdgcn_ballot_w64(ml.y < 0.0f) != 0ull;
  L = 1.0f;
  if constexpr (kKOnly) {
    const float lse = p.lse[u];
    err = err || !__builtin_isfinite(lse);
    M = lse * 1.44269504088896340736f;
  } else {
    float Lp = 0.0f;
    if (lane < items) {
      const float w = __builtin_amdgcn_exp2f(ml.x - M);
      if (s_w) s_w[lane] = w;
      Lp = fmaf(ml.y, w, Lp);
    }
    L = sel::wave_sum(Lp);
  }
}

// Wave 0: the output (NaN for a unit with bad data) and its error count.
// The LSE route writes no output; its selection wave counts its errors.
template <int D, bool kKOnly>
__device__ __forceinline__ void finish_output(const SplitParams &p, int u, int items, const float *s_acc,
                                              const float2 *s_ml, float *s_w, int lane) {
  if constexpr (!kKOnly) {
    float M, L;
    bool err;
    unit_norm<kKOnly>(p, u, items, s_ml, s_w, lane, M, L, err);
    sel::wave_lds_sync();
    constexpr int kOut = D / 64;  // output elements per lane
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int dd = lane + 64 * i;
      float a = 0.0f;
      for (int t = 0; t < items; ++t) a = fmaf(s_acc[t * D + dd], s_w[t], a);
      p.out[static_cast<int64_t>(u) * D + dd] = err ? __builtin_nanf("") : a / L;
    }
    if (err && lane == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, 1ull);
  }
}

// Short units of calls that read V split the finish the other way (see the
// fused kernel): wave 0 writes the output and sends the row's arrival before
// its output stores, so their round trips overlap, and the last head to
// arrive updates the tag and the causal-block count; wave 1 selects, writes
// the support and adds its own newly selected blocks to the density counter.
template <int D>
__device__ __forceinline__ void finish_output_arrive(const SplitParams &p, const RowPlan &rp, int u, int h, int nb,
                                                     int items, const float *s_acc, const float2 *s_ml, float *s_w,
                                                     int lane) {
  const bool stateful = p.support != nullptr && !rp.bad && rp.req != WISE_DENSE;
  const bool discover = stateful && (rp.eff == WISE_DISCOVER || rp.eff == WISE_DISCOVER_UNION);
  float M, L;
  bool err;
  unit_norm<false>(p, u, items, s_ml, s_w, lane, M, L, err);
  wise_tag *tag = stateful ? p.tags + static_cast<int64_t>(rp.slot) * p.layers + p.layer : nullptr;
  unsigned int *arrive = discover ? reinterpret_cast<unsigned int *>(&tag->reserved) : nullptr;
  unsigned int all = 0u;
  if (discover && lane == 0) {
    const unsigned int mine = 1u | (err ? 1u << 8 : 0u);
    all = atomicAdd(arrive, mine) + mine;
  }
  sel::wave_lds_sync();
  constexpr int kOut = D / 64;  // output elements per lane
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int dd = lane + 64 * i;
    float a = 0.0f;
    for (int t = 0; t < items; ++t) a = fmaf(s_acc[t * D + dd], s_w[t], a);
    p.out[static_cast<int64_t>(u) * D + dd] = err ? __builtin_nanf("") : a / L;
  }
  if (err && lane == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, 1ull);
  if (!stateful || lane != 0) return;
  if (!discover) {
    // a union row whose discovery window is broken ran dense: the rest of
    // this token runs dense too
    if (rp.req == WISE_DISCOVER_UNION && h == 0) tag->discoveries = 0;
    return;
  }
  if (static_cast<int>(all & 0xFFu) != p.heads) return;
  atomicExch(arrive, 0u);
  const int err_heads = static_cast<int>((all >> 8) & 0xFFu);
  if (p.counters && rp.eff == WISE_DISCOVER)
    atomicAdd(p.counters + WISE_CTR_CAUSAL, static_cast<unsigned long long>(nb) * (p.heads - err_heads));
  // a bad page in any head of the row breaks this discovery
  if (rp.eff == WISE_DISCOVER) {
    tag->request = p.row_request[rp.row];
    tag->position = p.row_position[rp.row];
    tag->discoveries = err_heads ? 0 : 1;
  } else {
    tag->discoveries = err_heads ? 0 : tag->discoveries + 1;
  }
}

// Wave 1: the eta selection of a discovery unit, the support words written
// (DISCOVER) or ORed (DISCOVER_UNION; into the words its plan loaded -- no
// other unit writes them) and its newly selected blocks counted; on the LSE
// route also the row's arrival and, for its last head, the tag and the
// density counters.
template <bool kKOnly, int MAXB, bool kArrives>
__device__ __forceinline__ void finish_row(const SplitParams &p, const RowPlan &rp, int u, int h, int nb, int items,
                                           const float2 *s_ml, const float2 *s_st, uint32_t *s_bits, int lane) {
  const bool stateful = p.support != nullptr && !rp.bad && rp.req != WISE_DENSE;
  const bool discover = stateful && (rp.eff == WISE_DISCOVER || rp.eff == WISE_DISCOVER_UNION);
  wise_tag *tag = stateful ? p.tags + static_cast<int64_t>(rp.slot) * p.layers + p.layer : nullptr;
  if (!discover) {
    // a union row whose discovery window is broken ran dense (on the LSE
    // route it did no work): the rest of this token runs dense too (done by
    // the wave that carries the arrival)
    if (kArrives && stateful && rp.req == WISE_DISCOVER_UNION && h == 0 && lane == 0) tag->discoveries = 0;
    if (!kKOnly || !rp.bad) return;
  }
  float M, L;
  bool err;
  unit_norm<kKOnly>(p, u, items, s_ml, nullptr, lane, M, L, err);
  if constexpr (kKOnly) {
    if (err && lane == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, 1ull);
    if (!discover) return;
  }
  int K = 0;
  uint32_t nw = 0u;  // lane w: new support word w (a unit has at most MAXB / 32 words)
  if (!err) {
    if (nb <= 64) {
      // one block per lane; the selected set comes back as a register mask
      const float2 st = lane < nb ? s_st[lane] : make_float2(0.0f, 0.0f);
      unsigned long long mask = 0ull;
      K = nb <= 16   ? sel::select_eta_mask<16>(st, p.eta, nb, M, L, lane, mask)
          : nb <= 32 ? sel::select_eta_mask<32>(st, p.eta, nb, M, L, lane, mask)
                     : sel::select_eta_mask<64>(st, p.eta, nb, M, L, lane, mask);
      nw = lane == 0 ? static_cast<uint32_t>(mask) : lane == 1 ? static_cast<uint32_t>(mask >> 32) : 0u;
    } else if constexpr (MAXB > 64) {
      // two or four blocks per lane (lane l holds blocks l*KPL ..); the
      // selected blocks' bits are ORed into LDS words
      static_assert(MAXB <= 256, "a long fused unit has at most 256 blocks");
      if (lane < MAXB / 32) s_bits[lane] = 0u;
      sel::wave_lds_sync();
      if (nb <= 128) {
        float2 st[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) st[j] = 2 * lane + j < nb ? s_st[2 * lane + j] : make_float2(0.0f, 0.0f);
        K = sel::select_eta<2, 128>(st, p.eta, nb, M, L, lane, s_bits);
      } else {
        float2 st[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) st[j] = 4 * lane + j < nb ? s_st[4 * lane + j] : make_float2(0.0f, 0.0f);
        K = sel::select_eta<4, 256>(st, p.eta, nb, M, L, lane, s_bits);
      }
      sel::wave_lds_sync();
      nw = lane < MAXB / 32 ? s_bits[lane] : 0u;
    }
  }
  const int selected = err ? 0 : rp.eff == WISE_DISCOVER ? K : sel::wave_sum_int(__popc(nw & ~rp.word));
  if constexpr (!kArrives) {
    // wave 0 carries the row's arrival; this wave adds its own newly
    // selected blocks to the density counter
    if (err) return;
    uint32_t *sw = p.support + ((static_cast<int64_t>(rp.slot) * p.layers + p.layer) * p.heads + h) * p.words;
    if (rp.eff == WISE_DISCOVER) {
      for (int w = lane; w < p.words; w += 64) sw[w] = w == lane ? nw : 0u;
    } else if (lane < p.words && (nw & ~rp.word) != 0u) {
      sw[lane] = rp.word | nw;  // the other words keep their bits
    }
    if (lane == 0 && p.counters && selected > 0)
      atomicAdd(p.counters + WISE_CTR_SELECTED, static_cast<unsigned long long>(selected));
    return;
  }
  // the arrival goes out before the support stores, which overlap its round trip
  unsigned int *arrive = reinterpret_cast<unsigned int *>(&tag->reserved);
  unsigned int all = 0u;
  if (lane == 0) {
    const unsigned int mine = 1u | (err ? 1u << 8 : 0u) | (static_cast<unsigned int>(selected) << 16);
    all = atomicAdd(arrive, mine) + mine;
  }
  if (!err) {
    uint32_t *sw = p.support + ((static_cast<int64_t>(rp.slot) * p.layers + p.layer) * p.heads + h) * p.words;
    if (rp.eff == WISE_DISCOVER) {
      for (int w = lane; w < p.words; w += 64) sw[w] = w == lane ? nw : 0u;
    } else if (lane < p.words && (nw & ~rp.word) != 0u) {
      sw[lane] = rp.word | nw;  // the other words keep their bits
    }
  }
  if (lane != 0 || static_cast<int>(all & 0xFFu) != p.heads) return;
  atomicExch(arrive, 0u);
  const int err_heads = static_cast<int>((all >> 8) & 0xFFu);
  if (p.counters) {
    atomicAdd(p.counters + WISE_CTR_SELECTED, static_cast<unsigned long long>(all >> 16));
    if (rp.eff == WISE_DISCOVER)
      atomicAdd(p.counters + WISE_CTR_CAUSAL, static_cast<unsigned long long>(nb) * (p.heads - err_heads));
  }
  // a bad page in any head of the row breaks this discovery
  if (rp.eff == WISE_DISCOVER) {
    tag->request = p.row_request[rp.row];
    tag->position = p.row_position[rp.row];
    tag->discoveries = err_heads ? 0 : 1;
  } else {
    tag->discoveries = err_heads ? 0 : tag->discoveries + 1;
  }
}

// MAXB: the most blocks a unit of the launch has (64, or 256 for contexts up
// to 8K); a wave's share of a unit is at most ceil(MAXB / W) list entries.
// The unit a fused workgroup takes.  A launch of per-row modes over at most
// 64 rows takes its rows heaviest first: rows that attend in full (dense,
// discovery) before sparse rows, then longer contexts first, then by index.
// The longest units then start in the first round of workgroups instead of
// queueing behind short ones that happened to come first (the order of a
// longest-processing-time-first schedule).  Other launches take the units in
// index order.  Every workgroup computes the same permutation from the same
// keys (unique, since the row index is part of each), so every unit is taken
// exactly once; the heads of a row stay on consecutive workgroups, spread
// over the XCDs.
__device__ __forceinline__ void fused_unit(const SplitParams &p, int lane, int &r, int &h) {
  const int b = blockIdx.x;
  const int pos = b / p.heads;
  h = b - pos * p.heads;
  r = pos;
  if (p.row_mode == nullptr || p.rows > 64) return;
  uint32_t key = 0xFFFFFFFFu;
  if (lane < p.rows) {
    const int n = min(max(p.ctx_len[lane], 0), kMaxCtx);
    key = (p.row_mode[lane] == WISE_SPARSE ? 1u << 23 : 0u) | (static_cast<uint32_t>(kMaxCtx - n) << 6) |
          static_cast<uint32_t>(lane);
  }
  int rank = 0;
  for (int j = 0; j < p.rows; ++j)
    rank += static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), j)) < key ? 1 : 0;
  const unsigned long long hit = __ballot(lane < p.rows && rank == pos);
  r = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(hit)) - 1);
}

template <bool kBf16, int D, int W, bool kKOnly, int MAXB>
__global__ __launch_bounds__(64 * W) void split_fused_kernel(const SplitParams p) {
  constexpr int kTiles = (MAXB + W - 1) / W > kMaxTilesPerItem ? (MAXB + W - 1) / W : kMaxTilesPerItem;
  static_assert(kTiles <= 64, "one lane per list entry of an item");
  static_assert(W >= 2, "waves 0 and 1 finish the unit");
  __shared__ int s_tiles[W][kTiles];
  __shared__ float s_acc[W * D];
  __shared__ float2 s_ml[W];
  __shared__ float2 s_st[MAXB];
  __shared__ float s_w[W];
  __shared__ uint32_t s_bits[MAXB / 32];
  const int lane = threadIdx.x & 63;
  const int k = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);  // item slot
  int r, h;
  fused_unit(p, lane, r, h);
  const int u = r * p.heads + h;  // unit = (row, head)
  const RowPlan rp = plan_row(p, r, h, lane);
  const int nb = rp.bad ? 0 : (rp.n + kBlock - 1) / kBlock;
  const bool sparse = !rp.bad && rp.eff == WISE_SPARSE;
  uint32_t word = 0u;
  int incl = 0;
  // K-only calls have nothing to do for a row whose discovery window broke
  const int count = (kKOnly && rp.eff == WISE_DENSE) ? 0
                    : sparse                         ? support_scan(rp.word, nb, lane, word, incl)
                                                     : nb;
  // the unit's list entries spread evenly over the workgroup's waves (the
  // partials stay in LDS, so the item size need not match the workspace's)
  const int T = max(1, (count + W - 1) / W);
  const int items = (count + T - 1) / T;
  if (k == 0 && lane == 0 && h == 0 && rp.fallback && p.counters)
    atomicAdd(p.counters + WISE_CTR_FALLBACKS, 1ull);
  const UnitLds lds{s_acc, s_ml, s_st};
  if (k < items)
    run_item<kBf16, D, kKOnly>(p, u, r, h, k, rp.n, sparse, count, word, incl, lane, s_tiles[k], T, &lds);
  __syncthreads();  // every wave of the workgroup reaches this once
  // short units of calls that read V: wave 0 carries the row's arrival
  // (long units: measured 1% slower at 8K, where twice as many workgroups
  // end with the selected-block counter atomics)
  constexpr bool kEarlyArrival = !kKOnly && MAXB <= kMaxFusedBlocks;
  if constexpr (kEarlyArrival) {
    if (k == 0) finish_output_arrive<D>(p, rp, u, h, nb, items, s_acc, s_ml, s_w, lane);
    if (k == 1) finish_row<kKOnly, MAXB, false>(p, rp, u, h, nb, items, s_ml, s_st, s_bits, lane);
  } else {
    if (k == 0) finish_output<D, kKOnly>(p, u, items, s_acc, s_ml, s_w, lane);
    if (k == 1) finish_row<kKOnly, MAXB, true>(p, rp, u, h, nb, items, s_ml, s_st, s_bits, lane);
  }
}

// ---------------------------------------------------------------------------
// Plan kernel (one workgroup) for calls with sparse rows: effective modes,
// per-unit tile counts, the call's item length, per-unit item counts, and
// the compact list of live items, so that the split grid carries no empty
// item slots.  The item length follows the rule of calls with no sparse
// rows, applied to the tiles the call really attends: 32 tiles when the
// launch still has at least kLongItemMinWaves items of 32, else 16 on the
// same condition, else eight.  A launch that large outlasts any one item
// many times over, so a dense row among sparse ones cannot set its length,
// while a smaller launch keeps the eight-tile items the split design
// prescribes.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanRegUnits = 4;  // units per thread whose tile counts stay in registers

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const SplitParams p) {
  // per-wave totals; each array is written once, so no wave can overwrite
  // a total another wave has yet to read
  __shared__ int s_wave_long[2][kPlanThreads / 64];  // items of 32 and of 16 tiles
  __shared__ int s_wave_full[kPlanThreads / 64];     // full-length items
  __shared__ int s_wave_tails[kPlanThreads / 64];    // short last items
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int U = p.rows * p.heads;
  const int per = (U + kPlanThreads - 1) / kPlanThreads;
  const int u0 = min(U, t * per), u1 = min(U, u0 + per);
  // tiles a unit attends (its item count is fixed once the item length is)
  auto unit_tiles = [&](int u) -> int {
    const int r = u / p.heads;
    const int h = u - r * p.heads;
    const RowPlan rp = plan_row(p, r);
    const int nb = rp.bad ? 0 : (rp.n + kBlock - 1) / kBlock;
    int count = nb;
    if (!rp.bad && rp.eff == WISE_SPARSE) {
      // popcount of the unit's support words, eight loads in flight at a time
      const uint32_t *sw = support_words(p, rp.slot, h);
      const int nw = (nb + 31) >> 5;
      count = 0;
      for (int w0 = 0; w0 < nw; w0 += 8) {
        uint32_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = w0 + j < nw ? sw[w0 + j] : 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int valid = nb - 32 * (w0 + j);
          count += __popc(valid < 32 ? x[j] & ((1u << max(valid, 0)) - 1u) : x[j]);
        }
      }
    }
    if (h == 0) {
      p.row_code[r] = encode_row(rp.bad ? kRowError : rp.eff, rp.req);
      p.row_done[r] = 0ull;
      if (rp.fallback && p.counters) atomicAdd(p.counters + WISE_CTR_FALLBACKS, 1ull);
    }
    return count;
  };
  int cnt[kPlanRegUnits];
  int n32 = 0, n16 = 0;
#pragma unroll
  for (int j = 0; j < kPlanRegUnits; ++j) {
    cnt[j] = u0 + j < u1 ? unit_tiles(u0 + j) : 0;
    n32 += (cnt[j] + 31) >> 5;
    n16 += (cnt[j] + 15) >> 4;
  }
  for (int u = u0 + kPlanRegUnits; u < u1; ++u) {
    const int c = unit_tiles(u);
    p.unit_items[u] = c;  // tile count until the item length is known
    n32 += (c + 31) >> 5;
    n16 += (c + 15) >> 4;
  }
  int T = p.tiles_per_item;
  if (p.long_items) {
    const int w32 = __builtin_amdgcn_readlane(wave_inclusive_scan(n32, lane), 63);
    const int w16 = __builtin_amdgcn_readlane(wave_inclusive_scan(n16, lane), 63);
    if (lane == 0) {
      s_wave_long[0][t >> 6] = w32;
      s_wave_long[1][t >> 6] = w16;
    }
    __syncthreads();
    int tot32 = 0, tot16 = 0;
    for (int wv = 0; wv < kPlanThreads / 64; ++wv) {
      tot32 += s_wave_long[0][wv];
      tot16 += s_wave_long[1][wv];
    }
    T = tot32 >= kLongItemMinWaves ? 32 : tot16 >= kLongItemMinWaves ? 16 : T;
  }
  // The list holds every unit's full-length items first, in unit order,
  // then the shorter last items of the units whose tile count T does not
  // divide.
  int full = 0, tails = 0;
#pragma unroll
  for (int j = 0; j < kPlanRegUnits; ++j) {
    full += cnt[j] / T;
    tails += cnt[j] % T != 0;
  }
  for (int u = u0 + kPlanRegUnits; u < u1; ++u) {
    const int c = p.unit_items[u];
    full += c / T;
    tails += c % T != 0;
  }
  // exclusive scans of the per-thread full and tail counts: within each
  // wave, then the totals of the waves before it
  const int incl_full = wave_inclusive_scan(full, lane);
  const int incl_tails = wave_inclusive_scan(tails, lane);
  if (lane == 63) {
    s_wave_full[t >> 6] = incl_full;
    s_wave_tails[t >> 6] = incl_tails;
  }
  __syncthreads();
  int before_full = 0, all_full = 0, before_tails = 0, all_tails = 0;
  for (int wv = 0; wv < kPlanThreads / 64; ++wv) {
    const bool earlier = wv < (t >> 6);
    before_full += earlier ? s_wave_full[wv] : 0;
    before_tails += earlier ? s_wave_tails[wv] : 0;
    all_full += s_wave_full[wv];
    all_tails += s_wave_tails[wv];
  }
  int at_full = before_full + incl_full - full;
  int at_tail = all_full + before_tails + incl_tails - tails;
  auto list_unit = [&](int u, int c) {
    const int nf = c / T;
    for (int kk = 0; kk < nf; ++kk) p.item_list[at_full + kk] = (static_cast<uint32_t>(u) << kItemBits) | kk;
    at_full += nf;
    if (nf * T < c) p.item_list[at_tail++] = (static_cast<uint32_t>(u) << kItemBits) | nf;
    p.unit_items[u] = (c + T - 1) / T;
  };
#pragma unroll
  for (int j = 0; j < kPlanRegUnits; ++j)
    if (u0 + j < u1) list_unit(u0 + j, cnt[j]);
  for (int u = u0 + kPlanRegUnits; u < u1; ++u) list_unit(u, p.unit_items[u]);
  if (t == 0) {
    p.n_items[0] = all_full + all_tails;
    p.n_items[1] = T;
  }
}

// ---------------------------------------------------------------------------
// Listed grid: persistent waves striding over the compact item list (full-
// length items first, so each stride of the grid takes items of about one
// length).
// ---------------------------------------------------------------------------
template <bool kBf16, int D>
__global__ __launch_bounds__(64 * kWavesPerGroup) __attribute__((amdgpu_waves_per_eu(Geo<kBf16, D>::kListedWavesPerEU)))
void split_listed_kernel(const SplitParams p) {
  __shared__ int s_tiles[kWavesPerGroup][kLongTiles];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stride = gridDim.x * kWavesPerGroup;
  const int n_items = p.n_items[0];
  const int T = p.n_items[1];  // the item length the plan kernel chose
  int i = blockIdx.x * kWavesPerGroup + wave;
  uint32_t it_next = i < n_items ? p.item_list[i] : 0u;
  for (; i < n_items; i += stride) {
    // this wave's next list entry is fetched one item ahead
    const uint32_t it = it_next;
    if (i + stride < n_items) it_next = p.item_list[i + stride];
    const int u = static_cast<int>(it >> kItemBits);
    const int k = static_cast<int>(it & ((1u << kItemBits) - 1u));
    const int r = u / p.heads;
    const int h = u - r * p.heads;
    const int n = p.ctx_len[r];
    const int code = p.row_code[r];
    const int slot = p.slot_of_row ? p.slot_of_row[r] : r;
    // the support word is loaded with the context and the row code, before
    // either is known (a slot out of range is not read; only sparse rows use
    // the word, and support_scan drops the words past the context)
    const int nb = (n + kBlock - 1) / kBlock;
    uint32_t raw = 0u;
    if (slot >= 0 && slot < p.slots && lane < p.words) raw = support_words(p, slot, h)[lane];
    const bool sparse = (code & 0xF) == WISE_SPARSE;
    uint32_t word = 0u;
    int incl = 0;
    const int count = sparse ? support_scan(raw, nb, lane, word, incl) : nb;
    run_item<kBf16, D, false>(p, u, r, h, k, n, sparse, count, word, incl, lane, s_tiles[wave], T, nullptr,
                              T > 8);
  }
}

}  // namespace

// Resident workgroups of the listed split kernel on one CU of the current
// device (occupancy query, cached per device and instantiation).
template <bool kBf16, int D>
static int listed_groups_per_cu() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, split_listed_kernel<kBf16, D>, 64 * kWavesPerGroup, 0) !=
            hipSuccess ||
        n < 1)
      return -1;
    cache[dev] = n;
  }
  return cache[dev];
}

// Launch of one split kernel.  With timing events, through the launch that
// stamps them with the kernel's own start and stop (hipExtLaunchKernel), so
// they measure the kernel rather than the queue around it.
template <typename... Args, typename F = void (*)(Args...)>
static hipError_t launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t ev_begin,
                               hipEvent_t ev_end, Args... args) {
  if (ev_begin)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev_begin, ev_end, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  return hipGetLastError();
}

// One workgroup per unit, p.fused_waves waves; units of up to 64 blocks use
// the short shape (one block per lane in the selection), longer ones the
// long shape.
template <bool kBf16, int D, bool kKOnly, int MAXB>
static hipError_t launch_fused_w(const SplitParams &p, hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream) {
  const dim3 units(static_cast<unsigned>(p.rows) * p.heads);
  switch (p.fused_waves) {
    case 4:
      if constexpr (MAXB <= 64)
        return launch_timed(split_fused_kernel<kBf16, D, 4, kKOnly, MAXB>, units, dim3(64 * 4), stream, ev_begin,
                            ev_end, p);
      break;
    case 8:
      return launch_timed(split_fused_kernel<kBf16, D, 8, kKOnly, MAXB>, units, dim3(64 * 8), stream, ev_begin,
                          ev_end, p);
    case 16:
      // fp32 at head_dim 128 needs more than the 128 registers a 16-wave workgroup allows
      if constexpr (kBf16 || D == 64)
        return launch_timed(split_fused_kernel<kBf16, D, 16, kKOnly, MAXB>, units, dim3(64 * 16), stream,
                            ev_begin, ev_end, p);
      break;
  }
  return hipErrorInvalidValue;
}

template <bool kBf16, int D>
static hipError_t launch_fused(const SplitParams &p, bool k_only, hipEvent_t ev_begin, hipEvent_t ev_end,
                               hipStream_t stream) {
  const bool wide = p.max_blocks > kMaxFusedBlocks;
  if (k_only)
    return wide ? launch_fused_w<kBf16, D, true, kWideFusedBlocks>(p, ev_begin, ev_end, stream)
                : launch_fused_w<kBf16, D, true, kMaxFusedBlocks>(p, ev_begin, ev_end, stream);
  return wide ? launch_fused_w<kBf16, D, false, kWideFusedBlocks>(p, ev_begin, ev_end, stream)
              : launch_fused_w<kBf16, D, false, kMaxFusedBlocks>(p, ev_begin, ev_end, stream);
}

template <bool kBf16, int D>
static hipError_t launch_typed(const SplitParams &p, bool listed, bool k_only, bool fused, int cus,
                               hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream) {
  const dim3 block(64 * kWavesPerGroup);
  if (listed) {
    const int per_cu = listed_groups_per_cu<kBf16, D>();
    if (per_cu < 1) return hipErrorInvalidValue;
    const int64_t slot_groups =
        (static_cast<int64_t>(p.rows) * p.heads * p.items_per_unit + kWavesPerGroup - 1) / kWavesPerGroup;
    const int groups = static_cast<int>(std::min<int64_t>(slot_groups, static_cast<int64_t>(cus) * per_cu));
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_timed(split_listed_kernel<kBf16, D>, dim3(groups), block, stream, ev_begin, ev_end, p);
  }
  if (fused) return launch_fused<kBf16, D>(p, k_only, ev_begin, ev_end, stream);
  const dim3 grid(static_cast<unsigned>(p.rows) * p.heads * p.chunk_groups);
  if (k_only) return launch_timed(split_static_kernel<kBf16, D, true>, grid, block, stream, ev_begin, ev_end, p);
  return launch_timed(split_static_kernel<kBf16, D, false>, grid, block, stream, ev_begin, ev_end, p);
}

hipError_t launch_split(const SplitParams &p, int dtype, int head_dim, bool listed, bool k_only, bool fused,
                        int cus, hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream) {
  if (listed && (k_only || fused)) return hipErrorInvalidValue;  // K-only and fused calls use the static grid
  if (fused && (p.fused_waves < 1 || p.max_blocks > kWideFusedBlocks || (k_only && !p.lse)))
    return hipErrorInvalidValue;
  if (dtype == WISE_BF16 && head_dim == 128)
    return launch_typed<true, 128>(p, listed, k_only, fused, cus, ev_begin, ev_end, stream);
  if (dtype == WISE_BF16 && head_dim == 64)
    return launch_typed<true, 64>(p, listed, k_only, fused, cus, ev_begin, ev_end, stream);
  if (dtype == WISE_F32 && head_dim == 128)
    return launch_typed<false, 128>(p, listed, k_only, fused, cus, ev_begin, ev_end, stream);
  if (dtype == WISE_F32 && head_dim == 64)
    return launch_typed<false, 64>(p, listed, k_only, fused, cus, ev_begin, ev_end, stream);
  return hipErrorInvalidValue;
}

}  // namespace wise
