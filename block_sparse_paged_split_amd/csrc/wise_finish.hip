// Finish kernel: split merge, eta selection, union, support bookkeeping.
//
// Method: WISE pull request page (vllm-rlt pull 143).  "What changes": a
// second kernel combines the split partials and picks the support of the
// discovery rows; the support is a bitmask indexed by (slot, layer, head,
// block) and carries the request and position it was found for.
// "Summary": 32-token blocks and a cumulative-mass target eta of 0.95.  The
// review thread and the author's reply on density: a union depth ORs its
// pick into the earlier one, and the density count takes the first depth's
// pick and causal blocks, then only the bits a union depth newly sets.
//
// One workgroup per row for units of up to 64 blocks (a row with more than
// 16 heads takes several), one per 4 heads for longer units; one wave64 per
// (row, head):
//  1. merge the unit's items: M = max m_i, w_i = 2^(m_i - M),
//     L = sum l_i w_i, out = sum acc_i w_i / L (fixed summation orders; the
//     loads of up to eight items are in flight together);
//  2. discovery units: block mass p_b = l_b 2^(m_b - M) / L (fp32) from the
//     tile stats; 64-bit keys (mass bits, ~block index) sorted descending by
//     a bitonic network held in registers (lane l owns sorted positions
//     [l*KPL, l*KPL+KPL)); running sum in fp64 (per-lane run, then a wave
//     scan); K = the first prefix reaching eta, at least 1, all blocks if
//     rounding never reaches eta;
//  3. write (DISCOVER) or OR (DISCOVER_UNION) the unit's support words; the
//     heads of the row add (error heads, newly selected blocks) through LDS
//     and one wave updates the row's tag and the density counters.  Only a
//     row split over several workgroups needs a device-scope atomic (an
//     arrival word per row; the last workgroup to arrive does the update).
// Cross-lane exchanges within 16 lanes use DPP; every load that does not
// depend on arithmetic (partials, tile stats, old support words) is issued
// before any of it.
#include "wise_internal.h"
#include "wise_select.h"

namespace wise {

namespace {

using namespace sel;

constexpr int kHeadsPerGroup = 16;  // waves (heads) per finish workgroup of short units
constexpr float kLog2e = 1.44269504088896340736f;

// Row facts the finish of one unit needs (all from scalar loads issued together).
struct UnitInfo {
  int u, r, h, eff, req, items, nb, slot;
  bool row_bad;
};

struct UnitResult {
  bool err;      // the unit read a bad page (its output is NaN)
  int selected;  // blocks this unit newly selected
};

// Finish of one unit by one wave.  No workgroup barrier in here: the waves
// of a workgroup take different paths through it.
template <int KPL, int NPOS>
__device__ __forceinline__ UnitResult finish_unit(const FinishParams &p, const UnitInfo &ui, float *s_w,
                                                  uint32_t *s_bits) {
  const int lane = threadIdx.x & (kLanes - 1);
  const int items = ui.items;
  const int64_t base = static_cast<int64_t>(ui.u) * p.items_per_unit;
  const int D = p.head_dim;
  const bool stateful = p.support != nullptr && !ui.row_bad && ui.req != WISE_DENSE;
  const bool discover = stateful && (ui.eff == WISE_DISCOVER || ui.eff == WISE_DISCOVER_UNION);
  // LSE route: no output; a row whose discovery window broke has nothing to do
  const bool lse_mode = p.lse != nullptr;
  if (lse_mode && !discover && !ui.row_bad) return UnitResult{false, 0};

  // ---- loads: partials, tile stats, old support words (and the LSE) ----
  // (the partials of kUnroll items are in flight at a time; units of long
  // rows have many items, so they keep more of them in flight)
  constexpr int kUnroll = KPL >= 2 ? 16 : 8;
  constexpr int kDims = 2;  // head_dim <= 2 * 64
  const float *acc = p.part_acc + base * D;
  float v[kDims][kUnroll];
#pragma unroll
  for (int q = 0; q < kDims; ++q) {
    const int dd = lane + q * kLanes;
#pragma unroll
    for (int t = 0; t < kUnroll; ++t) v[q][t] = (!lse_mode && dd < D && t < items) ? acc[t * D + dd] : 0.0f;
  }
  const float lse = lse_mode ? p.lse[ui.u] : 0.0f;
  float2 ml_own[kMaxItemsPerUnit / kLanes];
#pragma unroll
  for (int c = 0; c < kMaxItemsPerUnit / kLanes; ++c) {
    const int i = c * kLanes + lane;
    ml_own[c] = i < items ? p.part_ml[base + i] : make_float2(-INFINITY, 0.0f);
  }
  float2 st[KPL];
  const float2 *stp = p.stats + static_cast<int64_t>(ui.u) * p.max_blocks;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int b = lane * KPL + j;
    st[j] = (discover && b < ui.nb) ? stp[b] : make_float2(0.0f, 0.0f);
  }
  uint32_t *sw = discover ? p.support + ((static_cast<int64_t>(ui.slot) * p.layers + p.layer) * p.heads + ui.h) *
                                             p.words
                          : nullptr;
  const uint32_t old_word = (discover && ui.eff == WISE_DISCOVER_UNION && lane < p.words) ? sw[lane] : 0u;

  // ---- 1. merge: M, w_i, L, out (fixed orders) ----
  float M = -INFINITY;
  bool bad_item = false;
#pragma unroll
  for (int c = 0; c < kMaxItemsPerUnit / kLanes; ++c) {
    bad_item |= ml_own[c].y < 0.0f;
    M = fmaxf(M, ml_own[c].x);
  }
  M = wave_max(M);
  bool err = items == 0 || __builtin_amdgcn_ballot_w64(bad_item) != 0ull;
  float L = 1.0f;
  if (lse_mode) {
    // masses relative to the external kernel's normaliser: M = lse in base-2 units, L = 1
    err = err || !__builtin_isfinite(lse);
    M = lse * kLog2e;
  } else {
    float Lp = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxItemsPerUnit / kLanes; ++c) {
      const int i = c * kLanes + lane;
      if (i < items) {
        const float w = __builtin_amdgcn_exp2f(ml_own[c].x - M);
        s_w[i] = w;
        Lp = fmaf(ml_own[c].y, w, Lp);
      }
    }
    L = wave_sum(Lp);
  }
  if (discover)
    for (int w = lane; w < kMaxWords; w += kLanes) s_bits[w] = 0u;
  wave_lds_sync();
  if (!lse_mode) {
#pragma unroll
    for (int q = 0; q < kDims; ++q) {
      const int dd = lane + q * kLanes;
      if (dd >= D) break;
      float a = 0.0f;
#pragma unroll
      for (int t = 0; t < kUnroll; ++t)
        if (t < items) a = fmaf(v[q][t], s_w[t], a);
      for (int i0 = kUnroll; i0 < items; i0 += kUnroll) {
        float x[kUnroll];
#pragma unroll
        for (int t = 0; t < kUnroll; ++t) x[t] = i0 + t < items ? acc[(i0 + t) * D + dd] : 0.0f;
#pragma unroll
        for (int t = 0; t < kUnroll; ++t)
          if (i0 + t < items) a = fmaf(x[t], s_w[i0 + t], a);
      }
      p.out[static_cast<int64_t>(ui.u) * D + dd] = err ? __builtin_nanf("") : a / L;
    }
  }
  if (err && lane == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, 1ull);

  UnitResult res{err, 0};
  if (!discover || err) return res;

  // ---- 2. eta selection, 3. support write / union ----
  const int K = select_eta<KPL, NPOS>(st, p.eta, ui.nb, M, L, lane, s_bits);
  wave_lds_sync();
  int added = 0;
  for (int w = lane; w < p.words; w += kLanes) {
    const uint32_t nw = w < kMaxWords ? s_bits[w] : 0u;
    if (ui.eff == WISE_DISCOVER) {
      sw[w] = nw;
    } else {
      const uint32_t old = w == lane ? old_word : sw[w];
      sw[w] = old | nw;
      added += __popc(nw & ~old);
    }
  }
  res.selected = ui.eff == WISE_DISCOVER ? K : wave_sum_int(added);
  return res;
}

// The smallest sort size holding the unit's nb blocks, up to KMAX per lane.
template <int KPL, int KMAX>
__device__ __forceinline__ UnitResult finish_sized(const FinishParams &p, const UnitInfo &ui, float *s_w,
                                                   uint32_t *s_bits) {
  if constexpr (KPL >= KMAX) {
    return finish_unit<KMAX, KMAX * kLanes>(p, ui, s_w, s_bits);
  } else {
    if (ui.nb <= KPL * kLanes) return finish_unit<KPL, KPL * kLanes>(p, ui, s_w, s_bits);
    return finish_sized<2 * KPL, KMAX>(p, ui, s_w, s_bits);
  }
}

// Tag and density counters of a discovery row once all of its heads are
// done: err_heads of them read a bad page, `selected` blocks were newly set.
__device__ __forceinline__ void row_bookkeeping(const FinishParams &p, const UnitInfo &ui, int err_heads,
                                                unsigned long long selected) {
  wise_tag *tag = p.tags + static_cast<int64_t>(ui.slot) * p.layers + p.layer;
  if (p.counters) {
    atomicAdd(p.counters + WISE_CTR_SELECTED, selected);
    if (ui.eff == WISE_DISCOVER)
      atomicAdd(p.counters + WISE_CTR_CAUSAL, static_cast<unsigned long long>(ui.nb) * (p.heads - err_heads));
  }
  // a bad page in any head of the row breaks this discovery
  if (ui.eff == WISE_DISCOVER) {
    tag->request = p.row_request[ui.r];
    tag->position = p.row_position[ui.r];
    tag->discoveries = err_heads ? 0 : 1;
  } else {
    tag->discoveries = err_heads ? 0 : tag->discoveries + 1;
  }
}

// Waves per workgroup for units of up to 64*KMAX blocks: 16 (a row of up to
// 16 heads in one workgroup) while a wave fits 128 registers, else 4.
// Units of up to 64 blocks (few items each) finish 16 heads per workgroup;
// longer units, whose merges take longer, spread a row over workgroups of 4
// heads so that every CU takes a share.
constexpr int waves_for(int kmax) { return kmax <= 1 ? kHeadsPerGroup : 4; }

template <int KMAX>
__global__ __launch_bounds__(kLanes *waves_for(KMAX)) void finish_kernel(const FinishParams p, int waves,
                                                                         int groups) {
  __shared__ float s_w[kHeadsPerGroup][kMaxItemsPerUnit];
  __shared__ uint32_t s_bits[kHeadsPerGroup][kMaxWords];
  __shared__ int s_err[kHeadsPerGroup];
  __shared__ int s_sel[kHeadsPerGroup];

  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  UnitInfo ui;
  ui.r = blockIdx.x / groups;
  const int g = blockIdx.x - ui.r * groups;
  ui.h = g * waves + wave;
  const bool active = ui.h < p.heads;
  ui.u = ui.r * p.heads + (active ? ui.h : 0);
  // independent scalar loads, issued together
  const int code = p.row_code[ui.r];
  const int items = p.unit_items[ui.u];
  const int n = p.ctx_len[ui.r];
  const int slot = (p.support && p.slot_of_row) ? p.slot_of_row[ui.r] : ui.r;
  ui.eff = code & 0xF;
  ui.req = (code >> 4) & 0xF;
  ui.row_bad = ui.eff == kRowError;
  ui.items = ui.row_bad ? 0 : items;
  ui.nb = ui.row_bad ? 0 : (n + kBlock - 1) / kBlock;
  ui.slot = slot;

  UnitResult res{false, 0};
  if (active) {
    float *sw = s_w[wave];
    uint32_t *sb = s_bits[wave];
    if (ui.nb <= 16) res = finish_unit<1, 16>(p, ui, sw, sb);
    else if (ui.nb <= 32) res = finish_unit<1, 32>(p, ui, sw, sb);
    else res = finish_sized<1, KMAX>(p, ui, sw, sb);
  }
  if (lane == 0) {
    s_err[wave] = res.err ? 1 : 0;
    s_sel[wave] = res.selected;
  }
  __syncthreads();  // reached once by every wave of the workgroup

  const bool stateful = p.support != nullptr && !ui.row_bad && ui.req != WISE_DENSE;
  if (!stateful || wave != 0 || lane != 0) return;
  if (ui.eff != WISE_DISCOVER && ui.eff != WISE_DISCOVER_UNION) {
    // a union row whose discovery window is broken ran dense: the rest of
    // this token runs dense too
    if (ui.req == WISE_DISCOVER_UNION && g == 0)
      p.tags[static_cast<int64_t>(ui.slot) * p.layers + p.layer].discoveries = 0;
    return;
  }
  int err_heads = 0;
  unsigned long long selected = 0ull;
  for (int w = 0; w < waves; ++w) {
    err_heads += s_err[w];
    selected += static_cast<unsigned long long>(s_sel[w]);
  }
  if (groups == 1) {
    row_bookkeeping(p, ui, err_heads, selected);
    return;
  }
  // the row spans several workgroups: the last one to arrive does it
  const unsigned long long mine = 1ull | (static_cast<unsigned long long>(err_heads) << 16) | (selected << 32);
  const unsigned long long all = atomicAdd(p.row_done + ui.r, mine) + mine;
  if (static_cast<int>(all & 0xFFFFull) != groups) return;
  row_bookkeeping(p, ui, static_cast<int>((all >> 16) & 0xFFFFull), all >> 32);
}

}  // namespace

namespace {
template <int KMAX>
hipError_t launch_finish_typed(const FinishParams &p, hipStream_t stream) {
  constexpr int kWaves = waves_for(KMAX);
  const int waves = p.heads < kWaves ? p.heads : kWaves;
  const int groups = (p.heads + waves - 1) / waves;
  hipLaunchKernelGGL(finish_kernel<KMAX>, dim3(static_cast<unsigned>(p.rows) * groups), dim3(kLanes * waves), 0,
                     stream, p, waves, groups);
  return hipGetLastError();
}
}  // namespace

// The kernel is specialised on the largest unit the call can hold (from the
// host-known block bound), so short contexts do not pay for the registers
// of long ones.
hipError_t launch_finish(const FinishParams &p, hipStream_t stream) {
  const int nb = p.max_blocks;
  if (nb <= kLanes) return launch_finish_typed<1>(p, stream);
  if (nb <= 2 * kLanes) return launch_finish_typed<2>(p, stream);
  if (nb <= 4 * kLanes) return launch_finish_typed<4>(p, stream);
  if (nb <= 8 * kLanes) return launch_finish_typed<8>(p, stream);
  if (nb <= 16 * kLanes) return launch_finish_typed<16>(p, stream);
  return launch_finish_typed<32>(p, stream);
}

}  // namespace wise
