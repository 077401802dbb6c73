// Finish kernel: split merge, eta selection, union, support bookkeeping.
//
// WISE pull request page (vllm-rlt pull 143): "What changes" -- a finish
// kernel merges the splits and runs the selection for discovery rows; the
// support bitmask is [slot, layer, head, block] and tagged with (request,
// position); "Summary" -- B = 32 blocks and the eta = 0.95 cumulative-mass
// rule; review thread and the author's reply -- a union depth ORs its
// selection into the previous support, and the density count adds, for the
// first discovery depth, its selection and the causal blocks, and for a
// union depth only the newly set blocks.
//
// One wave64 per (row, head):
//  1. merge the unit's items: M = max m_i, w_i = 2^(m_i - M),
//     L = sum l_i w_i, out = sum acc_i w_i / L (fixed summation orders; the
//     loads of up to eight items are in flight together);
//  2. discovery units: block mass p_b = l_b 2^(m_b - M) / L (fp32) from the
//     tile stats; 64-bit keys (mass bits, ~block index) sorted descending by
//     a bitonic network held in registers (lane l owns sorted positions
//     [l*KPL, l*KPL+KPL)); running sum in fp64 (per-lane run, then a wave
//     scan); K = the first prefix reaching eta, at least 1, all blocks if
//     rounding never reaches eta;
//  3. write (DISCOVER) or OR (DISCOVER_UNION) the unit's support words; each
//     head adds (1 arrival, error flag, selected blocks) to its row's atomic
//     word, and the last head to arrive updates the row's tag and adds the
//     row's totals to the density counters (one global atomic per row, not
//     per head).
#include "wise_internal.h"

namespace wise {

namespace {

constexpr int kLanes = 64;
constexpr int kUnroll = 8;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ double wave_inclusive_scan(double x, int lane) {
#pragma unroll
  for (int d = 1; d < kLanes; d <<= 1) {
    const double y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}
__device__ __forceinline__ unsigned long long shfl_xor64(unsigned long long x, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), m);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ float key_mass(unsigned long long key) {
  return __uint_as_float(static_cast<uint32_t>(key >> 32));
}

// Block masses of one discovery unit from its tile stats (loaded by the
// caller, lane l holding blocks l*KPL .. l*KPL+KPL-1), sorted descending by
// (mass, ~block index) with a bitonic network held in registers; the fp64
// running sum picks K; the selected blocks' bits are ORed into s_bits.
template <int KPL>
__device__ __forceinline__ int select_eta(const float2 (&st)[KPL], float eta, int nb, float M, float L, int lane,
                                          uint32_t *s_bits) {
  unsigned long long key[KPL];
  const float invL = 1.0f / L;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int b = lane * KPL + j;
    key[j] = 0ull;  // padding sorts after every block
    if (b < nb) {
      const float mass = st[j].y * __builtin_amdgcn_exp2f(st[j].x - M) * invL;
      key[j] = (static_cast<unsigned long long>(__float_as_uint(mass)) << 32) |
               static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(b));
    }
  }
  // bitonic network over positions e = lane*KPL + j, descending keys
  constexpr int N = kLanes * KPL;
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < KPL) {
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          if (j & stride) continue;
          const int e = lane * KPL + j;
          const bool desc = (e & size) == 0;
          const unsigned long long a = key[j], b = key[j | stride];
          const bool swap = (a < b) == desc;
          key[j] = swap ? b : a;
          key[j | stride] = swap ? a : b;
        }
      } else {
        const int lm = stride / KPL;
        const bool lower = (lane & lm) == 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int e = lane * KPL + j;
          const bool desc = (e & size) == 0;
          const unsigned long long a = key[j], b = shfl_xor64(a, lm);
          const unsigned long long hi = a > b ? a : b, lo = a > b ? b : a;
          key[j] = (lower == desc) ? hi : lo;
        }
      }
    }
  }
  // fp64 running sum in sorted order
  double part = 0.0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) part += static_cast<double>(key_mass(key[j]));
  const double incl = wave_inclusive_scan(part, lane);
  const double prev = __shfl_up(incl, 1);
  double run = lane ? prev : 0.0;
  int kfound = nb;
  bool hit = false;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    run += static_cast<double>(key_mass(key[j]));
    if (!hit && run >= static_cast<double>(eta)) {
      kfound = lane * KPL + j + 1;
      hit = true;
    }
  }
  const unsigned long long hits = __builtin_amdgcn_ballot_w64(hit);
  const int K = min(nb, hits ? __builtin_amdgcn_readlane(kfound, __builtin_ctzll(hits)) : nb);
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    if (lane * KPL + j < K) {
      const uint32_t b = 0xFFFFFFFFu - static_cast<uint32_t>(key[j]);
      atomicOr(&s_bits[b >> 5], 1u << (b & 31));
    }
  }
  return K;
}

// Row facts the finish of one unit needs (all from scalar loads issued together).
struct UnitInfo {
  int u, r, h, eff, req, items, nb, slot;
  bool row_bad;
};

// Finish of one unit.  Every load that does not depend on arithmetic (item
// partials, tile stats, old support words) is issued up front, so the
// discovery path waits on memory about once instead of once per step.
template <int KPL>
__device__ __forceinline__ void finish_unit(const FinishParams &p, const UnitInfo &ui, float *s_w,
                                            uint32_t *s_bits) {
  const int lane = threadIdx.x;
  const int items = ui.items;
  const int64_t base = static_cast<int64_t>(ui.u) * p.items_per_unit;
  const int D = p.head_dim;
  const bool stateful = p.support != nullptr && !ui.row_bad && ui.req != WISE_DENSE;
  const bool discover = stateful && (ui.eff == WISE_DISCOVER || ui.eff == WISE_DISCOVER_UNION);

  // ---- loads: partials, tile stats, old support words ----
  constexpr int kDims = 2;  // head_dim <= 2 * 64
  const float *acc = p.part_acc + base * D;
  float v[kDims][kUnroll];
#pragma unroll
  for (int q = 0; q < kDims; ++q) {
    const int dd = lane + q * kLanes;
#pragma unroll
    for (int t = 0; t < kUnroll; ++t) v[q][t] = (dd < D && t < items) ? acc[t * D + dd] : 0.0f;
  }
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
  const bool err = items == 0 || __builtin_amdgcn_ballot_w64(bad_item) != 0ull;
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
  const float L = wave_sum(Lp);
  if (discover)
    for (int w = lane; w < kMaxWords; w += kLanes) s_bits[w] = 0u;
  __syncthreads();
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
  if (err && lane == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, 1ull);

  if (!stateful) return;
  const int slot = ui.slot;
  wise_tag *tag = p.tags + static_cast<int64_t>(slot) * p.layers + p.layer;
  if (!discover) {
    // a union row whose discovery window is broken ran dense: the rest of
    // this token runs dense too
    if (ui.req == WISE_DISCOVER_UNION && ui.h == 0 && lane == 0) tag->discoveries = 0;
    return;
  }

  // ---- 2. eta selection, 3. support write / union ----
  int selected = 0;
  if (!err) {
    const int K = select_eta<KPL>(st, p.eta, ui.nb, M, L, lane, s_bits);
    __syncthreads();
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
    selected = ui.eff == WISE_DISCOVER ? K : wave_sum_int(added);
  }

  // ---- the row's tag and density counts: by the last of its heads to arrive ----
  if (lane != 0) return;
  const unsigned long long mine =
      1ull | (err ? (1ull << 16) : 0ull) | (static_cast<unsigned long long>(selected) << 32);
  const unsigned long long all = atomicAdd(p.row_done + ui.r, mine) + mine;
  if (static_cast<int>(all & 0xFFFFull) != p.heads) return;
  const int err_heads = static_cast<int>((all >> 16) & 0xFFFFull);
  if (p.counters) {
    atomicAdd(p.counters + WISE_CTR_SELECTED, all >> 32);
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

__global__ __launch_bounds__(kLanes) void finish_kernel(const FinishParams p) {
  __shared__ float s_w[kMaxItemsPerUnit];
  __shared__ uint32_t s_bits[kMaxWords];
  UnitInfo ui;
  ui.u = blockIdx.x;
  ui.r = ui.u / p.heads;
  ui.h = ui.u - ui.r * p.heads;
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
  if (ui.nb <= kLanes) finish_unit<1>(p, ui, s_w, s_bits);
  else if (ui.nb <= 2 * kLanes) finish_unit<2>(p, ui, s_w, s_bits);
  else if (ui.nb <= 4 * kLanes) finish_unit<4>(p, ui, s_w, s_bits);
  else if (ui.nb <= 8 * kLanes) finish_unit<8>(p, ui, s_w, s_bits);
  else if (ui.nb <= 16 * kLanes) finish_unit<16>(p, ui, s_w, s_bits);
  else finish_unit<32>(p, ui, s_w, s_bits);
}

}  // namespace

hipError_t launch_finish(const FinishParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(finish_kernel, dim3(static_cast<unsigned>(p.rows) * p.heads), dim3(kLanes), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wise
