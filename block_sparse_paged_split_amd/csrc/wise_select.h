// Cross-lane helpers and the eta selection of one unit by one wave64,
// shared by the finish kernel and the fused split + finish kernel.
//
// WISE pull request page (vllm-rlt pull 143), "Summary": the support is the
// fewest 32-token blocks, heaviest first, whose softmax mass reaches eta.
// Block mass p_b = l_b 2^(m_b - M) / L (fp32); 64-bit keys (mass bits,
// ~block index) sorted descending by a bitonic network held in registers
// (lane l owns sorted positions [l*KPL, l*KPL+KPL)); running sum in fp64;
// K = the first prefix reaching eta, at least 1, all blocks if rounding never
// reaches eta.
#ifndef WISE_SELECT_H
#define WISE_SELECT_H

#include "wise_internal.h"

namespace wise {
namespace sel {

constexpr int kLanes = 64;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, true));
}
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1]; row_shr:n (lane i reads
// lane i-n of its 16-lane row, 0 where that leaves the row); row_ror:n (lane
// i reads lane (i-n) mod 16 of its row).
constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128, kRowRor12 = 0x12C;

// Value held by lane (lane ^ M).  For M = 16 and 32, v_permlane16_swap
// (v_permlane32_swap) with both operands x returns x of the lower lane of
// each pair (lane with bit M clear) first and x of the upper lane second, in
// both lanes of the pair; each lane keeps its partner's.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lane) {
  if constexpr (M == 16 || M == 32) {
    const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & M) ? r[0] : r[1];
  } else if constexpr (M == 1) {
    return dpp32<kQuadSwap1>(x);
  } else if constexpr (M == 2) {
    return dpp32<kQuadSwap2>(x);
  } else if constexpr (M == 4) {
    const uint32_t down = dpp32<kRowRor4>(x), up = dpp32<kRowRor12>(x);
    return (lane & 4) ? down : up;
  } else if constexpr (M == 8) {
    return dpp32<kRowRor8>(x);
  } else {
    static_assert(M < 0, "lane distance must be 1, 2, 4, 8, 16 or 32");
    return x;
  }
}
template <int M>
__device__ __forceinline__ unsigned long long xor_lane64(unsigned long long x, int lane) {
  const uint32_t lo = xor_lane<M>(static_cast<uint32_t>(x), lane);
  const uint32_t hi = xor_lane<M>(static_cast<uint32_t>(x >> 32), lane);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// All-lane reductions: rotations within each 16-lane row, then the four row
// results combined in a fixed order (every lane returns the same bits).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __uint_as_float(dpp32<kRowRor8>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp32<kRowRor4>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp32<kRowRor2>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp32<kRowRor1>(__float_as_uint(x))));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += __uint_as_float(dpp32<kRowRor8>(__float_as_uint(x)));
  x += __uint_as_float(dpp32<kRowRor4>(__float_as_uint(x)));
  x += __uint_as_float(dpp32<kRowRor2>(__float_as_uint(x)));
  x += __uint_as_float(dpp32<kRowRor1>(__float_as_uint(x)));
  return ((lane_f(x, 0) + lane_f(x, 16)) + lane_f(x, 32)) + lane_f(x, 48);
}
__device__ __forceinline__ int wave_sum_int(int x) {
  x += static_cast<int>(dpp32<kRowRor8>(static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp32<kRowRor4>(static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp32<kRowRor2>(static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp32<kRowRor1>(static_cast<uint32_t>(x)));
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
         __builtin_amdgcn_readlane(x, 48);
}

template <int CTRL>
__device__ __forceinline__ double dpp64(double x) {
  const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(x));
  const uint32_t lo = dpp32<CTRL>(static_cast<uint32_t>(b));
  const uint32_t hi = dpp32<CTRL>(static_cast<uint32_t>(b >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
__device__ __forceinline__ double lane_d(double x, int l) {
  const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(x));
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(b), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), l);
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
// Exclusive prefix sum over lanes 0..lane-1: a shift scan within each
// 16-lane row, then the totals of the lower rows added in row order.
__device__ __forceinline__ double wave_exclusive_scan(double x, int lane) {
  double s = x;
  s += dpp64<kRowShr1>(s);
  s += dpp64<kRowShr2>(s);
  s += dpp64<kRowShr4>(s);
  s += dpp64<kRowShr8>(s);
  const double t0 = lane_d(s, 15), t1 = lane_d(s, 31), t2 = lane_d(s, 47);
  const int row = lane >> 4;
  double off = 0.0;
  if (row >= 1) off += t0;
  if (row >= 2) off += t1;
  if (row >= 3) off += t2;
  return (s - x) + off;
}

__device__ __forceinline__ float key_mass(unsigned long long key) {
  return __uint_as_float(static_cast<uint32_t>(key >> 32));
}

// LDS written by some lanes of a wave and then read by other lanes of it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// One compare-exchange of the bitonic network between lanes lane and lane^LM.
template <int LM>
__device__ __forceinline__ unsigned long long bitonic_lanes(unsigned long long a, int lane, bool desc) {
  const unsigned long long b = xor_lane64<LM>(a, lane);
  const unsigned long long hi = a > b ? a : b, lo = a > b ? b : a;
  return (((lane & LM) == 0) == desc) ? hi : lo;
}

// The bitonic network over positions e = lane*KPL + j, descending keys;
// every step a compile-time (size, stride) pair.  The direction of position
// e within a merge of `SIZE` is bit SIZE of e: of j while SIZE < KPL, of
// lane*KPL otherwise.
template <int KPL, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_merge(unsigned long long (&key)[KPL], int lane, bool desc_lane) {
  if constexpr (STRIDE < KPL) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (j & STRIDE) continue;
      const bool desc = SIZE < KPL ? (j & SIZE) == 0 : desc_lane;
      const unsigned long long a = key[j], b = key[j | STRIDE];
      const bool swap = (a < b) == desc;
      key[j] = swap ? b : a;
      key[j | STRIDE] = swap ? a : b;
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) key[j] = bitonic_lanes<STRIDE / KPL>(key[j], lane, desc_lane);
  }
  if constexpr (STRIDE > 1) bitonic_merge<KPL, SIZE, STRIDE / 2>(key, lane, desc_lane);
}
template <int KPL, int SIZE, int NPOS>
__device__ __forceinline__ void bitonic_sort(unsigned long long (&key)[KPL], int lane) {
  bitonic_merge<KPL, SIZE, SIZE / 2>(key, lane, ((lane * KPL) & SIZE) == 0);
  if constexpr (SIZE < NPOS) bitonic_sort<KPL, 2 * SIZE, NPOS>(key, lane);
}

// Sorted keys and the cut of one discovery unit.  st[j] holds the tile
// stats (m_b, l_b) of block b = lane*KPL + j.  Keys (mass bits, ~b) are
// sorted descending over NPOS positions (NPOS >= nb, a power of two;
// positions beyond it belong to independent copies of the network holding
// only padding, which sorts after every block), and the fp64 running sum
// picks K: the blocks of sorted positions [0, K) are selected.
template <int KPL, int NPOS>
__device__ __forceinline__ int eta_sorted_cut(const float2 (&st)[KPL], float eta, int nb, float M, float L, int lane,
                                              unsigned long long (&key)[KPL]) {
  const float invL = 1.0f / L;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int b = lane * KPL + j;
    const float mass = st[j].y * __builtin_amdgcn_exp2f(st[j].x - M) * invL;
    key[j] = b < nb ? (static_cast<unsigned long long>(__float_as_uint(mass)) << 32) |
                          static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(b))
                    : 0ull;  // padding sorts after every block
  }
  bitonic_sort<KPL, 2, NPOS>(key, lane);
  // fp64 running sum in sorted order: each lane's own run, then the lanes below
  double part = 0.0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) part += static_cast<double>(key_mass(key[j]));
  double run = wave_exclusive_scan(part, lane);
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
  return min(nb, hits ? __builtin_amdgcn_readlane(kfound, __builtin_ctzll(hits)) : nb);
}

// Eta selection of one discovery unit: the selected blocks' bits are ORed
// into s_bits (LDS); returns K.
template <int KPL, int NPOS>
__device__ __forceinline__ int select_eta(const float2 (&st)[KPL], float eta, int nb, float M, float L, int lane,
                                          uint32_t *s_bits) {
  unsigned long long key[KPL];
  const int K = eta_sorted_cut<KPL, NPOS>(st, eta, nb, M, L, lane, key);
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    if (lane * KPL + j < K) {
      const uint32_t b = 0xFFFFFFFFu - static_cast<uint32_t>(key[j]);
      atomicOr(&s_bits[b >> 5], 1u << (b & 31));
    }
  }
  return K;
}

// Eta selection of a unit of at most 64 blocks, one per lane (st = the
// stats of block `lane`): the selected set comes back as a 64-bit block
// mask.  Sorted position p < nb holds block b_p, a permutation of [0, nb),
// and sends lane b_p whether p < K (one forward lane permute; positions of
// padding send to their own lanes, which hold no block).  Every lane of the
// wave must be active.  Returns K.
template <int NPOS>
__device__ __forceinline__ int select_eta_mask(float2 st, float eta, int nb, float M, float L, int lane,
                                               unsigned long long &mask) {
  const float2 st1[1] = {st};
  unsigned long long key[1];
  const int K = eta_sorted_cut<1, NPOS>(st1, eta, nb, M, L, lane, key);
  const int b = lane < nb ? static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key[0])) : lane;
  const int picked = __builtin_amdgcn_ds_permute(b << 2, lane < K ? 1 : 0);
  mask = __builtin_amdgcn_ballot_w64(picked != 0 && lane < nb);
  return K;
}

}  // namespace sel
}  // namespace wise

#endif  // WISE_SELECT_H
