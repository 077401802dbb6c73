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
// One 256-thread workgroup per (row, head):
//  1. merge the unit's items in item order (fixed order, fp32):
//     M = max m_i, w_i = 2^(m_i - M), L = sum l_i w_i, out = sum acc_i w_i / L;
//  2. discovery units: block mass p_b = l_b 2^(m_b - M) / L from the tile
//     stats (fp32), keys (mass descending, block index ascending) sorted by
//     an LDS bitonic network, running sum in fp64, K = first prefix reaching
//     eta (at least 1; all blocks if rounding never reaches eta);
//  3. write (DISCOVER) or OR (DISCOVER_UNION) the unit's support words; add
//     the density counts; the head-0 workgroup updates the row's tag.
#include <climits>

#include "wise_internal.h"

namespace wise {

namespace {

__global__ __launch_bounds__(kFinishThreads) void finish_kernel(const FinishParams p) {
  extern __shared__ unsigned long long s_keys[];  // [npow] selection keys
  __shared__ float s_w[kMaxItemsPerUnit];
  __shared__ float2 s_ml[kMaxItemsPerUnit];
  __shared__ double s_part[kFinishThreads];
  __shared__ uint32_t s_bits[kMaxWords];
  __shared__ float s_M, s_L;
  __shared__ int s_err, s_K, s_added, s_rowerr;

  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int r = u / p.heads;
  const int h = u - r * p.heads;
  const int code = p.row_code[r];
  const int eff = code & 0xF;
  const int req = (code >> 4) & 0xF;
  const bool row_bad = eff == kRowError;
  const int items = row_bad ? 0 : p.unit_items[u];
  const int64_t base = static_cast<int64_t>(u) * p.items_per_unit;
  const int D = p.head_dim;

  // ---- 1. merge ----
  for (int i = tid; i < items; i += kFinishThreads) s_ml[i] = p.part_ml[base + i];
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY;
    int err = items == 0;
    for (int i = 0; i < items; ++i) {
      err |= s_ml[i].y < 0.0f;
      M = fmaxf(M, s_ml[i].x);
    }
    float L = 0.0f;
    for (int i = 0; i < items; ++i) {
      const float w = __builtin_amdgcn_exp2f(s_ml[i].x - M);
      s_w[i] = w;
      L = fmaf(s_ml[i].y, w, L);
    }
    s_M = M;
    s_L = L;
    s_err = err;
    s_K = INT_MAX;
    s_added = 0;
    s_rowerr = 0;
  }
  __syncthreads();
  const float M = s_M, L = s_L;
  const bool err = s_err != 0;
  for (int dd = tid; dd < D; dd += kFinishThreads) {
    float a = 0.0f;
    for (int i = 0; i < items; ++i) a = fmaf(p.part_acc[(base + i) * D + dd], s_w[i], a);
    p.out[static_cast<int64_t>(u) * D + dd] = err ? __builtin_nanf("") : a / L;
  }
  if (err && tid == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, 1ull);

  if (p.support == nullptr || row_bad || req == WISE_DENSE) return;
  const int slot = p.slot_of_row ? p.slot_of_row[r] : r;

  // ---- 2. eta selection of a discovery unit ----
  const bool discover = eff == WISE_DISCOVER || eff == WISE_DISCOVER_UNION;
  if (discover && !err) {
    const int nb = (p.ctx_len[r] + kBlock - 1) / kBlock;
    int npow = 1;
    while (npow < nb) npow <<= 1;
    const float invL = 1.0f / L;
    for (int b = tid; b < npow; b += kFinishThreads) {
      unsigned long long key = 0ull;  // padding sorts after every block
      if (b < nb) {
        const float2 st = p.stats[static_cast<int64_t>(u) * p.max_blocks + b];
        const float mass = st.y * __builtin_amdgcn_exp2f(st.x - M) * invL;
        key = (static_cast<unsigned long long>(__float_as_uint(mass)) << 32) |
              static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(b));
      }
      s_keys[b] = key;
    }
    for (int w = tid; w < kMaxWords; w += kFinishThreads) s_bits[w] = 0u;
    __syncthreads();
    // bitonic sort, descending keys: mass descending, then block index ascending
    for (int size = 2; size <= npow; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (npow >> 1); t += kFinishThreads) {
          const int lo = 2 * stride * (t / stride) + (t % stride);
          const int hi = lo + stride;
          const bool desc = (lo & size) == 0;
          const unsigned long long a = s_keys[lo], bkey = s_keys[hi];
          if ((a < bkey) == desc) {
            s_keys[lo] = bkey;
            s_keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    // running sum in fp64: each thread owns a contiguous run of the order
    const int per = (nb + kFinishThreads - 1) / kFinishThreads;
    const int lo = min(nb, tid * per), hi = min(nb, lo + per);
    double sum = 0.0;
    for (int i = lo; i < hi; ++i) sum += static_cast<double>(__uint_as_float(static_cast<uint32_t>(s_keys[i] >> 32)));
    s_part[tid] = sum;
    __syncthreads();
    if (tid == 0) {
      double run = 0.0;
      for (int t = 0; t < kFinishThreads; ++t) {
        const double x = s_part[t];
        s_part[t] = run;
        run += x;
      }
    }
    __syncthreads();
    double run = s_part[tid];
    int kfound = INT_MAX;
    for (int i = lo; i < hi; ++i) {
      run += static_cast<double>(__uint_as_float(static_cast<uint32_t>(s_keys[i] >> 32)));
      if (run >= static_cast<double>(p.eta)) {
        kfound = i + 1;
        break;
      }
    }
    if (kfound != INT_MAX) atomicMin(&s_K, kfound);
    __syncthreads();
    const int K = s_K == INT_MAX ? nb : max(1, s_K);
    for (int i = tid; i < K; i += kFinishThreads) {
      const uint32_t b = 0xFFFFFFFFu - static_cast<uint32_t>(s_keys[i]);
      atomicOr(&s_bits[b >> 5], 1u << (b & 31));
    }
    __syncthreads();

    // ---- 3. support write / union, density counts ----
    uint32_t *sw = p.support + ((static_cast<int64_t>(slot) * p.layers + p.layer) * p.heads + h) * p.words;
    int added = 0;
    for (int w = tid; w < p.words; w += kFinishThreads) {
      const uint32_t nw = w < kMaxWords ? s_bits[w] : 0u;
      if (eff == WISE_DISCOVER) {
        sw[w] = nw;
      } else {
        const uint32_t old = sw[w];
        sw[w] = old | nw;
        added += __popc(nw & ~old);
      }
    }
    if (added) atomicAdd(&s_added, added);
    __syncthreads();
    if (tid == 0 && p.counters) {
      atomicAdd(p.counters + WISE_CTR_SELECTED,
                static_cast<unsigned long long>(eff == WISE_DISCOVER ? K : s_added));
      if (eff == WISE_DISCOVER) atomicAdd(p.counters + WISE_CTR_CAUSAL, static_cast<unsigned long long>(nb));
    }
  }

  // ---- tag of the row's (slot, layer), once per row ----
  if (h != 0) return;
  if (discover) {
    // a bad page in any head of the row breaks this discovery
    for (int hh = 0; hh < p.heads; ++hh) {
      const int uu = r * p.heads + hh;
      const int it = p.unit_items[uu];
      const int64_t bb = static_cast<int64_t>(uu) * p.items_per_unit;
      for (int i = tid; i < it; i += kFinishThreads)
        if (p.part_ml[bb + i].y < 0.0f) s_rowerr = 1;
    }
    __syncthreads();
  }
  if (tid != 0) return;
  wise_tag *t = p.tags + static_cast<int64_t>(slot) * p.layers + p.layer;
  if (eff == WISE_DISCOVER) {
    t->request = p.row_request[r];
    t->position = p.row_position[r];
    t->discoveries = s_rowerr ? 0 : 1;
  } else if (eff == WISE_DISCOVER_UNION) {
    t->discoveries = s_rowerr ? 0 : t->discoveries + 1;
  } else if (req == WISE_DISCOVER_UNION) {
    t->discoveries = 0;  // broken window: the rest of this token runs dense
  }
}

}  // namespace

hipError_t launch_finish(const FinishParams &p, hipStream_t stream) {
  int npow = 1;
  while (npow < p.max_blocks) npow <<= 1;
  const size_t lds = static_cast<size_t>(npow) * sizeof(unsigned long long);
  hipLaunchKernelGGL(finish_kernel, dim3(static_cast<unsigned>(p.rows) * p.heads), dim3(kFinishThreads), lds,
                     stream, p);
  return hipGetLastError();
}

}  // namespace wise
