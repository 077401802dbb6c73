// Read ceiling of the paged K/V access pattern, for the benchmark.
//
// A plain gather with no arithmetic: every work item reads the K and V rows
// of its tiles (32-token blocks of one (row, head)) through the block table,
// with the same 16-byte whole-token loads as the attention kernel, and folds
// them into one XOR word per wave so that no load is dead.  The item list
// (row, head, offset into a tile list, tile count) is built on the host from
// the same supports and contexts the attention call reads, so the probe
// moves the call's K/V bytes in items of the same length.  With no V cache
// it reads K only (the LSE route's pass).  It is not part of the attention
// library; only the benchmark loads it.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct ProbeParams {
  const char *k, *v;
  int64_t stride_page_b, stride_head_b, stride_token_b;
  const int32_t *block_table;
  int64_t bt_stride;
  const int32_t *ctx_len;
  int32_t page_shift;
  const int4 *items;    // row, head, first tile in `tiles`, tile count
  const int32_t *tiles; // block indices
  int32_t n_items;
  uint32_t *sink;       // one word per item
};

template <int ROW_BYTES>
__global__ __launch_bounds__(256) void read_probe_kernel(const ProbeParams p) {
  constexpr int LPT = ROW_BYTES / 16;  // lanes per token row
  constexpr int TPI = 64 / LPT;        // tokens per load instruction
  constexpr int NI = 32 / TPI;         // load instructions per tile and tensor
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  if (item >= p.n_items) return;
  const int4 it = p.items[item];
  const int r = it.x, h = it.y;
  const int n = p.ctx_len[r];
  const int c = lane % LPT, g = lane / LPT;
  const char *kh = p.k + h * p.stride_head_b + c * 16 + g * p.stride_token_b;
  const char *vh = p.v ? p.v + h * p.stride_head_b + c * 16 + g * p.stride_token_b : nullptr;
  const int32_t *bt = p.block_table + r * p.bt_stride;
  const int pmask = (1 << p.page_shift) - 1;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // The page of load instruction j of a tile sits in lane j of a vector
  // fetched one tile ahead (the TPI tokens of one load share a page: pages
  // hold a multiple of TPI tokens), as in the attention kernel.
  // the item's tile indices (at most 64), one per lane, loaded once
  const int my_tile = lane < it.w ? p.tiles[it.z + lane] : 0;
  auto fetch_pages = [&](int i) -> int {
    const int b = __builtin_amdgcn_readlane(my_tile, i);
    return bt[min(b * 32 + min(lane, NI - 1) * TPI, n - 1) >> p.page_shift];
  };
  int pages_next = fetch_pages(0);
  for (int i = 0; i < it.w; ++i) {
    const int b = __builtin_amdgcn_readlane(my_tile, i);
    const int pages = pages_next;
    if (i + 1 < it.w) pages_next = fetch_pages(i + 1);
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int t0 = b * 32 + j * TPI;
      const int page = __builtin_amdgcn_readlane(pages, j);
      const int64_t off = static_cast<int64_t>(page) * p.stride_page_b + (t0 & pmask) * p.stride_token_b;
      const bool valid = t0 + g < n;
      kr[j] = valid ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kh + off)) : u32x4{0u, 0u, 0u, 0u};
      vr[j] = (valid && p.v) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vh + off))
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) acc ^= kr[j] ^ vr[j];
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  x ^= __shfl_xor(x, 32);
  x ^= __shfl_xor(x, 16);
  if (lane == 0) p.sink[item] = x;
}

}  // namespace

extern "C" {

// Returns 0 on success, 1 for an unsupported row size, 2 for a launch error.
// Every pointer is a device pointer; items and tiles are as in ProbeParams.
int wise_read_probe(const void *k, const void *v, int64_t stride_page_b, int64_t stride_head_b,
                    int64_t stride_token_b, int32_t row_bytes, const int32_t *block_table, int64_t bt_stride,
                    const int32_t *ctx_len, int32_t page_shift, const int32_t *items, const int32_t *tiles,
                    int32_t n_items, uint32_t *sink, void *stream, void *ev_begin, void *ev_end) {
  ProbeParams p{static_cast<const char *>(k), static_cast<const char *>(v), stride_page_b, stride_head_b,
                stride_token_b, block_table, bt_stride, ctx_len, page_shift,
                reinterpret_cast<const int4 *>(items), tiles, n_items, sink};
  if (n_items < 1) return 0;
  const dim3 grid((n_items + 3) / 4), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t b = static_cast<hipEvent_t>(ev_begin), e = static_cast<hipEvent_t>(ev_end);
  switch (row_bytes) {
    case 128: hipExtLaunchKernelGGL(read_probe_kernel<128>, grid, block, 0, s, b, e, 0, p); break;
    case 256: hipExtLaunchKernelGGL(read_probe_kernel<256>, grid, block, 0, s, b, e, 0, p); break;
    case 512: hipExtLaunchKernelGGL(read_probe_kernel<512>, grid, block, 0, s, b, e, 0, p); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
