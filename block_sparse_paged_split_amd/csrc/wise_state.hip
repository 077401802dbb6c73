// Support/tag snapshot and restore across a KV offload.
//
// Method: WISE pull request page (vllm-rlt pull 143), review finding
// "Preserve WISE state across KV offload".  Restated: an offload after the
// discovery depths drops the request's slot, so its later reuse depths find
// no support for their token; the finding proposes saving the support and
// tags with the recurrent state and putting them back on resume.  These
// kernels copy whole slots (every layer and head) between the support state
// and caller-owned records; a restored tag names the same (request,
// position), so the resumed request reuses sparsely.
//
// Record layout (one per listed slot, record_bytes apart, 8-byte aligned):
//   support words [layers][heads][words] uint32, padded to 8 bytes,
//   then tags [layers] as 3 x 8-byte words each.
// One workgroup per record; the copies are plain 16-byte-or-smaller vector
// loads and stores.
#include "wise_internal.h"

namespace wise {

namespace {

constexpr int kStateThreads = 256;

__global__ __launch_bounds__(kStateThreads) void snapshot_kernel(const StateParams p) {
  const int i = blockIdx.x;
  const int slot = p.slots_list[i];
  const bool ok = slot >= 0 && slot < p.slots;
  char *rec = static_cast<char *>(p.records) + static_cast<int64_t>(i) * p.record_bytes;
  uint32_t *words = reinterpret_cast<uint32_t *>(rec);
  unsigned long long *tags = reinterpret_cast<unsigned long long *>(rec + p.tags_offset);
  const int64_t nw = static_cast<int64_t>(p.layers) * p.heads * p.words;
  const uint32_t *src = p.support + (ok ? static_cast<int64_t>(slot) * nw : 0);
  for (int64_t k = threadIdx.x; k < nw; k += kStateThreads) words[k] = ok ? src[k] : 0u;
  const unsigned long long *tsrc =
      reinterpret_cast<const unsigned long long *>(p.tags + (ok ? static_cast<int64_t>(slot) * p.layers : 0));
  for (int k = threadIdx.x; k < 3 * p.layers; k += kStateThreads) tags[k] = ok ? tsrc[k] : 0ull;
}

__global__ __launch_bounds__(kStateThreads) void restore_kernel(const StateParams p) {
  const int i = blockIdx.x;
  const int slot = p.slots_list[i];
  if (slot < 0 || slot >= p.slots) {
    if (threadIdx.x == 0 && p.counters) atomicAdd(p.counters + WISE_CTR_ERRORS, 1ull);
    return;
  }
  const char *rec = static_cast<const char *>(p.records) + static_cast<int64_t>(i) * p.record_bytes;
  const uint32_t *words = reinterpret_cast<const uint32_t *>(rec);
  const unsigned long long *tags = reinterpret_cast<const unsigned long long *>(rec + p.tags_offset);
  const int64_t nw = static_cast<int64_t>(p.layers) * p.heads * p.words;
  uint32_t *dst = p.support + static_cast<int64_t>(slot) * nw;
  for (int64_t k = threadIdx.x; k < nw; k += kStateThreads) dst[k] = words[k];
  unsigned long long *tdst = reinterpret_cast<unsigned long long *>(p.tags + static_cast<int64_t>(slot) * p.layers);
  for (int k = threadIdx.x; k < 3 * p.layers; k += kStateThreads) tdst[k] = tags[k];
}

}  // namespace

void state_record_layout(int layers, int heads, int words, size_t *tags_offset, size_t *record_bytes) {
  const size_t w = static_cast<size_t>(layers) * heads * words * sizeof(uint32_t);
  *tags_offset = (w + 7) & ~static_cast<size_t>(7);
  *record_bytes = *tags_offset + static_cast<size_t>(layers) * sizeof(wise_tag);
}

hipError_t launch_state_copy(const StateParams &p, bool restore, hipStream_t stream) {
  if (restore)
    hipLaunchKernelGGL(restore_kernel, dim3(p.count), dim3(kStateThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(snapshot_kernel, dim3(p.count), dim3(kStateThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wise
