// Opt-in device-side checks of the index data a call is about to trust
// (page ids, lengths, list counts, given scores).  Each check kernel reads
// only the arrays it checks, within their declared shapes (a count is
// clamped to its stride before the entries under it are read), and never
// dereferences the values it checks.  The first violation found is recorded
// in a small static device array, which the host reads back after the checks.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace sa {

// [0] violation code (0: none), [1..3] indices, [4] offending value (bits)
__device__ uint32_t validate_result[8];

namespace {

__device__ __forceinline__ void report(uint32_t* res, uint32_t code, uint32_t i0, uint32_t i1, uint32_t i2,
                                       uint32_t value) {
  if (atomicCAS(res, 0u, code) == 0u) {
    res[1] = i0;
    res[2] = i1;
    res[3] = i2;
    res[4] = value;
  }
}

__global__ void validate_clear_kernel(uint32_t* res) {
  if (threadIdx.x < 8) res[threadIdx.x] = 0u;
}

// seq_lens[b] in [0, max_pages * P]; block_table[b][lp] in [0, n_phys) for
// the sequence's logical pages.  Sequences [seq0, seq0 + batch).
__global__ void validate_kv_kernel(ValidateKV v, uint32_t* res) {
  const int b = v.seq0 + blockIdx.y;
  const int len = v.seq_lens[b];
  if (len < 0 || (long)len > (long)v.max_pages * v.P) {
    if (blockIdx.x == 0 && threadIdx.x == 0) report(res, kValSeqLen, b, 0, 0, (uint32_t)len);
    return;
  }
  if (!v.block_table) return;
  const int n = (len + v.P - 1) / v.P;
  for (int lp = blockIdx.x * blockDim.x + threadIdx.x; lp < n; lp += gridDim.x * blockDim.x) {
    const int ph = v.block_table[(size_t)b * v.max_pages + lp];
    if (ph < 0 || ph >= v.n_phys) report(res, kValBlockTable, b, lp, 0, (uint32_t)ph);
  }
}

// page_counts[b][s] in [0, list_stride]; critical_counts[b][s] in [0, count];
// list entries [0, count) in [0, n_pages(b)).
__global__ void validate_lists_kernel(ValidateLists v, uint32_t* res) {
  const int s = blockIdx.x, b = blockIdx.y;
  const int sel = b * v.n_sel + s;
  const int cnt = v.counts[sel];
  if (cnt < 0 || cnt > v.stride) {
    if (threadIdx.x == 0) report(res, kValCount, b, s, 0, (uint32_t)cnt);
    return;
  }
  if (v.ccounts) {
    const int cc = v.ccounts[sel];
    if ((cc < 0 || cc > cnt) && threadIdx.x == 0) report(res, kValCriticalCount, b, s, 0, (uint32_t)cc);
  }
  const int len = v.seq_lens[b];
  const int n = len > 0 ? (len + v.P - 1) / v.P : 0;
  const int32_t* list = v.lists + (size_t)sel * v.stride;
  for (int e = threadIdx.x; e < cnt; e += blockDim.x) {
    const int lp = list[e];
    if (lp < 0 || lp >= n) report(res, kValListEntry, b, s, e, (uint32_t)lp);
  }
}

// given scores finite over each sequence's pages
__global__ void validate_scores_kernel(ValidateScores v, uint32_t* res) {
  const int s = blockIdx.x, b = blockIdx.y;
  const int len = v.seq_lens[b];
  const int n = len > 0 ? min((len + v.P - 1) / v.P, v.max_pages) : 0;
  const float* row = v.scores + ((size_t)b * v.n_sel + s) * v.stride;
  for (int p = threadIdx.x; p < n; p += blockDim.x) {
    const float x = row[p];
    if (!isfinite(x)) report(res, kValScore, b, s, p, __float_as_uint(x));
  }
}

std::mutex g_res_mu;
uint32_t* g_res_dev[256];   // device address of validate_result, per device

}  // namespace

hipError_t validate_result_ptr(uint32_t** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_res_mu);
  if (!g_res_dev[dev]) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(validate_result));
    if (e != hipSuccess) return e;
    g_res_dev[dev] = reinterpret_cast<uint32_t*>(addr);
  }
  *ptr = g_res_dev[dev];
  return hipSuccess;
}

hipError_t launch_validate_clear(uint32_t* res, hipStream_t s) {
  hipLaunchKernelGGL(validate_clear_kernel, dim3(1), dim3(64), 0, s, res);
  return hipGetLastError();
}

hipError_t launch_validate_kv(const ValidateKV& v, int batch, uint32_t* res, hipStream_t s) {
  const int blocks = std::min((v.max_pages + 255) / 256, 64);
  hipLaunchKernelGGL(validate_kv_kernel, dim3(std::max(blocks, 1), batch), dim3(256), 0, s, v, res);
  return hipGetLastError();
}

hipError_t launch_validate_lists(const ValidateLists& v, int batch, uint32_t* res, hipStream_t s) {
  hipLaunchKernelGGL(validate_lists_kernel, dim3(v.n_sel, batch), dim3(256), 0, s, v, res);
  return hipGetLastError();
}

hipError_t launch_validate_scores(const ValidateScores& v, int batch, uint32_t* res, hipStream_t s) {
  hipLaunchKernelGGL(validate_scores_kernel, dim3(v.n_sel, batch), dim3(256), 0, s, v, res);
  return hipGetLastError();
}

}  // namespace sa
