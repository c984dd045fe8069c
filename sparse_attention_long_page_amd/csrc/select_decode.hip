// Page selection and sparse decode of one per-KV-head list in one workgroup:
// router scores of every page against the pooled query, the forced sink and
// local-window pages plus the top-k others ("Universal Attention Engine",
// sections "The Product" and "Content-Dependent Dynamic Routing"), then
// attention over exactly those pages' tokens (same page, "Key Design
// Decisions" 3: decode is memory-bound, only the selected blocks are loaded).
//
// The same computation as sa_select_pages followed by sa_sparse_decode with
// one split: score_keys_body and select_from_keys (select_body.h) on all 8
// waves, the list kept in LDS and written out, then the decode
// statements (decode_body.inc, the staged d 128 / pages of 64 path) on waves 0-3 while
// waves 4-7 only meet the decode's workgroup barriers, then end.
// Each list starts its decode as soon as its own selection is done, rather
// than when the slowest list's selection is, and no kernel boundary sits
// between the two steps.
#include "common.h"
#include "decode_body.h"
#include "select_body.h"

namespace sa {

template <int D, int P>
__global__ __launch_bounds__(kSelThreads, 1) void select_decode_kernel(ScoreParams sp, SelectParams sel,
                                                                       DecodeParams p,
                                                                       const int32_t* __restrict__ btab,
                                                                       const int32_t* __restrict__ seq_lens) {
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];   // [max_pages] keys, then the list [list_stride]
  __shared__ SelShared sh;
  // the decode's staging areas; before the decode they hold the newest
  // page's summary partials (refresh), which are dead once the scores are in
  __shared__ __attribute__((aligned(16))) uint16_t stg[4 * 16384];
  static_assert(refresh_ts<uint16_t, D>() * D * sizeof(double) <= sizeof(stg), "refresh partials fit");
  double* rpart = reinterpret_cast<double*>(stg);
  const int s = blockIdx.x, b = blockIdx.y;
  const ListShape L = list_shape(sel, b);
  score_keys_body<uint16_t, D>(sp, sel, L, b, s, keys, sh, rpart);
  __syncthreads();
  int32_t* list = reinterpret_cast<int32_t*>(keys + sp.max_pages);
  select_from_keys(sel, L, b, s, keys, sh, list);
  __syncthreads();
  const int count = L.n_forced + L.k_eff;
  int32_t* lrow = sel.lists + ((size_t)b * sel.n_sel + s) * sel.list_stride;
  for (int i = threadIdx.x; i < count; i += kSelThreads) lrow[i] = list[i];
  if (threadIdx.x >= 256) {
    // waves 4-7 have no decode work; they meet the decode's barriers and end
    for (int i = 0; i < decode_body_barriers(true); ++i) __syncthreads();
    return;
  }
  {
    constexpr bool TIERED = false, STAGED = true, FP8 = false;
    constexpr int KSTEPS = D / 32;
    constexpr int DTILES = D / 16;
    constexpr int E = 64 / P;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, kg = lane >> 4;
    const int split = 0;
    const int g = p.per_q ? s / p.G : s;
    const int R = p.per_q ? p.T : p.T * p.G;
    const int cc = count;
    uint16_t* const stg_area = stg;
#include "decode_body.inc"
  }
}

size_t select_decode_lds_bytes(int max_pages, int list_stride) {
  return (size_t)(max_pages + list_stride) * sizeof(uint32_t);
}

// LDS left for the keys and the list beside the kernel's static LDS (the
// decode's staging areas and the selection's working set), of the 160 KiB a
// workgroup may use
size_t select_decode_lds_limit() {
  static size_t limit = [] {
    hipFuncAttributes a{};
    if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&select_decode_kernel<128, 64>)) != hipSuccess)
      return (size_t)0;
    const size_t total = 160 * 1024;
    return a.sharedSizeBytes < total ? total - a.sharedSizeBytes : (size_t)0;
  }();
  return limit;
}

hipError_t launch_select_decode(const ScoreParams& sp, const SelectParams& p, const DecodeParams& dp, int batch,
                                hipStream_t s) {
  dim3 grid(p.n_sel, batch);
  hipLaunchKernelGGL((select_decode_kernel<128, 64>), grid, dim3(kSelThreads),
                     select_decode_lds_bytes(sp.max_pages, p.list_stride), s, sp, p, dp, dp.block_table,
                     dp.seq_lens);
  return hipGetLastError();
}

}  // namespace sa
