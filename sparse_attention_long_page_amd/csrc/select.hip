// Page selection: forced sink and local-window pages plus the top-k other
// pages by router score ("Universal Attention Engine", sections "The Product"
// and "Content-Dependent Dynamic Routing"; tiers from the TileSparse README,
// "Motivation": Critical tier of alpha pages, Ambient tier after it).
//
// One workgroup per (sequence, selection head).  Exact top-k by an MSB-first
// radix select over order-preserving 32-bit keys held in LDS (4 passes of 8
// bits, LDS histograms), then an index-ordered pass that takes the threshold
// ties lowest-index-first and compacts the chosen pages into an ascending
// list with workgroup prefix sums.  The result is a pure function of the fp32
// scores: same scores -> same list, bit for bit.
#include "common.h"

namespace sa {

constexpr int kSelThreads = 512;

// Non-candidate pages get key 0, NaN scores key 1, every other score a key
// >= 0x007fffff that orders like the float (-0 folded onto +0).
__device__ __forceinline__ uint32_t score_key(float x) {
  if (x != x) return 1u;
  if (x == 0.0f) x = 0.0f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (blockDim = kSelThreads), in thread
// order.  Returns the exclusive prefix; *total gets the sum over all threads.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const uint32_t t = wsum[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// k-th largest key among keys[0..n) (k >= 1): returns the key T and, in *need,
// how many keys equal to T belong to the top k.
__device__ uint32_t radix_select(const uint32_t* keys, int n, uint32_t k, uint32_t* need,
                                 uint32_t* hist, uint32_t* bcast) {
  uint32_t prefix = 0, pmask = 0, kk = k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
      const uint32_t key = keys[i];
      if (key != 0u && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[4 * lane + j];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      uint32_t suf = mine;                       // sum over lanes >= this one
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += y;
      }
      const uint32_t above = suf - mine;         // keys in higher lanes' bins
      if (suf >= kk && above < kk) {
        uint32_t acc = above;
        for (int j = 3; j >= 0; --j) {
          if (acc + c[j] >= kk) {
            bcast[0] = 4u * lane + j;
            bcast[1] = kk - acc;
            break;
          }
          acc += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= bcast[0] << shift;
    pmask |= 255u << shift;
    kk = bcast[1];
    __syncthreads();
  }
  *need = kk;
  return prefix;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t bcast[2];
  const int s = blockIdx.x, b = blockIdx.y;
  const int sel = b * p.n_sel + s;
  const int n = (p.seq_lens[b] + p.P - 1) / p.P;
  const int sink_hi = min(p.sink, n);
  const int win_lo = max(n - p.window, 0);
  const int n_forced = sink_hi + max(0, n - max(win_lo, sink_hi));
  const int n_cand = n - n_forced;
  const int k_eff = min(p.top_k, n_cand);
  const int k1 = p.tiered ? min(p.critical_k, k_eff) : k_eff;
  const float* sc = p.scores + (size_t)sel * p.scores_stride;

  for (int i = threadIdx.x; i < n; i += kSelThreads) {
    const bool forced = i < sink_hi || i >= win_lo;
    keys[i] = forced ? 0u : score_key(sc[i]);
  }
  __syncthreads();

  uint32_t T1 = 0xffffffffu, r1 = 0, T2 = 0xffffffffu, r2 = 0;
  if (k_eff > 0) T2 = radix_select(keys, n, (uint32_t)k_eff, &r2, hist, bcast);
  if (p.tiered && k1 > 0) T1 = radix_select(keys, n, (uint32_t)k1, &r1, hist, bcast);
  if (!p.tiered) { T1 = T2; r1 = r2; }

  // pass 1: rank ties at the thresholds by index; replace keys with flags
  // bit0 forced, bit1 in top-k1 (Critical), bit2 in top-k_eff
  uint32_t run1 = 0, run2 = 0;
  for (int base0 = 0; base0 < n; base0 += kSelThreads) {
    const int i = base0 + threadIdx.x;
    const uint32_t key = i < n ? keys[i] : 0u;
    const uint32_t e1 = (key != 0u && key == T1) ? 1u : 0u;
    const uint32_t e2 = (key != 0u && key == T2) ? 1u : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(e1 | (e2 << 16), &tot, wsum);
    const uint32_t rank1 = run1 + (ex & 0xffffu), rank2 = run2 + (ex >> 16);
    const bool top1 = key != 0u && (key > T1 || (e1 && rank1 < r1));
    const bool top2 = key != 0u && (key > T2 || (e2 && rank2 < r2));
    const bool forced = i < n && (i < sink_hi || i >= win_lo);
    if (i < n) keys[i] = (forced ? 1u : 0u) | (top1 ? 2u : 0u) | (top2 ? 4u : 0u);
    run1 += tot & 0xffffu;
    run2 += tot >> 16;
  }
  __syncthreads();

  // pass 2: ascending compaction; segment A (forced + Critical, or the whole
  // untiered list), segment B (Ambient) after it
  int32_t* out = p.lists + (size_t)sel * p.list_stride;
  const int countA = n_forced + k1;
  uint32_t runA = 0, runB = 0;
  for (int base0 = 0; base0 < n; base0 += kSelThreads) {
    const int i = base0 + threadIdx.x;
    const uint32_t f = i < n ? keys[i] : 0u;
    uint32_t a, bb;
    if (p.tiered) { a = (f & 3u) ? 1u : 0u; bb = ((f & 4u) && !(f & 2u)) ? 1u : 0u; }
    else { a = (f & 5u) ? 1u : 0u; bb = 0u; }
    uint32_t tot;
    const uint32_t ex = block_excl_scan(a | (bb << 16), &tot, wsum);
    if (a) out[runA + (ex & 0xffffu)] = i;
    if (bb) out[countA + runB + (ex >> 16)] = i;
    runA += tot & 0xffffu;
    runB += tot >> 16;
  }
  if (threadIdx.x == 0) {
    p.counts[sel] = n_forced + k_eff;
    if (p.tiered && p.ccounts) p.ccounts[sel] = countA;
  }
}

hipError_t launch_select(const SelectParams& p, int batch, int max_pages, hipStream_t s) {
  dim3 grid(p.n_sel, batch);
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), (size_t)max_pages * sizeof(uint32_t), s, p);
  return hipGetLastError();
}

}  // namespace sa
