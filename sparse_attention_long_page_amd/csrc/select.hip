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

// Forced pages and candidate counts of list (b, s).
struct ListShape {
  int n, sink_hi, win_lo, n_forced, k_eff, k1;
};

__device__ __forceinline__ ListShape list_shape(const SelectParams& p, int b) {
  ListShape L;
  L.n = (p.seq_lens[b] + p.P - 1) / p.P;
  L.sink_hi = min(p.sink, L.n);
  L.win_lo = max(L.n - p.window, 0);
  L.n_forced = L.sink_hi + max(0, L.n - max(L.win_lo, L.sink_hi));
  L.k_eff = min(p.top_k, L.n - L.n_forced);
  L.k1 = p.tiered ? min(p.critical_k, L.k_eff) : L.k_eff;
  return L;
}

// Select from keys[0..n) in LDS (0 = forced page, else score_key) and write
// the list of (b, s).  Called by the whole workgroup after a barrier.
__device__ void select_from_keys(const SelectParams& p, const ListShape& L, int b, int s, uint32_t* keys,
                                 uint32_t* hist, uint32_t* wsum, uint32_t* bcast) {
  const int sel = b * p.n_sel + s;
  const int n = L.n, sink_hi = L.sink_hi, win_lo = L.win_lo, n_forced = L.n_forced, k_eff = L.k_eff, k1 = L.k1;
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

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t bcast[2];
  const int s = blockIdx.x, b = blockIdx.y;
  const ListShape L = list_shape(p, b);
  const float* sc = p.scores + ((size_t)b * p.n_sel + s) * p.scores_stride;
  for (int i = threadIdx.x; i < L.n; i += kSelThreads) {
    const bool forced = i < L.sink_hi || i >= L.win_lo;
    keys[i] = forced ? 0u : score_key(sc[i]);
  }
  __syncthreads();
  select_from_keys(p, L, b, s, keys, hist, wsum, bcast);
}

// Router scores and selection in one workgroup per list (used when there are
// enough lists to fill the GPU).  The pooled query sits in LDS; each wave
// scores 32 pages per round at d <= 128 (16 lanes per page, 4 pages per step,
// the 8 steps' mean-row loads in flight together), writing order-preserving
// keys into LDS.
// The score arithmetic is the same as page_score_kernel's: float64 products
// of the pooled query with the fp32 mean row, summed over 16 lanes in a fixed
// butterfly, rounded once to fp32.
template <typename T, int D>
__global__ __launch_bounds__(kSelThreads) void score_select_kernel(ScoreParams sp, SelectParams p) {
  constexpr int PL = D / 16;
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t bcast[2];
  __shared__ double qbar[D];
  const int s = blockIdx.x, b = blockIdx.y;
  const ListShape L = list_shape(p, b);
  const int n = L.n;
  const T* q = reinterpret_cast<const T*>(sp.q);
  const int rows = sp.per_q ? sp.T : sp.T * sp.G;
  for (int e = threadIdx.x; e < D; e += kSelThreads) {
    double v = 0.0;
    for (int r = 0; r < rows; ++r) {
      int t, h;
      if (sp.per_q) { t = r; h = s; } else { t = r / sp.G; h = s * sp.G + r % sp.G; }
      const size_t i = (((size_t)b * sp.T + t) * sp.Hq + h) * D + e;
      if constexpr (sizeof(T) == 2) v += (double)bf16_bits_to_f32(q[i]);
      else v += (double)q[i];
    }
    qbar[e] = v;
  }
  __syncthreads();
  const int g = sp.per_q ? s / sp.G : s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, slot = lane >> 4;
  const int32_t* bt = sp.block_table + (size_t)b * sp.max_pages;
  float* sout = sp.scores ? sp.scores + ((size_t)b * sp.n_sel + s) * sp.max_pages : nullptr;
  constexpr int kWaves = kSelThreads / 64;
  constexpr int kSteps = D <= 128 ? 8 : 2;           // 4-page steps whose loads are in flight together
  for (int r0 = 4 * kSteps * wave; r0 < n; r0 += 4 * kSteps * kWaves) {
    const int my_phys = (lane < 4 * kSteps && r0 + lane < n) ? bt[r0 + lane] : -1;
    f32x4 v[kSteps][PL / 4];
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int ph = __shfl(my_phys, it * 4 + slot, 64);
      const float* m = sp.mu + ((size_t)max(ph, 0) * sp.Hkv + g) * D + sub * PL;
#pragma unroll
      for (int i = 0; i < PL / 4; ++i) v[it][i] = ph >= 0 ? *reinterpret_cast<const f32x4*>(m + 4 * i) : f32x4{};
    }
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int lp = r0 + it * 4 + slot;
      const double* qq = qbar + sub * PL;
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < PL / 4; ++i) {
        acc += qq[4 * i] * (double)v[it][i][0];
        acc += qq[4 * i + 1] * (double)v[it][i][1];
        acc += qq[4 * i + 2] * (double)v[it][i][2];
        acc += qq[4 * i + 3] * (double)v[it][i][3];
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (sub == 0 && lp < n) {
        const float sc = (float)acc;
        const bool forced = lp < L.sink_hi || lp >= L.win_lo;
        keys[lp] = forced ? 0u : score_key(sc);
        if (sout) sout[lp] = sc;
      }
    }
  }
  if (sout)
    for (int lp = n + threadIdx.x; lp < sp.max_pages; lp += kSelThreads) sout[lp] = __builtin_nanf("");
  __syncthreads();
  select_from_keys(p, L, b, s, keys, hist, wsum, bcast);
}

hipError_t launch_select(const SelectParams& p, int batch, int max_pages, hipStream_t s) {
  dim3 grid(p.n_sel, batch);
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), (size_t)max_pages * sizeof(uint32_t), s, p);
  return hipGetLastError();
}

hipError_t launch_score_select(const ScoreParams& sp, const SelectParams& p, int batch, int bf16, hipStream_t s) {
  dim3 grid(p.n_sel, batch);
  const size_t lds = (size_t)sp.max_pages * sizeof(uint32_t);
#define SA_SS_LAUNCH(T_, D_) hipLaunchKernelGGL((score_select_kernel<T_, D_>), grid, dim3(kSelThreads), lds, s, sp, p)
  if (bf16) {
    if (sp.d == 64) SA_SS_LAUNCH(uint16_t, 64);
    else if (sp.d == 128) SA_SS_LAUNCH(uint16_t, 128);
    else SA_SS_LAUNCH(uint16_t, 576);
  } else {
    if (sp.d == 64) SA_SS_LAUNCH(float, 64);
    else SA_SS_LAUNCH(float, 128);
  }
#undef SA_SS_LAUNCH
  return hipGetLastError();
}

}  // namespace sa
