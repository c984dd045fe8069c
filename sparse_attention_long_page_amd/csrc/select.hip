// Page selection: forced sink and local-window pages plus the top-k other
// pages by router score ("Universal Attention Engine", sections "The Product"
// and "Content-Dependent Dynamic Routing"; tiers from the TileSparse README,
// "Motivation": Critical tier of alpha pages, Ambient tier after it).
//
// One workgroup per (sequence, selection head).  Exact top-k by an MSB-first
// radix select over order-preserving 32-bit keys held in LDS (4 passes of 8
// bits, LDS histograms, one barrier per pass), then index-ordered passes over
// per-thread ranges of consecutive pages that take the threshold ties
// lowest-index-first and compact the chosen pages into an ascending list (one
// workgroup prefix sum each).  The result is a pure function of the fp32
// scores: same scores -> same list, bit for bit.
#include "common.h"
#include "select_body.h"

namespace sa {

// 4-page steps per wave of the few-lists scoring kernel (its pages per workgroup: 4 x this x 8 waves)
constexpr int kLastSelSteps = 4;

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];
  __shared__ SelShared sh;
  const int s = blockIdx.x, b = blockIdx.y;
  const ListShape L = list_shape(p, b);
  const float* sc = p.scores + ((size_t)b * p.n_sel + s) * p.scores_stride;
  for (int i = threadIdx.x; i < 512; i += kSelThreads) sh.hist[0][0][i] = 0u;
  for (int i0 = threadIdx.x; i0 < L.n; i0 += 8 * kSelThreads) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * kSelThreads;
      v[j] = i < L.n ? sc[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * kSelThreads;
      const bool forced = i < L.sink_hi || i >= L.win_lo;
      if (i < L.n) keys[i] = forced ? 0u : score_key(v[j]);
    }
  }
  __syncthreads();
  select_from_keys(p, L, b, s, keys, sh, p.lists + ((size_t)b * p.n_sel + s) * p.list_stride);
}

// Router scores and selection in one workgroup per list (used when there are
// enough lists to fill the GPU).
template <typename T, int D>
__global__ __launch_bounds__(kSelThreads) void score_select_kernel(ScoreParams sp, SelectParams p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];
  __shared__ SelShared sh;
  __shared__ double rpart[refresh_ts<T, D>() * D];
  const int s = blockIdx.x, b = blockIdx.y;
  const ListShape L = list_shape(p, b);
  score_keys_body<T, D>(sp, p, L, b, s, keys, sh, rpart);
  __syncthreads();
  select_from_keys(p, L, b, s, keys, sh, p.lists + ((size_t)b * p.n_sel + s) * p.list_stride);
}

// Router scores and selection of long lists on few selection heads (too few
// lists to fill the GPU with one workgroup each): grid (block of 128 pages,
// selection head, sequence), 512 threads.  Each workgroup scores its pages
// with the arithmetic of the fused kernel (lane `sub` of a page's 16 takes
// dims 64 i + 4 sub + 0..3, float64 products summed in that order, then over
// the 16 lanes in a fixed butterfly, rounded once to fp32) into the list's
// score row; the last workgroup of the list to finish, counted on the list's
// arrival counter (cleared by the prep kernel), selects from the whole row.
// A forced page's mean row is read only when the caller asked for the scores.
template <typename T, int D>
__global__ __launch_bounds__(kSelThreads) void score_lastsel_kernel(ScoreParams sp, SelectParams p,
                                                                    const double* qpart, uint32_t* arrivals) {
  constexpr int kWaves = kSelThreads / 64;
  constexpr int kSteps = kLastSelSteps;              // 4-page steps per wave
  constexpr int kPages = 4 * kSteps * kWaves;
  constexpr int PL = D / 16;
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];
  __shared__ SelShared sh;
  __shared__ double qbar[D];
  __shared__ int phys_s[kPages];
  __shared__ int last_s;
  const int s = blockIdx.y, b = blockIdx.z;
  const ListShape L = list_shape(p, b);
  const int n = L.n;
  const int page0 = blockIdx.x * kPages;
  const int g = sp.per_q ? s / sp.G : s;
  if (threadIdx.x < kPages) {
    const int lp = page0 + threadIdx.x;
    const bool forced = lp < L.sink_hi || lp >= L.win_lo;
    phys_s[threadIdx.x] = (lp < n && !(sp.skip_forced && forced)) ? sp.block_table[(size_t)b * sp.max_pages + lp] : -1;
  }
  // pooled query: the row-chunk partials in chunk order, or the rows in order
  if (qpart) {
    const double* qp = qpart + ((size_t)b * sp.n_sel + s) * kQChunks * D;
    for (int e = threadIdx.x; e < D; e += kSelThreads) {
      double v = 0.0;
#pragma unroll
      for (int c = 0; c < kQChunks; ++c) v += qp[(size_t)c * D + e];
      qbar[e] = v;
    }
  } else {
    // rows 8 at a time, all 8 loads in flight (rows past the end re-read the
    // last one and add +0.0: the sum starts at +0.0 and never becomes -0.0)
    const T* q = reinterpret_cast<const T*>(sp.q);
    const int rows = sp.per_q ? sp.T : sp.T * sp.G;
    for (int e = threadIdx.x; e < D; e += kSelThreads) {
      double v = 0.0;
      for (int r0 = 0; r0 < rows; r0 += 8) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = min(r0 + j, rows - 1);
          int t, h;
          if (sp.per_q) { t = r; h = s; } else { t = r / sp.G; h = s * sp.G + r % sp.G; }
          const size_t i = (((size_t)b * sp.T + t) * sp.Hq + h) * D + e;
          if constexpr (sizeof(T) == 2) w[j] = bf16_bits_to_f32(q[i]);
          else w[j] = q[i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v += r0 + j < rows ? (double)w[j] : 0.0;
      }
      qbar[e] = v;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, slot = lane >> 4;
  // A lane whose page needs no row (forced without scores written out, or
  // past the sequence) reads the row of the block's first page that needs
  // one, so every load is unconditional (a load under a per-lane condition is
  // waited for before the next is issued); its score lands only where it is
  // not used (a forced page's key is 0, a page past the end gets NaN).  A
  // block with no such page reads nothing.
  int safe = -1;
  for (int j = 0; j < kPages && safe < 0; ++j) safe = phys_s[j];
  f32x4 v[kSteps][PL / 4];
  if (safe >= 0) {
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int ph = phys_s[wave * 4 * kSteps + it * 4 + slot];
      const float* m = sp.mu + ((size_t)(ph >= 0 ? ph : safe) * sp.Hkv + g) * D + 4 * sub;
#pragma unroll
      for (int i = 0; i < PL / 4; ++i) v[it][i] = *reinterpret_cast<const f32x4*>(m + 64 * i);
    }
  } else {
#pragma unroll
    for (int it = 0; it < kSteps; ++it)
#pragma unroll
      for (int i = 0; i < PL / 4; ++i) v[it][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float* out = sp.scores + ((size_t)b * sp.n_sel + s) * sp.max_pages;
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int lp = page0 + wave * 4 * kSteps + it * 4 + slot;
    const double* qq = qbar + 4 * sub;
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < PL / 4; ++i) {
      acc += qq[64 * i] * (double)v[it][i][0];
      acc += qq[64 * i + 1] * (double)v[it][i][1];
      acc += qq[64 * i + 2] * (double)v[it][i][2];
      acc += qq[64 * i + 3] * (double)v[it][i][3];
    }
    acc = row16_sum(acc);
    // (device-coherent stores: the list's last workgroup, possibly on
    // another XCD, reads them back)
    if (sub == 0 && lp < sp.max_pages)
      __hip_atomic_store(&out[lp], lp < n ? (float)acc : __builtin_nanf(""), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  // The list's last workgroup selects.  The workgroup's score stores are
  // ordered before its count on the list's counter by the barrier and the
  // count's device-scope release; the workgroup that counts last takes a
  // device-scope acquire before it reads all the scores back (device-coherent
  // loads), so it sees every other workgroup's stores.
  __syncthreads();
  if (threadIdx.x == 0)
    last_s = __hip_atomic_fetch_add(&arrivals[(size_t)b * sp.n_sel + s], 1u, __ATOMIC_RELEASE,
                                    __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!last_s) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int i = threadIdx.x; i < 512; i += kSelThreads) sh.hist[0][0][i] = 0u;
  // 8 scores per thread in flight, loaded before any is used (indices past
  // the end re-read the last score)
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * kSelThreads) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[j] = __hip_atomic_load(&out[min(i0 + j * kSelThreads, n - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * kSelThreads;
      const bool forced = i < L.sink_hi || i >= L.win_lo;
      if (i < n) keys[i] = forced ? 0u : score_key(x[j]);
    }
  }
  __syncthreads();
  select_from_keys(p, L, b, s, keys, sh, p.lists + ((size_t)b * p.n_sel + s) * p.list_stride);
}

hipError_t launch_score_lastsel(const ScoreParams& sp, const SelectParams& p, int bf16, const double* qpart,
                                uint32_t* arrivals, hipStream_t s) {
  constexpr int kPages = 4 * kLastSelSteps * (kSelThreads / 64);
  dim3 grid((sp.max_pages + kPages - 1) / kPages, p.n_sel, sp.B);
  const size_t lds = (size_t)sp.max_pages * sizeof(uint32_t);
#define SA_LS_LAUNCH(T_, D_) \
  hipLaunchKernelGGL((score_lastsel_kernel<T_, D_>), grid, dim3(kSelThreads), lds, s, sp, p, qpart, arrivals)
  if (bf16) {
    if (sp.d == 64) SA_LS_LAUNCH(uint16_t, 64);
    else if (sp.d == 128) SA_LS_LAUNCH(uint16_t, 128);
    else SA_LS_LAUNCH(uint16_t, 576);
  } else {
    if (sp.d == 64) SA_LS_LAUNCH(float, 64);
    else SA_LS_LAUNCH(float, 128);
  }
#undef SA_LS_LAUNCH
  return hipGetLastError();
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
