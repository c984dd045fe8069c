// AutoTuner of the tiered (Critical / Ambient) selection, and the Ambient
// head mask it implies (TileSparse README, "Motivation": Critical pages with
// all query heads, Ambient pages with h heads, an online per-layer search
// that maximises an estimated attention-mass coverage; "Configuration":
// token_budget, critical_top_count, ambient_head_count).  The estimate is not
// defined on the pages; the reading taken:
//   * a page stands in for its n_p tokens by its mean key, so query row (t, h)
//     gives page p the log-weight sm_scale * q . mu_p + ln n_p, and the row's
//     estimated mass on p is the softmax of those over the sequence's pages;
//     M[b][h][p] sums it over the query tokens;
//   * a configuration (alpha, h) under a budget B of (page, query head)
//     entries per KV head affords beta = floor((B - alpha*G) / h) Ambient
//     pages; it covers the forced pages and the first alpha ranked candidates
//     with all G heads and the next beta with the h heads of largest M; its
//     coverage is that mass over q_tokens*G, averaged over sequences and KV
//     heads; the search keeps the first configuration of largest coverage.
//
// Kernels:
//  * mass_logits_kernel: the log-weights of a 64-page x 64-row tile per
//    workgroup on v_mfma_f32_16x16x32_bf16, the tile's query rows staged in
//    LDS once for its four waves.  The fp32 mean keys are split as hi + lo
//    bf16 (two MFMAs per step, residual below 2^-17 relative), the bf16
//    queries are exact, so the products are fp32-accurate.
//  * mass_softmax_kernel: per (sequence, query head), the softmax over pages
//    of each query token's row, summed into M.
//  * tier_page_kernel: per (sequence, KV head, page) the page's mass over the
//    group and the sums of its top-h head masses for each searched h (the
//    group's masses bitonic-sorted across one wave).
//  * tier_cover_kernel: per (sequence, KV head, 64-page chunk) each page's
//    rank among the candidates (router score descending, page ascending, NaN
//    last; by counting over all keys) and every configuration's covered mass.
//  * tier_choose_kernel: the sums in a fixed order, mean over sequences and
//    KV heads, first maximum.
//  * ambient_mask_kernel: the top-h heads of every Ambient page of a list.
#include "common.h"

namespace sa {

// ------------------------------------------------------------ mass logits
// One wave-wide copy of 16 bytes per lane from per-lane global addresses into
// LDS: lane l's bytes land at lds + 16 l.
__device__ __forceinline__ void copy16_global_to_lds(const uint16_t* src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}
// grid (page tiles of 64, row tiles of 64, B*Hkv), 256 threads: wave w takes
// pages 16w..16w+15 of the tile against the tile's 64 query rows of KV head
// g (row r = t*G + head-in-group).  The tile's query rows are copied once
// into LDS (rows of D + 8 bf16: one pad chunk per row spreads a column's 16
// rows over distinct 16-byte slots) and every wave reads its B operands
// there; each wave loads only its own pages' mean rows from global memory.
template <int D>
__global__ __launch_bounds__(256) void mass_logits_kernel(MassParams p) {
  constexpr int kRowChunks = D / 8 + 1;                  // 16-byte chunks per LDS row (one pad)
  __shared__ __attribute__((aligned(16))) uint16_t qs[64 * kRowChunks * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int b = blockIdx.z / p.Hkv, g = blockIdx.z % p.Hkv;
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  if ((int)blockIdx.x * 64 >= n) return;
  const int p0 = blockIdx.x * 64 + wave * 16;
  const int TG = p.T * p.G;
  const int r0 = blockIdx.y * 64;
  const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(p.q);

  // the tile's query rows into LDS: wave-wide copy i covers LDS chunks
  // [64 i, 64 i + 64), chunk c = row c / kRowChunks, column c % kRowChunks
  // (the pad column re-reads column 0); rows past the group read the
  // group's first row (their results are never written)
  for (int i = wave; i < kRowChunks; i += 4) {
    const int c = 64 * i + lane, rr = c / kRowChunks, ch = c % kRowChunks;
    const int r = r0 + rr < TG ? r0 + rr : 0;
    const int t = r / p.G, hl = r % p.G;
    copy16_global_to_lds(qbase + (((size_t)b * p.T + t) * p.Hq + (size_t)g * p.G + hl) * D + 8 * (ch < D / 8 ? ch : 0),
                         qs + 512 * i);
  }

  // A operand: mean key of page p0 + col, dims 32*ks + 8*kq .. +7
  const int pg = p0 + col;
  const float* murow = p.mu + ((size_t)bt[pg < n ? pg : 0] * p.Hkv + g) * D;
  bool row_ok[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) row_ok[rt] = r0 + 16 * rt + col < TG;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x4 acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 6
  for (int ks = 0; ks < D / 32; ++ks) {
    const float4 x0 = *reinterpret_cast<const float4*>(murow + 32 * ks + 8 * kq);
    const float4 x1 = *reinterpret_cast<const float4*>(murow + 32 * ks + 8 * kq + 4);
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    bf16x8 hi, lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hi[i] = (__bf16)x[i];
      lo[i] = (__bf16)(x[i] - (float)hi[i]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const bf16x8 bq = *reinterpret_cast<const bf16x8*>(qs + 8 * ((16 * rt + col) * kRowChunks + 4 * ks + kq));
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bq, acc[rt], 0, 0, 0);
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bq, acc[rt], 0, 0, 0);
    }
  }
  // lane holds pages p0 + 4*kq + i of row r0 + 16*rt + col
  float lnn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pp = p0 + 4 * kq + i;
    lnn[i] = pp < n ? __logf((float)page_valid(len, pp, p.P)) : 0.f;
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if (!row_ok[rt]) continue;
    const int r = r0 + 16 * rt + col;
    const int t = r / p.G, hl = r % p.G;
    float* dst = p.est + (((size_t)b * p.T + t) * p.Hq + (size_t)g * p.G + hl) * p.stride + p0 + 4 * kq;
    if (p0 + 4 * kq + 3 < n) {                     // 16-byte aligned: the row stride is a multiple of 4
      *reinterpret_cast<float4*>(dst) = float4{acc[rt][0] * p.sm_scale + lnn[0], acc[rt][1] * p.sm_scale + lnn[1],
                                               acc[rt][2] * p.sm_scale + lnn[2], acc[rt][3] * p.sm_scale + lnn[3]};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p0 + 4 * kq + i < n) dst[i] = acc[rt][i] * p.sm_scale + lnn[i];
    }
  }
}

// ---------------------------------------------------------- mass softmax
__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// grid (Hq, B), 256 threads
__global__ __launch_bounds__(256) void mass_softmax_kernel(MassParams p) {
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = (p.seq_lens[b] + p.P - 1) / p.P;
  if (n == 0) return;
  float* M = p.mass + ((size_t)b * p.Hq + h) * p.max_pages;
  for (int t = 0; t < p.T; ++t) {
    const float* e = p.est + (((size_t)b * p.T + t) * p.Hq + h) * p.stride;
    float mx = -INFINITY;
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += 256) mx = fmaxf(mx, e[i]);
    mx = block_max_256(mx, red);
    float sm = 0.f;
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += 256) sm += __expf(e[i] - mx);
    const float lse = mx + __logf(block_sum_256(sm, red));
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += 256) {
      const float v = __expf(e[i] - lse);
      M[i] = t == 0 ? v : M[i] + v;
    }
  }
}

hipError_t launch_head_mass(const MassParams& p, hipStream_t s) {
  dim3 g1((p.max_pages + 63) / 64, (p.T * p.G + 63) / 64, p.B * p.Hkv);
  if (p.d == 64) hipLaunchKernelGGL(mass_logits_kernel<64>, g1, dim3(256), 0, s, p);
  else if (p.d == 128) hipLaunchKernelGGL(mass_logits_kernel<128>, g1, dim3(256), 0, s, p);
  else if (p.d == 576) hipLaunchKernelGGL(mass_logits_kernel<576>, g1, dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  hipLaunchKernelGGL(mass_softmax_kernel, dim3(p.Hq, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

// The search grid (alphas, head counts, betas) copied from the kernel
// arguments into LDS in one round trip: indexed in a loop, each argument
// would be a scalar load of its own from the argument segment.
struct TuneGrid {
  int alpha[kTuneMaxGrid], heads[kTuneMaxGrid], beta[kTuneMaxGrid * kTuneMaxGrid];
};
__device__ __forceinline__ void load_grid(const TuneParams& p, TuneGrid& gr) {
  for (int i = threadIdx.x; i < kTuneMaxGrid * kTuneMaxGrid; i += blockDim.x) gr.beta[i] = p.beta[i];
  if (threadIdx.x < kTuneMaxGrid) {
    gr.alpha[threadIdx.x] = p.alpha[threadIdx.x];
    gr.heads[threadIdx.x] = p.heads[threadIdx.x];
  }
}

// ------------------------------------------------------------ page stats
// Rank of head i's mass among the group's G masses in vals: mass descending,
// head index ascending.
__device__ __forceinline__ int head_rank(const float* vals, int G, int i) {
  const float v = vals[i];
  int r = 0;
  for (int j = 0; j < G; ++j) {
    const float w = vals[j];
    r += (w > v || (w == v && j < i)) ? 1 : 0;
  }
  return r;
}

// Bitonic sorts of NS independent sets of 128 values, each held two per lane
// (element lane in a[q], element lane + 64 in b[q]), into descending order
// across the wave.  The sets' compare-exchange chains interleave, so the
// cross-lane exchanges of one hide the latency of the others'.
template <int NS>
__device__ __forceinline__ void sort128_desc(float (&a)[NS], float (&b)[NS]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1) {
      if (j == 64) {                                // pairs (lane, lane + 64)
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          const float hi = fmaxf(a[q], b[q]), lo = fminf(a[q], b[q]);
          a[q] = hi;
          b[q] = lo;
        }
      } else {
        const bool lower = (lane & j) == 0;
        const bool desc_a = (lane & size) == 0, desc_b = ((lane + 64) & size) == 0;
        float pa[NS], pb[NS];
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          pa[q] = __shfl_xor(a[q], j, 64);
          pb[q] = __shfl_xor(b[q], j, 64);
        }
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          a[q] = (lower == desc_a) ? fmaxf(a[q], pa[q]) : fminf(a[q], pa[q]);
          b[q] = (lower == desc_b) ? fmaxf(b[q], pb[q]) : fminf(b[q], pb[q]);
        }
      }
    }
  }
}

// grid (ceil(max_pages/64), B*Hkv), 256 threads: the group's masses of 64
// consecutive pages are read row by row (coalesced) into LDS, then each wave
// takes 16 of the pages: a page's G masses are sorted across the wave (masses
// are >= 0; padding -1 sorts last), so a top-h sum is a prefix.
__global__ __launch_bounds__(256) void tier_page_kernel(TuneParams p) {
  __shared__ float vals[kTuneMaxGroup][65];
  __shared__ TuneGrid gr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y / p.Hkv, g = blockIdx.y % p.Hkv;
  const int n = (p.seq_lens[b] + p.P - 1) / p.P;
  const int p0 = blockIdx.x * 64;
  if (p0 >= n) return;                               // whole workgroup
  load_grid(p, gr);
  const float* m = p.mass + ((size_t)b * p.Hq + (size_t)g * p.G) * p.max_pages + p0;
  const int cols = min(64, n - p0);
  // the loads of 8 rows are issued before their LDS stores
  const int j = threadIdx.x & 63, h0 = threadIdx.x >> 6;
  for (int hb = 0; hb < p.G; hb += 32) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int h = min(hb + h0 + 4 * u, p.G - 1);
      v[u] = m[(size_t)h * p.max_pages + min(j, cols - 1)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (hb + h0 + 4 * u < p.G) vals[hb + h0 + 4 * u][j] = v[u];
  }
  __syncthreads();
  // 4 pages at a time per wave (pages past the sequence sort padding and are
  // not written)
  for (int j0 = wave * 16; j0 < wave * 16 + 16; j0 += 4) {
    float a[4], c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = min(j0 + q, 63);
      a[q] = lane < p.G ? vals[lane][j] : -1.f;
      c[q] = lane + 64 < p.G ? vals[lane + 64][j] : -1.f;
    }
    sort128_desc<4>(a, c);
    // inclusive prefix sums of the sorted masses (a: ranks 0-63, c: 64-127;
    // padding counted as 0): a top-h sum is one prefix value
    float sa[4], sc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sa[q] = a[q] > 0.f ? a[q] : 0.f;
      sc[q] = c[q] > 0.f ? c[q] : 0.f;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float ta = __shfl_up(sa[q], off, 64), tc = __shfl_up(sc[q], off, 64);
        if (lane >= off) {
          sa[q] += ta;
          sc[q] += tc;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float tot_a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sa[q]), 63));
      const float tot_c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[q]), 63));
      const size_t row = ((size_t)b * p.Hkv + g) * p.max_pages + p0 + j0 + q;
      if (lane == 0 && j0 + q < cols) p.mall[row] = tot_a + tot_c;
      for (int k = 0; k < p.n_h; ++k) {
        const int h = __builtin_amdgcn_readfirstlane(min(gr.heads[k], p.G));
        const float v = h <= 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sa[q]), h - 1))
                                : tot_a + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[q]), h - 65));
        if (lane == 0 && j0 + q < cols) p.tsum[row * p.n_h + k] = v;
      }
    }
  }
}

// ------------------------------------------------------------- coverage
// Key whose ascending order is (score descending, page ascending), NaN after
// every number, -0 == +0.
__device__ __forceinline__ uint64_t rank_key(float s, int page) {
  uint32_t hi;
  if (s != s) {
    hi = 0xffffffffu;
  } else {
    uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // increasing in s
    hi = ~ord;
  }
  return ((uint64_t)hi << 32) | (uint32_t)page;
}

// grid (ceil(max_pages/64), B*Hkv), 256 threads: page 64*blockIdx.x + j is
// ranked among its sequence's candidates by four threads (j, part), each
// counting the smaller keys in a quarter of the key array in LDS; wave 0 then
// adds the chunk's covered mass to every configuration, and the workgroup's
// sums go to part[bg][chunk][config].
__global__ __launch_bounds__(256) void tier_cover_kernel(TuneParams p) {
  __shared__ uint64_t key[kTuneMaxPages];
  __shared__ int rank_part[4][64];
  __shared__ TuneGrid gr;
  load_grid(p, gr);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bg = blockIdx.y;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int n = (p.seq_lens[b] + p.P - 1) / p.P;
  const int sink = min(p.sink, n), win_lo = max(0, n - p.window);
  const float* sc = p.scores + ((size_t)b * p.Hkv + g) * p.scores_stride;
  for (int i0 = 0; i0 < n; i0 += 1024) {              // 4 score loads in flight per thread
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = sc[min(i0 + (int)threadIdx.x + 256 * u, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + (int)threadIdx.x + 256 * u;
      if (i < n) key[i] = (i < sink || i >= win_lo) ? ~0ull : rank_key(v[u], i);
    }
  }
  __syncthreads();
  const int i = blockIdx.x * 64 + lane;
  const uint64_t ki = i < n ? key[i] : ~0ull;
  {
    const int q = (n + 3) / 4, lo = wave * q, hi = min(n, lo + q);
    int r = 0;
    for (int j = lo; j < hi; ++j) r += key[j] < ki ? 1 : 0;
    rank_part[wave][lane] = r;
  }
  __syncthreads();
  if (wave != 0) return;
  const int n_forced = n == 0 ? 0 : sink + (n - max(win_lo, sink));
  const int nc = n - n_forced;
  const bool forced = ki == ~0ull;
  const int rank = (rank_part[0][lane] + rank_part[1][lane]) + (rank_part[2][lane] + rank_part[3][lane]);
  float mall = 0.f;
  const float* ts = p.tsum;
  const size_t row = (size_t)bg * p.max_pages + (i < n ? i : 0);
  if (i < n) mall = p.mall[row];
  ts += row * p.n_h;
  const int n_cfg = p.n_a * p.n_h;
  const int nchunk = gridDim.x;
  for (int c = 0; c < n_cfg; ++c) {
    const int ia = c / p.n_h, ih = c % p.n_h;
    const int beta = gr.beta[c];
    float acc = 0.f;
    if (beta >= 0 && i < n) {
      const int a_eff = min(gr.alpha[ia], nc);
      const int b_eff = min(beta, nc - a_eff);
      if (forced || rank < a_eff) acc = mall;
      else if (rank < a_eff + b_eff) acc = ts[ih];
    }
    acc = wave_sum(acc);
    if (lane == 0) p.part[((size_t)bg * nchunk + blockIdx.x) * n_cfg + c] = acc;
  }
}

// one workgroup of 256 threads: the layer's coverage of each configuration
// (one wave per configuration, its partial sums reduced in a fixed order) and
// the first maximum
__global__ __launch_bounds__(256) void tier_choose_kernel(TuneParams p, int nchunk) {
  __shared__ float cov[kTuneMaxGrid * kTuneMaxGrid];
  __shared__ TuneGrid gr;
  load_grid(p, gr);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_cfg = p.n_a * p.n_h;
  const int nbg = p.B * p.Hkv;
  const int nparts = nbg * nchunk;
  for (int c = wave; c < n_cfg; c += 4) {
    float s = 0.f;
#pragma unroll 4
    for (int k = lane; k < nparts; k += 64) s += p.part[(size_t)k * n_cfg + c];
    s = wave_sum(s) / (float)(p.T * p.G);
    const float v = gr.beta[c] >= 0 ? s / (float)nbg : __builtin_nanf("");
    if (lane == 0) {
      cov[c] = v;
      p.coverage[c] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = -1;
    for (int c = 0; c < n_cfg; ++c) {
      if (gr.beta[c] < 0) continue;
      if (best < 0 || cov[c] > cov[best]) best = c;
    }
    p.choice[0] = best < 0 ? -1 : best / p.n_h;
    p.choice[1] = best < 0 ? -1 : best % p.n_h;
    p.choice[2] = best < 0 ? -1 : gr.beta[best];
  }
}

int autotune_chunks(int max_pages) { return (max_pages + 63) / 64; }

hipError_t launch_autotune(const TuneParams& p, hipStream_t s) {
  if (p.G > kTuneMaxGroup || p.max_pages > kTuneMaxPages || p.n_a > kTuneMaxGrid || p.n_h > kTuneMaxGrid)
    return hipErrorInvalidValue;
  const int nchunk = autotune_chunks(p.max_pages);
  hipLaunchKernelGGL(tier_page_kernel, dim3((p.max_pages + 63) / 64, p.B * p.Hkv), dim3(256), 0, s, p);
  hipLaunchKernelGGL(tier_cover_kernel, dim3(nchunk, p.B * p.Hkv), dim3(256), 0, s, p);
  hipLaunchKernelGGL(tier_choose_kernel, dim3(1), dim3(256), 0, s, p, nchunk);
  return hipGetLastError();
}

// ------------------------------------------------------------ ambient mask
__global__ void clear_words_kernel(uint32_t* w, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    w[i] = 0u;
}

// grid (B*Hkv, ceil(list_stride/4)), 256 threads: wave w takes Ambient entry
// cc + 4*blockIdx.y + w of KV head g's list
__global__ __launch_bounds__(256) void ambient_mask_kernel(AmbientMaskParams p) {
  __shared__ float vals[4][kTuneMaxGroup];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x / p.Hkv, g = blockIdx.x % p.Hkv;
  const int cnt = p.counts[(size_t)b * p.Hkv + g];
  const int cc = p.ccounts[(size_t)b * p.Hkv + g];
  const int32_t* list = p.lists + ((size_t)b * p.Hkv + g) * p.list_stride;
  const int e = cc + 4 * (int)blockIdx.y + wave;
  const bool ok = e >= cc && e < min(cnt, p.list_stride);
  int pg = ok ? list[e] : 0;
  const bool in_range = ok && pg >= 0 && pg < p.max_pages;
  if (!in_range) pg = 0;
  for (int i = lane; i < p.G; i += 64)
    vals[wave][i] = in_range ? p.mass[((size_t)b * p.Hq + (size_t)g * p.G + i) * p.max_pages + pg] : 0.f;
  __syncthreads();
  if (!in_range) return;
  for (int i = lane; i < p.G; i += 64) {
    if (head_rank(vals[wave], p.G, i) < p.h) {
      const int hq = g * p.G + i;
      atomicOr(p.mask + ((size_t)b * p.max_pages + pg) * p.words + (hq >> 5), 1u << (hq & 31));
    }
  }
}

hipError_t launch_ambient_mask(const AmbientMaskParams& p, hipStream_t s) {
  if (p.G > kTuneMaxGroup) return hipErrorInvalidValue;
  const size_t words = (size_t)p.B * p.max_pages * p.words;
  hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)std::min<size_t>((words + 255) / 256, 4096)), dim3(256), 0,
                     s, p.mask, words);
  hipLaunchKernelGGL(ambient_mask_kernel, dim3(p.B * p.Hkv, (p.list_stride + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
