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
//    workgroup on v_mfma_f32_16x16x32_bf16.  The fp32 mean keys are split as
//    hi + lo bf16 (two MFMAs per step, residual below 2^-17 relative), the
//    bf16 queries are exact, so the products are fp32-accurate.
//  * mass_softmax_kernel: per (sequence, query head), the softmax over pages
//    of each query token's row, summed into M.
//  * tier_page_kernel: per (sequence, KV head, page) the page's mass over the
//    group and the sums of its top-h head masses for each searched h (rank by
//    counting: mass descending, head ascending).
//  * tier_coverage_kernel: per (sequence, KV head) the candidates' rank order
//    (router score descending, page ascending, NaN last; rank by counting)
//    and every configuration's covered mass.
//  * tier_choose_kernel: mean over sequences and KV heads, first maximum.
//  * ambient_mask_kernel: the top-h heads of every Ambient page of a list.
#include "common.h"

namespace sa {

// ------------------------------------------------------------ mass logits
// grid (page tiles of 64, row tiles of 64, B*Hkv), 256 threads: wave w takes
// pages 16w..16w+15 of the tile against the tile's 64 query rows of KV head
// g (row r = t*G + head-in-group).
template <int D>
__global__ __launch_bounds__(256) void mass_logits_kernel(MassParams p) {
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

  // A operand: mean key of page p0 + col, dims 32*ks + 8*kq .. +7
  const int pg = p0 + col;
  const float* murow = p.mu + ((size_t)bt[pg < n ? pg : 0] * p.Hkv + g) * D;
  // B operands: query rows r0 + 16*rt + col
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(p.q);
  bool row_ok[4];
  size_t qoff[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int r = r0 + 16 * rt + col;
    row_ok[rt] = r < TG;
    const int t = row_ok[rt] ? r / p.G : 0, hl = row_ok[rt] ? r % p.G : 0;
    qoff[rt] = (((size_t)b * p.T + t) * p.Hq + (size_t)g * p.G + hl) * D;
  }
  f32x4 acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
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
      bf16x8 bq;
      if (row_ok[rt]) {
        bq = *reinterpret_cast<const bf16x8*>(qbase + qoff[rt] + 32 * ks + 8 * kq);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) bq[i] = (__bf16)0.f;
      }
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
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (p0 + 4 * kq + i < n) dst[i] = acc[rt][i] * p.sm_scale + lnn[i];
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
    for (int i = threadIdx.x; i < n; i += 256) mx = fmaxf(mx, e[i]);
    mx = block_max_256(mx, red);
    float sm = 0.f;
    for (int i = threadIdx.x; i < n; i += 256) sm += __expf(e[i] - mx);
    const float lse = mx + __logf(block_sum_256(sm, red));
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

// grid (ceil(max_pages/4), B*Hkv), 256 threads: wave w takes one page
__global__ __launch_bounds__(256) void tier_page_kernel(TuneParams p) {
  __shared__ float vals[4][kTuneMaxGroup];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y / p.Hkv, g = blockIdx.y % p.Hkv;
  const int n = (p.seq_lens[b] + p.P - 1) / p.P;
  const int pg = blockIdx.x * 4 + wave;
  const bool ok = pg < n;
  for (int i = lane; i < p.G; i += 64)
    vals[wave][i] = ok ? p.mass[((size_t)b * p.Hq + (size_t)g * p.G + i) * p.max_pages + pg] : 0.f;
  __syncthreads();
  if (!ok) return;
  float v[2] = {0.f, 0.f};
  int rk[2] = {kTuneMaxGroup, kTuneMaxGroup};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    if (i < p.G) {
      v[k] = vals[wave][i];
      rk[k] = head_rank(vals[wave], p.G, i);
    }
  }
  const size_t row = ((size_t)b * p.Hkv + g) * p.max_pages + pg;
  const float all = wave_sum(v[0] + v[1]);
  if (lane == 0) p.mall[row] = all;
  for (int k = 0; k < p.n_h; ++k) {
    const int h = p.heads[k];
    const float part = wave_sum((rk[0] < h ? v[0] : 0.f) + (rk[1] < h ? v[1] : 0.f));
    if (lane == 0) p.tsum[row * p.n_h + k] = part;
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

// grid (B*Hkv), 1024 threads
__global__ __launch_bounds__(1024) void tier_coverage_kernel(TuneParams p) {
  __shared__ uint64_t key[kTuneMaxPages];
  __shared__ float wpart[16][kTuneMaxGrid * kTuneMaxGrid];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bg = blockIdx.x;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int n = (p.seq_lens[b] + p.P - 1) / p.P;
  const int sink = min(p.sink, n), win_lo = max(0, n - p.window);
  const float* sc = p.scores + ((size_t)b * p.Hkv + g) * p.scores_stride;
  for (int i = threadIdx.x; i < n; i += 1024) {
    const bool forced = i < sink || i >= win_lo;
    key[i] = forced ? ~0ull : rank_key(sc[i], i);
  }
  __syncthreads();
  const int n_forced = n == 0 ? 0 : sink + (n - max(win_lo, sink));
  const int nc = n - n_forced;
  // this thread's pages: forced flag, rank among the candidates
  constexpr int kPer = kTuneMaxPages / 1024;
  int rank[kPer];
  bool forced[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = threadIdx.x + 1024 * k;
    rank[k] = 0;
    forced[k] = false;
    if (i < n) {
      const uint64_t ki = key[i];
      forced[k] = ki == ~0ull;
      if (!forced[k]) {
        int r = 0;
        for (int j = 0; j < n; ++j) r += key[j] < ki ? 1 : 0;
        rank[k] = r;
      }
    }
  }
  const size_t row0 = (size_t)bg * p.max_pages;
  const int n_cfg = p.n_a * p.n_h;
  for (int c = 0; c < n_cfg; ++c) {
    const int ia = c / p.n_h, ih = c % p.n_h;
    const int beta = p.beta[c];
    float acc = 0.f;
    if (beta >= 0) {
      const int a_eff = min(p.alpha[ia], nc);
      const int b_eff = min(beta, nc - a_eff);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + 1024 * k;
        if (i >= n) continue;
        if (forced[k] || rank[k] < a_eff) acc += p.mall[row0 + i];
        else if (rank[k] < a_eff + b_eff) acc += p.tsum[(row0 + i) * p.n_h + ih];
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) wpart[wave][c] = acc;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < n_cfg; c += 1024) {
    float s = 0.f;
    for (int w = 0; w < 16; ++w) s += wpart[w][c];
    p.part[(size_t)bg * n_cfg + c] = p.beta[c] >= 0 ? s / (float)(p.T * p.G) : __builtin_nanf("");
  }
}

// one workgroup of 256 threads
__global__ __launch_bounds__(256) void tier_choose_kernel(TuneParams p) {
  __shared__ float cov[kTuneMaxGrid * kTuneMaxGrid];
  const int n_cfg = p.n_a * p.n_h;
  const int nbg = p.B * p.Hkv;
  for (int c = threadIdx.x; c < n_cfg; c += 256) {
    float s = 0.f;
    for (int i = 0; i < nbg; ++i) s += p.part[(size_t)i * n_cfg + c];
    const float v = p.beta[c] >= 0 ? s / (float)nbg : __builtin_nanf("");
    cov[c] = v;
    p.coverage[c] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = -1;
    for (int c = 0; c < n_cfg; ++c) {
      if (p.beta[c] < 0) continue;
      if (best < 0 || cov[c] > cov[best]) best = c;
    }
    p.choice[0] = best < 0 ? -1 : best / p.n_h;
    p.choice[1] = best < 0 ? -1 : best % p.n_h;
    p.choice[2] = best < 0 ? -1 : p.beta[best];
  }
}

hipError_t launch_autotune(const TuneParams& p, hipStream_t s) {
  if (p.G > kTuneMaxGroup || p.max_pages > kTuneMaxPages || p.n_a > kTuneMaxGrid || p.n_h > kTuneMaxGrid)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(tier_page_kernel, dim3((p.max_pages + 3) / 4, p.B * p.Hkv), dim3(256), 0, s, p);
  hipLaunchKernelGGL(tier_coverage_kernel, dim3(p.B * p.Hkv), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(tier_choose_kernel, dim3(1), dim3(256), 0, s, p);
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
