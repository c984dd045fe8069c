// Page summaries (mean key per page) and router scores (pooled query . page
// mean), the block-granular routing step of "Universal Attention Engine",
// section "Content-Dependent Dynamic Routing": score = q @ mean(k_blocks).
//
// Both kernels are HBM-bound streams: the summary reads each page's keys once
// (16-byte vector loads), the score kernel reads one fp32 mean row per (page,
// KV head).  Both are written for memory-level parallelism: every load a
// thread needs is issued before its sums are formed.  Accumulation is float64
// (exact for sums of bf16 values of ordinary range), rounded once to fp32, so
// the scores that top-k ranks do not depend on summation order.
#include "common.h"

namespace sa {

// ------------------------------------------------------------------ summary
// grid (KV head, page slot, batch), block 256.  Thread (cg, ts) owns one
// 16-byte column group of the head's rows and every TS-th token; the TS
// partial sums are combined through LDS in a fixed order, so each page's mean
// is computed from all its loads in flight at once.
constexpr int kSumMaxPart = 2048;    // doubles: TS * d <= 16 * 128, 3 * 576

template <typename T, int VW>
__global__ __launch_bounds__(256) void page_summary_kernel(SummaryParams p) {
  __shared__ double part[kSumMaxPart];
  const int g = blockIdx.x, b = blockIdx.z;
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  int lp = blockIdx.y;
  if (p.last_pages > 0) lp = n - p.last_pages + (int)blockIdx.y;
  if (lp < 0 || lp >= n) return;                    // whole workgroup
  const int phys = p.block_table[(size_t)b * p.max_pages + lp];
  const int nv = page_valid(len, lp, p.P);
  const int CG = p.d / VW;
  const int TS = min(16, 256 / CG);
  const int t = threadIdx.x;
  if (t < CG * TS) {
    const int cg = t % CG, ts = t / CG;
    const T* base = reinterpret_cast<const T*>(p.k_pool) + (((size_t)phys * p.n_kv + g) * p.P) * p.d + cg * VW;
    double acc[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) acc[i] = 0.0;
#pragma unroll 4
    for (int j = ts; j < nv; j += TS) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + (size_t)j * p.d);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += (double)bf16_lo(w[i]);
          acc[2 * i + 1] += (double)bf16_hi(w[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += (double)__uint_as_float(w[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < VW; ++i) part[ts * p.d + cg * VW + i] = acc[i];
  }
  __syncthreads();
  float* out = p.mu + ((size_t)phys * p.n_kv + g) * p.d;
  for (int e = t; e < p.d; e += 256) {
    double sum = 0.0;
    for (int ts = 0; ts < TS; ++ts) sum += part[ts * p.d + e];
    out[e] = (float)(sum / (double)nv);
  }
}

hipError_t launch_page_summary(const SummaryParams& p, int batch, int bf16, hipStream_t s) {
  const int slots = p.last_pages > 0 ? p.last_pages : p.max_pages;
  dim3 grid(p.n_kv, slots, batch);
  if (bf16)
    hipLaunchKernelGGL((page_summary_kernel<uint16_t, 8>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((page_summary_kernel<float, 4>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------- scores
template <typename T>
__device__ __forceinline__ double load_q(const T* q, size_t i) {
  if constexpr (sizeof(T) == 2) return (double)bf16_bits_to_f32(q[i]);
  else return (double)q[i];
}

// Query row r (0 .. rows) of selection head s -> (token, head).
__device__ __forceinline__ void pooled_row(const ScoreParams& p, int s, int r, int* t, int* h) {
  if (p.per_q) { *t = r; *h = s; }
  else { *t = r / p.G; *h = s * p.G + r % p.G; }
}

// Pooled query for selection heads with many rows (e.g. 2 tokens x 128 heads):
// grid (row chunk, n_sel, B), block 256.  Chunk c sums rows
// [c*rpc, (c+1)*rpc) into qpart[b][s][c][d] (float64; exact for sums of bf16
// values of ordinary range); the score kernel adds the chunks in order.
constexpr int kQChunks = 8;

template <typename T>
__global__ __launch_bounds__(256) void pooled_q_kernel(ScoreParams p, double* qpart) {
  __shared__ double part[kSumMaxPart];
  const int c = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int rows = p.per_q ? p.T : p.T * p.G;
  const int rpc = (rows + kQChunks - 1) / kQChunks;
  const int r0 = c * rpc, r1 = min(rows, r0 + rpc);
  const T* q = reinterpret_cast<const T*>(p.q);
  constexpr int VW = 16 / sizeof(T);
  const int CG = p.d / VW;
  const int RS = min(16, 256 / CG);
  const int t = threadIdx.x;
  if (t < CG * RS) {
    const int cg = t % CG, rs = t / CG;
    double acc[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) acc[i] = 0.0;
    // 8 rows' loads in flight, then added in row order
    for (int rb = r0 + rs; rb < r1; rb += 8 * RS) {
      u32x4 w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = rb + j * RS;
        int tt = 0, h = 0;
        if (r < r1) pooled_row(p, s, r, &tt, &h);
        w[j] = r < r1 ? *reinterpret_cast<const u32x4*>(q + (((size_t)b * p.T + tt) * p.Hq + h) * p.d + cg * VW)
                      : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (rb + j * RS >= r1) break;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += (double)bf16_lo(w[j][i]);
            acc[2 * i + 1] += (double)bf16_hi(w[j][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += (double)__uint_as_float(w[j][i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VW; ++i) part[rs * p.d + cg * VW + i] = acc[i];
  }
  __syncthreads();
  double* out = qpart + (((size_t)b * p.n_sel + s) * kQChunks + c) * p.d;
  for (int e = t; e < p.d; e += 256) {
    double sum = 0.0;
    for (int rs = 0; rs < RS; ++rs) sum += part[rs * p.d + e];
    out[e] = sum;
  }
}

// grid (page chunk of 64, n_sel, B), block 256.  The 64 pages' physical ids
// are read first; then every wave issues the mean-row loads of its 16 pages
// (4 pages of 16 lanes per step, all 4 steps in flight) before reducing.
// Lane `sub` of a page's 16 takes dims 64 i + 4 sub + 0..3, so each load
// instruction reads 256 contiguous bytes of the mean row; the float64
// products are summed in that order, then over the 16 lanes in a fixed
// butterfly, and rounded once to fp32.
template <typename T, int D>
__global__ __launch_bounds__(256) void page_score_kernel(ScoreParams p, const double* qpart) {
  constexpr int kPagesPerBlock = 64;
  constexpr int PL = D / 16;               // floats of a mean row per lane: 4, 8 or 36
  __shared__ double qbar[D];
  __shared__ int phys_s[kPagesPerBlock];
  const int b = blockIdx.z, s = blockIdx.y;
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  const int page0 = blockIdx.x * kPagesPerBlock;
  if (threadIdx.x < kPagesPerBlock) {
    // forced pages (first sink, last window) are scored only when the caller
    // asked for the scores; otherwise their mean rows are not read
    const int lp = page0 + threadIdx.x;
    const bool forced = lp < min(p.sink, n) || lp >= max(n - p.window, 0);
    phys_s[threadIdx.x] = (lp < n && !(p.skip_forced && forced)) ? p.block_table[(size_t)b * p.max_pages + lp] : -1;
  }
  if (qpart) {
    const double* qp = qpart + ((size_t)b * p.n_sel + s) * kQChunks * D;
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
      double v = 0.0;
      for (int c = 0; c < kQChunks; ++c) v += qp[(size_t)c * D + e];
      qbar[e] = v;
    }
  } else {
    const T* q = reinterpret_cast<const T*>(p.q);
    const int rows = p.per_q ? p.T : p.T * p.G;
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
      double v = 0.0;
      for (int r = 0; r < rows; ++r) {
        int tt, h;
        pooled_row(p, s, r, &tt, &h);
        v += load_q(q, (((size_t)b * p.T + tt) * p.Hq + h) * D + e);
      }
      qbar[e] = v;
    }
  }
  __syncthreads();
  const int g = p.per_q ? s / p.G : s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, slot = lane >> 4;
  f32x4 v[4][PL / 4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int ph = phys_s[wave * 16 + it * 4 + slot];
    const float* m = p.mu + ((size_t)max(ph, 0) * p.Hkv + g) * D + 4 * sub;
#pragma unroll
    for (int i = 0; i < PL / 4; ++i) v[it][i] = ph >= 0 ? *reinterpret_cast<const f32x4*>(m + 64 * i) : f32x4{};
  }
  float* out = p.scores + ((size_t)b * p.n_sel + s) * p.max_pages;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int lp = page0 + wave * 16 + it * 4 + slot;
    const double* qq = qbar + 4 * sub;
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < PL / 4; ++i) {
      acc += qq[64 * i] * (double)v[it][i][0];
      acc += qq[64 * i + 1] * (double)v[it][i][1];
      acc += qq[64 * i + 2] * (double)v[it][i][2];
      acc += qq[64 * i + 3] * (double)v[it][i][3];
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (sub == 0 && lp < p.max_pages) out[lp] = lp < n ? (float)acc : __builtin_nanf("");
  }
}

hipError_t launch_page_scores_ws(const ScoreParams& p, int bf16, double* qpart_ws, hipStream_t s) {
  const int rows = p.per_q ? p.T : p.T * p.G;
  const bool big = rows > 32;
  if (big) {
    dim3 g(kQChunks, p.n_sel, p.B);
    if (bf16) hipLaunchKernelGGL((pooled_q_kernel<uint16_t>), g, dim3(256), 0, s, p, qpart_ws);
    else hipLaunchKernelGGL((pooled_q_kernel<float>), g, dim3(256), 0, s, p, qpart_ws);
  }
  dim3 grid((p.max_pages + 63) / 64, p.n_sel, p.B);
  const double* qw = big ? qpart_ws : nullptr;
#define SA_SCORE_LAUNCH(T_, D_) hipLaunchKernelGGL((page_score_kernel<T_, D_>), grid, dim3(256), 0, s, p, qw)
  if (bf16) {
    if (p.d == 64) SA_SCORE_LAUNCH(uint16_t, 64);
    else if (p.d == 128) SA_SCORE_LAUNCH(uint16_t, 128);
    else SA_SCORE_LAUNCH(uint16_t, 576);
  } else {
    if (p.d == 64) SA_SCORE_LAUNCH(float, 64);
    else SA_SCORE_LAUNCH(float, 128);
  }
#undef SA_SCORE_LAUNCH
  return hipGetLastError();
}

}  // namespace sa
