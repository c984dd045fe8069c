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

// Mean of page lp of sequence b, KV head g, by one 256-thread workgroup
// (part: kSumMaxPart doubles of LDS).
template <typename T, int VW>
__device__ __forceinline__ void summary_page(const SummaryParams& p, int g, int b, int lp, int len, double* part) {
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
    // all of this thread's rows (tokens ts, ts + TS, ... of a page of at most
    // 64) are loaded before any is added, then added in token order; rows
    // past nv re-read row nv - 1 and add +0.0 instead (exact: the sums start at
    // +0.0 and never become -0.0), so no load sits behind a branch
    auto rows = [&](auto rc) {
      constexpr int R = decltype(rc)::value;
      u32x4 w[R];
#pragma unroll
      for (int i = 0; i < R; ++i) w[i] = *reinterpret_cast<const u32x4*>(base + (size_t)min(ts + i * TS, nv - 1) * p.d);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const uint32_t keep = ts + i * TS < nv ? 0xffffffffu : 0u;
        if constexpr (sizeof(T) == 1) {
          // OCP E4M3 bytes -> exact values (via bf16); the page scale is applied to the sum
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t v = w[i][c] & keep;
            const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false));
            const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true));
            acc[4 * c] += (double)bf16_lo(lo);
            acc[4 * c + 1] += (double)bf16_hi(lo);
            acc[4 * c + 2] += (double)bf16_lo(hi);
            acc[4 * c + 3] += (double)bf16_hi(hi);
          }
        } else if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[2 * c] += (double)bf16_lo(w[i][c] & keep);
            acc[2 * c + 1] += (double)bf16_hi(w[i][c] & keep);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] += (double)__uint_as_float(w[i][c] & keep);
        }
      }
    };
    if (TS >= 16) rows(std::integral_constant<int, 4>{});
    else if (TS >= 8) rows(std::integral_constant<int, 8>{});
    else rows(std::integral_constant<int, 22>{});          // d 576: TS = 3
#pragma unroll
    for (int i = 0; i < VW; ++i) part[ts * p.d + cg * VW + i] = acc[i];
  }
  __syncthreads();
  float* out = p.mu + ((size_t)phys * p.n_kv + g) * p.d;
  // FP8: sum of the page's values times its scale (both exact in float64:
  // E4M3 values carry 4 significant bits, the scale 24)
  const double scale = sizeof(T) == 1 ? (double)p.k_scale[(size_t)phys * p.n_kv + g] : 1.0;
  for (int e = t; e < p.d; e += 256) {
    double sum = 0.0;
    for (int ts = 0; ts < TS; ++ts) sum += part[ts * p.d + e];
    out[e] = (float)(sum * scale / (double)nv);
  }
}

template <typename T, int VW>
__global__ __launch_bounds__(256) void page_summary_kernel(SummaryParams p) {
  __shared__ double part[kSumMaxPart];
  const int g = blockIdx.x, b = blockIdx.z;
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  int lp = blockIdx.y;
  if (p.last_pages > 0) lp = n - p.last_pages + (int)blockIdx.y;
  if (lp < 0 || lp >= n) return;                    // whole workgroup
  summary_page<T, VW>(p, g, b, lp, len, part);
}

hipError_t launch_page_summary(const SummaryParams& p, int batch, int bf16, hipStream_t s) {
  const int slots = p.last_pages > 0 ? p.last_pages : p.max_pages;
  dim3 grid(p.n_kv, slots, batch);
  if (p.k_scale)
    hipLaunchKernelGGL((page_summary_kernel<uint8_t, 16>), grid, dim3(256), 0, s, p);
  else if (bf16)
    hipLaunchKernelGGL((page_summary_kernel<uint16_t, 8>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((page_summary_kernel<float, 4>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------- scores
// Query row r (0 .. rows) of selection head s -> (token, head).
__device__ __forceinline__ void pooled_row(const ScoreParams& p, int s, int r, int* t, int* h) {
  if (p.per_q) { *t = r; *h = s; }
  else { *t = r / p.G; *h = s * p.G + r % p.G; }
}

// Pooled query for selection heads with many rows (e.g. 2 tokens x 128 heads):
// grid (row chunk, n_sel, B), block 256.  Chunk c sums rows
// [c*rpc, (c+1)*rpc) into qpart[b][s][c][d] (float64; exact for sums of bf16
// values of ordinary range); the score kernel adds the chunks in order.

// Row chunk c of the pooled query of selection head s, sequence b, by one
// 256-thread workgroup (part: kSumMaxPart doubles of LDS).
template <typename T>
__device__ __forceinline__ void pooled_chunk(const ScoreParams& p, double* qpart, int c, int s, int b, double* part) {
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
    // 16 rows' loads in flight, then added in row order
    for (int rb = r0 + rs; rb < r1; rb += 16 * RS) {
      u32x4 w[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // (unconditional loads: rows past the chunk re-read its last row)
        int tt, h;
        pooled_row(p, s, min(rb + j * RS, r1 - 1), &tt, &h);
        w[j] = *reinterpret_cast<const u32x4*>(q + (((size_t)b * p.T + tt) * p.Hq + h) * p.d + cg * VW);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // rows past the chunk add +0.0 (exact, see summary_page)
        const uint32_t keep = rb + j * RS < r1 ? 0xffffffffu : 0u;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += (double)bf16_lo(w[j][i] & keep);
            acc[2 * i + 1] += (double)bf16_hi(w[j][i] & keep);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += (double)__uint_as_float(w[j][i] & keep);
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

// Everything the selection of long lists needs before its scoring kernel, in
// one launch: workgroups [0, n_pooled) sum the pooled-query row chunks
// (chunk, selection head, sequence), the next n_refresh ones recompute each
// sequence's newest-page summary (KV head, sequence) exactly as
// page_summary_kernel does, and workgroup 0 also clears the per-list arrival
// counters the scoring kernel counts its workgroups with.
template <typename T, int VW>
__global__ __launch_bounds__(256) void select_prep_kernel(SummaryParams smp, ScoreParams sp, double* qpart,
                                                          uint32_t* arrivals, int n_pooled, int n_refresh,
                                                          int n_arrivals) {
  __shared__ double part[kSumMaxPart];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_arrivals; i += 256) arrivals[i] = 0u;
  int w = blockIdx.x;
  if (w < n_pooled) {
    const int c = w % kQChunks;
    w /= kQChunks;
    pooled_chunk<T>(sp, qpart, c, w % sp.n_sel, w / sp.n_sel, part);
    return;
  }
  w -= n_pooled;
  if (w >= n_refresh) return;                       // (the one workgroup of a launch with neither)
  const int g = w % smp.n_kv, b = w / smp.n_kv;
  const int len = smp.seq_lens[b];
  const int n = (len + smp.P - 1) / smp.P;
  if (n > 0) summary_page<T, VW>(smp, g, b, n - 1, len, part);
}

hipError_t launch_select_prep(const SummaryParams& smp, const ScoreParams& sp, int bf16, bool refresh, double* qpart,
                              uint32_t* arrivals, hipStream_t s) {
  const int rows = sp.per_q ? sp.T : sp.T * sp.G;
  const int n_pooled = rows > kScoreInlineRows ? kQChunks * sp.n_sel * sp.B : 0;
  const int n_refresh = refresh ? smp.n_kv * sp.B : 0;
  const int n_arrivals = sp.n_sel * sp.B;
  const dim3 grid(max(1, n_pooled + n_refresh));
  if (bf16)
    hipLaunchKernelGGL((select_prep_kernel<uint16_t, 8>), grid, dim3(256), 0, s, smp, sp, qpart, arrivals, n_pooled,
                       n_refresh, n_arrivals);
  else
    hipLaunchKernelGGL((select_prep_kernel<float, 4>), grid, dim3(256), 0, s, smp, sp, qpart, arrivals, n_pooled,
                       n_refresh, n_arrivals);
  return hipGetLastError();
}

}  // namespace sa
