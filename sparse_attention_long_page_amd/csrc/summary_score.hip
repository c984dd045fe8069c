// Page summaries (mean key per page) and router scores (pooled query . page
// mean), the block-granular routing step of "Universal Attention Engine",
// section "Content-Dependent Dynamic Routing": score = q @ mean(k_blocks).
//
// Both kernels are HBM-bound streams: the summary reads each page's keys once
// (16-byte vector loads, consecutive threads on consecutive columns), the
// score kernel reads one fp32 mean row per (page, KV head).  Accumulation is
// float64 (exact for sums of bf16 values), rounded once to fp32, so the
// scores that top-k ranks do not depend on summation order.
#include "common.h"

namespace sa {

// ------------------------------------------------------------------ summary
// grid (page slot, batch), block 256.  Thread handles VW consecutive columns
// of one KV head and walks the page's valid tokens.
template <typename T, int VW>
__global__ __launch_bounds__(256) void page_summary_kernel(SummaryParams p) {
  const int b = blockIdx.y;
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  int lp = blockIdx.x;
  if (p.last_pages > 0) lp = n - p.last_pages + (int)blockIdx.x;
  if (lp < 0 || lp >= n) return;
  const int phys = p.block_table[(size_t)b * p.max_pages + lp];
  const int nv = page_valid(len, lp, p.P);
  const int groups_per_head = p.d / VW;
  const int groups = p.n_kv * groups_per_head;
  const T* kp = reinterpret_cast<const T*>(p.k_pool);
  for (int c = threadIdx.x; c < groups; c += blockDim.x) {
    const int g = c / groups_per_head;
    const int e0 = (c % groups_per_head) * VW;
    const T* base = kp + (((size_t)phys * p.n_kv + g) * p.P) * p.d + e0;
    double acc[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) acc[i] = 0.0;
    for (int j = 0; j < nv; ++j) {
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
    float* out = p.mu + ((size_t)phys * p.n_kv + g) * p.d + e0;
#pragma unroll
    for (int i = 0; i < VW; ++i) out[i] = (float)(acc[i] / (double)nv);
  }
}

hipError_t launch_page_summary(const SummaryParams& p, int batch, int bf16, hipStream_t s) {
  const int slots = p.last_pages > 0 ? p.last_pages : p.max_pages;
  dim3 grid(slots, batch);
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

// Pooled query of selection head s: sum over query tokens and the head's
// query heads, float64.  Row r of the pool -> (t, h).
template <typename T>
__device__ __forceinline__ double pooled_q(const ScoreParams& p, const T* q, int b, int s, int e) {
  double acc = 0.0;
  if (p.per_q) {
    for (int t = 0; t < p.T; ++t) acc += load_q(q, (((size_t)b * p.T + t) * p.Hq + s) * p.d + e);
  } else {
    for (int t = 0; t < p.T; ++t)
      for (int hg = 0; hg < p.G; ++hg)
        acc += load_q(q, (((size_t)b * p.T + t) * p.Hq + s * p.G + hg) * p.d + e);
  }
  return acc;
}

// grid (column chunk of 64, n_sel, B), block 256 (4 row lanes x 64 columns):
// pooled query for configurations with many pooled rows (e.g. 2 tokens x 128
// heads); written to a float64 workspace the score kernel reads.
template <typename T>
__global__ __launch_bounds__(256) void pooled_q_kernel(ScoreParams p, double* qbar) {
  const int b = blockIdx.z, s = blockIdx.y;
  const int e = blockIdx.x * 64 + (threadIdx.x & 63);
  const int r0 = threadIdx.x >> 6;
  const T* q = reinterpret_cast<const T*>(p.q);
  const int rows = p.per_q ? p.T : p.T * p.G;
  double acc = 0.0;
  if (e < p.d) {
    for (int r = r0; r < rows; r += 4) {
      int t, h;
      if (p.per_q) { t = r; h = s; } else { t = r / p.G; h = s * p.G + r % p.G; }
      acc += load_q(q, (((size_t)b * p.T + t) * p.Hq + h) * p.d + e);
    }
  }
  __shared__ double part[4][64];
  part[r0][threadIdx.x & 63] = acc;
  __syncthreads();
  if (r0 == 0 && e < p.d) {
    // fixed order (r0 = 0..3) so the result is deterministic; exact for bf16 sums
    double v = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] + part[3][threadIdx.x];
    qbar[((size_t)b * p.n_sel + s) * p.d + e] = v;
  }
}

// grid (page chunk of 64, n_sel, B), block 256.  16 lanes per page, 4 pages
// per wave per step; each lane owns d/16 consecutive dims of the mean row.
template <typename T>
__global__ __launch_bounds__(256) void page_score_kernel(ScoreParams p, const double* qbar_ws) {
  constexpr int kPagesPerBlock = 64;
  __shared__ double qbar[576];
  const int b = blockIdx.z, s = blockIdx.y;
  const T* q = reinterpret_cast<const T*>(p.q);
  if (qbar_ws) {
    for (int e = threadIdx.x; e < p.d; e += blockDim.x) qbar[e] = qbar_ws[((size_t)b * p.n_sel + s) * p.d + e];
  } else {
    for (int e = threadIdx.x; e < p.d; e += blockDim.x) qbar[e] = pooled_q(p, q, b, s, e);
  }
  __syncthreads();
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  const int g = p.per_q ? s / p.G : s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, slot = lane >> 4;
  const int per_lane = p.d / 16;          // 4, 8 or 36 floats
  float* out = p.scores + ((size_t)b * p.n_sel + s) * p.max_pages;
  const int page0 = blockIdx.x * kPagesPerBlock;
  for (int it = 0; it < kPagesPerBlock; it += 16) {
    const int lp = page0 + it + wave * 4 + slot;
    double acc = 0.0;
    const bool valid = lp < n;
    if (valid) {
      const int phys = p.block_table[(size_t)b * p.max_pages + lp];
      const float* m = p.mu + ((size_t)phys * p.Hkv + g) * p.d + sub * per_lane;
      const double* qq = qbar + sub * per_lane;
      for (int i = 0; i < per_lane; i += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(m + i);
        acc += qq[i] * (double)v[0];
        acc += qq[i + 1] * (double)v[1];
        acc += qq[i + 2] * (double)v[2];
        acc += qq[i + 3] * (double)v[3];
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (sub == 0 && lp < p.max_pages) out[lp] = valid ? (float)acc : __builtin_nanf("");
  }
}

hipError_t launch_page_scores_ws(const ScoreParams& p, int bf16, double* qbar_ws, hipStream_t s) {
  const int rows = p.per_q ? p.T : p.T * p.G;
  const bool big = rows > 32;
  if (big) {
    dim3 g((p.d + 63) / 64, p.n_sel, p.B);
    if (bf16) hipLaunchKernelGGL((pooled_q_kernel<uint16_t>), g, dim3(256), 0, s, p, qbar_ws);
    else hipLaunchKernelGGL((pooled_q_kernel<float>), g, dim3(256), 0, s, p, qbar_ws);
  }
  dim3 grid((p.max_pages + 63) / 64, p.n_sel, p.B);
  const double* qw = big ? qbar_ws : nullptr;
  if (bf16) hipLaunchKernelGGL((page_score_kernel<uint16_t>), grid, dim3(256), 0, s, p, qw);
  else hipLaunchKernelGGL((page_score_kernel<float>), grid, dim3(256), 0, s, p, qw);
  return hipGetLastError();
}

}  // namespace sa
