// Mean correction of a block-sparse chunked prefill, and the per-page mean
// value rows it needs (block-sparse prefill brief on the Paperraft page: a
// mean correction term beside pattern discovery and thresholding, bounding the
// error of the blocks left out).  Reading of the unstated formula: every
// causal block the group's union table skips that lies wholly at or before the
// query stands in for its n_b tokens by its mean key mu_b and mean value nu_b,
// i.e. one extra softmax term of log-weight sm_scale * q . mu_b + ln n_b and
// value nu_b.
//
// mean_correct_kernel: workgroup = (64-query tile, query head), 4 waves of 16
// query rows.  The prefill's (o, lse) of a row is one term of log-weight lse
// and value o; the skipped blocks are further terms, taken 16 at a time:
// their mean keys and values (fp32 page summaries, rounded to bf16) are staged
// in LDS, S^T = Mu Q^T and O^T += Nu^T P^T run on v_mfma_f32_16x16x16_bf16
// (the S^T fragment a lane holds is exactly its B operand of the PV product),
// with an online softmax per row.  The corrected (o, lse) overwrite the
// prefill's.
#include "common.h"

namespace sa {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ value means
// grid (KV head, page slot, batch), block 128: thread e sums dim e of the
// page's valid tokens (contiguous in the page-transposed pool) in float64.
template <typename T>
__global__ __launch_bounds__(128) void page_value_summary_kernel(ValueSummaryParams p) {
  const int g = blockIdx.x, b = blockIdx.z;
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  int lp = blockIdx.y;
  if (p.last_pages > 0) lp = n - p.last_pages + (int)blockIdx.y;
  if (lp < 0 || lp >= n) return;
  const int phys = p.block_table[(size_t)b * p.max_pages + lp];
  const int nv = page_valid(len, lp, p.P);
  for (int e = threadIdx.x; e < p.d_v; e += 128) {
    const T* row = reinterpret_cast<const T*>(p.v_pool) + (((size_t)phys * p.n_kv + g) * p.d_v + e) * p.P;
    double acc = 0.0;
    for (int j = 0; j < nv; ++j) {
      if constexpr (sizeof(T) == 1) {
        const uint32_t bits = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                                               (uint32_t)row[j], 1.0f, false));
        acc += (double)bf16_lo(bits);
      } else if constexpr (sizeof(T) == 2) {
        acc += (double)bf16_bits_to_f32(row[j]);
      } else {
        acc += (double)row[j];
      }
    }
    const double scale = sizeof(T) == 1 ? (double)p.v_scale[(size_t)phys * p.n_kv + g] : 1.0;
    p.nu[((size_t)phys * p.n_kv + g) * p.d_v + e] = (float)(acc * scale / (double)nv);
  }
}

hipError_t launch_page_value_summary(const ValueSummaryParams& p, int batch, int elem_bytes, hipStream_t s) {
  const int slots = p.last_pages > 0 ? p.last_pages : p.max_pages;
  dim3 grid(p.n_kv, slots, batch);
  if (elem_bytes == 1) hipLaunchKernelGGL((page_value_summary_kernel<uint8_t>), grid, dim3(128), 0, s, p);
  else if (elem_bytes == 2) hipLaunchKernelGGL((page_value_summary_kernel<uint16_t>), grid, dim3(128), 0, s, p);
  else hipLaunchKernelGGL((page_value_summary_kernel<float>), grid, dim3(128), 0, s, p);
  return hipGetLastError();
}

// -------------------------------------------------------- mean correction
constexpr int kMcD = 128;               // head dim
constexpr int kMcChunk = 16;            // skipped blocks per MFMA tile
constexpr int kMcKRow = kMcD + 8;       // LDS row of a mean key, bf16 (padded)

__global__ __launch_bounds__(256) void mean_correct_kernel(MeanCorrParams p) {
  __shared__ int skip[kPrefillMaxBlocks];
  __shared__ uint8_t in_table[kPrefillMaxBlocks];
  __shared__ int n_skip_s;
  __shared__ __attribute__((aligned(16))) uint16_t mk[kMcChunk * kMcKRow];     // [block][dim]
  __shared__ __attribute__((aligned(16))) uint16_t nvT[kMcD * kMcChunk];       // [dim][block]
  __shared__ int blk_nv[kMcChunk];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int g = h / p.G;
  const int seq_len = *p.seq_len;
  const int n_seq = seq_len > 0 ? (seq_len + p.P - 1) / p.P : 0;
  const int q0 = tile * 64;
  const int last_pos = p.q_start + min(q0 + 64, p.q_len) - 1;

  // the skipped causal blocks wholly at or before the tile's last position, ascending
  const int n_blk = min(n_seq, p.nkb);
  for (int kb = threadIdx.x; kb < n_blk; kb += 256) in_table[kb] = 0;
  __syncthreads();
  const int cnt = p.counts[g];
  for (int t = threadIdx.x; t < cnt; t += 256) {
    const int kb = p.table[(size_t)g * p.nkb + t];
    if (kb >= 0 && kb < n_blk) in_table[kb] = 1;
  }
  if (threadIdx.x == 0) n_skip_s = 0;
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int kb0 = 0; kb0 < n_blk; kb0 += 64) {
      const int kb = kb0 + lane;
      bool take = false;
      if (kb < n_blk && !in_table[kb]) take = kb * p.P + page_valid(seq_len, kb, p.P) - 1 <= last_pos;
      const unsigned long long m = __ballot(take);
      const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (take) skip[base + before] = kb;
      base += __popcll(m);
    }
    if (lane == 0) n_skip_s = base;
  }
  __syncthreads();
  const int n_skip = n_skip_s;
  if (n_skip == 0) return;                           // nothing to correct: (o, lse) stand

  // this wave's 16 query rows: row col of the MFMA tiles
  const int i = q0 + 16 * wave + col;
  const bool row_ok = i < p.q_len;
  const int pos = p.q_start + i;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  // Q^T operand of k-step ks: row col, dims 16*ks + 4*kq .. +3
  bf16x4 qreg[kMcD / 16];
#pragma unroll
  for (int ks = 0; ks < kMcD / 16; ++ks) {
    const size_t off = ((size_t)(row_ok ? i : 0) * p.Hq + h) * kMcD + 16 * ks + 4 * kq;
    qreg[ks] = *reinterpret_cast<const bf16x4*>(qp + off);
  }
  // the prefill's result as the first term: log-weight lse, value o.  O^T
  // accumulator of dim tile dt: dims 16*dt + 4*kq .. +3 of row col
  uint16_t* op = reinterpret_cast<uint16_t*>(p.out);
  const size_t orow = ((size_t)(row_ok ? i : 0) * p.Hq + h);
  float m = row_ok ? p.out_lse[orow] * kLog2e : -INFINITY;     // base 2
  float l = m == -INFINITY ? 0.f : 1.f;
  f32x4 oacc[kMcD / 16];
#pragma unroll
  for (int dt = 0; dt < kMcD / 16; ++dt) {
    const uint2 w = *reinterpret_cast<const uint2*>(op + orow * kMcD + 16 * dt + 4 * kq);
    const bool keep = l > 0.f;
    oacc[dt] = f32x4{keep ? bf16_lo(w.x) : 0.f, keep ? bf16_hi(w.x) : 0.f, keep ? bf16_lo(w.y) : 0.f,
                     keep ? bf16_hi(w.y) : 0.f};
  }

  for (int c0 = 0; c0 < n_skip; c0 += kMcChunk) {
    // stage the chunk's mean keys (rows) and mean values (transposed) as bf16
    __syncthreads();
    for (int idx = threadIdx.x; idx < kMcChunk * kMcD; idx += 256) {
      const int jb = idx / kMcD, e = idx % kMcD;
      const int c = c0 + jb;
      float kv = 0.f, vv = 0.f;
      if (c < n_skip) {
        const int phys = p.bt_row[skip[c]];
        const size_t off = ((size_t)phys * p.Hkv + g) * kMcD + e;
        kv = p.mu[off];
        vv = p.nu[off];
      }
      mk[jb * kMcKRow + e] = f32_to_bf16_bits(kv);
      nvT[e * kMcChunk + jb] = f32_to_bf16_bits(vv);
      if (e == 0) blk_nv[jb] = c < n_skip ? page_valid(seq_len, skip[c], p.P) : 0;
    }
    __syncthreads();
    // S^T[block][row] over the 16 blocks: lane holds blocks 4*kq .. +3 of row col
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kMcD / 16; ++ks) {
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(&mk[col * kMcKRow + 16 * ks + 4 * kq]);
      s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, qreg[ks], s, 0, 0, 0);
    }
    // log-weights (base 2): scale * s + log2(n_b); blocks not wholly at or
    // before this row's position (or past the list) take no part
    float z[4], zmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jb = 4 * kq + r, c = c0 + jb;
      const int nvb = blk_nv[jb];
      const bool vis = row_ok && c < n_skip && skip[c] * p.P + nvb - 1 <= pos;
      z[r] = vis ? s[r] * p.scale_log2 + __log2f((float)nvb) : -INFINITY;
      zmax = fmaxf(zmax, z[r]);
    }
    // row maximum over the 4 lane groups holding the row's 16 blocks
    zmax = max_over_row_groups(zmax);
    const float m_new = fmaxf(m, zmax);
    // a row with no term yet keeps alpha 1 and adds zeros (every lane takes
    // part in the MFMAs below)
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
    const float msub = none ? 0.f : m_new;
    float psum = 0.f;
    bf16x4 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = __builtin_amdgcn_exp2f(z[r] - msub);
      psum += pv;
      pb[r] = (__bf16)pv;
    }
    psum = sum_over_row_groups(psum);
    l = l * alpha + psum;
    m = m_new;
    // O^T[dim][row] += Nu^T[dim][block] P^T[block][row]
#pragma unroll
    for (int dt = 0; dt < kMcD / 16; ++dt) {
      oacc[dt][0] *= alpha; oacc[dt][1] *= alpha; oacc[dt][2] *= alpha; oacc[dt][3] *= alpha;
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(&nvT[(16 * dt + col) * kMcChunk + 4 * kq]);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, oacc[dt], 0, 0, 0);
    }
  }
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int dt = 0; dt < kMcD / 16; ++dt) {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16_bits(oacc[dt][0] * inv) | ((uint32_t)f32_to_bf16_bits(oacc[dt][1] * inv) << 16);
    w.y = (uint32_t)f32_to_bf16_bits(oacc[dt][2] * inv) | ((uint32_t)f32_to_bf16_bits(oacc[dt][3] * inv) << 16);
    *reinterpret_cast<uint2*>(op + orow * kMcD + 16 * dt + 4 * kq) = w;
  }
  if (kq == 0) p.out_lse[orow] = m == -INFINITY ? -INFINITY : (m + __log2f(l)) * kLn2;
}

hipError_t launch_mean_correct(const MeanCorrParams& p, hipStream_t s) {
  dim3 grid((p.q_len + 63) / 64, p.Hq);
  hipLaunchKernelGGL(mean_correct_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
