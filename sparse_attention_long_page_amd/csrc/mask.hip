// Block-level pattern discovery for a prefill chunk: the 2D block mask that
// the Q-block / intra-group union consumes (block-sparse prefill brief on the
// Paperraft page: instantaneous pattern discovery and max-based dynamic
// thresholding; score form of the "Universal Attention Engine" router,
// "Content-Dependent Dynamic Routing": pooled query against the block's mean
// key; mask structure of the CompactAttention abstract).
//
// One workgroup per (Q-block, KV head): the pooled queries (mean over the
// Q-block's queries, float64) of the head's query group are scored against
// the mean key of every causal KV block, read once for the whole group; each
// query head then keeps the sink block, its diagonal blocks and either the
// top-k other blocks or those within max_gap of its largest score, with the
// exact radix selection of the decode path (lowest block index first on
// ties), and writes its mask row.
#include "common.h"
#include "select_body.h"

namespace sa {

template <typename T, int D>
__global__ __launch_bounds__(kSelThreads) void block_mask_kernel(MaskParams mp) {
  constexpr int kMaxG = 8;
  constexpr int PL = D / 16;                 // dims per lane of a 16-lane block group
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ SelShared sh;
  __shared__ double qbar[kMaxG][D];
  __shared__ float red[kSelThreads / 64];
  __shared__ int32_t s_count[kMaxG];
  const int qb = blockIdx.x, g = blockIdx.y;
  const int G = mp.G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nkb = mp.nkb;
  float* scores = reinterpret_cast<float*>(dyn);                 // [G][nkb]
  uint32_t* keys = dyn + (size_t)G * nkb;                        // [nkb]
  int32_t* list = reinterpret_cast<int32_t*>(keys + nkb);        // [nkb]

  const int i0 = qb * mp.block_q, i1 = min(i0 + mp.block_q, mp.q_len);
  const int seq_len = *mp.seq_len;
  const int n_seq = seq_len > 0 ? (seq_len + mp.P - 1) / mp.P : 0;
  const int n = min(min((mp.q_start + i1 - 1) / mp.P + 1, n_seq), nkb);
  const int kb_lo = max(0, min((mp.q_start + i0) / mp.P, n - 1));

  // pooled queries: mean over the Q-block's rows, float64, rows added in
  // order.  The rows are loaded 16 at a time, unconditionally from clamped
  // indices (a load under a per-lane condition is waited for at once), and
  // rows past the Q-block add +0.0, which leaves the sum unchanged (it starts
  // at +0.0 and never becomes -0.0).
  const T* q = reinterpret_cast<const T*>(mp.q);
  for (int idx = threadIdx.x; idx < G * D; idx += kSelThreads) {
    const int hh = idx / D, e = idx % D;
    const int h = g * G + hh;
    double acc = 0.0;
    for (int i = i0; i < i1; i += 16) {
      float w[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const size_t off = ((size_t)min(i + u, i1 - 1) * mp.Hq + h) * D + e;
        if constexpr (sizeof(T) == 2) w[u] = bf16_bits_to_f32(q[off]);
        else w[u] = q[off];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += i + u < i1 ? (double)w[u] : 0.0;
    }
    qbar[hh][e] = acc / (double)(i1 - i0);
  }
  __syncthreads();

  // block scores: 16 lanes per block, lane `sub` takes dims 64*i + 4*sub + 0..3.
  // A round covers kRounds steps of 4 blocks per wave: the block-table
  // entries of the round are loaded together, then all its mean rows, then
  // the scores are computed (two memory round trips per round instead of
  // two per step); loads past the causal blocks re-read the last one.
  const int sub = lane & 15, slot = lane >> 4;
  const double sc = (double)mp.sm_scale;
  constexpr int kRounds = 8;
  constexpr int kStep = 4 * (kSelThreads / 64);             // blocks per step over the workgroup
  for (int kb0 = 0; kb0 < n; kb0 += kRounds * kStep) {
    int phys[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) phys[r] = mp.bt_row[min(kb0 + r * kStep + wave * 4 + slot, n - 1)];
    f32x4 v[kRounds][PL / 4];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const float* m = mp.mu + ((size_t)phys[r] * mp.Hkv + g) * D + 4 * sub;
#pragma unroll
      for (int i = 0; i < PL / 4; ++i) v[r][i] = *reinterpret_cast<const f32x4*>(m + 64 * i);
    }
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int kb = kb0 + r * kStep + wave * 4 + slot;
      for (int hh = 0; hh < G; ++hh) {
        const double* qq = &qbar[hh][4 * sub];
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < PL / 4; ++i) {
          acc += qq[64 * i] * (double)v[r][i][0];
          acc += qq[64 * i + 1] * (double)v[r][i][1];
          acc += qq[64 * i + 2] * (double)v[r][i][2];
          acc += qq[64 * i + 3] * (double)v[r][i][3];
        }
        acc = row16_sum(acc);
        if (sub == 0 && kb < n) scores[(size_t)hh * nkb + kb] = (float)(sc * acc);
      }
    }
  }
  __syncthreads();

  SelectParams p{};
  p.n_sel = G;
  p.list_stride = nkb;
  p.counts = s_count;
  p.ccounts = nullptr;
  p.tiered = 0;
  for (int hh = 0; hh < G; ++hh) {
    const float* row = scores + (size_t)hh * nkb;
    // largest score over the causal blocks (threshold mode)
    float mx = -INFINITY;
    for (int kb = threadIdx.x; kb < n; kb += kSelThreads) mx = fmaxf(mx, row[kb]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    for (int i = threadIdx.x; i < 512; i += kSelThreads) sh.hist[0][0][i] = 0u;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < kSelThreads / 64; ++w) mx = fmaxf(mx, red[w]);
    const float thr = mx - mp.max_gap;
    // keys: 0 for the sink and diagonal blocks, the order-preserving image of
    // the score otherwise; in threshold mode count the candidates at or above it
    uint32_t above = 0;
    for (int kb = threadIdx.x; kb < n; kb += kSelThreads) {
      const bool forced = kb == 0 || kb >= kb_lo;
      keys[kb] = forced ? 0u : score_key(row[kb]);
      above += (!forced && row[kb] >= thr) ? 1u : 0u;
    }
    uint32_t total = 0;
    block_excl_scan(above, &total, sh.wsum[0]);
    ListShape L;
    L.n = n;
    L.sink_hi = min(1, n);
    L.win_lo = kb_lo;
    L.n_forced = L.sink_hi + max(0, n - max(L.win_lo, L.sink_hi));
    const int k = mp.top_k >= 0 ? mp.top_k : (int)total;
    L.k_eff = max(0, min(k, n - L.n_forced));
    L.k1 = L.k_eff;
    __syncthreads();
    if (n > 0) select_from_keys(p, L, 0, hh, keys, sh, list);   // counts land in s_count[hh]
    __syncthreads();
    // the mask row: zero, then the listed blocks
    uint8_t* mrow = mp.mask + ((size_t)(g * G + hh) * mp.nqb + qb) * nkb;
    for (int kb = threadIdx.x; kb < nkb; kb += kSelThreads) mrow[kb] = 0;
    __syncthreads();
    const int cnt = n > 0 ? s_count[hh] : 0;
    for (int j = threadIdx.x; j < cnt; j += kSelThreads) mrow[list[j]] = 1;
    __syncthreads();
  }
}

size_t block_mask_lds_bytes(int G, int nkb) { return ((size_t)G * nkb + 2 * (size_t)nkb) * sizeof(uint32_t); }

hipError_t launch_block_mask(const MaskParams& mp, int bf16, int d, hipStream_t s) {
  const dim3 grid(mp.nqb, mp.Hkv), block(kSelThreads);
  const size_t lds = block_mask_lds_bytes(mp.G, mp.nkb);
  if (bf16) {
    if (d == 64) hipLaunchKernelGGL((block_mask_kernel<uint16_t, 64>), grid, block, lds, s, mp);
    else hipLaunchKernelGGL((block_mask_kernel<uint16_t, 128>), grid, block, lds, s, mp);
  } else {
    if (d == 64) hipLaunchKernelGGL((block_mask_kernel<float, 64>), grid, block, lds, s, mp);
    else hipLaunchKernelGGL((block_mask_kernel<float, 128>), grid, block, lds, s, mp);
  }
  return hipGetLastError();
}

}  // namespace sa
