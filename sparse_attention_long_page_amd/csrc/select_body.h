// Page selection device code shared by the selection kernels and the fused
// selection + decode kernel; the method and design are described in
// select.hip.
#pragma once
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

// LDS working set of one selection: three pairs of 256-bin histograms used
// round robin by consecutive radix passes (one barrier per pass; a pair
// serves the two thresholds of a tiered list), and one per-wave partial-sum
// array for each of the two workgroup scans.
struct alignas(16) SelShared {
  uint32_t hist[3][2][256];
  uint32_t wsum[2][kSelThreads / 64];
};

// Inclusive prefix sum over the 64 lanes of a wave from DPP lane moves:
// row shifts by 1, 2, 4, 8 (zero past the row start) sum each 16-lane row,
// then the last lane of row 0 is added into row 1 and of row 2 into row 3
// (row_bcast:15), and the last lane of row 1 into rows 2 and 3
// (row_bcast:31).  No LDS round trip.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);    // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);    // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);    // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);    // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Exclusive prefix sum over the workgroup in thread order.  `wsum` serves this
// one call only, so a single barrier suffices.  *total gets the sum over all
// threads.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const uint32_t t = wsum[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + x - v;
}

// One radix digit of a k-th-largest search, found by every wave from the
// 256-bin histogram h of the keys that match the search's prefix: the bin
// holding the kk-th largest of them (returned), and in *kk its rank within
// that bin.  Lane l holds bins 255 - 4l - j, j = 0..3 (higher bins hold
// larger keys), so a prefix sum over the lanes counts the keys in this lane's
// bins and all higher ones.
__device__ __forceinline__ uint32_t find_digit(const uint32_t* h, uint32_t* kk) {
  const int lane = threadIdx.x & 63;
  const u32x4 w = *reinterpret_cast<const u32x4*>(h + 252 - 4 * lane);
  const uint32_t c[4] = {w[3], w[2], w[1], w[0]};
  const uint32_t mine = (c[0] + c[1]) + (c[2] + c[3]);
  const uint32_t incl = wave_incl_scan(mine);
  const uint32_t above = incl - mine;            // keys in higher lanes' bins
  const uint32_t k = *kk;
  const bool here = incl >= k && above < k;      // exactly one lane
  uint32_t bin = 0, rest = 0, acc = above;
  bool found = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool hit = !found && acc + c[j] >= k;
    if (hit) {
      bin = 255u - 4u * lane - j;
      rest = k - acc;
    }
    found |= hit;
    acc += c[j];
  }
  const int src = __builtin_ctzll(__ballot(here));
  *kk = (uint32_t)__builtin_amdgcn_readlane((int)rest, src);
  return (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
}

// Thresholds of the kA-th and (when kB > 0) the kB-th largest of the nonzero
// keys[0..n) (1 <= kA, kB <= their number), both in the same four MSB-first
// passes of 8 bits.  Each returns the key T and, in need, how many keys equal
// to T belong to the top k.  Pass p counts into hist[p % 3] (zeroed
// beforehand, with a barrier since) and zeroes hist[(p + 1) % 3], which no
// wave reads any more: its last readers finished before the previous pass's
// barrier.  In pass 0 both searches share one histogram.
__device__ inline void radix_select2(const uint32_t* keys, int n, uint32_t kA, uint32_t kB, uint32_t* TA, uint32_t* needA,
                              uint32_t* TB, uint32_t* needB, SelShared& sh) {
  uint32_t preA = 0, preB = 0, pmask = 0, kkA = kA, kkB = kB;
  const bool two = kB > 0;
  int pass = 0;
  for (int shift = 24; shift >= 0; shift -= 8, ++pass) {
    uint32_t* hA = sh.hist[pass % 3][0];
    uint32_t* hB = pass == 0 ? hA : sh.hist[pass % 3][1];
    uint32_t* hn = sh.hist[(pass + 1) % 3][0];
    for (int i = threadIdx.x; i < 512; i += kSelThreads) hn[i] = 0u;   // both bins of the pair
    const bool countB = two && pass > 0;
    auto count = [&](uint32_t key) {
      if (key == 0u) return;
      const uint32_t bin = (key >> shift) & 255u;
      if ((key & pmask) == preA) atomicAdd(&hA[bin], 1u);
      if (countB && (key & pmask) == preB) atomicAdd(&hB[bin], 1u);
    };
    // long lists: 8 keys read before their atomics; then the rest one by one
    const int n8 = n - n % (8 * kSelThreads);
    for (int i0 = threadIdx.x; i0 < n8; i0 += 8 * kSelThreads) {
      uint32_t kv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) kv[j] = keys[i0 + j * kSelThreads];
#pragma unroll
      for (int j = 0; j < 8; ++j) count(kv[j]);
    }
    for (int i = n8 + threadIdx.x; i < n; i += kSelThreads) count(keys[i]);
    __syncthreads();
    preA |= find_digit(hA, &kkA) << shift;
    if (two) preB |= find_digit(hB, &kkB) << shift;
    pmask |= 255u << shift;
  }
  *TA = preA;
  *needA = kkA;
  *TB = preB;
  *needB = kkB;
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
// the list of (b, s) into the row `out` (global memory or LDS), its counts to
// p.counts / p.ccounts.  Called by the whole workgroup after a barrier that
// follows the keys' writes and the zeroing of the pair sh.hist[0].  Each thread owns
// the consecutive keys [lo, hi), so ranking the threshold ties by index and
// compacting the chosen pages in ascending order take one workgroup scan each.
__device__ inline void select_from_keys(const SelectParams& p, const ListShape& L, int b, int s, uint32_t* keys,
                                        SelShared& sh, int32_t* out) {
  const int sel = b * p.n_sel + s;
  const int n = L.n, sink_hi = L.sink_hi, win_lo = L.win_lo, n_forced = L.n_forced, k_eff = L.k_eff, k1 = L.k1;
  uint32_t T1 = 0xffffffffu, r1 = 0, T2 = 0xffffffffu, r2 = 0;
  if (k_eff > 0) {
    const uint32_t kB = (p.tiered && k1 > 0) ? (uint32_t)k1 : 0u;
    uint32_t TB = 0xffffffffu, rB = 0;
    radix_select2(keys, n, (uint32_t)k_eff, kB, &T2, &r2, &TB, &rB, sh);
    if (kB > 0) { T1 = TB; r1 = rB; }
  }
  if (!p.tiered) { T1 = T2; r1 = r2; }

  const int m = (n + kSelThreads - 1) / kSelThreads;
  const int lo = min(n, (int)threadIdx.x * m), hi = min(n, lo + m);

  // ties at the thresholds before this thread's range (counts < 2^16: n <= 16384)
  uint32_t t1 = 0, t2 = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    t1 += (key != 0u && key == T1) ? 1u : 0u;
    t2 += (key != 0u && key == T2) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan(t1 | (t2 << 16), &tot, sh.wsum[0]);

  // flags: bit0 forced, bit1 in top-k1 (Critical), bit2 in top-k_eff; count
  // this thread's entries of segment A (forced + Critical, or the whole
  // untiered list) and segment B (Ambient)
  uint32_t rank1 = ex & 0xffffu, rank2 = ex >> 16;
  uint32_t ca = 0, cb = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    const bool e1 = key != 0u && key == T1, e2 = key != 0u && key == T2;
    const bool top1 = key != 0u && (key > T1 || (e1 && rank1 < r1));
    const bool top2 = key != 0u && (key > T2 || (e2 && rank2 < r2));
    rank1 += e1 ? 1u : 0u;
    rank2 += e2 ? 1u : 0u;
    const bool forced = i < sink_hi || i >= win_lo;
    const bool a = p.tiered ? (forced || top1) : (forced || top2);
    const bool bb = p.tiered && top2 && !top1;
    ca += a ? 1u : 0u;
    cb += bb ? 1u : 0u;
    keys[i] = (a ? 1u : 0u) | (bb ? 2u : 0u);
  }
  const uint32_t ex2 = block_excl_scan(ca | (cb << 16), &tot, sh.wsum[1]);

  // ascending compaction of this thread's range
  const int countA = n_forced + k1;
  // (positions stay below n_forced + k_eff <= list_stride; the bound only
  // keeps the stores inside the row should that ever fail)
  const uint32_t stride = (uint32_t)p.list_stride;
  uint32_t posA = ex2 & 0xffffu, posB = countA + (ex2 >> 16);
  for (int i = lo; i < hi; ++i) {
    const uint32_t f = keys[i];
    if ((f & 1u) && posA < stride) out[posA] = i;
    if ((f & 2u) && posB < stride) out[posB] = i;
    posA += f & 1u;
    posB += (f >> 1) & 1u;
  }
  if (threadIdx.x == 0) {
    p.counts[sel] = n_forced + k_eff;
    if (p.tiered && p.ccounts) p.ccounts[sel] = countA;
  }
}

// Router scores of list (b, s) into order-preserving keys in LDS, by one
// workgroup of kSelThreads threads (the selection follows after a barrier;
// the zeroing of sh.hist[0] it needs is done here).  The pooled query sits in LDS; each wave
// scores 32 pages per round at d <= 128 (16 lanes per page, 4 pages per step,
// the 8 steps' mean-row loads in flight together), writing order-preserving
// keys into LDS.
// The score arithmetic is the same as page_score_kernel's: lane `sub` of a
// page's 16 takes dims 64 i + 4 sub + 0..3 (each load instruction reads 256
// contiguous bytes of the mean row), float64 products of the pooled query
// with the fp32 mean row summed in that order, then over the 16 lanes in a
// fixed butterfly, rounded once to fp32.
// newest-page summary refresh: the thread partition of page_summary_kernel
// (thread (cg, ts): 16-byte column group cg, tokens ts, ts + TS, ...); the
// refresh needs TS * D doubles of LDS
template <typename T, int D>
constexpr int refresh_ts() {
  return (256 / (D / (16 / (int)sizeof(T))) < 16) ? 256 / (D / (16 / (int)sizeof(T))) : 16;
}

template <typename T, int D>
__device__ __forceinline__ void score_keys_body(const ScoreParams& sp, const SelectParams& p, const ListShape& L,
                                                int b, int s, uint32_t* keys, SelShared& sh, double* rpart) {
  constexpr int PL = D / 16;
  constexpr int VW = 16 / sizeof(T), CG = D / VW, TS = refresh_ts<T, D>();
  __shared__ double qbar[D];
  __shared__ float fresh[D];
  const int n = L.n;
  const int g = sp.per_q ? s / sp.G : s;
  const int32_t* bt = sp.block_table + (size_t)b * sp.max_pages;
  // With refresh, the newest page's mean row (KV head g) is recomputed here,
  // summed in the same order as page_summary_kernel (same bits), written by
  // one list per head, and used for this list's score of that page from LDS.
  const bool refresh = sp.refresh && n > 0;
  const int last_phys = refresh ? bt[n - 1] : 0;
  const int last_nv = refresh ? page_valid(sp.seq_lens[b], n - 1, sp.P) : 0;
  if (refresh && threadIdx.x < CG * TS) {
    const int cg = threadIdx.x % CG, ts = threadIdx.x / CG;
    const T* base = reinterpret_cast<const T*>(sp.k_pool) + (((size_t)last_phys * sp.Hkv + g) * sp.P) * D + cg * VW;
    double acc[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) acc[i] = 0.0;
#pragma unroll 4
    for (int j = ts; j < last_nv; j += TS) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + (size_t)j * D);
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
    for (int i = 0; i < VW; ++i) rpart[ts * D + cg * VW + i] = acc[i];
  }
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
  for (int i = threadIdx.x; i < 512; i += kSelThreads) sh.hist[0][0][i] = 0u;
  __syncthreads();
  if (refresh) {
    const bool writer = !sp.per_q || s % sp.G == 0;
    float* mrow = sp.mu_out + ((size_t)last_phys * sp.Hkv + g) * D;
    for (int e = threadIdx.x; e < D; e += kSelThreads) {
      double sum = 0.0;
      for (int ts = 0; ts < TS; ++ts) sum += rpart[ts * D + e];
      const float m = (float)(sum / (double)last_nv);
      fresh[e] = m;
      if (writer) mrow[e] = m;
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, slot = lane >> 4;
  float* sout = sp.scores ? sp.scores + ((size_t)b * sp.n_sel + s) * sp.max_pages : nullptr;
  constexpr int kWaves = kSelThreads / 64;
  constexpr int kSteps = D <= 128 ? 8 : 2;           // 4-page steps whose loads are in flight together
  for (int r0 = 4 * kSteps * wave; r0 < n; r0 += 4 * kSteps * kWaves) {
    // forced pages' scores are not needed unless the caller asked for the
    // scores: their mean rows are then not read at all (the newest page's row
    // may be rewritten concurrently by a summary update on another stream)
    const int lp_l = r0 + lane;
    const bool need = lane < 4 * kSteps && lp_l < n && (sout || !(lp_l < L.sink_hi || lp_l >= L.win_lo)) &&
                      !(refresh && lp_l == n - 1);    // the refreshed row comes from LDS
    const int my_phys = need ? bt[lp_l] : -1;
    f32x4 v[kSteps][PL / 4];
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int ph = __shfl(my_phys, it * 4 + slot, 64);
      const float* m = sp.mu + ((size_t)max(ph, 0) * sp.Hkv + g) * D + 4 * sub;
#pragma unroll
      for (int i = 0; i < PL / 4; ++i) v[it][i] = ph >= 0 ? *reinterpret_cast<const f32x4*>(m + 64 * i) : f32x4{};
    }
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int lp = r0 + it * 4 + slot;
      if (refresh && lp == n - 1) {
#pragma unroll
        for (int i = 0; i < PL / 4; ++i) {
          const float* f = fresh + 64 * i + 4 * sub;
          v[it][i] = f32x4{f[0], f[1], f[2], f[3]};
        }
      }
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
}

}  // namespace sa
