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

// Sum of a double over the 16 lanes of each DPP row, rotating the row by 8,
// 4, 2 and 1 lanes (no LDS round trip).  The first lane of the row adds the
// same values in the same order as an xor butterfly over 8, 4, 2, 1 (for every
// lane it depends on, rotating by k reaches lane ^ k), so its result has the
// same bits; the other lanes hold the sum in another order.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long v = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)v, CTRL, 0xf, 0xf, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(v >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double row16_sum(double x) {
  x += dpp_f64<0x128>(x);   // row_ror:8
  x += dpp_f64<0x124>(x);   // row_ror:4
  x += dpp_f64<0x122>(x);   // row_ror:2
  x += dpp_f64<0x121>(x);   // row_ror:1
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
__device__ __forceinline__ uint32_t find_digit(const uint32_t* h, uint32_t* kk, uint32_t* in_bin) {
  const int lane = threadIdx.x & 63;
  const u32x4 w = *reinterpret_cast<const u32x4*>(h + 252 - 4 * lane);
  const uint32_t c[4] = {w[3], w[2], w[1], w[0]};
  const uint32_t mine = (c[0] + c[1]) + (c[2] + c[3]);
  const uint32_t incl = wave_incl_scan(mine);
  const uint32_t above = incl - mine;            // keys in higher lanes' bins
  const uint32_t k = *kk;
  const bool here = incl >= k && above < k;      // exactly one lane
  uint32_t bin = 0, rest = 0, cnt = 0, acc = above;
  bool found = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool hit = !found && acc + c[j] >= k;
    if (hit) {
      bin = 255u - 4u * lane - j;
      rest = k - acc;
      cnt = c[j];
    }
    found |= hit;
    acc += c[j];
  }
  const int src = __builtin_ctzll(__ballot(here));
  *kk = (uint32_t)__builtin_amdgcn_readlane((int)rest, src);
  *in_bin = (uint32_t)__builtin_amdgcn_readlane((int)cnt, src);
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
    uint32_t cntA = 0, cntB = 0;
    preA |= find_digit(hA, &kkA, &cntA) << shift;
    if (two) preB |= find_digit(hB, &kkB, &cntB) << shift;
    pmask |= 255u << shift;
    // Every key of the chosen bin is needed (and the bin's lowest key is not
    // 0): the top k are exactly the keys >= that lowest key, so the
    // threshold is the key just below it, with no ties taken; the remaining
    // passes are skipped.  (Uniform: the counts come from one lane.)
    const bool doneA = kkA == cntA && preA != 0u;
    const bool doneB = !two || (kkB == cntB && preB != 0u);
    if (shift > 0 && doneA && doneB) {
      *TA = preA - 1u;
      *needA = 0u;
      *TB = two ? preB - 1u : preB;
      *needB = two ? 0u : kkB;
      return;
    }
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

  const int countA = n_forced + k1;
  // (positions stay below n_forced + k_eff <= list_stride; the bound only
  // keeps the stores inside the row should that ever fail)
  const uint32_t stride = (uint32_t)p.list_stride;
  uint32_t tot;
  // Ranges of 4 to 16 keys made of whole 16-byte groups (e.g. 8,192 pages on
  // 512 threads): each thread reads its keys once, 16 bytes at a time, and
  // keeps them and their flags in registers.  (Threads' ranges sit 64 bytes
  // apart, so single-word reads of them conflict 16-way in the LDS banks,
  // 16-byte reads 4-way.)  Same ranks, flags and order as the loops below.
  if ((m & 3) == 0 && m <= 16 && (n & 3) == 0 && (reinterpret_cast<uintptr_t>(keys) & 15u) == 0) {
    const int cnt = hi - lo;
    uint32_t kr[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (4 * q < cnt) w = *reinterpret_cast<const u32x4*>(keys + lo + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) kr[4 * q + e] = w[e];
    }
    uint32_t t1 = 0, t2 = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t key = j < cnt ? kr[j] : 0u;
      t1 += (key != 0u && key == T1) ? 1u : 0u;
      t2 += (key != 0u && key == T2) ? 1u : 0u;
    }
    const uint32_t ex = block_excl_scan(t1 | (t2 << 16), &tot, sh.wsum[0]);
    uint32_t rank1 = ex & 0xffffu, rank2 = ex >> 16;
    uint32_t ca = 0, cb = 0, fl = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t key = j < cnt ? kr[j] : 0u;
      const bool e1 = key != 0u && key == T1, e2 = key != 0u && key == T2;
      const bool top1 = key != 0u && (key > T1 || (e1 && rank1 < r1));
      const bool top2 = key != 0u && (key > T2 || (e2 && rank2 < r2));
      rank1 += e1 ? 1u : 0u;
      rank2 += e2 ? 1u : 0u;
      const int i = lo + j;
      const bool forced = j < cnt && (i < sink_hi || i >= win_lo);
      const bool fa = p.tiered ? (forced || top1) : (forced || top2);
      const bool fb = p.tiered && top2 && !top1;
      ca += fa ? 1u : 0u;
      cb += fb ? 1u : 0u;
      fl |= ((fa ? 1u : 0u) | (fb ? 2u : 0u)) << (2 * j);
    }
    const uint32_t ex2 = block_excl_scan(ca | (cb << 16), &tot, sh.wsum[1]);
    uint32_t posA = ex2 & 0xffffu, posB = countA + (ex2 >> 16);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t f = (fl >> (2 * j)) & 3u;
      if ((f & 1u) && posA < stride) out[posA] = lo + j;
      if ((f & 2u) && posB < stride) out[posB] = lo + j;
      posA += f & 1u;
      posB += (f >> 1) & 1u;
    }
  } else {
    // ties at the thresholds before this thread's range (counts < 2^16: n <= 16384)
    uint32_t t1 = 0, t2 = 0;
    for (int i = lo; i < hi; ++i) {
      const uint32_t key = keys[i];
      t1 += (key != 0u && key == T1) ? 1u : 0u;
      t2 += (key != 0u && key == T2) ? 1u : 0u;
    }
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
    uint32_t posA = ex2 & 0xffffu, posB = countA + (ex2 >> 16);
    for (int i = lo; i < hi; ++i) {
      const uint32_t f = keys[i];
      if ((f & 1u) && posA < stride) out[posA] = i;
      if ((f & 2u) && posB < stride) out[posB] = i;
      posA += f & 1u;
      posB += (f >> 1) & 1u;
    }
  }
  if (threadIdx.x == 0) {
    p.counts[sel] = n_forced + k_eff;
    if (p.tiered && p.ccounts) p.ccounts[sel] = countA;
  }
}

// Router scores of list (b, s) into order-preserving keys in LDS, by one
// workgroup of kSelThreads threads (the selection follows after a barrier;
// the zeroing of sh.hist[0] it needs is done here).  The pooled query sits in
// LDS.  Each wave scores 4 pages per step with 16 lanes per page; at d <= 128
// a round is 16 steps, so the 8 waves cover 512 pages per round.
// The score arithmetic is the same as score_lastsel_kernel's: lane `sub` of a
// page's 16 takes dims 64 i + 4 sub + 0..3 (each load instruction reads 256
// contiguous bytes of the mean row), float64 products of the pooled query
// with the fp32 mean row summed in that order, then over the 16 lanes in a
// fixed butterfly (row16_sum), rounded once to fp32.
// Memory round trips: the block-table entries of the first round, the
// newest page's keys and the query rows are loaded together; the first
// round's mean rows are issued as soon as the block-table entries arrive,
// while the pooled query and the refreshed mean are summed.  Every load is
// unconditional, from a clamped valid index: rows past the query rows and
// tokens past the newest page's valid ones add +0.0 (exact: the float64 sums
// start at +0.0 and never become -0.0), and a lane whose page is forced, past
// the sequence or refreshed re-reads the mean row of the nearest page the list
// does score, and does not use it.  Forced pages' rows are thus read only
// when the scores are written out, or when the list scores no page at all
// (page 0's row is then read and ignored).  (A load under a per-lane
// condition makes the compiler wait for it at once, and a wait after a branch
// waits for every load of either path.)
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
  constexpr int kWaves = kSelThreads / 64;
  constexpr int kSteps = D <= 128 ? 16 : 2;           // 4-page steps whose loads are in flight together
  constexpr int kRound = 4 * kSteps * kWaves;         // pages per round
  constexpr int kQPer = (D + kSelThreads - 1) / kSelThreads;   // pooled-query dims per thread
  constexpr int kQRows = 8;                            // query rows loaded together
  __shared__ double qbar[D];
  __shared__ float fresh[D];
  const int n = L.n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, slot = lane >> 4;
  float* sout = sp.scores ? sp.scores + ((size_t)b * sp.n_sel + s) * sp.max_pages : nullptr;
  for (int i = threadIdx.x; i < 512; i += kSelThreads) sh.hist[0][0][i] = 0u;
  if (sout)
    for (int lp = n + threadIdx.x; lp < sp.max_pages; lp += kSelThreads) sout[lp] = __builtin_nanf("");
  if (n == 0) return;                                   // nothing to score (uniform)
  const int g = sp.per_q ? s / sp.G : s;
  const int32_t* bt = sp.block_table + (size_t)b * sp.max_pages;
  const float* mu_g = sp.mu + (size_t)g * D + 4 * sub;
  const size_t mu_page = (size_t)sp.Hkv * D;
  // this lane's page in a round: round base + 4 kSteps wave + lane (lanes
  // past 4 kSteps carry no page)
  const int lane_pg = 4 * kSteps * wave + min(lane, 4 * kSteps - 1);
  const bool refresh = sp.refresh != 0;
  // the pages whose mean rows this list uses: all with the scores written
  // out, else those not forced; the refreshed newest page's row comes from LDS
  const int rd_lo = sout ? 0 : L.sink_hi;
  const int rd_hi = min(sout ? n : L.win_lo, refresh ? n - 1 : n);
  auto row_page = [&](int lp) __attribute__((always_inline)) {
    return rd_lo < rd_hi ? min(max(lp, rd_lo), rd_hi - 1) : 0;
  };

  // (1) block-table entries of the first round
  const int phys0 = bt[row_page(lane_pg)];

  // (2) the newest page's keys (refresh) and the query rows
  // With refresh, the newest page's mean row (KV head g) is recomputed here,
  // summed in the same order as page_summary_kernel (same bits), written by
  // one list per head, and used for this list's score of that page from LDS.
  const int last_phys = bt[n - 1];
  const int last_nv = page_valid(sp.seq_lens[b], n - 1, sp.P);
  const int rcg = (threadIdx.x & 255) % CG, rts = min((threadIdx.x & 255) / CG, TS - 1);
  constexpr int kTokMax = 4;                            // tokens per thread per refresh chunk
  u32x4 rw[kTokMax];
  const T* rbase = reinterpret_cast<const T*>(sp.k_pool) + (((size_t)last_phys * sp.Hkv + g) * sp.P) * D + rcg * VW;
  if (refresh) {
#pragma unroll
    for (int j = 0; j < kTokMax; ++j)
      rw[j] = *reinterpret_cast<const u32x4*>(rbase + (size_t)min(rts + j * TS, last_nv - 1) * D);
  }
  const T* q = reinterpret_cast<const T*>(sp.q);
  const int rows = sp.per_q ? sp.T : sp.T * sp.G;
  auto q_index = [&](int r, int e) __attribute__((always_inline)) {
    int t, h;
    if (sp.per_q) { t = r; h = s; } else { t = r / sp.G; h = s * sp.G + r % sp.G; }
    return (((size_t)b * sp.T + t) * sp.Hq + h) * D + e;
  };
  float qv[kQPer][kQRows];
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int e = min((int)threadIdx.x + k * kSelThreads, D - 1);
#pragma unroll
    for (int r = 0; r < kQRows; ++r) {
      const size_t i = q_index(min(r, rows - 1), e);
      if constexpr (sizeof(T) == 2) qv[k][r] = bf16_bits_to_f32(q[i]);
      else qv[k][r] = q[i];
    }
  }

  // (3) mean rows of the first round
  f32x4 v[kSteps][PL / 4];
  auto load_round = [&](int phys) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int ph = __shfl(phys, it * 4 + slot, 64);
      const float* m = mu_g + (size_t)ph * mu_page;
#pragma unroll
      for (int i = 0; i < PL / 4; ++i) v[it][i] = *reinterpret_cast<const f32x4*>(m + 64 * i);
    }
  };
  load_round(phys0);

  // pooled query (rows in order; rows past `rows` add +0.0) and refresh partials
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int e = threadIdx.x + k * kSelThreads;
    double acc = 0.0;
#pragma unroll
    for (int r = 0; r < kQRows; ++r) acc += r < rows ? (double)qv[k][r] : 0.0;
    for (int r0 = kQRows; r0 < rows; r0 += kQRows) {     // more rows than one batch
      float w[kQRows];
#pragma unroll
      for (int r = 0; r < kQRows; ++r) {
        const size_t i = q_index(min(r0 + r, rows - 1), min(e, D - 1));
        if constexpr (sizeof(T) == 2) w[r] = bf16_bits_to_f32(q[i]);
        else w[r] = q[i];
      }
#pragma unroll
      for (int r = 0; r < kQRows; ++r) acc += r0 + r < rows ? (double)w[r] : 0.0;
    }
    if (e < D) qbar[e] = acc;
  }
  if (refresh) {
    double acc[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) acc[i] = 0.0;
    for (int j0 = 0; j0 * TS < last_nv; j0 += kTokMax) {
      if (j0 > 0) {                                     // pages of more than kTokMax * TS tokens
#pragma unroll
        for (int j = 0; j < kTokMax; ++j)
          rw[j] = *reinterpret_cast<const u32x4*>(rbase + (size_t)min(rts + (j0 + j) * TS, last_nv - 1) * D);
      }
#pragma unroll
      for (int j = 0; j < kTokMax; ++j) {
        const bool ok = rts + (j0 + j) * TS < last_nv;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += ok ? (double)bf16_lo(rw[j][i]) : 0.0;
            acc[2 * i + 1] += ok ? (double)bf16_hi(rw[j][i]) : 0.0;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += ok ? (double)__uint_as_float(rw[j][i]) : 0.0;
        }
      }
    }
    if (threadIdx.x < CG * TS)
#pragma unroll
      for (int i = 0; i < VW; ++i) rpart[rts * D + rcg * VW + i] = acc[i];
  }
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

  // (4) scores of each round; the next round's block-table entries and mean
  // rows are loaded after this round's scores
  for (int base = 0; base < n; base += kRound) {
    if (base > 0) load_round(bt[row_page(base + lane_pg)]);
    const int r0 = base + 4 * kSteps * wave;
#pragma unroll
    for (int it = 0; it < kSteps; ++it) {
      const int lp = r0 + it * 4 + slot;
      if (refresh && lp == n - 1) {                     // the refreshed row comes from LDS
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
      acc = row16_sum(acc);
      if (sub == 0 && lp < n) {
        const float sc = (float)acc;
        const bool forced = lp < L.sink_hi || lp >= L.win_lo;
        keys[lp] = forced ? 0u : score_key(sc);
        if (sout) sout[lp] = sc;
      }
    }
  }
}

}  // namespace sa
