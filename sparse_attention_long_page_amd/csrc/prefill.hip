// Chunked block-sparse prefill: 2D block mask -> GQA-union KV block tables,
// then causal attention in place over the paged KV (CompactAttention abstract,
// on the page titled "Causal Attention on CPU: A Cache-Aware and Load-Balanced
// Scheduling Kernel for Prefill": Q-block union then intra-group union, KV
// blocks read in place with no compaction; "Universal Attention Engine",
// "Key Design Decisions" 3: prefill is compute-bound, optimise FLOPs).
//
// Union kernel: one workgroup per KV head; each thread ORs four KV-block
// columns over the group's heads and Q-blocks (4-byte loads, many in flight),
// then an index-ordered workgroup prefix sum writes the ascending table.
//
// Attention kernel (bf16, d 128, pages of 64):
//  * workgroup = (KV head g, tile of 64 query positions); two waves per query
//    head of the group (32 query rows each), so every K/V tile staged in LDS
//    serves all G heads (GQA packing: 64*G rows per tile);
//  * workgroup ids are remapped so the tiles of one KV head run on one XCD
//    and share its L2 while they sweep the same KV blocks;
//  * per KV block: K (token-major) and V^T (page-transposed) are copied from
//    the pool into padded LDS rows (conflict-free 16-byte reads) by
//    buffer-to-LDS copies, three stages: the copy of block t+2 is issued at
//    the end of block t, and only by the first four waves (one per SIMD);
//    those win the SIMD's issue arbitration over the other wave, finish
//    their block first and would wait at the block's barrier, so their copy
//    issue (which stalls a wave while the memory pipeline drains the
//    burst) overlaps that wait instead of delaying the other waves' MFMAs;
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 (Q^T resident
//    in registers), with the token permutation that makes the S^T fragments
//    the PV operand directly; the row sums of P are one more MFMA per PV
//    step with an all-ones operand (the sums of the bf16 weights the PV
//    product uses);
//  * causal and sequence-end masks only on blocks that cross a row's
//    position; the ascending table stops the sweep past the tile's last row;
//  * online softmax in base 2 with a lazily moved reference maximum: the
//    accumulators are rescaled only when a row's maximum grows by more than
//    2^8 (exact: the final normalisation uses the same reference).
#include <type_traits>

#include "common.h"

namespace sa {

// ------------------------------------------------------------------- union
constexpr int kUnionThreads = 1024;

// One workgroup per KV head.  Thread t owns KV-block columns 4t .. 4t+3 of a
// 4096-column pass and ORs them over the group's heads and Q-blocks with
// 4-byte loads (16 loads in flight per step); an index-ordered workgroup
// prefix sum over the per-thread counts writes the ascending table.
template <bool VEC4>
__global__ __launch_bounds__(kUnionThreads) void union_kernel(UnionParams p) {
  __shared__ uint32_t wsum[kUnionThreads / 64];
  const int g = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrows = p.G * p.nqb;                       // (head, Q-block) rows of this group
  const uint8_t* mbase = p.mask + (size_t)g * p.G * p.nqb * p.nkb;
  uint32_t run = 0;
  int32_t* out = p.table + (size_t)g * p.nkb;
  for (int base = 0; base < p.nkb; base += 4 * kUnionThreads) {
    const int kb0 = base + 4 * threadIdx.x;
    uint32_t any = 0;                                   // byte j nonzero <=> column kb0 + j kept
    if (kb0 < p.nkb) {
      if (VEC4) {
        int r = 0;
        for (; r + 16 <= nrows; r += 16) {
          uint32_t w[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) w[j] = *reinterpret_cast<const uint32_t*>(mbase + (size_t)(r + j) * p.nkb + kb0);
#pragma unroll
          for (int j = 0; j < 16; ++j) any |= w[j];
        }
        for (; r < nrows; ++r) any |= *reinterpret_cast<const uint32_t*>(mbase + (size_t)r * p.nkb + kb0);
      } else {
        for (int r = 0; r < nrows; ++r)
          for (int j = 0; j < 4; ++j)
            if (kb0 + j < p.nkb && mbase[(size_t)r * p.nkb + kb0 + j]) any |= 1u << (8 * j);
      }
    }
    uint32_t flags = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (kb0 + j < p.nkb && ((any >> (8 * j)) & 0xffu)) flags |= 1u << j;
    const uint32_t f = __popc(flags);
    // exclusive prefix over the workgroup in thread (= column) order
    uint32_t x = f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < kUnionThreads / 64; ++w) {
      const uint32_t t = wsum[w];
      if (w < wave) before += t;
      all += t;
    }
    __syncthreads();
    uint32_t pos = run + before + x - f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((flags >> j) & 1u) out[pos++] = kb0 + j;
    run += all;
  }
  if (threadIdx.x == 0) p.counts[g] = (int32_t)run;
}

hipError_t launch_union(const UnionParams& p, hipStream_t s) {
  if (p.nkb % 4 == 0 && reinterpret_cast<uintptr_t>(p.mask) % 4 == 0)
    hipLaunchKernelGGL(union_kernel<true>, dim3(p.Hkv), dim3(kUnionThreads), 0, s, p);
  else
    hipLaunchKernelGGL(union_kernel<false>, dim3(p.Hkv), dim3(kUnionThreads), 0, s, p);
  return hipGetLastError();
}

// --------------------------------------------------------------- attention
constexpr int kPD = 128;          // head dim
constexpr int kPP = 64;           // page (KV block) size
constexpr int kBQ = 64;           // query positions per tile
constexpr int kRT = 2;            // 16-row MFMA tiles per wave: 32 query rows
constexpr int kKRow = kPD + 8;    // padded K row in LDS (bf16 elements): 272 B
constexpr int kVRow = kPP + 8;    // padded V^T row in LDS: 144 B
constexpr int kKTile = kPP * kKRow;
constexpr int kVTile = kPD * kVRow;
// One pipeline stage holds a block's K tile (64 rows of 16 data chunks + 1 pad
// chunk) followed by its V^T tile (128 rows of 8 data chunks + 1 pad chunk):
// 2240 16-byte chunks, filled by 35 wave-wide LDS-DMA loads.
constexpr int kKChunks = kPP * (kKRow / 8);      // 1088
constexpr int kVChunks = kPD * (kVRow / 8);      // 1152
constexpr int kStageInstr = (kKChunks + kVChunks) / 64;   // 35
constexpr int kStageElems = kKTile + kVTile;     // bf16 elements per stage (35840 B)
static_assert((kKChunks + kVChunks) % 64 == 0, "stage must be whole wave loads");
constexpr float kRescaleThreshold = 8.0f;   // log2 units

// LDS layout and operand orders, chosen for the LDS bank rules of gfx950
// (measured): a 16-byte read serves a 64-lane instruction in four cycles,
// lanes 0-31 in the first two and 32-63 in the last two, split within each
// half by the parity of lane bits 2..4; the 16 lanes of one cycle must fall
// in distinct 16-byte slots modulo 256 bytes.
//
// Token order: the 16x16 MFMA row m of token tile j4 is token ptok(j4, m).
// The S^T fragment a lane holds for PV step kp and lane group kg is then
// tokens 8*pchunk(kp, kg) .. +8, one 16-byte chunk of a V^T row.
__device__ __forceinline__ int pchunk(int kp, int kg) { return 2 * kp + (kg >> 1) + 4 * (kg & 1); }
__device__ __forceinline__ int ptok(int j4, int m) {
  return 8 * pchunk(j4 >> 1, m >> 2) + 4 * (j4 & 1) + (m & 3);
}
// K rows (272 bytes, 17 slots) hold their 16 dim-chunks in order; k-step kk
// of QK^T gives lane group kg dim-chunk kk + 4*kg (Q uses the same order).
// V^T rows (144 bytes, 9 slots) hold token-chunk q at slot q ^ vsw(d) for
// dim d.  With these, both the K and the V^T reads are free of conflicts.
__device__ __forceinline__ int vsw(int d) { return 4 * (((d >> 2) ^ (d >> 3)) & 1); }

// a value every lane of the wave holds, moved to a scalar register
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int V>
struct Stage {
  static constexpr int value = V;
};

// HW query heads per workgroup, two waves per head (query rows 0-31 and
// 32-63 of the tile).  A group larger than HW is split over G/HW workgroups.
template <int HW>
__global__ __launch_bounds__(128 * HW) void prefill_kernel(PrefillParams p) {
  // three pipeline stages as distinct LDS objects (so the wait-count pass
  // can tell a copy into one from reads of another): blocks t+1 and t+2 are
  // in flight while block t is computed
  __shared__ __attribute__((aligned(16))) uint16_t st0[kStageElems];
  __shared__ __attribute__((aligned(16))) uint16_t st1[kStageElems];
  __shared__ __attribute__((aligned(16))) uint16_t st2[kStageElems];
  __shared__ int kb_s[kPrefillMaxBlocks], ph_s[kPrefillMaxBlocks];
  constexpr int NW = 2 * HW;                                  // waves per workgroup
  constexpr int NCW = NW < 4 ? NW : 4;                        // waves that issue the copies
  constexpr int NI = (kStageInstr + NCW - 1) / NCW;           // copy loads per copying wave per block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kg = lane >> 4;

  const int nwg = gridDim.x, w = blockIdx.x;
  const int logical = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;
  const int hsplit = p.G / HW;                       // workgroups per (KV head, tile)
  const int g = logical / (p.n_qtiles * hsplit);
  const int rem = logical % (p.n_qtiles * hsplit);
  const int qt = rem / hsplit;
  const int h = g * p.G + (rem % hsplit) * HW + (wave >> 1);
  const int q0 = qt * kBQ;                           // tile's first query
  const int qw = q0 + 32 * (wave & 1);               // this wave's first query
  const int rows_valid = min(kBQ, p.q_len - q0);
  const int seq_len = *p.seq_len;
  const int pos_hi = p.q_start + q0 + rows_valid - 1;
  const int wpos_lo = p.q_start + qw;
  const int count = p.counts[g];
  const int32_t* table = p.table + (size_t)g * p.nkb;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(p.v_pool);
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);

  // Q^T operand: row-tile rt, k-step kk: query qw + 16*rt + col, dims 8*(kk + 4*kg) .. +8
  bf16x8 qreg[kRT][4];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int i = qw + 16 * rt + col;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qreg[rt][kk] = i < p.q_len
          ? *reinterpret_cast<const bf16x8*>(qp + ((size_t)i * p.Hq + h) * kPD + 8 * (kk + 4 * kg))
          : bf16x8{};
  }

  f32x4 oacc[8][kRT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) oacc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // row sums of P on MFMA: an all-ones A operand puts the column sums of
  // P^T (the sum over the row's tokens) in every element of lacc[rt]
  float m_ref[kRT];
  f32x4 lacc[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) { m_ref[rt] = -INFINITY; lacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // table entries at or before the tile's last position (the table ascends)
  int nblk = 0;
  {
    int lo = 0, hi = count;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (table[mid] * kPP > pos_hi) hi = mid; else lo = mid + 1;
    }
    nblk = lo;
  }

  // LDS-DMA copy of table entry t into a stage: wave-wide load i covers stage
  // chunks [64 i, 64 i + 64); loads 0-16 hold the K tile, 17-34 the V^T tile.
  // K slots copy straight; V^T slot c of row d receives token-chunk
  // c ^ vsw(d) (an involution); pad slots re-read chunk 0 of their row.  Each
  // copying wave issues NI loads (the last real load is repeated to fill).  Each
  // lane's byte offset within the (page, head) tile is fixed per load and
  // computed once; per block only the tile's base address (scalar) changes.
  static_assert(kKChunks % 64 == 0, "loads hold K or V^T chunks only");
  constexpr int kKInstr = kKChunks / 64;
  uint32_t lane_off[NI];     // bytes
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int i = min(wave + NCW * j, kStageInstr - 1);
    const int c = 64 * i + lane;
    if (c < kKChunks) {
      const int r = c / (kKRow / 8), slot = c % (kKRow / 8);
      lane_off[j] = 2 * (r * kPD + 8 * (slot < 16 ? slot : 0));
    } else {
      const int cv = c - kKChunks;
      const int r = cv / (kVRow / 8), slot = cv % (kVRow / 8);
      lane_off[j] = 2 * (r * kPP + 8 * (slot < 8 ? (slot ^ vsw(r)) : 0));
    }
  }
  // buffer-to-LDS copies: the tile bases live in scalar resources, the lane
  // offsets stay fixed, so a block's copy costs no vector instructions
  auto stage_copy = [&](uint16_t* st, int t) __attribute__((always_inline)) {
    const int phys = wave_uniform(ph_s[t]);
    const size_t tile = ((size_t)phys * p.Hkv + g) * kPP * kPD;     // same size for K and V^T tiles
    const auto rk = buffer_rsrc(kpool + tile, kPP * kPD * 2);
    const auto rv = buffer_rsrc(vpool + tile, kPP * kPD * 2);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = min(wave + NCW * j, kStageInstr - 1);
      copy16_to_lds(i < kKInstr ? rk : rv, st + i * 512, lane_off[j]);
    }
  };

  // A block's work in two parts.  qk: S^T = K Q^T into sacc.  sm_pv: masks,
  // softmax and O^T += V^T P^T from the sacc of the same block.  A block
  // entirely past this wave's rows contributes nothing (the tile's other wave
  // may still need it).
  f32x4 sacc[4][kRT];
  auto active = [&](int t) __attribute__((always_inline)) { return kb_s[t] * kPP <= p.q_start + min(qw + 31, p.q_len - 1); };
  auto qk = [&](const uint16_t* K, int t) __attribute__((always_inline)) {
    if (!active(t)) return;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) sacc[j4][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // k-steps outer: the eight accumulators of a k-step are independent,
    // so an MFMA never waits on the one just issued
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(K + ptok(j4, col) * kKRow + 8 * (kk + 4 * kg));
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          sacc[j4][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rt][kk], sacc[j4][rt], 0, 0, 0);
      }
    }
  };
  auto sm_pv = [&](const uint16_t* V, int t) __attribute__((always_inline)) {
    if (!active(t)) return;
    const int tok0 = kb_s[t] * kPP;
    // softmax (lane: row 16*rt + col, tokens ptok(j4, 4*kg + i)).
    // The row maximum is taken on the raw logits (the scale is positive),
    // then p = 2^(s * scale_log2 - m) is one FMA and one v_exp_f32
    // (results below 2^-126 flush to zero: their weight relative to the
    // row maximum is below 2^-126).
    // causal and sequence-end masks, only on blocks that cross a row (the
    // empty volatile asm keeps this a branch: if-converted, the masking
    // would run as per-element compares and selects on every block)
    const bool full = (tok0 + kPP - 1 <= wpos_lo) && (tok0 + kPP <= seq_len);
    if (!full) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const int row_pos = wpos_lo + 16 * rt + col;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = tok0 + ptok(j4, 4 * kg + i);
            if (j > row_pos || j >= seq_len) sacc[j4][rt][i] = -INFINITY;
          }
      }
    }
    bf16x8 pb[kRT][2];
    float alpha[kRT];
    bool need_rescale = false;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      float mraw = -INFINITY;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
        for (int i = 0; i < 4; ++i) mraw = fmaxf(mraw, sacc[j4][rt][i]);
      mraw = max_over_row_groups(mraw);
      const float mloc = mraw * p.scale_log2;      // -inf stays -inf (the scale is positive)
      // move the reference only when the row maximum outgrows it (the
      // first finite maximum always does: -inf + threshold = -inf); the
      // factor for a reference of -inf is 2^-inf = 0
      float mref = m_ref[rt];
      alpha[rt] = 1.f;
      if (mloc > mref + kRescaleThreshold) {
        alpha[rt] = __builtin_amdgcn_exp2f(mref - mloc);
        mref = mloc;
        need_rescale = true;
      }
      m_ref[rt] = mref;
      const float msub = mref == -INFINITY ? 0.f : mref;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j4][rt][i], p.scale_log2, -msub));
          pb[rt][j4 >> 1][4 * (j4 & 1) + i] = (__bf16)pv;
        }
    }
    if (__any(need_rescale)) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          oacc[dt][rt][0] *= alpha[rt]; oacc[dt][rt][1] *= alpha[rt];
          oacc[dt][rt][2] *= alpha[rt]; oacc[dt][rt][3] *= alpha[rt];
        }
        lacc[rt][0] *= alpha[rt]; lacc[rt][1] *= alpha[rt];
        lacc[rt][2] *= alpha[rt]; lacc[rt][3] *= alpha[rt];
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(V + (16 * dt + col) * kVRow + 8 * (pchunk(kp, kg) ^ vsw(col)));
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          oacc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt][kp], oacc[dt][rt], 0, 0, 0);
      }
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        lacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[rt][kp], lacc[rt], 0, 0, 0);
    }
  };

  // One block: wait for this wave's part of its copy (the copy of block t+1,
  // issued after it, may stay in flight), barrier (then every part has
  // landed and every wave has finished block t-1), compute, then copy block
  // t+2 into the stage block t-1 used.  Every copying wave issues exactly
  // NI loads per block (past the last block it repeats the last block's
  // page into a stage no one reads again), so the wait is a fixed count.
  // The wait is the s_waitcnt builtin (other counters free), which the
  // compiler's wait-count pass sees, so it adds no wait of its own; the
  // barrier is a plain s_barrier with a memory clobber (a __syncthreads()
  // fence would also wait for the copies in flight).
  auto block = [&](auto sidx, auto copying, int t) __attribute__((always_inline)) {
    constexpr int k = decltype(sidx)::value;
    constexpr bool CP = decltype(copying)::value;
    uint16_t* cur = k == 0 ? st0 : (k == 1 ? st1 : st2);
    uint16_t* ahead2 = k == 0 ? st2 : (k == 1 ? st0 : st1);
    __builtin_amdgcn_s_waitcnt((NI & 15) | ((NI >> 4) << 14) | 0x0f70);   // vmcnt(NI)
    asm volatile("s_barrier" ::: "memory");
    qk(cur, t);
    sm_pv(cur + kKTile, t);
    if constexpr (CP) stage_copy(ahead2, min(t + 2, nblk - 1));
  };

  // the tile's table entries and their physical pages, read once into LDS so
  // that no global load is waited on while block copies are in flight (the
  // load counter completes in issue order)
  for (int t = tid; t < nblk; t += 128 * HW) kb_s[t] = table[t];
  __syncthreads();
  for (int t = tid; t < nblk; t += 128 * HW) ph_s[t] = p.bt_row[kb_s[t]];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // the copying waves and the others run the same loop in two copies, so
  // that no branch on the wave sits inside it (the wait-count pass would
  // merge the two paths and wait for every copy in flight)
  auto sweep = [&](auto copying) __attribute__((always_inline)) {
    constexpr bool CP = decltype(copying)::value;
    if (CP && nblk > 0) {
      stage_copy(st0, 0);
      stage_copy(st1, min(1, nblk - 1));
    }
    int t3 = 0;
    for (; t3 + 3 <= nblk; t3 += 3) {
      block(Stage<0>{}, copying, t3);
      block(Stage<1>{}, copying, t3 + 1);
      block(Stage<2>{}, copying, t3 + 2);
    }
    if (t3 < nblk) block(Stage<0>{}, copying, t3);
    if (t3 + 1 < nblk) block(Stage<1>{}, copying, t3 + 1);
  };
  if (wave < NCW) sweep(std::true_type{});
  else sweep(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0x0f70);     // no copy into LDS outlives the loop

  // epilogue: O = O^T / l per row
  uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const float l = lacc[rt][0];
    const int i = qw + 16 * rt + col;
    if (i >= p.q_len) continue;
    const bool empty = m_ref[rt] == -INFINITY;
    const float inv = empty ? 0.f : 1.f / l;
    const size_t orow = (size_t)i * p.Hq + h;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint16_t v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = f32_to_bf16_bits(oacc[dt][rt][e] * inv);
      uint2 pk;
      pk.x = (uint32_t)v4[0] | ((uint32_t)v4[1] << 16);
      pk.y = (uint32_t)v4[2] | ((uint32_t)v4[3] << 16);
      *reinterpret_cast<uint2*>(out + orow * kPD + 16 * dt + 4 * kg) = pk;
    }
    if (kg == 0 && p.out_lse) p.out_lse[orow] = empty ? -INFINITY : (m_ref[rt] + log2f(l)) * kLn2;
  }
}

hipError_t launch_prefill(const PrefillParams& p0, hipStream_t s) {
  PrefillParams p = p0;
  p.n_qtiles = (p.q_len + kBQ - 1) / kBQ;
  const int hw = p.G % 4 == 0 ? 4 : (p.G % 2 == 0 ? 2 : 1);
  const int nwg = p.Hkv * p.n_qtiles * (p.G / hw);
  if (hw == 4) hipLaunchKernelGGL(prefill_kernel<4>, dim3(nwg), dim3(512), 0, s, p);
  else if (hw == 2) hipLaunchKernelGGL(prefill_kernel<2>, dim3(nwg), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(prefill_kernel<1>, dim3(nwg), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
