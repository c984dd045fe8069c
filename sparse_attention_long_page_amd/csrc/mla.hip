// Tiered sparse decode over a latent (MLA) paged cache.
//
// Method: TileSparse README, "Motivation" (Tiered QK 2D sparsity): a Critical
// tier of alpha pages computed with every query head and an Ambient tier of
// beta pages, each computed only by the h query heads chosen for it; "Two
// implementations, by design": a true per-head page-list Flash-decode.  With
// multi-token prediction and many heads sharing one latent KV row, decode
// attention becomes compute-heavy ("Motivation": arithmetic intensity of MLA
// decode with MTP), so the QK^T and PV contractions run on MFMA.
//
// Shapes: one latent KV head, K row = 576 dims (512 latent + 64 rope), V = the
// first 512 dims of the same row; pages of 64 tokens; rows = (head, token).
//
// Design (bf16 in, fp32 accumulate):
//  * workgroup = (sequence, group of 128 query rows, split of the page list),
//    4 waves of 32 rows (two 16-row MFMA column tiles) each; a row tile holds
//    16/T heads x T query tokens, so both MTP tokens of a head share a tile
//    and the head's Ambient bit;
//  * each page's 64 x 576 K tile is copied once into LDS by the LDS-DMA path
//    (global_load_lds_dwordx4, no registers), double-buffered: the copy of the
//    next page runs while the current one is computed; rows are padded to
//    1168 bytes so the 16-byte K reads and the 2-byte transposed V reads both
//    spread over the banks;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with Q^T resident in registers
//    (576 dims x 32 rows); the S^T fragments are the P^T operand of the PV
//    product directly; V^T operands (8 tokens of one dim) are gathered from
//    the token-major tile with 2-byte LDS reads;
//  * rows whose head is not in an Ambient page's head set see that page as
//    masked (-inf); a page none of the wave's rows attends is skipped;
//  * softmax in base 2 against a per-row reference maximum fixed at the first
//    page the row attends; the accumulators are never rescaled (a rescale of
//    256 accumulation registers per wave would cost as much VALU time as the
//    page's MFMAs).  Logits may exceed the reference by up to 2^64 before a
//    workgroup falls back to an exact-maximum pass and a recompute;
//  * fp32 partials (o_s, lse_s) per split go to the workspace and are merged
//    by the LSE-merge kernel; with one split the output is written directly.
#include "common.h"

namespace sa {

constexpr int kMD = 576;                 // QK dims
constexpr int kMDV = 512;                // V dims
constexpr int kMP = 64;                  // page size
constexpr int kMRowChunks = 73;          // 72 data chunks of 16 B + 1 pad chunk
constexpr int kMRS = kMRowChunks * 8;    // LDS row stride, bf16 elements (1168 B)
constexpr int kMTile = kMP * kMRS;       // elements per staged page
constexpr int kMInstr = kMP * kMRowChunks / 64;   // 73 wave-wide 16-byte DMA loads per page
constexpr int kMKSteps = kMD / 32;       // 18
constexpr int kMHalfInstr = 37;          // copy instructions covering rows 0-31 (37 * 64 >= 32 * 73)
constexpr int kMDTiles = kMDV / 16;      // 32
constexpr int kMetaWin = 256;            // pages of page metadata held in LDS
constexpr float kMMargin = 64.0f;         // log2 units a logit may exceed its row's reference

// Token of row m (0..15) of the 16-token MFMA tile j4 of a page.  Rows
// 4*g .. 4*g+3 (g = m/4) hold tokens 16*j4 + 8*(g/2) + g%2 + {0, 2, 4, 6}.
// With 1168-byte LDS rows (292 dwords, 4 mod 32) this keeps both the 16-byte
// K reads (8 rows per pass, distinct row mod 8) and the transposing V reads
// (4 rows 2 apart per 16-lane group) free of bank conflicts.
__device__ __forceinline__ int tok_of(int j4, int m) {
  const int g = m >> 2;
  return 16 * j4 + 8 * (g >> 1) + (g & 1) + 2 * (m & 3);
}

template <int V>
struct Parity {
  static constexpr int value = V;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ lds_v4i16* lds_v4(const uint16_t* p) {
  return (lds_v4i16*)(const_cast<uint16_t*>(p));
}

__global__ __launch_bounds__(256, 1) void mla_decode_kernel(DecodeParams p) {
  // two page buffers as distinct LDS objects, so the wait-count pass can
  // tell an LDS-DMA into one from reads of the other
  __shared__ __attribute__((aligned(16))) uint16_t sk0[kMTile];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[kMTile];
  // metadata of a window of the split's pages: physical page, valid tokens,
  // and the Ambient head-mask words covering this workgroup's heads
  __shared__ int m_phys[kMetaWin], m_nv[kMetaWin];
  __shared__ uint32_t m_word[kMetaWin][4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int col = lane & 15, kg = lane >> 4;
  const int T = p.T;
  const int heads_per_wg = 128 / T, heads_per_tile = 16 / T;
  const int n_rg = (p.Hq + heads_per_wg - 1) / heads_per_wg;

  // XCD-aware order: consecutive logical ids (the row groups of one
  // (sequence, split), which stream the same pages) share an XCD and its L2.
  const int nwg = gridDim.x, w = blockIdx.x;
  int u = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + w / 8 : w;
  const int rg = u % n_rg;
  u /= n_rg;
  const int split = u % p.splits;
  const int b = u / p.splits;

  const int sel = b;                       // one latent KV head: one list per sequence
  const int count = p.counts[sel];
  const int cc = p.ccounts ? p.ccounts[sel] : count;
  const int32_t* list = p.lists + (size_t)sel * p.list_stride;
  const int32_t* btab = p.block_table + (size_t)b * p.max_pages;
  const int sbase = count / p.splits, sextra = count % p.splits;
  const int beg = split * sbase + min(split, sextra);
  const int end = beg + sbase + (split < sextra ? 1 : 0);
  const int seq_len = p.seq_lens[b];

  // this lane's query row in each of the wave's two row tiles; a tile's
  // 16/T heads lie in one 32-bit word of the Ambient head mask
  int h_row[2], t_row[2], tile_word[2];
  bool row_ok[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int tile_h0 = rg * heads_per_wg + wave * 2 * heads_per_tile + rt * heads_per_tile;
    tile_word[rt] = tile_h0 >> 5;
    h_row[rt] = tile_h0 + col / T;
    t_row[rt] = col % T;
    row_ok[rt] = h_row[rt] < p.Hq;
  }
  const bool wave_rows = rg * heads_per_wg + wave * 2 * heads_per_tile < p.Hq;   // uniform
  const int word0 = (rg * heads_per_wg) >> 5;      // the workgroup's heads span words word0 .. word0+3

  // Q^T operand, resident: tile rt, k-step kk -> row col, dims 8*kg + 32*kk .. +8
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  bf16x8 qreg[2][kMKSteps];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    // rows past the last head read row 0: their logits are masked in the
    // softmax and their outputs never stored, so the loads need no select
    // (a select would wait for each load before the page metadata is read)
    const size_t qrow = row_ok[rt] ? ((size_t)b * T + t_row[rt]) * p.Hq + h_row[rt] : 0;
#pragma unroll
    for (int kk = 0; kk < kMKSteps; ++kk)
      qreg[rt][kk] = *reinterpret_cast<const bf16x8*>(qp + qrow * kMD + 8 * kg + 32 * kk);
  }

  f32x4 oacc[kMDTiles][2];
#pragma unroll
  for (int dt = 0; dt < kMDTiles; ++dt)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) oacc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);

  // LDS-DMA copy of one page's K tile: wave-wide instruction i covers LDS
  // chunks [64 i, 64 i + 64); chunk c is row c / 73, 16-byte column c % 73
  // (column 72 is row padding and re-reads column 0 of the row).  Wave w
  // issues the instructions i = w mod 4 of [i_lo, i_hi).
  auto stage = [&](uint16_t* buf, int phys, int i_lo, int i_hi) {
    const uint16_t* src = kpool + (size_t)phys * p.Hkv * kMP * kMD;
    for (int i = i_lo + ((wave - i_lo) & 3); i < i_hi; i += 4) {
      const int c = 64 * i + lane;
      const int r = c / kMRowChunks, ch = c % kMRowChunks;
      const int sch = ch < kMRowChunks - 1 ? ch : 0;
      __builtin_amdgcn_global_load_lds(src + (size_t)r * kMD + 8 * sch, buf + i * 512, 16, 0, 0);
    }
  };

  // Pass structure.  Attempt 0 sets each row's reference maximum from the
  // first page it attends and never moves it: later logits may exceed it by
  // up to 2^64 (exp2 stays finite in fp32), so the accumulators are never
  // rescaled.  If any row of the workgroup outgrows that margin, attempt 1
  // finds every row's exact maximum over the split (QK^T only) and attempt 2
  // recomputes with that fixed reference.  Inputs with ordinary logit ranges
  // take attempt 0 only.
  //
  // Within a page, every global load the page needs (list entry, block
  // table, head-mask words) is issued and consumed before the next page's
  // LDS-DMA is issued: completions are counted in issue order, so a wait for
  // a later load would also wait for the whole copy.
  bool overflow = false;
  for (int attempt = 0; attempt < 3; ++attempt) {
    if (attempt == 1) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) m_ref[rt] = -INFINITY;
    }
    if (attempt == 2) {
#pragma unroll
      for (int dt = 0; dt < kMDTiles; ++dt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) oacc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) l_run[rt] = 0.f;
    }
    const bool do_pv = attempt != 1;

    // metadata of the page being computed (cur_*) and of the next one
    // page metadata for pages [w0, w0 + kMetaWin) of the split, read into LDS
    // while no page copy is in flight (global loads complete in issue order)
    int w0 = beg;
    auto load_meta = [&](int first) {
      for (int i = threadIdx.x; i < kMetaWin && first + i < end; i += 256) {
        const int e = first + i;
        const int lp = list[e];
        // the block-table entry and the mask words are loaded together,
        // unconditionally (lp is a page of the sequence, the word index is
        // clamped), and chosen afterwards: a load under a condition would be
        // waited for before the next one is issued
        const int ph = btab[lp];
        uint32_t wd[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        if (p.ccounts) {
          const uint32_t* mrow = p.amask + ((size_t)b * p.max_pages + lp) * p.mask_words;
#pragma unroll
          for (int k = 0; k < 4; ++k) wd[k] = mrow[min(word0 + k, p.mask_words - 1)];
        }
        const int nv = page_valid(seq_len, lp, kMP);
        m_nv[i] = nv;
        m_phys[i] = nv > 0 ? ph : 0;
        const bool ambient = p.ccounts && e >= cc;
#pragma unroll
        for (int k = 0; k < 4; ++k) m_word[i][k] = (ambient && word0 + k < p.mask_words) ? wd[k] : 0xffffffffu;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    load_meta(beg);
    if (beg < end && m_nv[0] > 0) stage(sk0, m_phys[0], 0, kMInstr);

    // one page: compute from `cur` while the next page is copied into `nxt`
    auto page = [&](auto parity, int e) {
      uint16_t* cur = parity.value ? sk1 : sk0;
      uint16_t* nxt = parity.value ? sk0 : sk1;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int nv = m_nv[e - w0];
      uint32_t word[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) word[rt] = m_word[e - w0][tile_word[rt] - word0];
      if (nv > 0 && nv < kMP) {
        // tokens past the sequence end: zero their rows (V operand must be finite)
        for (int idx = threadIdx.x; idx < (kMP - nv) * 72; idx += 256) {
          const int r = nv + idx / 72, ch = idx % 72;
          *reinterpret_cast<u32x4*>(&cur[r * kMRS + 8 * ch]) = u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
      }
      if (e + 1 < end) {
        if (e + 1 - w0 == kMetaWin) {           // next window (long splits only)
          __syncthreads();
          w0 = e + 1;
          load_meta(w0);
        }
      }
      // the next page's copy in two parts: rows 0-31 now, the rest between
      // this page's two halves (issued at once, the copy stalls the wave on
      // the memory pipeline for thousands of cycles)
      const bool stage_next = e + 1 < end && m_nv[e + 1 - w0] > 0;
      auto copy_rest = [&]() {
        if (stage_next) stage(nxt, m_phys[e + 1 - w0], kMHalfInstr, kMInstr);
      };
      if (stage_next) stage(nxt, m_phys[e + 1 - w0], 0, kMHalfInstr);
      // which of this wave's rows attend the page
      bool act[2];
      bool any_row = false;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        act[rt] = row_ok[rt] && ((word[rt] >> (h_row[rt] & 31)) & 1u);
        any_row |= __any(act[rt]) != 0;
      }
      // a wave none of whose rows attend the page skips the work but still
      // passes the copy point between the halves
      const bool compute = nv > 0 && wave_rows && any_row;

      const uint16_t* K = cur;
      constexpr int kAhead = 3;            // operand reads in flight ahead of use
      auto half_page = [&](int half) {
        // S^T = K Q^T over tokens 32*half .. +32 (tiles j4 = 2*half, 2*half + 1)
        f32x4 sacc[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) sacc[j][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        constexpr int nsq = 2 * kMKSteps;
        // A row m of tile j4 is token tok_of(j4, m): the 8 lanes of one LDS
        // pass read 8 rows with distinct (row mod 8), i.e. distinct banks.
        auto kload = [&](int step) {
          const int kk = step >> 1, j4 = 2 * half + (step & 1);
          return *reinterpret_cast<const bf16x8*>(K + tok_of(j4, col) * kMRS + 8 * kg + 32 * kk);
        };
        bf16x8 ka[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) ka[i] = kload(i);
#pragma unroll
        for (int step = 0; step < nsq; ++step) {
          if (step + kAhead < nsq) ka[(step + kAhead) % (kAhead + 1)] = kload(step + kAhead);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            sacc[step & 1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % (kAhead + 1)],
                                                                         qreg[rt][step >> 1], sacc[step & 1][rt],
                                                                         0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }

        // softmax: lane holds S^T[token tok_of(2*half + j, 4*kg + i)][row col]
        bf16x8 pb[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          // row maximum on the raw logits (the scale is positive); then
          // p = 2^(s * scale_log2 - m) is one FMA and one v_exp_f32
          float mraw = -INFINITY;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tok = tok_of(2 * half + j, 4 * kg + i);
              if (!(act[rt] && tok < nv)) sacc[j][rt][i] = -INFINITY;
              mraw = fmaxf(mraw, sacc[j][rt][i]);
            }
          mraw = max_over_row_groups(mraw);
          const float mloc = mraw == -INFINITY ? -INFINITY : mraw * p.scale_log2;
          if (attempt == 1) {
            m_ref[rt] = fmaxf(m_ref[rt], mloc);
            continue;
          }
          if (attempt == 0) {
            if (m_ref[rt] == -INFINITY) m_ref[rt] = mloc;
            else if (mloc > m_ref[rt] + kMMargin) overflow = true;
          }
          const float msub = m_ref[rt] == -INFINITY ? 0.f : m_ref[rt];
          float psum = 0.f;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][rt][i], p.scale_log2, -msub));
              psum += pv;
              pb[rt][4 * j + i] = (__bf16)pv;
            }
          l_run[rt] += psum;
        }
        if (!do_pv) return;

        // O^T += V^T P^T over the same 32 tokens.  k-slot 8*kg + 4*j + i of
        // this product is token tok_of(2*half + j, 4*kg + i), the S^T fragment
        // element the lane already holds.  Two transposing LDS reads per
        // operand (j = 0, 1): within each 16-lane group, lane c gets element i
        // from the 4-element row that lane 4*i + c/4 addresses, at column c%4.
        // Lane col therefore addresses token tok_of(2*half + j, 4*kg + col/4),
        // dims 16*dt + 4*(col%4) .. +4, and receives dim 16*dt + col of the
        // tokens of k-slots 8*kg + 4*j + 0..3.  The 4 rows of one group are 2
        // apart, which puts them in distinct banks.
        const uint16_t* vb0 = K + tok_of(2 * half, 4 * kg + (col >> 2)) * kMRS + 4 * (col & 3);
        const uint16_t* vb1 = K + tok_of(2 * half + 1, 4 * kg + (col >> 2)) * kMRS + 4 * (col & 3);
        auto vload = [&](int dt) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4(vb0 + 16 * dt));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4(vb1 + 16 * dt));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 va[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) va[i] = vload(i);
#pragma unroll
        for (int dt = 0; dt < kMDTiles; ++dt) {
          if (dt + kAhead < kMDTiles) va[(dt + kAhead) % (kAhead + 1)] = vload(dt + kAhead);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            oacc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt % (kAhead + 1)], pb[rt], oacc[dt][rt],
                                                                   0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (compute) half_page(half);
        if (half == 0) copy_rest();
      }
    };
    for (int e = beg; e < end; e += 2) {
      page(Parity<0>{}, e);
      if (e + 1 < end) page(Parity<1>{}, e + 1);
    }
    // every wave has finished reading the last staged page before a new
    // attempt restages buffer 0
    if (attempt == 0 && !__syncthreads_or(overflow ? 1 : 0)) break;
    if (attempt == 1) __syncthreads();
  }

  // epilogue: O = O^T / l per row; lane holds dims 16*dt + 4*kg + 0..3 of row col
  float lse_row[2];
  size_t orow[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float l = l_run[rt];
    l = sum_over_row_groups(l);
    const bool empty = m_ref[rt] == -INFINITY;
    const float inv = empty ? 0.f : 1.f / l;
    lse_row[rt] = empty ? -INFINITY : (m_ref[rt] + log2f(l)) * kLn2;
    orow[rt] = ((size_t)b * T + t_row[rt]) * p.Hq + h_row[rt];
    if (!row_ok[rt]) continue;
    if (p.splits == 1) {
      uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + orow[rt] * kMDV;
#pragma unroll
      for (int dt = 0; dt < kMDTiles; ++dt) {
        f32x4 v = oacc[dt][rt];
        v[0] *= inv; v[1] *= inv; v[2] *= inv; v[3] *= inv;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(out + 16 * dt + 4 * kg) = pk;
      }
    } else if (p.part_bf16) {
      uint16_t* po = reinterpret_cast<uint16_t*>(p.part_o) + (orow[rt] * p.splits + split) * kMDV;
#pragma unroll
      for (int dt = 0; dt < kMDTiles; ++dt) {
        f32x4 v = oacc[dt][rt];
        v[0] *= inv; v[1] *= inv; v[2] *= inv; v[3] *= inv;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(po + 16 * dt + 4 * kg) = pk;
      }
    } else {
      float* po = p.part_o + (orow[rt] * p.splits + split) * kMDV;
#pragma unroll
      for (int dt = 0; dt < kMDTiles; ++dt) {
        f32x4 v = oacc[dt][rt];
        v[0] *= inv; v[1] *= inv; v[2] *= inv; v[3] *= inv;
        *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * kg) = v;
      }
    }
  }
  // One lane per row stores the log-sum-exp, after every output store: with
  // no register live past this branch, none can be restored from a spill
  // under its narrowed lane mask (the compiler in use did that, clobbering
  // accumulators of the other 48 lanes, when these stores sat between the
  // two row tiles).
  if (kg == 0) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (!row_ok[rt]) continue;
      if (p.splits == 1) {
        if (p.out_lse) p.out_lse[orow[rt]] = lse_row[rt];
      } else {
        p.part_lse[orow[rt] * p.splits + split] = lse_row[rt];
      }
    }
  }
}

hipError_t launch_mla_decode(const DecodeParams& p, hipStream_t s) {
  const int heads_per_wg = 128 / p.T;
  const int n_rg = (p.Hq + heads_per_wg - 1) / heads_per_wg;
  const dim3 grid(p.B * n_rg * p.splits), block(256);
  hipLaunchKernelGGL(mla_decode_kernel, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
