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
//  * workgroup = (sequence, row group, split of the page list), 8 row tiles of
//    16 rows (MFMA columns): 8 waves of one tile each, so that two waves share
//    a SIMD (256 registers each) and one runs while the other waits on its
//    copy instructions or LDS reads (4 waves of two tiles with 512 registers,
//    the RT = 2 form of the kernel, measured 2 us slower); a tile holds 16/T
//    heads x T query tokens, so the MTP tokens of a head share a tile and the
//    head's Ambient bit;
//  * a split takes a contiguous chunk of the Critical segment and a contiguous
//    chunk of the Ambient segment of the list (chunk sizes differ by at most
//    one), so every split holds a few Ambient pages;
//  * the Ambient tier saves compute: every workgroup of a (sequence, split)
//    ranks the sequence's heads by their membership pattern over the split's
//    Ambient pages (heads attending the same pages become neighbours), and
//    deals the ranked heads out in tiles; a tile computes an Ambient page only
//    if one of its heads attends it, so each Ambient page runs on few tiles
//    instead of on every tile with a member head somewhere;
//  * each page's 64 x 576 K tile is copied once into LDS by buffer-to-LDS
//    copies (16 bytes per lane, no registers), double-buffered: the copy of the
//    next page runs while the current one is computed; rows are padded to
//    1168 bytes so the 16-byte K reads and the 2-byte transposed V reads both
//    spread over the banks;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with Q^T resident in registers
//    (576 dims x 16 rows per tile); the S^T fragments are the P^T operand of the PV
//    product directly; V^T operands (8 tokens of one dim) come from the
//    token-major tile with transposing LDS reads; with two row tiles per wave,
//    when both attend a page each K and V operand read feeds both tiles' MFMAs;
//  * the first page's copy is issued right behind the query-row loads, so
//    the two land together;
//  * rows of an active tile whose head is not in an Ambient page's head set
//    see that page as masked (-inf);
//  * softmax in base 2 against a per-row reference maximum fixed at the first
//    page the row attends; the accumulators are never rescaled (a rescale of
//    256 accumulation registers per wave would cost as much VALU time as the
//    page's MFMAs).  Logits may exceed the reference by up to 2^64 before a
//    workgroup falls back to an exact-maximum pass and a recompute;
//  * bf16 partials (o_s) and fp32 lse_s per split go to the workspace and are
//    merged by the LSE-merge kernel; with one split the output is written
//    directly.
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
constexpr int kMetaWin = 128;            // pages of page metadata held in LDS
constexpr int kMaxMaskWords = 8;         // Ambient head-mask words per page (n_q_heads <= 256)
constexpr float kMMargin = 64.0f;         // log2 units a logit may exceed its row's reference
constexpr int kOutRS = kMDV + 8;          // LDS row stride of the staged bf16 output rows (1040 B)

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

// Chunk s of [0, n) cut into S contiguous chunks whose sizes differ by at most one.
__device__ __forceinline__ void split_chunk(int n, int S, int s, int& lo, int& hi) {
  const int base = n / S, extra = n % S;
  lo = s * base + min(s, extra);
  hi = lo + base + (s < extra ? 1 : 0);
}

// RT row tiles per wave (1: 8 waves, two per SIMD; 2: 4 waves, one per SIMD)
template <int RT>
__global__ __launch_bounds__(512 / RT, RT == 1 ? 2 : 1) void mla_decode_kernel(DecodeParams p) {
  constexpr int NWV = 8 / RT;                            // waves per workgroup (8 row tiles)
  constexpr int NT = 64 * NWV;                           // threads
  // two page buffers as distinct LDS objects, so the wait-count pass can
  // tell an LDS-DMA into one from reads of the other
  __shared__ __attribute__((aligned(16))) uint16_t sk0[kMTile];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[kMTile];
  // metadata of a window of the split's pages: physical page, valid tokens,
  // and the page's Ambient head-mask words (all ones for a Critical page)
  __shared__ int m_phys[kMetaWin], m_nv[kMetaWin];
  __shared__ uint32_t m_word[kMetaWin][kMaxMaskWords];
  // heads ranked by their Ambient membership pattern over the split
  __shared__ __attribute__((aligned(16))) uint32_t h_key[256];
  __shared__ uint16_t h_rank[256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int col = lane & 15, kg = lane >> 4;
  const int T = p.T;
  const int hpt = 16 / T;                                // heads per 16-row tile
  const int n_tiles = (p.Hq + hpt - 1) / hpt;
  const int n_rg = (n_tiles + 7) / 8;                    // 8 tiles per workgroup

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
  const int cc = p.ccounts ? min(p.ccounts[sel], count) : count;
  const int32_t* list = p.lists + (size_t)sel * p.list_stride;
  const int32_t* btab = p.block_table + (size_t)b * p.max_pages;
  // this split's pages: chunk `split` of the Critical segment, then chunk
  // `split` of the Ambient segment
  int cb, ce, ab, ae;
  split_chunk(cc, p.splits, split, cb, ce);
  split_chunk(count - cc, p.splits, split, ab, ae);
  ab += cc;
  ae += cc;
  const int n_crit = ce - cb;
  const int n_pg = n_crit + (ae - ab);
  const int seq_len = p.seq_lens[b];

  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);

  // The copies are buffer loads to LDS over a resource spanning the page
  // (lanes past it would read 0): as buffer instructions they count on the
  // vector-memory counter only, so the compiler keeps its partial waits on
  // the LDS reads of the page being computed while a copy is in flight (with
  // the global-load form it waits for every LDS read at once).
  auto stage = [&](uint16_t* buf, int phys, int i_lo, int i_hi) {
    const uint16_t* src = kpool + (size_t)phys * p.Hkv * kMP * kMD;
    const auto rsrc = buffer_rsrc(src, kMP * kMD * 2);
    for (int i = i_lo + ((wave - i_lo) & (NWV - 1)); i < i_hi; i += NWV) {
      const int c = 64 * i + lane;
      const int r = c / kMRowChunks, ch = c % kMRowChunks;
      const int sch = ch < kMRowChunks - 1 ? ch : 0;
      copy16_to_lds(rsrc, buf + i * 512, (r * kMD + 8 * sch) * 2);
    }
  };

  // page metadata for pages [w0, w0 + kMetaWin) of the split, read into LDS
  // while no page copy is in flight (global loads complete in issue order)
  int w0 = 0;
  auto load_meta = [&](int first) {
    for (int i = threadIdx.x; i < kMetaWin && first + i < n_pg; i += NT) {
      const int k = first + i;
      const int e = k < n_crit ? cb + k : ab + (k - n_crit);
      const int lp = list[e];
      // the block-table entry and the mask words are loaded together,
      // unconditionally (lp is a page of the sequence, the word index is
      // clamped), and chosen afterwards: a load under a condition would be
      // waited for before the next one is issued
      const int ph = btab[lp];
      uint32_t wd[kMaxMaskWords];
#pragma unroll
      for (int j = 0; j < kMaxMaskWords; ++j) wd[j] = 0xffffffffu;
      if (p.ccounts) {
        const uint32_t* mrow = p.amask + ((size_t)b * p.max_pages + lp) * p.mask_words;
#pragma unroll
        for (int j = 0; j < kMaxMaskWords; ++j) wd[j] = mrow[min(j, p.mask_words - 1)];
      }
      const int nv = page_valid(seq_len, lp, kMP);
      m_nv[i] = nv;
      m_phys[i] = nv > 0 ? ph : 0;
      const bool ambient = k >= n_crit;
#pragma unroll
      for (int j = 0; j < kMaxMaskWords; ++j) m_word[i][j] = ambient ? wd[j] : 0xffffffffu;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  load_meta(0);

  // Rank the heads: key bit j = the head attends Ambient page j of the split
  // (first 32 held in the first window); ranked by (key, head index), so the
  // ranking is the same in every workgroup of the (sequence, split).  Slots
  // past the last head hold the largest key and never count.
  const bool ranked = p.ccounts != nullptr;
  if (ranked) {
    const int na = min(min(n_pg - n_crit, 32), kMetaWin - n_crit);
    for (int h = threadIdx.x; h < 256; h += NT) {
      uint32_t key = 0xffffffffu;
      if (h < p.Hq) {
        key = 0;
        // all 32 words are read from clamped indices and the bits past na
        // dropped afterwards, so the reads are in flight together (the empty
        // asm keeps each read unconditional: otherwise the compiler sinks it
        // into a branch on j < na with a wait of its own)
        uint32_t wv[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) wv[j] = m_word[min(n_crit + j, kMetaWin - 1)][h >> 5];
#pragma unroll
        for (int j = 0; j < 32; ++j) asm volatile("" : "+v"(wv[j]));
#pragma unroll
        for (int j = 0; j < 32; ++j) key |= (j < na ? (wv[j] >> (h & 31)) & 1u : 0u) << j;
      }
      h_key[h] = key;
    }
    // (the ranking exchanges LDS data only, so its barriers wait on LDS only)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const uint4* keys4 = reinterpret_cast<const uint4*>(h_key);
    const int n4 = (p.Hq + 3) >> 2;
    for (int h = threadIdx.x; h < p.Hq; h += NT) {
      const uint32_t kh = h_key[h];
      int r = 0;
      // 16 key quads per round, read unconditionally from clamped indices
      // (slots past the last head hold the largest key and never count)
      for (int i0 = 0; i0 < n4; i0 += 16) {
        uint4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = keys4[min(i0 + u, n4 - 1)];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int hb = 4 * (i0 + u);
          int c = (v[u].x < kh || (v[u].x == kh && hb < h)) ? 1 : 0;
          c += (v[u].y < kh || (v[u].y == kh && hb + 1 < h)) ? 1 : 0;
          c += (v[u].z < kh || (v[u].z == kh && hb + 2 < h)) ? 1 : 0;
          c += (v[u].w < kh || (v[u].w == kh && hb + 3 < h)) ? 1 : 0;
          r += i0 + u < n4 ? c : 0;
        }
      }
      h_rank[r] = (uint16_t)h;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // This lane's query row in each of the wave's row tiles.  Ranked tile
  // t (heads of ranks t*hpt ..) goes to row group, wave and slot in a snake
  // order, so every wave gets a mix of rarely and often attending tiles.
  int h_row[RT], t_row[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int j = rt * NWV + ((rt & 1) ? NWV - 1 - wave : wave);
    const int t = j * n_rg + ((j & 1) ? n_rg - 1 - rg : rg);
    const int pos = t * hpt + col / T;
    row_ok[rt] = t < n_tiles && pos < p.Hq;
    h_row[rt] = row_ok[rt] ? (ranked ? (int)h_rank[pos] : pos) : 0;
    t_row[rt] = col % T;
  }

  // Q^T operand, resident: tile rt, k-step kk -> row col, dims 8*kg + 32*kk .. +8
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  bf16x8 qreg[RT][kMKSteps];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // rows past the last head read row 0: their logits are masked in the
    // softmax and their outputs never stored, so the loads need no select
    // (a select would wait for each load before the page metadata is read)
    const size_t qrow = row_ok[rt] ? ((size_t)b * T + t_row[rt]) * p.Hq + h_row[rt] : 0;
#pragma unroll
    for (int kk = 0; kk < kMKSteps; ++kk)
      qreg[rt][kk] = *reinterpret_cast<const bf16x8*>(qp + qrow * kMD + 8 * kg + 32 * kk);
  }
  // the first page's copy goes out right behind the query-row loads, so the
  // two land together (issued before the ranking, the copy held the issuing
  // waves and delayed the ranking by as long)
  if (n_pg > 0 && m_nv[0] > 0) stage(sk0, m_phys[0], 0, kMInstr);

  f32x4 oacc[kMDTiles][RT];
#pragma unroll
  for (int dt = 0; dt < kMDTiles; ++dt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) oacc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) { m_ref[rt] = -INFINITY; l_run[rt] = 0.f; }

  // LDS-DMA copy of one page's K tile: wave-wide instruction i covers LDS
  // chunks [64 i, 64 i + 64); chunk c is row c / 73, 16-byte column c % 73
  // (column 72 is row padding and re-reads column 0 of the row).  Wave w
  // issues the instructions i of [i_lo, i_hi) with i = w mod NWV (the
  // stage lambda above).
  // Pass structure.  Attempt 0 sets each row's reference maximum from the
  // first page it attends and never moves it: later logits may exceed it by
  // up to 2^64 (exp2 stays finite in fp32), so the accumulators are never
  // rescaled.  If any row of the workgroup outgrows that margin, attempt 1
  // finds every row's exact maximum over the split (QK^T only) and attempt 2
  // recomputes with that fixed reference.  Inputs with ordinary logit ranges
  // take attempt 0 only.
  //
  // Within a page, every global load the page needs is issued and consumed
  // before the next page's LDS-DMA is issued: completions are counted in
  // issue order, so a wait for a later load would also wait for the whole
  // copy.  The page metadata comes from LDS.
  bool overflow = false;
  for (int attempt = 0; attempt < 3; ++attempt) {
    if (attempt == 1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) m_ref[rt] = -INFINITY;
    }
    if (attempt == 2) {
#pragma unroll
      for (int dt = 0; dt < kMDTiles; ++dt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) oacc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) l_run[rt] = 0.f;
    }
    if (attempt > 0 && w0 != 0) {
      __syncthreads();
      w0 = 0;
      load_meta(0);
    }
    if (attempt > 0 && n_pg > 0 && m_nv[0] > 0) stage(sk0, m_phys[0], 0, kMInstr);

    // one page: compute from `cur` while the next page is copied into `nxt`
    auto page = [&](auto parity, int k) {
      uint16_t* cur = parity.value ? sk1 : sk0;
      uint16_t* nxt = parity.value ? sk0 : sk1;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int nv = m_nv[k - w0];
      bool act[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t word = m_word[k - w0][h_row[rt] >> 5];
        act[rt] = row_ok[rt] && ((word >> (h_row[rt] & 31)) & 1u);
      }
      if (nv > 0 && nv < kMP) {
        // tokens past the sequence end: zero their rows (V operand must be finite)
        for (int idx = threadIdx.x; idx < (kMP - nv) * 72; idx += NT) {
          const int r = nv + idx / 72, ch = idx % 72;
          *reinterpret_cast<u32x4*>(&cur[r * kMRS + 8 * ch]) = u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
      }
      if (k + 1 < n_pg && k + 1 - w0 == kMetaWin) {   // next window (long splits only)
        __syncthreads();
        w0 = k + 1;
        load_meta(w0);
      }
      // the next page's copy in two parts: rows 0-31 now, the rest between
      // this page's two halves (issued at once, the copy stalls the wave on
      // the memory pipeline for thousands of cycles)
      const bool stage_next = k + 1 < n_pg && m_nv[k + 1 - w0] > 0;
      auto copy_part = [&](int half) {
        if (stage_next) stage(nxt, m_phys[k + 1 - w0], half ? kMHalfInstr : 0, half ? kMInstr : kMHalfInstr);
      };
      copy_part(0);
      // tiles of this wave with a row that attends the page (wave-uniform)
      int tmask = nv > 0 && __any(act[0]) ? 1 : 0;
      if constexpr (RT > 1) tmask |= nv > 0 && __any(act[RT - 1]) ? 2 : 0;

      const uint16_t* K = cur;
      constexpr int kAhead = RT == 1 ? 3 : 5;   // operand reads in flight ahead of use
      // The row tiles in MASK (bit rt) over half a page: S^T = K Q^T over
      // tokens 32*half .. +32 (MFMA tiles j4 = 2*half, 2*half + 1), softmax,
      // O^T += V^T P^T.  With both tiles, each K and V operand read from LDS
      // feeds the MFMAs of both.  A tile none of whose rows attends the page
      // is left out.
      auto tile_pass = [&](auto maskc, int half) {
        constexpr int MASK = decltype(maskc)::value;
        constexpr bool on[2] = {(MASK & 1) != 0, (MASK & 2) != 0};
        f32x4 sacc[2][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[rt][0] = sacc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
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
          for (int rt = 0; rt < RT; ++rt)
            if (on[rt])
              sacc[rt][step & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % (kAhead + 1)],
                                                                          qreg[rt][step >> 1], sacc[rt][step & 1],
                                                                          0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }

        // softmax: lane holds S^T[token tok_of(2*half + j, 4*kg + i)][row col].
        // Row maximum on the raw logits (the scale is positive); then
        // p = 2^(s * scale_log2 - m) is one FMA and one v_exp_f32.
        bf16x8 pb[2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (!on[rt]) continue;
          float mraw = -INFINITY;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tok = tok_of(2 * half + j, 4 * kg + i);
              if (!(act[rt] && tok < nv)) sacc[rt][j][i] = -INFINITY;
              mraw = fmaxf(mraw, sacc[rt][j][i]);
            }
          mraw = max_over_row_groups(mraw);
          const float mloc = mraw * p.scale_log2;     // -inf stays -inf (the scale is positive)
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
              const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rt][j][i], p.scale_log2, -msub));
              psum += pv;
              pb[rt][4 * j + i] = (__bf16)pv;
            }
          l_run[rt] += psum;
        }
        if (attempt == 1) return;

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
          for (int rt = 0; rt < RT; ++rt)
            if (on[rt])
              oacc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt % (kAhead + 1)], pb[rt], oacc[dt][rt],
                                                                     0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // a wave with no active tile skips the work but still passes the copy
      // point between the halves (tmask is wave-uniform)
      auto halfpage = [&](int half) {
        // (independent ifs: as an if-else chain the compiler spilled most of
        // the accumulators)
        if constexpr (RT > 1)
          if (tmask == 3) tile_pass(std::integral_constant<int, 3>{}, half);
        if (tmask == 1) tile_pass(std::integral_constant<int, 1>{}, half);
        if constexpr (RT > 1)
          if (tmask == 2) tile_pass(std::integral_constant<int, 2>{}, half);
      };
      halfpage(0);
      copy_part(1);
      halfpage(1);
    };
    for (int k = 0; k < n_pg; k += 2) {
      page(Parity<0>{}, k);
      if (k + 1 < n_pg) page(Parity<1>{}, k + 1);
    }
    // every wave has finished reading the last staged page before a new
    // attempt restages buffer 0
    if (attempt == 0 && !__syncthreads_or(overflow ? 1 : 0)) break;
    if (attempt == 1) __syncthreads();
  }

  // epilogue: O = O^T / l per row; lane holds dims 16*dt + 4*kg + 0..3 of row col.
  // bf16 rows (the output, or bf16 split partials) go through LDS: each tile's
  // 16 rows are written to a free page buffer, then stored row by row, 1 KiB
  // per wave-wide store, instead of 16 rows x 32 bytes per store.  The page
  // buffers are free once every wave has passed the barrier below (no copy is
  // issued after the last page).
  const bool staged_out = p.splits == 1 || p.part_bf16;     // uniform
  if (staged_out) __syncthreads();
  auto out_area = [&](int rt) {
    const int ti = wave * RT + rt;                          // 8 tiles, 4 per page buffer
    return (ti < 4 ? sk0 : sk1) + (ti & 3) * 16 * kOutRS;
  };
  static_assert(4 * 16 * kOutRS <= kMTile, "four tiles' output rows fit one page buffer");
  float lse_row[RT];
  size_t orow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = l_run[rt];
    l = sum_over_row_groups(l);
    const bool empty = m_ref[rt] == -INFINITY;
    const float inv = empty ? 0.f : 1.f / l;
    lse_row[rt] = empty ? -INFINITY : (m_ref[rt] + log2f(l)) * kLn2;
    orow[rt] = ((size_t)b * T + t_row[rt]) * p.Hq + h_row[rt];
    if (!row_ok[rt]) continue;
    if (staged_out) {
      uint16_t* ar = out_area(rt) + col * kOutRS;
#pragma unroll
      for (int dt = 0; dt < kMDTiles; ++dt) {
        f32x4 v = oacc[dt][rt];
        v[0] *= inv; v[1] *= inv; v[2] *= inv; v[3] *= inv;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(ar + 16 * dt + 4 * kg) = pk;
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
  if (staged_out) {
    __syncthreads();
    // row r of a tile is lane r's row (kg 0): its validity and output row are
    // taken from that lane, and the wave stores the row's 1 KiB at once
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint16_t* ar = out_area(rt);
      for (int r = 0; r < 16; ++r) {
        const int ok = __shfl(row_ok[rt] ? 1 : 0, r, 64);
        const size_t orr = ((size_t)(uint32_t)__shfl((int)(orow[rt] >> 32), r, 64) << 32) |
                           (size_t)(uint32_t)__shfl((int)(uint32_t)orow[rt], r, 64);
        if (ok) {
          const uint4 v = *reinterpret_cast<const uint4*>(ar + r * kOutRS + 8 * lane);
          uint16_t* dst = p.splits == 1 ? reinterpret_cast<uint16_t*>(p.out) + orr * kMDV
                                        : reinterpret_cast<uint16_t*>(p.part_o) + (orr * p.splits + split) * kMDV;
          *reinterpret_cast<uint4*>(dst + 8 * lane) = v;
        }
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
    for (int rt = 0; rt < RT; ++rt) {
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
  const int hpt = 16 / p.T;
  const int n_rg = ((p.Hq + hpt - 1) / hpt + 7) / 8;
  const dim3 grid(p.B * n_rg * p.splits);
  hipLaunchKernelGGL(mla_decode_kernel<1>, grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
