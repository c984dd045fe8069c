// Split-K paged flash-decode over per-head page lists, and the LSE merge.
//
// Method: each query row attends exactly the valid tokens of its selected
// pages ("Universal Attention Engine", "Content-Dependent Dynamic Routing":
// selected blocks get full attention, only they are loaded; TileSparse README,
// "Two implementations, by design": a true per-head page-list Flash-decode;
// "Motivation": Tiered QK 2D sparsity, Ambient pages on a subset of heads).
//
// bf16 kernel (d 64/128).  Decode is HBM-bound ("Key Design Decisions" 3:
// optimise bytes loaded), so the design goal is streaming each selected
// (page, KV head) exactly once with full 16-byte loads, straight into MFMA
// operand registers (no LDS staging; nothing is reused across waves):
//  * workgroup = (sequence, selection head, split), 4 waves; the query rows
//    that share the KV head (GQA group x query tokens, or one head's tokens)
//    form the 16 columns of one MFMA tile, so each K/V element is read once
//    for all of them;
//  * the split's list is walked in 64-token chunks (1 page of 64 or 4 pages
//    of 16), chunk c by wave c % 4;
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: K rows are the A operand
//    read directly from the token-major page; the token->row assignment is
//    permuted so that the fp32 S^T accumulators of two tiles are exactly the
//    B operand layout of the PV product (no shuffle between QK and PV);
//  * O^T += V^T P^T with V^T read directly from the page-transposed V pool
//    (8 consecutive tokens of one dim = one 16-byte load);
//  * online softmax in base 2 on the S^T fragments (max/sum over the 16
//    tokens a lane holds, then 2 cross-lane steps);
//  * the 4 waves' (m, l, O) are combined in LDS; with one split the result
//    is written directly, otherwise fp32 partials go to the workspace and a
//    merge kernel combines the splits.
#include "common.h"

namespace sa {

// ---------------------------------------------------------------- bf16 / MFMA
// The list, block table, lengths and counts arrive as restrict kernel
// arguments: the kernel never writes them, so their wave-uniform reads compile
// to scalar loads, which complete on their own counter and never wait behind
// the K/V vector loads in flight.
// STAGED (d 128, per-KV-head lists): each wave copies its next 64-token
// chunk (K rows and V^T rows, 32 KiB) into its own LDS area with non-temporal
// load-to-LDS instructions of 1 KiB contiguous each, and reads the MFMA
// operands from there.  Streaming reads whose instructions cover whole cache
// lines run at ~6.1-6.4 TB/s on this HBM against ~5.4-6.0 TB/s for the
// operand-shaped register loads (16 rows x 64 B per instruction), which
// cannot use the non-temporal hint.  Every page of a per-KV-head list is read
// by one workgroup only, so nothing is lost by not keeping it in L2.
// LDS rows are XOR-swizzled so the operand reads are free of bank conflicts
// (gfx950 16-byte reads: four cycles per 64 lanes, lanes of a cycle by
// half-wave and the parity of lane bits 2..4, distinct 16-byte slots modulo
// 256 bytes):
//   K row r (256 B):   16-byte chunk c sits at slot c ^ (2 (r & 3) + 8 ((r >> 3) & 1))
//   V^T row d (128 B): token chunk c sits at slot c ^ (d & 6)
__device__ __forceinline__ int stg_kswz(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }
__device__ __forceinline__ int stg_vswz(int d) { return d & 6; }

template <int D, int P, bool TIERED, bool STAGED>
__global__ __launch_bounds__(256, 2) void decode_bf16_kernel(DecodeParams p, const int32_t* __restrict__ lists,
                                                            const int32_t* __restrict__ btab,
                                                            const int32_t* __restrict__ seq_lens,
                                                            const int32_t* __restrict__ counts) {
  constexpr int KSTEPS = D / 32;
  constexpr int DTILES = D / 16;
  constexpr int E = 64 / P;            // list entries per 64-token chunk
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;

  int u = blockIdx.x;
  const int split = u % p.splits;
  u /= p.splits;
  const int s = u % p.n_sel;
  const int b = u / p.n_sel;
  const int g = p.per_q ? s / p.G : s;
  const int R = p.per_q ? p.T : p.T * p.G;
  const int sel = b * p.n_sel + s;
  const int count = counts[sel];
  const int32_t* list = lists + (size_t)sel * p.list_stride;
  const int cc = TIERED ? p.ccounts[sel] : count;
  const int sbase = count / p.splits, sextra = count % p.splits;
  const int beg = split * sbase + min(split, sextra);
  const int len = sbase + (split < sextra ? 1 : 0);
  const int end = beg + len;
  const int seq_len = seq_lens[b];
  const int32_t* bt = btab + (size_t)b * p.max_pages;

  // query row of this lane's MFMA column
  const bool row_ok = col < R;
  int t_row = 0, h_row = 0;
  if (row_ok) {
    if (p.per_q) { t_row = col; h_row = s; }
    else { t_row = col / p.G; h_row = s * p.G + col % p.G; }
  }
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    if (row_ok)
      qreg[kk] = *reinterpret_cast<const bf16x8*>(
          qp + (((size_t)b * p.T + t_row) * p.Hq + h_row) * D + 8 * kg + 32 * kk);
    else
      qreg[kk] = bf16x8{};
  }

  f32x4 oacc[DTILES];
#pragma unroll
  for (int i = 0; i < DTILES; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(p.v_pool);
  const int nchunks = seq_len > 0 ? (len + E - 1) / E : 0;

  // Chunk metadata is pipelined over two iterations with no branches, so its
  // scalar loads never wait in the middle of a chunk: the list entries of
  // chunk c+8 and the block-table entries of chunk c+4 are read while chunk c
  // computes.  Entries past the split, or pages with no valid token, point at
  // the sequence's first page (allocated whenever seq_len > 0) so that every
  // K/V load is unconditional; their tokens are masked, and their V rows only
  // meet zero probabilities.
  const int bt0 = seq_len > 0 ? bt[0] : 0;
  auto load_lps = [&](int c, int* lp) {
    const int e0 = beg + c * E;
#pragma unroll
    for (int j = 0; j < E; ++j) lp[j] = list[min(e0 + j, end - 1)];
  };
  auto resolve = [&](int c, const int* lp, int* phys, int* nval, bool* act) {
    const int e0 = beg + c * E;
#pragma unroll
    for (int j = 0; j < E; ++j) phys[j] = bt[lp[j]];   // used only where nval > 0 (see page_of)
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = e0 + j;
      nval[j] = e < end ? page_valid(seq_len, lp[j], P) : 0;
      bool a = e < end;
      if (TIERED && e < end && e >= cc) {
        const uint32_t w = p.amask[((size_t)b * p.max_pages + lp[j]) * p.mask_words + (h_row >> 5)];
        a = row_ok && ((w >> (h_row & 31)) & 1u);
      }
      act[j] = a;
    }
  };

  // K: A operand of tile j4, row m = col holds token
  //   tau = 32*(j4/2) + 8*(m/4) + 4*(j4%2) + m%4
  // The K loads of a wave's next chunk are issued as soon as this chunk's
  // QK^T has consumed its K registers, so the vector-memory queue never runs
  // dry while the chunk's softmax and PV compute.
  bf16x8 kreg[4][KSTEPS];
  uint16_t* stage_buf = nullptr;        // this wave's 32 KiB staging area (STAGED)
  if constexpr (STAGED) {
    __shared__ __attribute__((aligned(16))) uint16_t stg[4 * 16384];
    stage_buf = stg + wave * 16384;
  }
  // STAGED: copy of one chunk into the wave's staging area.  Wave-wide
  // instruction i covers slots [64 i, 64 i + 64) of the K part (row s / 16,
  // slot s % 16) and of the V^T part (row s / 8, slot s % 8).
  auto stage_copy = [&](const int* ph, const int* nv) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int sl = 64 * i + lane, r = sl >> 4;
      const int c = (sl & 15) ^ stg_kswz(r);
      const int ent = r / P, rr = r % P;
      const int pg = nv[ent] > 0 ? ph[ent] : bt0;
      __builtin_amdgcn_global_load_lds(kpool + (((size_t)pg * p.Hkv + g) * P + rr) * D + 8 * c, stage_buf + 512 * i,
                                       16, 0, 2 /* nt */);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int sl = 64 * i + lane, d = sl >> 3;
      const int c = (sl & 7) ^ stg_vswz(d);
      const int t0 = 8 * c, ent = t0 / P, r0 = t0 % P;
      const int pg = nv[ent] > 0 ? ph[ent] : bt0;
      __builtin_amdgcn_global_load_lds(vpool + (((size_t)pg * p.Hkv + g) * D + d) * P + r0,
                                       stage_buf + 8192 + 512 * i, 16, 0, 2 /* nt */);
    }
  };
  // STAGED: the chunk's operands from the staging area (its copy complete)
  auto read_staged = [&](bf16x8 (&vreg)[DTILES][2]) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int tau = 32 * (j4 >> 1) + 8 * (col >> 2) + 4 * (j4 & 1) + (col & 3);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        kreg[j4][kk] = *reinterpret_cast<const bf16x8*>(stage_buf + 8 * (16 * tau + ((kg + 4 * kk) ^ stg_kswz(tau))));
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const int d = 16 * dt + col;
        vreg[dt][kp] = *reinterpret_cast<const bf16x8*>(stage_buf + 8192 + 8 * (8 * d + ((4 * kp + kg) ^ stg_vswz(d))));
      }
  };
  auto load_k = [&](const int* ph, const int* nv) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int tau = 32 * (j4 >> 1) + 8 * (col >> 2) + 4 * (j4 & 1) + (col & 3);
      const int ent = tau / P, r = tau % P;
      const int pg = nv[ent] > 0 ? ph[ent] : bt0;
      const uint16_t* kb = kpool + (((size_t)pg * p.Hkv + g) * P + r) * D + 8 * kg;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) kreg[j4][kk] = *reinterpret_cast<const bf16x8*>(kb + 32 * kk);
    }
  };

  int phys[E], nval[E], lp_next[E];
  bool act[E];
  if (wave < nchunks) {
    int lp0[E];
    load_lps(wave, lp0);
    resolve(wave, lp0, phys, nval, act);
    if (wave + 4 < nchunks) load_lps(wave + 4, lp_next);
    if constexpr (STAGED) stage_copy(phys, nval);
    else load_k(phys, nval);
  }
  // one chunk; `prefetch` (a compile-time constant in each instantiation)
  // issues the next chunk's K loads.  The wave's last chunk is peeled off so
  // that no chunk carries a branch around the prefetch: the wait-count pass
  // would merge both paths and wait for the prefetch before PV.
  auto chunk = [&](auto prefetch, int c) {
    // physical page of chunk entry j: the sequence's first page stands in for
    // entries with no valid token
    auto page_of = [&](int j) { return nval[j] > 0 ? phys[j] : bt0; };

    // V^T: A operand of PV tile dt, k-step kp: dim 16*dt + col, tokens 32*kp + 8*kg + 0..7
    bf16x8 vreg[DTILES][2];
    if constexpr (!STAGED) {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const int t0 = 32 * kp + 8 * kg;
        const int ent = t0 / P, r0 = t0 % P;
        const uint16_t* vb = vpool + (((size_t)page_of(ent) * p.Hkv + g) * D + col) * P + r0;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) vreg[dt][kp] = *reinterpret_cast<const bf16x8*>(vb + (size_t)16 * dt * P);
      }
    }

    // metadata of the next two chunks (scalar loads) while this one computes
    int nphys[E], nnval[E], lp_after[E];
    bool nact[E];
    if (c + 4 < nchunks) resolve(c + 4, lp_next, nphys, nnval, nact);
    if (c + 8 < nchunks) load_lps(c + 8, lp_after);
    if constexpr (STAGED) {
      // this chunk's copy has landed; take its operands, then reuse the
      // staging area for the next chunk while this one computes
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      read_staged(vreg);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (decltype(prefetch)::value) stage_copy(nphys, nnval);
    }

    f32x4 sacc[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      sacc[j4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        sacc[j4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kreg[j4][kk], qreg[kk], sacc[j4], 0, 0, 0);
    }
    if constexpr (!STAGED && decltype(prefetch)::value) load_k(nphys, nnval);

    // lane holds S^T[token 32*(j4/2) + 8*kg + 4*(j4%2) + i][row col]; the
    // row maximum is taken on the raw logits (the scale is positive), then
    // p = 2^(s * scale_log2 - m) is one FMA and one v_exp_f32
    float mraw = -INFINITY;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 32 * (j4 >> 1) + 8 * kg + 4 * (j4 & 1) + i;
        const int ent = tau / P, r = tau % P;
        const bool ok = (r < nval[ent]) && act[ent];
        if (!ok) sacc[j4][i] = -INFINITY;
        mraw = fmaxf(mraw, sacc[j4][i]);
      }
    }
    mraw = max_over_row_groups(mraw);
    const float mloc = mraw == -INFINITY ? -INFINITY : mraw * p.scale_log2;
    const float m_new = fmaxf(m_run, mloc);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float msub = none ? 0.f : m_new;
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j4][i], p.scale_log2, -msub));
        psum += pv;
        pb[j4 >> 1][4 * (j4 & 1) + i] = (__bf16)pv;
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      oacc[dt][0] *= alpha; oacc[dt][1] *= alpha; oacc[dt][2] *= alpha; oacc[dt][3] *= alpha;
    }
    m_run = m_new;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vreg[dt][kp], pb[kp], oacc[dt], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      phys[j] = nphys[j];
      nval[j] = nnval[j];
      act[j] = nact[j];
      lp_next[j] = lp_after[j];
    }
  };
  int c = wave;
  for (; c + 4 < nchunks; c += 4) chunk(std::true_type{}, c);
  if (c < nchunks) chunk(std::false_type{}, c);

  // combine the 4 waves
  l_run = sum_over_row_groups(l_run);
  __shared__ float sm_m[4][16], sm_l[4][16];
  float (*sm_o)[16][D + 4];              // [4][16][D + 4]
  if constexpr (STAGED) {
    // the staging areas are free once every wave has left the loop (its last
    // operand reads waited for, no copy in flight after the peeled last
    // chunk); the barrier keeps a fast wave's partial O out of an area
    // another wave may still be reading
    sm_o = reinterpret_cast<float (*)[16][D + 4]>(stage_buf - wave * 16384);
    static_assert(4 * 16 * (D + 4) * sizeof(float) <= 4 * 16384 * sizeof(uint16_t), "partial O fits the staging areas");
    __syncthreads();
  } else {
    __shared__ float sm_o_s[4][16][D + 4];
    sm_o = sm_o_s;
  }
  if (kg == 0) { sm_m[wave][col] = m_run; sm_l[wave][col] = l_run; }
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[wave][col][16 * dt + 4 * kg + i] = oacc[dt][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    float M = fmaxf(fmaxf(sm_m[0][r], sm_m[1][r]), fmaxf(sm_m[2][r], sm_m[3][r]));
    float o = 0.f, lse = -INFINITY;
    if (M != -INFINITY) {
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = exp2f(sm_m[w][r] - M);
        L += sc * sm_l[w][r];
        acc += sc * sm_o[w][r][d];
      }
      o = acc / L;
      lse = (M + log2f(L)) * kLn2;
    }
    int t, h;
    if (p.per_q) { t = r; h = s; } else { t = r / p.G; h = s * p.G + r % p.G; }
    const size_t orow = ((size_t)b * p.T + t) * p.Hq + h;
    if (p.splits == 1) {
      reinterpret_cast<uint16_t*>(p.out)[orow * D + d] = f32_to_bf16_bits(o);
      if (d == 0 && p.out_lse) p.out_lse[orow] = lse;
    } else {
      p.part_o[(orow * p.splits + split) * D + d] = o;
      if (d == 0) p.part_lse[orow * p.splits + split] = lse;
    }
  }
}

// ------------------------------------------------------------------- fp32
// Plain VALU kernel for fp32 caches: one wave per query row, one lane per
// token of a page for the logits, one lane per output dim for PV.
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeParams p) {
  constexpr int DPL = D / 64;          // output dims per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int u = blockIdx.x;
  const int split = u % p.splits;
  u /= p.splits;
  const int s = u % p.n_sel;
  const int b = u / p.n_sel;
  const int g = p.per_q ? s / p.G : s;
  const int R = p.per_q ? p.T : p.T * p.G;
  const int sel = b * p.n_sel + s;
  const int count = p.counts[sel];
  const int32_t* list = p.lists + (size_t)sel * p.list_stride;
  const int cc = p.ccounts ? p.ccounts[sel] : count;
  const int sbase = count / p.splits, sextra = count % p.splits;
  const int beg = split * sbase + min(split, sextra);
  const int end = beg + sbase + (split < sextra ? 1 : 0);
  const int seq_len = p.seq_lens[b];
  const int P = p.P;
  const float* kpool = reinterpret_cast<const float*>(p.k_pool);
  const float* vpool = reinterpret_cast<const float*>(p.v_pool);

  for (int r = wave; r < R; r += 4) {
    int t, h;
    if (p.per_q) { t = r; h = s; } else { t = r / p.G; h = s * p.G + r % p.G; }
    const size_t orow = ((size_t)b * p.T + t) * p.Hq + h;
    const float* qrow = reinterpret_cast<const float*>(p.q) + orow * D;   // broadcast reads
    float m_run = -INFINITY, l_run = 0.f;
    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = 0.f;
    for (int e = beg; e < end; ++e) {
      const int lp = list[e];
      const int phys = p.block_table[(size_t)b * p.max_pages + lp];
      const int nv = page_valid(seq_len, lp, P);
      bool act = true;
      if (p.ccounts && e >= cc) {
        const uint32_t w = p.amask[((size_t)b * p.max_pages + lp) * p.mask_words + (h >> 5)];
        act = (w >> (h & 31)) & 1u;
      }
      if (!act || nv == 0) continue;
      float z = -INFINITY;
      if (lane < nv) {
        const float* krow = kpool + (((size_t)phys * p.Hkv + g) * P + lane) * D;
        float acc = 0.f;
        for (int d = 0; d < D; d += 4) {
          const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + d);
          const f32x4 qv = *reinterpret_cast<const f32x4*>(qrow + d);
          acc += kv[0] * qv[0] + kv[1] * qv[1] + kv[2] * qv[2] + kv[3] * qv[3];
        }
        z = acc * p.scale_log2;
      }
      const float mc = wave_max(z);
      const float m_new = fmaxf(m_run, mc);
      const float alpha = exp2f(m_run - m_new);
      const float pz = lane < nv ? exp2f(z - m_new) : 0.f;
      l_run = l_run * alpha + wave_sum(pz);
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = lane + 64 * i;
        const float* vrow = vpool + (((size_t)phys * p.Hkv + g) * D + d) * P;
        float acc = o[i] * alpha;
        for (int j = 0; j < nv; ++j) acc += __shfl(pz, j, 64) * vrow[j];
        o[i] = acc;
      }
      m_run = m_new;
    }
    const bool empty = m_run == -INFINITY;
    const float lse = empty ? -INFINITY : (m_run + log2f(l_run)) * kLn2;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int d = lane + 64 * i;
      const float val = empty ? 0.f : o[i] / l_run;
      if (p.splits == 1) reinterpret_cast<float*>(p.out)[orow * D + d] = val;
      else p.part_o[(orow * p.splits + split) * D + d] = val;
    }
    if (lane == 0) {
      if (p.splits == 1) { if (p.out_lse) p.out_lse[orow] = lse; }
      else p.part_lse[orow * p.splits + split] = lse;
    }
  }
}

// ------------------------------------------------------------------- merge
// One wave per query row: o = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max).
// Lanes own 4 consecutive dims (16-byte fp32 or 8-byte bf16 loads); the loads
// of up to 8 splits are issued before any is consumed.
template <bool BF16P>
__device__ __forceinline__ f32x4 load_partial4(const float* po, size_t off) {
  if constexpr (BF16P) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(po) + off);
    return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
  } else {
    return *reinterpret_cast<const f32x4*>(po + off);
  }
}

template <bool BF16P>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const float* pl = p.part_lse + (size_t)row * p.splits;
  const float mine = lane < p.splits ? pl[lane] : -INFINITY;
  const float M = wave_max(mine);
  float w = 0.f;
  if (M != -INFINITY && lane < p.splits) w = __expf(mine - M);
  const float L = wave_sum(w);
  const float inv = M == -INFINITY ? 0.f : 1.f / L;
  const float* po = p.part_o;
  const size_t row_off = (size_t)row * p.splits * p.d_v;
  for (int d4 = lane; d4 < p.d_v / 4; d4 += 64) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.splits; s0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = s0 + j < p.splits ? load_partial4<BF16P>(po, row_off + (size_t)(s0 + j) * p.d_v + 4 * d4)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ws = __shfl(w, (s0 + j) & 63, 64);
        if (s0 + j < p.splits && ws != 0.f) {
          acc[0] += ws * v[j][0]; acc[1] += ws * v[j][1]; acc[2] += ws * v[j][2]; acc[3] += ws * v[j][3];
        }
      }
    }
    const size_t o = (size_t)row * p.d_v + 4 * d4;
    if (p.out_fp32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + o) =
          f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    } else {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16_bits(acc[0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16_bits(acc[2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[3] * inv) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o) = pk;
    }
  }
  if (lane == 0 && p.out_lse) p.out_lse[row] = M == -INFINITY ? -INFINITY : M + __logf(L);
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  if (p.part_bf16) hipLaunchKernelGGL(lse_merge_kernel<true>, dim3((p.rows + 3) / 4), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(lse_merge_kernel<false>, dim3((p.rows + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int bf16, hipStream_t s) {
  const dim3 grid(p.B * p.n_sel * p.splits), block(256);
  const bool tiered = p.ccounts != nullptr;
  if (!bf16) {
    if (p.d_qk == 64) hipLaunchKernelGGL(decode_f32_kernel<64>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(decode_f32_kernel<128>, grid, block, 0, s, p);
    return hipGetLastError();
  }
#define SA_DECODE_LAUNCH(D_, P_, ST_)                                                                   \
  do {                                                                                                  \
    if (tiered)                                                                                         \
      hipLaunchKernelGGL((decode_bf16_kernel<D_, P_, true, ST_>), grid, block, 0, s, p, p.lists,            \
                         p.block_table, p.seq_lens, p.counts);                                          \
    else                                                                                                \
      hipLaunchKernelGGL((decode_bf16_kernel<D_, P_, false, ST_>), grid, block, 0, s, p, p.lists,           \
                         p.block_table, p.seq_lens, p.counts);                                          \
  } while (0)
  // staged operands for per-KV-head lists at d 128 (pages read by one
  // workgroup only); register operands otherwise
  const bool staged = !p.per_q;
  if (p.d_qk == 64 && p.P == 16) SA_DECODE_LAUNCH(64, 16, false);
  else if (p.d_qk == 64 && p.P == 64) SA_DECODE_LAUNCH(64, 64, false);
  else if (p.d_qk == 128 && p.P == 16) {
    if (staged) SA_DECODE_LAUNCH(128, 16, true);
    else SA_DECODE_LAUNCH(128, 16, false);
  } else {
    if (staged) SA_DECODE_LAUNCH(128, 64, true);
    else SA_DECODE_LAUNCH(128, 64, false);
  }
#undef SA_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace sa
