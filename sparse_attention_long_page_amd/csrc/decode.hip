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
#include "decode_body.h"

namespace sa {

// ---------------------------------------------------------------- bf16 / MFMA
template <int D, int P, bool TIERED, bool STAGED, bool FP8>
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
  __shared__ __attribute__((aligned(16))) uint16_t stg[STAGED ? 4 * 16384 : 8];
  uint16_t* const stg_area = stg;
#include "decode_body.inc"
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
// Lanes own VPL consecutive dims (16-byte loads: 4 fp32 or 8 bf16 partial
// values); the loads of a group of 8 splits are issued before any is
// consumed, and the first group's go out together with the row's lse loads,
// before the weights are formed.
template <bool BF16P>
struct MergeLanes {
  static constexpr int VPL = BF16P ? 8 : 4;         // dims per lane per load
  typedef u32x4 raw_t;                              // 16 bytes of partial values
  __device__ static float val(const raw_t& v, int e) {
    if constexpr (BF16P) return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
    else return __uint_as_float(v[e]);
  }
};

template <bool BF16P>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeParams p) {
  using ML = MergeLanes<BF16P>;
  constexpr int VPL = ML::VPL;
  typedef typename ML::raw_t raw_t;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const float* pl = p.part_lse + (size_t)row * p.splits;
  const size_t row_off = (size_t)row * p.splits * p.d_v;
  const uint16_t* pob = reinterpret_cast<const uint16_t*>(p.part_o);
  // group of 8 splits from s0 at dims d0.. (unconditional loads from clamped
  // indices: a split past the last re-reads the last one, dims past d_v the
  // row's last VPL; neither is used)
  auto load_group = [&](int d0, int s0, raw_t (&v)[8]) __attribute__((always_inline)) {
    const int dd = min(d0, p.d_v - VPL);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t off = row_off + (size_t)min(s0 + j, p.splits - 1) * p.d_v + dd;
      if constexpr (BF16P) v[j] = *reinterpret_cast<const raw_t*>(pob + off);
      else v[j] = *reinterpret_cast<const raw_t*>(p.part_o + off);
    }
  };
  const int d_first = VPL * lane;
  raw_t v[8];
  const float lv = pl[min(lane, p.splits - 1)];
  load_group(d_first, 0, v);
  const float mine = lane < p.splits ? lv : -INFINITY;
  const float M = wave_max(mine);
  float w = 0.f;
  if (M != -INFINITY && lane < p.splits) w = __expf(mine - M);
  const float L = wave_sum(w);
  const float inv = M == -INFINITY ? 0.f : 1.f / L;
  // a split that takes no part adds +0.0, which leaves acc unchanged (it
  // starts at +0.0 and never becomes -0.0); an empty split's partial,
  // whatever it holds, is never used
  auto accumulate = [&](const raw_t (&vv)[8], int s0, float (&acc)[VPL]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float ws = __shfl(w, (s0 + j) & 63, 64);
      const bool use = s0 + j < p.splits && ws != 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) acc[e] += use ? ws * ML::val(vv[j], e) : 0.f;
    }
  };
  auto store = [&](int d0, const float (&acc)[VPL]) __attribute__((always_inline)) {
    const size_t o = (size_t)row * p.d_v + d0;
    if (p.out_fp32) {
      float* of = reinterpret_cast<float*>(p.out) + o;
#pragma unroll
      for (int e = 0; e < VPL; e += 4)
        *reinterpret_cast<f32x4*>(of + e) = f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
    } else {
      uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + o;
#pragma unroll
      for (int e = 0; e < VPL; e += 4) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(acc[e] * inv) | ((uint32_t)f32_to_bf16_bits(acc[e + 1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(acc[e + 2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[e + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(ob + e) = pk;
      }
    }
  };
  for (int d0 = d_first; d0 < p.d_v; d0 += 64 * VPL) {
    float acc[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) acc[e] = 0.f;
    for (int s0 = 0; s0 < p.splits; s0 += 8) {
      if (d0 != d_first || s0 != 0) load_group(d0, s0, v);
      accumulate(v, s0, acc);
    }
    store(d0, acc);
  }
  if (lane == 0 && p.out_lse) p.out_lse[row] = M == -INFINITY ? -INFINITY : M + __logf(L);
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  // whole 16-byte loads per lane: d_v a multiple of 8 (bf16 partials) or 4 (fp32)
  if (p.d_v % (p.part_bf16 ? 8 : 4) != 0) return hipErrorInvalidValue;
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
#define SA_DECODE_LAUNCH3(D_, P_, ST_, F8_)                                                             \
  do {                                                                                                  \
    if (tiered)                                                                                         \
      hipLaunchKernelGGL((decode_bf16_kernel<D_, P_, true, ST_, F8_>), grid, block, 0, s, p, p.lists,       \
                         p.block_table, p.seq_lens, p.counts);                                          \
    else                                                                                                \
      hipLaunchKernelGGL((decode_bf16_kernel<D_, P_, false, ST_, F8_>), grid, block, 0, s, p, p.lists,      \
                         p.block_table, p.seq_lens, p.counts);                                          \
  } while (0)
#define SA_DECODE_LAUNCH(D_, P_, ST_) SA_DECODE_LAUNCH3(D_, P_, ST_, false)
  if (p.fp8) {
    // FP8 pages: register operands (d 128)
    if (p.P == 16) SA_DECODE_LAUNCH3(128, 16, false, true);
    else SA_DECODE_LAUNCH3(128, 64, false, true);
    return hipGetLastError();
  }
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
#undef SA_DECODE_LAUNCH3
  return hipGetLastError();
}

}  // namespace sa
