// Mean correction of a block-sparse chunked prefill, and the per-page mean
// value rows it needs (block-sparse prefill brief on the Paperraft page: a
// mean correction term beside pattern discovery and thresholding, bounding the
// error of the blocks left out).  Reading of the unstated formula: every
// causal block the group's union table skips that lies wholly at or before the
// query stands in for its n_b tokens by its mean key mu_b and mean value nu_b,
// i.e. one extra softmax term of log-weight sm_scale * q . mu_b + ln n_b and
// value nu_b.
//
// Three kernels:
//  * mean_skip_kernel (one workgroup per KV head g): the blocks of the
//    sequence that g's union table leaves out and that lie wholly at or
//    before the chunk's last query, ascending.  A query tile's blocks (those
//    wholly before its last position) are a prefix of this list.
//  * mean_pack_kernel (32-block chunk, g): their mean keys and values rounded
//    to bf16 and packed chunk by chunk in the order the MFMAs read them, with
//    log2(n_b) and the block's last token position.
//  * mean_correct_kernel: workgroup = (query tile, g) covering the tile's rows
//    of every query head of g (256 rows: 256/G queries x G heads), 32 rows per
//    wave as two 16-row MFMA tiles; the packed chunks stream through a double
//    buffer in LDS by buffer-to-LDS copies.  The prefill's (o, lse) of a row
//    is one term of log-weight lse and value o; each chunk adds 32 terms:
//    S^T = Mu Q^T and O^T += Nu^T P^T on v_mfma_f32_16x16x32_bf16 with an
//    online softmax per row.  The corrected (o, lse) overwrite the prefill's.
#include "common.h"

namespace sa {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ value means
// grid (KV head, page slot, batch), 256 threads.  A page's values of KV head
// g are d_v rows of P contiguous elements (page-transposed pool); a thread
// loads 16-byte vectors, vpr = P*elem/16 consecutive lanes cover one row and
// add their parts in float64 with xor shuffles.
template <typename T>
__device__ __forceinline__ double sum_vec16(const uint4 w, int first, int nv) {
  constexpr int per = 16 / (int)sizeof(T);
  double acc = 0.0;
  const uint32_t word[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int t = 0; t < per; ++t) {
    float x;
    if constexpr (sizeof(T) == 1) {
      const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                                          word[t / 4] >> (8 * (t % 4)), 1.0f, false));
      x = bf16_lo(b);
    } else if constexpr (sizeof(T) == 2) {
      x = (t & 1) ? bf16_hi(word[t / 2]) : bf16_lo(word[t / 2]);
    } else {
      x = __uint_as_float(word[t]);
    }
    acc += (first + t < nv) ? (double)x : 0.0;
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(256) void page_value_summary_kernel(ValueSummaryParams p) {
  const int g = blockIdx.x, b = blockIdx.z;
  const int len = p.seq_lens[b];
  const int n = (len + p.P - 1) / p.P;
  int lp = blockIdx.y;
  if (p.last_pages > 0) lp = n - p.last_pages + (int)blockIdx.y;
  if (lp < 0 || lp >= n) return;
  const int phys = p.block_table[(size_t)b * p.max_pages + lp];
  const int nv = page_valid(len, lp, p.P);
  constexpr int per = 16 / (int)sizeof(T);               // elements per vector
  const int vpr = p.P / per;                            // vectors per row: 1..16, divides 64
  const uint4* page = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(p.v_pool) +
                                                     ((size_t)phys * p.n_kv + g) * p.d_v * p.P);
  const double scale = sizeof(T) == 1 ? (double)p.v_scale[(size_t)phys * p.n_kv + g] : 1.0;
  float* dst = p.nu + ((size_t)phys * p.n_kv + g) * p.d_v;
  const int total = p.d_v * vpr;
  // four vectors per lane are loaded together, unconditionally from clamped
  // indices (a load under a per-lane condition is waited for at once); the
  // trip counts are uniform, so every lane takes part in the shuffles
  for (int v0 = 0; v0 < total; v0 += 4 * 256) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = page[min(v0 + 256 * u + (int)threadIdx.x, total - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (v0 + 256 * u >= total) break;
      const int v = v0 + 256 * u + threadIdx.x;
      double acc = v < total ? sum_vec16<T>(w[u], (v % vpr) * per, nv) : 0.0;
      for (int o = vpr >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (v < total && v % vpr == 0) dst[v / vpr] = (float)(acc * scale / (double)nv);
    }
  }
}

hipError_t launch_page_value_summary(const ValueSummaryParams& p, int batch, int elem_bytes, hipStream_t s) {
  const int slots = p.last_pages > 0 ? p.last_pages : p.max_pages;
  dim3 grid(p.n_kv, slots, batch);
  if (elem_bytes == 1) hipLaunchKernelGGL((page_value_summary_kernel<uint8_t>), grid, dim3(256), 0, s, p);
  else if (elem_bytes == 2) hipLaunchKernelGGL((page_value_summary_kernel<uint16_t>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((page_value_summary_kernel<float>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// -------------------------------------------------------- mean correction
constexpr int kMcD = 128;               // head dim
constexpr int kMcChunk = 32;            // skipped blocks per chunk
constexpr int kMcRows = 256;            // query rows (queries x heads) per workgroup, at most
constexpr int kMcMetaWords = 64;        // per chunk: 32 log2(n_b), 32 last positions

// Position of block jb of a chunk in the PV contraction: lane group kq holds
// S^T blocks 4kq..4kq+3 (tile 0) and 16+4kq..16+4kq+3 (tile 1) and feeds them
// as its contraction entries 8kq..8kq+7.
__device__ __forceinline__ int mc_pv_pos(int jb) { return 8 * ((jb & 15) >> 2) + 4 * (jb >> 4) + (jb & 3); }

size_t mean_correct_workspace(int Hkv, int nkb, void* base, MeanCorrParams* p) {
  const size_t nch = (size_t)(nkb + kMcChunk - 1) / kMcChunk;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t b_skip = al((size_t)Hkv * nkb * 4), b_cnt = al((size_t)Hkv * 4);
  const size_t b_pk = al((size_t)Hkv * nch * kMcChunk * kMcD * 2), b_pv = b_pk;
  const size_t b_meta = al((size_t)Hkv * nch * kMcMetaWords * 4);
  if (base && p) {
    char* c = static_cast<char*>(base);
    p->skip = reinterpret_cast<int32_t*>(c); c += b_skip;
    p->n_skip = reinterpret_cast<int32_t*>(c); c += b_cnt;
    p->pk = reinterpret_cast<uint16_t*>(c); c += b_pk;
    p->pv = reinterpret_cast<uint16_t*>(c); c += b_pv;
    p->meta = reinterpret_cast<uint32_t*>(c);
    p->nch = (int)nch;
  }
  return b_skip + b_cnt + b_pk + b_pv + b_meta;
}

// grid Hkv, 256 threads
__global__ __launch_bounds__(256) void mean_skip_kernel(MeanCorrParams p) {
  __shared__ uint8_t in_table[kPrefillMaxBlocks];
  const int g = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seq_len = *p.seq_len;
  const int n_seq = seq_len > 0 ? (seq_len + p.P - 1) / p.P : 0;
  const int n_blk = min(n_seq, p.nkb);
  const int last_pos = p.q_start + p.q_len - 1;
  for (int kb = threadIdx.x; kb < n_blk; kb += 256) in_table[kb] = 0;
  __syncthreads();
  const int cnt = p.counts[g];
  for (int t = threadIdx.x; t < cnt; t += 256) {
    const int kb = p.table[(size_t)g * p.nkb + t];
    if (kb >= 0 && kb < n_blk) in_table[kb] = 1;
  }
  __syncthreads();
  if (wave != 0) return;
  int base = 0;
  for (int kb0 = 0; kb0 < n_blk; kb0 += 64) {
    const int kb = kb0 + lane;
    bool take = false;
    if (kb < n_blk && !in_table[kb]) take = kb * p.P + page_valid(seq_len, kb, p.P) - 1 <= last_pos;
    const unsigned long long m = __ballot(take);
    const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (take) p.skip[(size_t)g * p.nkb + base + before] = kb;
    base += __popcll(m);
  }
  if (lane == 0) p.n_skip[g] = base;
}

// grid (nch, Hkv), 256 threads: chunk ch of KV head g.  Entries past the list
// get zero means, log2 weight 0 and last position INT_MAX (never visible).
__global__ __launch_bounds__(256) void mean_pack_kernel(MeanCorrParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kMcD * kMcChunk];    // [dim][PV position]
  const int ch = blockIdx.x, g = blockIdx.y;
  const int n = p.n_skip[g];
  if (ch * kMcChunk >= n) return;
  const int seq_len = *p.seq_len;
  uint16_t* pk = p.pk + ((size_t)g * p.nch * kMcChunk + (size_t)ch * kMcChunk) * kMcD;
  uint32_t* meta = p.meta + ((size_t)g * p.nch + ch) * kMcMetaWords;
  for (int idx = threadIdx.x; idx < kMcChunk * (kMcD / 4); idx += 256) {
    const int jb = idx / (kMcD / 4), e4 = idx % (kMcD / 4);
    const int c = ch * kMcChunk + jb;
    float4 kv = float4{0.f, 0.f, 0.f, 0.f}, vv = kv;
    int kb = 0;
    if (c < n) {
      kb = p.skip[(size_t)g * p.nkb + c];
      const size_t off = ((size_t)p.bt_row[kb] * p.Hkv + g) * kMcD + 4 * e4;
      kv = *reinterpret_cast<const float4*>(p.mu + off);
      vv = *reinterpret_cast<const float4*>(p.nu + off);
    }
    uint2 kw;
    kw.x = (uint32_t)f32_to_bf16_bits(kv.x) | ((uint32_t)f32_to_bf16_bits(kv.y) << 16);
    kw.y = (uint32_t)f32_to_bf16_bits(kv.z) | ((uint32_t)f32_to_bf16_bits(kv.w) << 16);
    *reinterpret_cast<uint2*>(pk + (size_t)jb * kMcD + 4 * e4) = kw;
    const int pp = mc_pv_pos(jb);
    vt[(4 * e4 + 0) * kMcChunk + pp] = f32_to_bf16_bits(vv.x);
    vt[(4 * e4 + 1) * kMcChunk + pp] = f32_to_bf16_bits(vv.y);
    vt[(4 * e4 + 2) * kMcChunk + pp] = f32_to_bf16_bits(vv.z);
    vt[(4 * e4 + 3) * kMcChunk + pp] = f32_to_bf16_bits(vv.w);
    if (e4 == 0) {
      const int nvb = c < n ? page_valid(seq_len, kb, p.P) : 0;
      meta[jb] = __float_as_uint(c < n ? __log2f((float)nvb) : 0.f);
      meta[32 + jb] = c < n ? (uint32_t)(kb * p.P + nvb - 1) : (uint32_t)INT_MAX;
    }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(p.pv + ((size_t)g * p.nch + ch) * kMcD * kMcChunk);
  const uint4* src = reinterpret_cast<const uint4*>(vt);
  for (int i = threadIdx.x; i < kMcD * kMcChunk / 8; i += 256) dst[i] = src[i];
}

// LDS layouts of a staged chunk (16-byte segments XOR-swizzled so that the
// MFMA operand reads of 16 lanes fall in distinct banks):
//   keys:   row jb (256 B), segment s at position s ^ (jb & 15)
//   values: row dim (64 B), segment s at position s ^ ((dim >> 2) & 3)
__device__ __forceinline__ int mc_k_seg(int row, int seg) { return row * 16 + (seg ^ (row & 15)); }
__device__ __forceinline__ int mc_v_seg(int row, int seg) { return row * 4 + (seg ^ ((row >> 2) & 3)); }

__global__ __launch_bounds__(512) void mean_correct_kernel(MeanCorrParams p) {
  // two chunk buffers as distinct arrays (the loop alternates them by name),
  // so the compiler sees that reads of one never wait for copies into the other
  __shared__ __attribute__((aligned(16))) uint16_t sk0[kMcChunk * kMcD], sk1[kMcChunk * kMcD];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[kMcD * kMcChunk], sv1[kMcD * kMcChunk];
  __shared__ __attribute__((aligned(16))) uint32_t sm0[256], sm1[256];   // one wave-wide copy: 1 KiB
  const int nwaves = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  // consecutive workgroups take consecutive KV heads, so with 8 KV heads each
  // XCD serves one head and its L2 holds that head's packed means
  const int g = blockIdx.x % p.Hkv;
  const int qt = p.q_tile;
  const int q0 = (blockIdx.x / p.Hkv) * qt;
  const int last_pos = p.q_start + min(q0 + qt, p.q_len) - 1;
  const int n = p.n_skip[g];
  if (n == 0) return;                                // nothing to correct: (o, lse) stand
  const int nch_g = (n + kMcChunk - 1) / kMcChunk;

  // this wave's two 16-row tiles; tile t holds queries qoff..qoff+15 of head hh
  const int tiles_per_head = qt / 16;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  uint16_t* op = reinterpret_cast<uint16_t*>(p.out);
  bool row_ok[2];
  int pos[2];
  size_t orow[2];
  int wave_min_pos = INT_MAX;                        // earliest position among the wave's tiles
  bf16x8 qreg[2][kMcD / 32];
  f32x4 oacc[2][kMcD / 16];
  float m[2], l[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int t = 2 * wave + rt;
    const int hh = t / tiles_per_head;
    const int qoff = (t % tiles_per_head) * 16;
    const int i = q0 + qoff + col;
    row_ok[rt] = hh < p.G && i < p.q_len;
    if (hh < p.G && q0 + qoff < p.q_len) wave_min_pos = min(wave_min_pos, p.q_start + q0 + qoff);
    pos[rt] = p.q_start + i;
    orow[rt] = row_ok[rt] ? (size_t)i * p.Hq + (size_t)g * p.G + hh : 0;
    // Q^T operand of k-step ks: dims 32*ks + 8*kq .. +7 of the row
#pragma unroll
    for (int ks = 0; ks < kMcD / 32; ++ks)
      qreg[rt][ks] = *reinterpret_cast<const bf16x8*>(qp + orow[rt] * kMcD + 32 * ks + 8 * kq);
    // the prefill's result as the first term: log-weight lse, value o.  O^T
    // accumulator of dim tile dt: dims 16*dt + 4*kq .. +3 of the row
    m[rt] = row_ok[rt] ? p.out_lse[orow[rt]] * kLog2e : -INFINITY;   // base 2
    l[rt] = m[rt] == -INFINITY ? 0.f : 1.f;
#pragma unroll
    for (int dt = 0; dt < kMcD / 16; ++dt) {
      const uint2 w = *reinterpret_cast<const uint2*>(op + orow[rt] * kMcD + 16 * dt + 4 * kq);
      const bool keep = l[rt] > 0.f;
      oacc[rt][dt] = f32x4{keep ? bf16_lo(w.x) : 0.f, keep ? bf16_hi(w.x) : 0.f, keep ? bf16_lo(w.y) : 0.f,
                           keep ? bf16_hi(w.y) : 0.f};
    }
  }

  // chunk copies: 8 wave-wide copies of keys, 8 of values, 1 of metadata
  const size_t chunk_elems = (size_t)kMcChunk * kMcD;
  const auto rk = buffer_rsrc(p.pk + (size_t)g * p.nch * chunk_elems, (uint32_t)(p.nch * chunk_elems * 2));
  const auto rv = buffer_rsrc(p.pv + (size_t)g * p.nch * chunk_elems, (uint32_t)(p.nch * chunk_elems * 2));
  const auto rm = buffer_rsrc(p.meta + (size_t)g * p.nch * kMcMetaWords, (uint32_t)(p.nch * kMcMetaWords * 4));
  auto stage = [&](uint16_t* skd, uint16_t* svd, uint32_t* smd, int ch) __attribute__((always_inline)) {
    for (int i = wave; i < 17; i += nwaves) {
      const int s = 64 * (i & 7) + lane;             // destination segment of this lane
      if (i < 8) {
        const int row = s >> 4, seg = (s & 15) ^ (row & 15);
        copy16_to_lds(rk, skd + 64 * 8 * i, (uint32_t)(((size_t)ch * chunk_elems + row * kMcD + seg * 8) * 2));
      } else if (i < 16) {
        const int row = s >> 2, seg = (s & 3) ^ ((row >> 2) & 3);
        copy16_to_lds(rv, svd + 64 * 8 * (i - 8),
                      (uint32_t)(((size_t)ch * chunk_elems + row * kMcChunk + seg * 8) * 2));
      } else {
        copy16_to_lds(rm, smd, (uint32_t)((ch * kMcMetaWords + 4 * lane) * 4));
      }
    }
  };

  bool any[2] = {false, false};
  // one chunk from (skb, svb, smb) while the next is copied into (skn, svn,
  // smn); false once the list has passed the tile
  auto step = [&](const uint16_t* skb, const uint16_t* svb, const uint32_t* smb, uint16_t* skn, uint16_t* svn,
                  uint32_t* smn, int ch) __attribute__((always_inline)) -> bool {
    // the list is ascending: stop at the first chunk that starts past the tile
    if ((int)smb[32] > last_pos) return false;
    if (ch + 1 < nch_g) stage(skn, svn, smn, ch + 1);   // in flight over this chunk's products

    const float* lg = reinterpret_cast<const float*>(smb);
    const int* bend = reinterpret_cast<const int*>(smb + 32);
    // every term of the chunk visible to every row of the wave
    const bool full = bend[kMcChunk - 1] <= wave_min_pos;
    // S^T[block][row] for the chunk's two 16-block tiles: lane holds blocks
    // 16*st + 4*kq .. +3 of row col
    f32x4 s[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int st = 0; st < 2; ++st) s[rt][st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ks = 0; ks < kMcD / 32; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(skb + 8 * mc_k_seg(16 * st + col, 4 * ks + kq));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          s[rt][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rt][ks], s[rt][st], 0, 0, 0);
      }
    const float4 lg0 = *reinterpret_cast<const float4*>(&lg[4 * kq]);
    const float4 lg1 = *reinterpret_cast<const float4*>(&lg[16 + 4 * kq]);
    const float lgv[8] = {lg0.x, lg0.y, lg0.z, lg0.w, lg1.x, lg1.y, lg1.z, lg1.w};
    bf16x8 pb[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      // log-weights (base 2): scale * s + log2(n_b); terms not wholly at or
      // before this row's position take no part
      float z[8], zmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 8; ++t) z[t] = s[rt][t >> 2][t & 3] * p.scale_log2 + lgv[t];
      if (!full) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int jb = 16 * (t >> 2) + 4 * kq + (t & 3);
          const bool vis = (bend[jb] <= pos[rt]) & row_ok[rt];
          z[t] = vis ? z[t] : -INFINITY;
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) zmax = fmaxf(zmax, z[t]);
      zmax = max_over_row_groups(zmax);
      any[rt] |= zmax != -INFINITY;
      // the running maximum moves only for rows where a term exceeds it; the
      // rescale is skipped when no row of the wave moves (the common case once
      // the prefill's own term leads)
      const bool grow = zmax > m[rt];
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m[rt] - zmax) : 1.f;
        if (grow) m[rt] = zmax;
        l[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kMcD / 16; ++dt) {
          oacc[rt][dt][0] *= alpha; oacc[rt][dt][1] *= alpha;
          oacc[rt][dt][2] *= alpha; oacc[rt][dt][3] *= alpha;
        }
      }
      const float msub = m[rt] == -INFINITY ? 0.f : m[rt];
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float pv = __builtin_amdgcn_exp2f(z[t] - msub);
        psum += pv;
        pb[rt][t] = (__bf16)pv;
      }
      l[rt] += sum_over_row_groups(psum);
    }
    // O^T[dim][row] += Nu^T[dim][block] P^T[block][row]
#pragma unroll
    for (int dt = 0; dt < kMcD / 16; ++dt) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(svb + 8 * mc_v_seg(16 * dt + col, kq));
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        oacc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], oacc[rt][dt], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                                 // next chunk staged; this one's reads done
    return true;
  };
  stage(sk0, sv0, sm0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int ch = 0; ch < nch_g; ch += 2) {
    if (!step(sk0, sv0, sm0, sk1, sv1, sm1, ch)) break;
    if (ch + 1 >= nch_g || !step(sk1, sv1, sm1, sk0, sv0, sm0, ch + 1)) break;
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    if (!row_ok[rt] || !any[rt]) continue;          // no mean term: (o, lse) stand as they are
    const float inv = l[rt] > 0.f ? 1.f / l[rt] : 0.f;
#pragma unroll
    for (int dt = 0; dt < kMcD / 16; ++dt) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16_bits(oacc[rt][dt][0] * inv) |
            ((uint32_t)f32_to_bf16_bits(oacc[rt][dt][1] * inv) << 16);
      w.y = (uint32_t)f32_to_bf16_bits(oacc[rt][dt][2] * inv) |
            ((uint32_t)f32_to_bf16_bits(oacc[rt][dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + orow[rt] * kMcD + 16 * dt + 4 * kq) = w;
    }
    if (kq == 0) p.out_lse[orow[rt]] = m[rt] == -INFINITY ? -INFINITY : (m[rt] + __log2f(l[rt])) * kLn2;
  }
}

// Query tile of a workgroup: 256/G queries rounded down to a multiple of 16
// (G <= 8, so at least 32), i.e. G*qt <= 256 rows over ceil(G*qt/32) waves.
static int mean_correct_q_tile(int G) { return (kMcRows / G) / 16 * 16; }

hipError_t launch_mean_correct(const MeanCorrParams& p_in, hipStream_t s) {
  MeanCorrParams p = p_in;
  if (p.G < 1 || p.G > 8 || p.nch != (p.nkb + kMcChunk - 1) / kMcChunk) return hipErrorInvalidValue;
  p.q_tile = mean_correct_q_tile(p.G);
  const int waves = (p.G * p.q_tile + 31) / 32;
  hipLaunchKernelGGL(mean_skip_kernel, dim3(p.Hkv), dim3(256), 0, s, p);
  hipLaunchKernelGGL(mean_pack_kernel, dim3(p.nch, p.Hkv), dim3(256), 0, s, p);
  dim3 grid((p.q_len + p.q_tile - 1) / p.q_tile * p.Hkv);
  hipLaunchKernelGGL(mean_correct_kernel, grid, dim3(64 * waves), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
