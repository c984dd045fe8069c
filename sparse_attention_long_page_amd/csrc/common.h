// Internal definitions shared by the library's host layer and its gfx950
// kernels.  Not part of the public interface (include/sparse_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (native v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// Full-wave (64 lanes) reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48: the rows an MFMA 16x16 accumulator spreads over), by the gfx950 lane
// swap instructions instead of LDS round trips.  Swapping a value with itself
// leaves each lane holding its own and its partner's value (l^16, then l^32);
// the pairing and order of operations match a butterfly over xor 16 then
// xor 32, so the results are the same bits in all four lanes.
__device__ __forceinline__ float max_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle,
// offsets bounds-checked against the record count).
constexpr uint32_t kBufferRsrcWord3 = 0x00020000u;

// A shared-memory pointer as the LDS address-space pointer that the
// buffer-load-to-LDS builtins take.
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) void*)(const_cast<void*>(p));
}

// Raw buffer resource over [base, base + bytes): lanes whose offset falls past
// it read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferRsrcWord3);
}

// One wave-wide 16-byte-per-lane copy from global memory into LDS: lane l's
// 16 bytes at byte offset voff of the resource land at lds + 16 l.  A buffer
// instruction counts on the vector-memory counter only (the global-load form
// of the same copy also makes the compiler wait for every LDS read at once).
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, const void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(lds), 16, voff, 0, 0, 0);
}

// Number of valid tokens of logical page `lp` in a sequence of `len` tokens.
__device__ __forceinline__ int page_valid(int len, int lp, int P) {
  int r = len - lp * P;
  return r < 0 ? 0 : (r > P ? P : r);
}

// ---------------------------------------------------------------- launch params
// Pooled queries of more than kScoreInlineRows rows are summed by a kernel of
// their own in kQChunks row chunks (float64 partials) before scoring; fewer
// rows are summed inside the scoring kernel.
constexpr int kQChunks = 8;
constexpr int kScoreInlineRows = 32;

struct SummaryParams {
  const void* k_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* mu;
  int n_kv, P, d, max_pages, last_pages;
  const float* k_scale;      // FP8 pages: [n_phys][n_kv] scales (null otherwise)
};

struct ScoreParams {
  const void* q;             // [B][T][Hq][d]
  const float* mu;           // [n_phys][Hkv][d]
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* scores;             // [B][n_sel][max_pages]
  int B, T, Hq, Hkv, G, n_sel, d, P, max_pages;
  int per_q;                 // 1: PER_Q_HEAD
  int sink, window;          // forced pages: the first sink and the last window of a sequence
  int skip_forced;           // forced pages' mean rows are not read (their scores are unused)
  const void* k_pool;        // refresh: keys of the newest pages
  float* mu_out;             // refresh: the summary rows rewritten (same array as mu)
  int refresh;               // recompute each sequence's newest-page summary before scoring
};

struct SelectParams {
  const float* scores;       // [B][n_sel][stride]
  const int32_t* seq_lens;
  int32_t* lists;            // [B][n_sel][list_stride]
  int32_t* counts;           // [B][n_sel]
  int32_t* ccounts;          // [B][n_sel] or null
  int scores_stride, n_sel, P, list_stride;
  int sink, window, top_k, critical_k, tiered;
};

struct DecodeParams {
  const void* q;             // [B][T][Hq][d_qk]
  const void* k_pool;        // [n_phys][Hkv][P][d_qk]
  const void* v_pool;        // [n_phys][Hkv][d_v][P]  (null: latent)
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* lists;      // [B][n_sel][list_stride]
  const int32_t* counts;     // [B][n_sel]
  const int32_t* ccounts;    // [B][n_sel] or null
  const uint32_t* amask;     // [B][max_pages][mask_words] or null
  void* out;                 // [B][T][Hq][d_v]
  float* out_lse;            // [B][T][Hq] or null
  float* part_o;             // [B][T][Hq][splits][d_v], fp32 or (part_bf16) bf16
  float* part_lse;           // [B][T][Hq][splits]
  int part_bf16;             // split partials of o stored as bf16 (latent path)
  int B, T, Hq, Hkv, G, n_sel, per_q, list_stride, max_pages, mask_words;
  int P, d_qk, d_v, splits;
  float scale_log2;          // sm_scale * log2(e)
  int fp8;                   // K/V pools hold OCP E4M3 bytes with per-(page, KV head) scales
  const float* k_scale;      // [n_phys][Hkv] (fp8 only)
  const float* v_scale;
};

struct MergeParams {
  const float* part_o;       // fp32, or bf16 when part_bf16
  const float* part_lse;
  void* out;
  float* out_lse;
  int rows, splits, d_v, out_fp32, part_bf16;
};

struct UnionParams {
  const uint8_t* mask;       // [Hq][nqb][nkb]
  int32_t* table;            // [Hkv][nkb]
  int32_t* counts;           // [Hkv]
  int Hq, Hkv, G, nqb, nkb;
};

struct PrefillParams {
  const void* q;             // [q_len][Hq][d]
  const void* k_pool;
  const void* v_pool;
  const int32_t* bt_row;     // block_table row of the sequence
  const int32_t* seq_len;    // pointer to seq_lens[seq]
  const int32_t* table;      // [Hkv][nkb]
  const int32_t* counts;     // [Hkv]
  void* out;                 // [q_len][Hq][d]
  float* out_lse;            // [q_len][Hq] or null
  int q_len, q_start, Hq, Hkv, G, nkb, P;
  int n_qtiles;
  float scale_log2;
};

constexpr int kPrefillMaxBlocks = 4096;     // KV blocks of a prefill chunk (262144 tokens at pages of 64)

struct ValueSummaryParams {
  const void* v_pool;        // [n_phys][n_kv][d_v][P]
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* v_scale;      // FP8 pages: [n_phys][n_kv] (null otherwise)
  float* nu;                 // out [n_phys][n_kv][d_v]
  int n_kv, P, d_v, max_pages, last_pages;
};

struct MeanCorrParams {
  const void* q;             // [q_len][Hq][128] bf16
  const float* mu;           // mean keys [n_phys][Hkv][128]
  const float* nu;           // mean values [n_phys][Hkv][128]
  const int32_t* bt_row;
  const int32_t* seq_len;
  const int32_t* table;      // union tables [Hkv][nkb] and counts [Hkv]
  const int32_t* counts;
  void* out;                 // [q_len][Hq][128] bf16, read and rewritten
  float* out_lse;            // [q_len][Hq], read and rewritten
  // workspace (mean_correct_workspace): the skipped blocks of each KV head,
  // ascending, and their means packed as bf16 in 32-block chunks
  int32_t* skip;             // [Hkv][nkb]
  int32_t* n_skip;           // [Hkv]
  uint16_t* pk;              // [Hkv][nch * 32][128] mean keys
  uint16_t* pv;              // [Hkv][nch][128][32] mean values, dim-major, PV contraction order
  uint32_t* meta;            // [Hkv][nch][64]: log2(n_b) (float bits) x 32, last token position x 32
  int q_len, q_start, Hq, Hkv, G, nkb, P;
  int nch;                   // ceil(nkb / 32)
  int q_tile;                // queries per workgroup (set by the launcher)
  float scale_log2;
};

// Bytes of the mean-correction workspace for Hkv KV heads and nkb blocks;
// with `base` set, also points p's workspace arrays into it.
size_t mean_correct_workspace(int Hkv, int nkb, void* base, MeanCorrParams* p);

constexpr int kTuneMaxGrid = 16;      // alphas and head counts per search, each at most
constexpr int kTuneMaxPages = 4096;    // pages per sequence a search ranks
constexpr int kTuneMaxGroup = 128;     // query heads per KV head

struct MassParams {
  const void* q;             // [B][T][Hq][d] bf16
  const float* mu;           // [n_phys][Hkv][d]
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* est;                // workspace [B][T*Hq][stride]: page log-weights
  float* mass;               // out [B][Hq][max_pages]
  int B, T, Hq, Hkv, G, d, P, max_pages, stride;
  float sm_scale;
};

struct TuneParams {
  const float* mass;         // [B][Hq][max_pages]
  const float* scores;       // [B][Hkv][scores_stride]
  const int32_t* seq_lens;
  float* mall;               // workspace [B][Hkv][max_pages]: a page's mass over the group
  float* tsum;               // workspace [B][Hkv][max_pages][n_h]: its top-h head masses
  float* part;               // workspace [B*Hkv][chunks][n_a*n_h]: covered mass per 64-page chunk
  float* coverage;           // out [n_a][n_h]
  int32_t* choice;           // out [3]: alpha index, head-count index, beta
  int B, T, Hq, Hkv, G, P, max_pages, scores_stride, sink, window;
  int n_a, n_h;
  int alpha[kTuneMaxGrid], heads[kTuneMaxGrid];
  int beta[kTuneMaxGrid * kTuneMaxGrid];   // -1: infeasible
};

struct AmbientMaskParams {
  const float* mass;         // [B][Hq][max_pages]
  const int32_t* lists;      // [B][Hkv][list_stride]
  const int32_t* counts;     // [B][Hkv]
  const int32_t* ccounts;    // [B][Hkv]
  uint32_t* mask;            // out [B][max_pages][words]
  int B, Hq, Hkv, G, max_pages, list_stride, words, h;
};

// ------------------------------------------------------------- launchers
hipError_t launch_page_value_summary(const ValueSummaryParams& p, int batch, int elem_bytes, hipStream_t s);
hipError_t launch_mean_correct(const MeanCorrParams& p, hipStream_t s);
hipError_t launch_head_mass(const MassParams& p, hipStream_t s);
hipError_t launch_autotune(const TuneParams& p, hipStream_t s);
int autotune_chunks(int max_pages);
hipError_t launch_ambient_mask(const AmbientMaskParams& p, hipStream_t s);
hipError_t launch_page_summary(const SummaryParams& p, int batch, int bf16, hipStream_t s);
hipError_t launch_select(const SelectParams& p, int batch, int max_pages, hipStream_t s);
hipError_t launch_score_select(const ScoreParams& sp, const SelectParams& p, int batch, int bf16, hipStream_t s);
size_t select_decode_lds_bytes(int max_pages, int list_stride);
size_t select_decode_lds_limit();
hipError_t launch_select_decode(const ScoreParams& sp, const SelectParams& p, const DecodeParams& dp, int batch,
                                hipStream_t s);
hipError_t launch_select_prep(const SummaryParams& smp, const ScoreParams& sp, int bf16, bool refresh, double* qpart,
                              uint32_t* arrivals, hipStream_t s);
hipError_t launch_score_lastsel(const ScoreParams& sp, const SelectParams& p, int bf16, const double* qpart,
                                uint32_t* arrivals, hipStream_t s);
struct MaskParams {
  const void* q;             // [q_len][Hq][d]
  const float* mu;           // page summaries [n_phys][Hkv][d]
  const int32_t* bt_row;     // block_table row of the sequence
  const int32_t* seq_len;    // pointer to seq_lens[seq]
  uint8_t* mask;             // out [Hq][nqb][nkb]
  int q_len, q_start, Hq, Hkv, G, P, block_q, nqb, nkb, top_k;
  float sm_scale, max_gap;   // top_k < 0: keep candidates with score >= max - max_gap
};
size_t block_mask_lds_bytes(int G, int nkb);
hipError_t launch_block_mask(const MaskParams& mp, int bf16, int d, hipStream_t s);

// Device-side data checks (debug validation mode).  Violation codes:
constexpr uint32_t kValSeqLen = 1;         // seq_lens[b] outside [0, max_pages * page_size]
constexpr uint32_t kValBlockTable = 2;     // block_table[b][lp] outside [0, n_phys_pages)
constexpr uint32_t kValCount = 3;          // page_counts[b][s] outside [0, list_stride]
constexpr uint32_t kValListEntry = 4;      // page_lists[b][s][e] outside [0, n_pages(b))
constexpr uint32_t kValCriticalCount = 5;  // critical_counts[b][s] outside [0, page_counts[b][s]]
constexpr uint32_t kValScore = 6;          // a given score that is not finite

struct ValidateKV {
  const int32_t* block_table;  // null: only the lengths are checked
  const int32_t* seq_lens;
  int seq0, max_pages, P, n_phys;
};

struct ValidateLists {
  const int32_t* lists;
  const int32_t* counts;
  const int32_t* ccounts;    // or null
  const int32_t* seq_lens;
  int n_sel, stride, P;
};

struct ValidateScores {
  const float* scores;
  const int32_t* seq_lens;
  int n_sel, stride, P, max_pages;
};

hipError_t validate_result_ptr(uint32_t** ptr);
hipError_t launch_validate_clear(uint32_t* res, hipStream_t s);
hipError_t launch_validate_kv(const ValidateKV& v, int batch, uint32_t* res, hipStream_t s);
hipError_t launch_validate_lists(const ValidateLists& v, int batch, uint32_t* res, hipStream_t s);
hipError_t launch_validate_scores(const ValidateScores& v, int batch, uint32_t* res, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int bf16, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_mla_decode(const DecodeParams& p, hipStream_t s);
hipError_t launch_union(const UnionParams& p, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);

}  // namespace sa
