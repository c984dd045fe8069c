// Host side of the C ABI declared in include/sparse_attn.h: argument
// validation (before anything is launched), workspace sizing, launch-shape
// choice and dispatch to the gfx950 kernels.  Allocates no device memory and
// keeps no device state beyond a cached compute-unit count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/sparse_attn.h"
#include "common.h"

namespace {

thread_local std::string g_last_error;

sa_status fail(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sa_status ok() {
  g_last_error.clear();
  return SA_OK;
}

sa_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int device_cu_count() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached_dev = dev;
    cached_cus = cus;
  }
  return cached_cus;
}

bool is_latent(const sa_paged_kv* kv) { return kv->v_pool == nullptr; }

// Shape checks shared by every call.  `need_pools`: k_pool/v_pool must be set.
sa_status check_kv(const sa_paged_kv* kv, bool need_pools) {
  if (!kv) return fail(SA_ERR_INVALID_ARGUMENT, "kv is NULL");
  if (!kv->block_table || !kv->seq_lens) return fail(SA_ERR_INVALID_ARGUMENT, "block_table/seq_lens NULL");
  if (need_pools && !kv->k_pool) return fail(SA_ERR_INVALID_ARGUMENT, "k_pool is NULL");
  if (kv->n_phys_pages <= 0 || kv->n_kv_heads <= 0 || kv->max_pages <= 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_phys_pages/n_kv_heads/max_pages must be positive");
  if (kv->dtype != SA_DTYPE_BF16 && kv->dtype != SA_DTYPE_FP32 && kv->dtype != SA_DTYPE_FP8_E4M3)
    return fail(SA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)kv->dtype);
  if (kv->dtype == SA_DTYPE_FP8_E4M3) {
    if (!kv->v_pool || kv->d_qk != 128 || kv->d_v != 128)
      return fail(SA_ERR_UNSUPPORTED, "FP8 pages need a V pool and d_qk == d_v == 128");
    if (!kv->k_scale || !kv->v_scale) return fail(SA_ERR_INVALID_ARGUMENT, "FP8 pages need k_scale and v_scale");
  }
  if (kv->page_size != 16 && kv->page_size != 64)
    return fail(SA_ERR_UNSUPPORTED, "page_size %d unsupported (16 or 64)", kv->page_size);
  const bool latent = kv->v_pool == nullptr;
  if (latent) {
    if (!(kv->d_qk == 576 && kv->d_v == 512))
      return fail(SA_ERR_UNSUPPORTED, "a latent cache (v_pool NULL) needs d_qk 576 / d_v 512, got %d/%d",
                  kv->d_qk, kv->d_v);
    if (kv->dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "latent cache must be bf16");
  } else {
    if (!((kv->d_qk == 64 && kv->d_v == 64) || (kv->d_qk == 128 && kv->d_v == 128)))
      return fail(SA_ERR_UNSUPPORTED, "(d_qk, d_v) = (%d, %d) unsupported with a V pool", kv->d_qk, kv->d_v);
  }
  return SA_OK;
}

int n_sel_of(const sa_paged_kv* kv, int n_q_heads, sa_sel_mode mode) {
  return mode == SA_SEL_PER_KV_HEAD ? kv->n_kv_heads : n_q_heads;
}

// Splits per selection head for the decode kernels.
int choose_splits(const sa_paged_kv* kv, int batch, int n_sel, int list_stride, int q_tokens, int n_q_heads) {
  int units = std::max(1, batch * n_sel);
  if (is_latent(kv)) units = batch * ((n_q_heads * q_tokens + 127) / 128);
  const int cus = device_cu_count();
  if (is_latent(kv)) {
    // latent path: units are (sequence, group of 128 query rows); one
    // workgroup per CU, at least 2 pages per split
    const int target = cus;
    int s = (target + units - 1) / units;
    s = std::min(s, std::max(1, list_stride / 2));
    return std::max(1, std::min(s, 64));
  }
  // The decode kernel is bound by its K/V loads once every CU holds one
  // workgroup (4 waves, 32 KiB of loads in flight each); more splits then
  // only add partials and the merge.
  const int per_chunk = 64 / kv->page_size;
  const int chunks = (list_stride + per_chunk - 1) / per_chunk;
  const int target = cus;
  int s = (target + units - 1) / units;
  s = std::min(s, std::max(1, chunks / 4));  // at least one chunk per wave
  return std::max(1, std::min(s, 64));
}

// Split partials of o: bf16 for a latent cache (512-wide rows for 128+ heads
// make fp32 partials the largest traffic of that path), fp32 otherwise.
size_t partial_elem_bytes(const sa_paged_kv* kv) { return is_latent(kv) ? 2 : sizeof(float); }

size_t decode_partials_bytes(const sa_paged_kv* kv, int batch, int q_tokens, int n_q_heads, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)batch * q_tokens * n_q_heads;
  return align_up(rows * splits * kv->d_v * partial_elem_bytes(kv)) + align_up(rows * splits * sizeof(float));
}

// Debug validation: off unless SA_DEBUG_VALIDATE is set in the environment
// (to anything but "0") or sa_set_debug_validate(1) was called.
std::atomic<int> g_validate{-1};   // -1: environment not read yet

bool validate_on() {
  int v = g_validate.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* env = std::getenv("SA_DEBUG_VALIDATE");
    int want = (env && *env && std::strcmp(env, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_validate.compare_exchange_strong(expected, want);
    v = g_validate.load(std::memory_order_relaxed);
  }
  return v != 0;
}

// Runs the device checks of one call on its stream, then waits for them and
// turns the first violation into SA_ERR_DATA.  Nothing else is enqueued in
// between, so a call that fails here launches none of its own kernels.
struct Validator {
  hipStream_t stream;
  uint32_t* res = nullptr;
  hipError_t err = hipSuccess;

  explicit Validator(hipStream_t s) : stream(s) {
    err = sa::validate_result_ptr(&res);
    if (err == hipSuccess) err = sa::launch_validate_clear(res, stream);
  }
  void kv(const sa_paged_kv* kv, int seq0, int batch, bool block_table = true) {
    if (err != hipSuccess) return;
    sa::ValidateKV v{block_table ? kv->block_table : nullptr, kv->seq_lens, seq0, kv->max_pages, kv->page_size,
                     kv->n_phys_pages};
    err = sa::launch_validate_kv(v, batch, res, stream);
  }
  void lists(const sa_paged_kv* kv, int batch, int n_sel, const int32_t* lists, const int32_t* counts,
             const int32_t* ccounts, int stride) {
    if (err != hipSuccess) return;
    sa::ValidateLists v{lists, counts, ccounts, kv->seq_lens, n_sel, stride, kv->page_size};
    err = sa::launch_validate_lists(v, batch, res, stream);
  }
  void scores(const sa_paged_kv* kv, int batch, int n_sel, const float* scores, int stride) {
    if (err != hipSuccess) return;
    sa::ValidateScores v{scores, kv->seq_lens, n_sel, stride, kv->page_size, kv->max_pages};
    err = sa::launch_validate_scores(v, batch, res, stream);
  }
  sa_status finish(const sa_paged_kv* kv, int list_stride) {
    uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (err == hipSuccess) err = hipMemcpyAsync(h, res, sizeof(h), hipMemcpyDeviceToHost, stream);
    if (err == hipSuccess) err = hipStreamSynchronize(stream);
    if (err != hipSuccess) return device_status(err, "debug validation");
    const int v = (int)h[4];
    switch (h[0]) {
      case 0: return SA_OK;
      case sa::kValSeqLen:
        return fail(SA_ERR_DATA, "seq_lens[%u] = %d outside [0, max_pages * page_size = %ld]", h[1], v,
                    (long)kv->max_pages * kv->page_size);
      case sa::kValBlockTable:
        return fail(SA_ERR_DATA, "block_table[%u][%u] = %d outside [0, n_phys_pages = %d)", h[1], h[2], v,
                    kv->n_phys_pages);
      case sa::kValCount:
        return fail(SA_ERR_DATA, "page_counts[%u][%u] = %d outside [0, list_stride = %d]", h[1], h[2], v,
                    list_stride);
      case sa::kValListEntry:
        return fail(SA_ERR_DATA, "page_lists[%u][%u][%u] = %d is not a page of sequence %u", h[1], h[2], h[3], v,
                    h[1]);
      case sa::kValCriticalCount:
        return fail(SA_ERR_DATA, "critical_counts[%u][%u] = %d outside [0, page_counts[%u][%u]]", h[1], h[2], v,
                    h[1], h[2]);
      case sa::kValScore: {
        float x;
        std::memcpy(&x, &h[4], sizeof(x));
        return fail(SA_ERR_DATA, "scores[%u][%u][%u] = %g is not finite", h[1], h[2], h[3], (double)x);
      }
    }
    return fail(SA_ERR_DATA, "debug validation reported code %u", h[0]);
  }
};

}  // namespace

extern "C" {

int sa_set_debug_validate(int on) {
  const int prev = validate_on() ? 1 : 0;
  g_validate.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARGUMENT: return "SA_ERR_INVALID_ARGUMENT";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE_TOO_SMALL: return "SA_ERR_WORKSPACE_TOO_SMALL";
    case SA_ERR_DEVICE: return "SA_ERR_DEVICE";
    case SA_ERR_DATA: return "SA_ERR_DATA";
  }
  return "SA_ERR_UNKNOWN";
}

const char* sa_last_error_message(void) { return g_last_error.c_str(); }

int sa_version(void) { return 100; }   // 0.1.0

// --------------------------------------------------------- prefill block mask
sa_status sa_prefill_block_mask(const sa_paged_kv* kv, int32_t seq, const void* q, int32_t q_len, int32_t q_start,
                                int32_t n_q_heads, const float* page_summary, int32_t block_q, int32_t n_kv_blocks,
                                float sm_scale, int32_t top_k, float max_gap, uint8_t* block_mask_out,
                                hipStream_t stream) {
  sa_status st = check_kv(kv, false);
  if (st != SA_OK) return st;
  if (is_latent(kv)) return fail(SA_ERR_UNSUPPORTED, "the block mask needs a V-pool cache (d 64 or 128)");
  if (seq < 0) return fail(SA_ERR_INVALID_ARGUMENT, "seq must be >= 0");
  if (!q || !page_summary || !block_mask_out)
    return fail(SA_ERR_INVALID_ARGUMENT, "q, page_summary and block_mask_out must be set");
  if (q_len <= 0 || q_start < 0 || block_q <= 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "q_len and block_q must be positive, q_start >= 0");
  if (n_q_heads <= 0 || n_q_heads % kv->n_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / kv->n_kv_heads;
  if (G > 8) return fail(SA_ERR_UNSUPPORTED, "the block mask supports up to 8 query heads per KV head");
  const long need_blocks = ((long)q_start + q_len + kv->page_size - 1) / kv->page_size;
  if (n_kv_blocks < need_blocks || n_kv_blocks > kv->max_pages)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_kv_blocks %d must cover q_start+q_len (%ld) and be <= max_pages %d",
                n_kv_blocks, need_blocks, kv->max_pages);
  if (sa::block_mask_lds_bytes(G, n_kv_blocks) > 144 * 1024)
    return fail(SA_ERR_UNSUPPORTED, "%d heads per KV head x %d KV blocks of scores exceed the LDS budget", G,
                n_kv_blocks);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  if (top_k < 0 && !(max_gap >= 0.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "threshold mode (top_k < 0) needs max_gap >= 0 (+inf allowed)");
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, seq, 1);
    st = v.finish(kv, 0);
    if (st != SA_OK) return st;
  }
  sa::MaskParams mp{};
  mp.q = q;
  mp.mu = page_summary;
  mp.bt_row = kv->block_table + (size_t)seq * kv->max_pages;
  mp.seq_len = kv->seq_lens + seq;
  mp.mask = block_mask_out;
  mp.q_len = q_len;
  mp.q_start = q_start;
  mp.Hq = n_q_heads;
  mp.Hkv = kv->n_kv_heads;
  mp.G = G;
  mp.P = kv->page_size;
  mp.block_q = block_q;
  mp.nqb = (q_len + block_q - 1) / block_q;
  mp.nkb = n_kv_blocks;
  mp.top_k = top_k < 0 ? -1 : top_k;
  mp.sm_scale = sm_scale;
  mp.max_gap = top_k < 0 ? max_gap : 0.f;
  return device_status(sa::launch_block_mask(mp, kv->dtype != SA_DTYPE_FP32, kv->d_qk, stream), "block mask launch");
}

// ------------------------------------------------------------------ summary
sa_status sa_page_summary(const sa_paged_kv* kv, int32_t batch, int32_t last_pages, float* page_summary,
                          hipStream_t stream) {
  sa_status st = check_kv(kv, true);
  if (st != SA_OK) return st;
  if (batch <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "batch must be positive");
  if (last_pages < 0) return fail(SA_ERR_INVALID_ARGUMENT, "last_pages must be >= 0");
  if (!page_summary) return fail(SA_ERR_INVALID_ARGUMENT, "page_summary is NULL");
  sa::SummaryParams p{};
  p.k_pool = kv->k_pool;
  p.block_table = kv->block_table;
  p.seq_lens = kv->seq_lens;
  p.mu = page_summary;
  p.n_kv = kv->n_kv_heads;
  p.P = kv->page_size;
  p.d = kv->d_qk;
  p.max_pages = kv->max_pages;
  p.last_pages = std::min(last_pages, kv->max_pages);
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, 0, batch);
    st = v.finish(kv, 0);
    if (st != SA_OK) return st;
  }
  p.k_scale = kv->dtype == SA_DTYPE_FP8_E4M3 ? kv->k_scale : nullptr;
  return device_status(sa::launch_page_summary(p, batch, kv->dtype == SA_DTYPE_BF16, stream), "page_summary launch");
}

// ------------------------------------------------------------ value summary
sa_status sa_page_value_summary(const sa_paged_kv* kv, int32_t batch, int32_t last_pages, float* value_summary,
                                hipStream_t stream) {
  sa_status st = check_kv(kv, true);
  if (st != SA_OK) return st;
  if (is_latent(kv)) return fail(SA_ERR_UNSUPPORTED, "value summaries need a V pool");
  if (batch <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "batch must be positive");
  if (last_pages < 0) return fail(SA_ERR_INVALID_ARGUMENT, "last_pages must be >= 0");
  if (!value_summary) return fail(SA_ERR_INVALID_ARGUMENT, "value_summary is NULL");
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, 0, batch);
    st = v.finish(kv, 0);
    if (st != SA_OK) return st;
  }
  sa::ValueSummaryParams p{};
  p.v_pool = kv->v_pool;
  p.block_table = kv->block_table;
  p.seq_lens = kv->seq_lens;
  p.v_scale = kv->dtype == SA_DTYPE_FP8_E4M3 ? kv->v_scale : nullptr;
  p.nu = value_summary;
  p.n_kv = kv->n_kv_heads;
  p.P = kv->page_size;
  p.d_v = kv->d_v;
  p.max_pages = kv->max_pages;
  p.last_pages = std::min(last_pages, kv->max_pages);
  const int eb = kv->dtype == SA_DTYPE_FP8_E4M3 ? 1 : kv->dtype == SA_DTYPE_BF16 ? 2 : 4;
  return device_status(sa::launch_page_value_summary(p, batch, eb, stream), "value summary launch");
}

// ------------------------------------------------------------------- select
size_t sa_select_pages_workspace_size(int32_t batch, int32_t n_sel, int32_t max_pages) {
  if (batch <= 0 || n_sel <= 0 || max_pages <= 0) return 0;
  // router scores + float64 pooled-query partials (8 row chunks, d_qk <= 576)
  // + one arrival counter per list
  return align_up((size_t)batch * n_sel * max_pages * sizeof(float)) +
         align_up((size_t)batch * n_sel * 8 * 576 * sizeof(double)) + align_up((size_t)batch * n_sel * sizeof(uint32_t));
}

sa_status sa_select_pages(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                          int32_t n_q_heads, float* page_summary, int32_t refresh_newest_page, const float* scores,
                          int32_t scores_stride, sa_sel_mode mode, int32_t sink_pages, int32_t window_pages,
                          int32_t top_k, int32_t critical_k, int32_t* page_lists, int32_t list_stride,
                          int32_t* page_counts, int32_t* critical_counts, float* scores_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  sa_status st = check_kv(kv, false);
  if (st != SA_OK) return st;
  if (batch <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "batch must be positive");
  if (mode != SA_SEL_PER_KV_HEAD && mode != SA_SEL_PER_Q_HEAD)
    return fail(SA_ERR_INVALID_ARGUMENT, "unknown selection mode %d", (int)mode);
  if (n_q_heads <= 0 || n_q_heads % kv->n_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                n_q_heads, kv->n_kv_heads);
  if (sink_pages < 0 || window_pages < 0 || top_k < 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "sink_pages, window_pages and top_k must be >= 0");
  if (critical_counts && critical_k < 0) return fail(SA_ERR_INVALID_ARGUMENT, "critical_k must be >= 0");
  if (!page_lists || !page_counts) return fail(SA_ERR_INVALID_ARGUMENT, "page_lists/page_counts NULL");
  if (kv->max_pages > 16384) return fail(SA_ERR_UNSUPPORTED, "max_pages %d > 16384", kv->max_pages);
  const long need_stride = std::min<long>(kv->max_pages, (long)sink_pages + window_pages + top_k);
  if (list_stride < need_stride)
    return fail(SA_ERR_INVALID_ARGUMENT, "list_stride %d < min(max_pages, sink+window+top_k) = %ld", list_stride,
                need_stride);
  const int n_sel = n_sel_of(kv, n_q_heads, mode);
  if (refresh_newest_page && kv->dtype == SA_DTYPE_FP8_E4M3)
    return fail(SA_ERR_UNSUPPORTED, "refresh_newest_page is not supported for FP8 pages (use sa_page_summary)");
  if (refresh_newest_page && (scores || !page_summary))
    return fail(SA_ERR_INVALID_ARGUMENT, "refresh_newest_page needs page_summary and router scores (no scores)");
  if (scores) {
    if (scores_stride < kv->max_pages)
      return fail(SA_ERR_INVALID_ARGUMENT, "scores_stride %d < max_pages %d", scores_stride, kv->max_pages);
  } else {
    if (!q || !page_summary) return fail(SA_ERR_INVALID_ARGUMENT, "q and page_summary needed without scores");
    if (q_tokens <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "q_tokens must be positive");
    const size_t need = sa_select_pages_workspace_size(batch, n_sel, kv->max_pages);
    if (workspace_bytes < need || (!workspace && need))
      return fail(SA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  }

  sa::SelectParams sp{};
  sp.seq_lens = kv->seq_lens;
  sp.lists = page_lists;
  sp.counts = page_counts;
  sp.ccounts = critical_counts;
  sp.n_sel = n_sel;
  sp.P = kv->page_size;
  sp.list_stride = list_stride;
  sp.sink = sink_pages;
  sp.window = window_pages;
  sp.top_k = top_k;
  sp.critical_k = critical_k;
  sp.tiered = critical_counts != nullptr;

  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, 0, batch, scores == nullptr);   // given scores: the block table is not read
    if (scores) v.scores(kv, batch, n_sel, scores, scores_stride);
    st = v.finish(kv, list_stride);
    if (st != SA_OK) return st;
  }

  const int pooled_rows = mode == SA_SEL_PER_KV_HEAD ? q_tokens * (n_q_heads / kv->n_kv_heads) : q_tokens;
  if (!scores && batch * n_sel >= 128 && pooled_rows <= sa::kScoreInlineRows) {
    // enough lists to fill the GPU: score and select in one workgroup per list
    sa::ScoreParams p{};
    p.q = q;
    p.mu = page_summary;
    p.block_table = kv->block_table;
    p.seq_lens = kv->seq_lens;
    p.scores = scores_out;
    p.B = batch;
    p.T = q_tokens;
    p.Hq = n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.G = n_q_heads / kv->n_kv_heads;
    p.n_sel = n_sel;
    p.d = kv->d_qk;
    p.P = kv->page_size;
    p.max_pages = kv->max_pages;
    p.per_q = mode == SA_SEL_PER_Q_HEAD;
    p.refresh = refresh_newest_page ? 1 : 0;
    p.k_pool = kv->k_pool;
    p.mu_out = page_summary;
    return device_status(sa::launch_score_select(p, sp, batch, kv->dtype != SA_DTYPE_FP32, stream),
                         "score_select launch");
  }
  if (!scores) {
    // too few lists for one workgroup each: a prep kernel (pooled query,
    // newest-page summaries, arrival counters), then scoring over blocks of
    // pages whose last workgroup per list selects
    float* buf = scores_out ? scores_out : reinterpret_cast<float*>(workspace);
    char* ws = reinterpret_cast<char*>(workspace);
    const size_t sc_bytes = align_up((size_t)batch * n_sel * kv->max_pages * sizeof(float));
    double* qbar = reinterpret_cast<double*>(ws + sc_bytes);
    uint32_t* arrivals = reinterpret_cast<uint32_t*>(ws + sc_bytes + align_up((size_t)batch * n_sel * 8 * 576 * sizeof(double)));
    sa::ScoreParams p{};
    p.q = q;
    p.mu = page_summary;
    p.block_table = kv->block_table;
    p.seq_lens = kv->seq_lens;
    p.scores = buf;
    p.sink = sink_pages;
    p.window = window_pages;
    p.skip_forced = scores_out ? 0 : 1;
    p.B = batch;
    p.T = q_tokens;
    p.Hq = n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.G = n_q_heads / kv->n_kv_heads;
    p.n_sel = n_sel;
    p.d = kv->d_qk;
    p.P = kv->page_size;
    p.max_pages = kv->max_pages;
    p.per_q = mode == SA_SEL_PER_Q_HEAD;
    sa::SummaryParams smp{};
    smp.k_pool = kv->k_pool;
    smp.block_table = kv->block_table;
    smp.seq_lens = kv->seq_lens;
    smp.mu = page_summary;
    smp.n_kv = kv->n_kv_heads;
    smp.P = kv->page_size;
    smp.d = kv->d_qk;
    smp.max_pages = kv->max_pages;
    smp.last_pages = 1;
    const bool bf16 = kv->dtype != SA_DTYPE_FP32;   // the query's type (bf16 for FP8 pages)
    hipError_t e = sa::launch_select_prep(smp, p, bf16, refresh_newest_page != 0, qbar, arrivals, stream);
    if (e != hipSuccess) return device_status(e, "select prep launch");
    const bool pooled = pooled_rows > sa::kScoreInlineRows;
    return device_status(sa::launch_score_lastsel(p, sp, bf16, pooled ? qbar : nullptr, arrivals, stream),
                         "score/select launch");
  }
  sp.scores = scores;
  sp.scores_stride = scores_stride;
  return device_status(sa::launch_select(sp, batch, kv->max_pages, stream), "select launch");
}

// ------------------------------------------------------------------- decode
static sa_status check_decode_shape(const sa_paged_kv* kv, int32_t batch, int32_t q_tokens, int32_t n_q_heads,
                                    sa_sel_mode mode) {
  if (batch <= 0 || q_tokens <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "batch and q_tokens must be positive");
  if (mode != SA_SEL_PER_KV_HEAD && mode != SA_SEL_PER_Q_HEAD)
    return fail(SA_ERR_INVALID_ARGUMENT, "unknown selection mode %d", (int)mode);
  if (n_q_heads <= 0 || n_q_heads % kv->n_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                n_q_heads, kv->n_kv_heads);
  const int G = n_q_heads / kv->n_kv_heads;
  if (is_latent(kv)) {
    if (kv->n_kv_heads != 1) return fail(SA_ERR_UNSUPPORTED, "latent decode needs n_kv_heads == 1");
    if (mode != SA_SEL_PER_KV_HEAD) return fail(SA_ERR_UNSUPPORTED, "latent decode uses per-KV-head lists");
    if (16 % q_tokens != 0)
      return fail(SA_ERR_UNSUPPORTED, "latent decode needs q_tokens in {1, 2, 4, 8, 16}, got %d", q_tokens);
    if (kv->page_size != 64) return fail(SA_ERR_UNSUPPORTED, "latent decode needs page_size 64");
    if (n_q_heads > 256) return fail(SA_ERR_UNSUPPORTED, "latent decode supports up to 256 query heads");
  } else if (kv->dtype != SA_DTYPE_FP32) {
    const int rows = mode == SA_SEL_PER_KV_HEAD ? q_tokens * G : q_tokens;
    if (rows > 16)
      return fail(SA_ERR_UNSUPPORTED, "%d query rows share a KV head; the bf16 decode tile holds 16", rows);
  }
  return SA_OK;
}

size_t sa_sparse_decode_workspace_size(const sa_paged_kv* kv, int32_t batch, int32_t q_tokens, int32_t n_q_heads,
                                       int32_t list_stride, sa_sel_mode mode, int32_t num_splits) {
  if (!kv || batch <= 0 || q_tokens <= 0 || n_q_heads <= 0 || list_stride <= 0 || kv->n_kv_heads <= 0) return 0;
  const int n_sel = n_sel_of(kv, n_q_heads, mode);
  const int splits = num_splits > 0 ? num_splits : choose_splits(kv, batch, n_sel, list_stride, q_tokens, n_q_heads);
  return decode_partials_bytes(kv, batch, q_tokens, n_q_heads, splits);
}

// Host validation of a decode call; on success `splits` and the workspace
// bytes it needs are set.  Touches no device memory.
static sa_status decode_validate(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                                 int32_t n_q_heads, const int32_t* page_lists, const int32_t* page_counts,
                                 int32_t list_stride, sa_sel_mode mode, const int32_t* critical_counts,
                                 const uint32_t* ambient_head_mask, float sm_scale, int32_t num_splits, void* out,
                                 int* splits_out, size_t* need_out) {
  sa_status st = check_kv(kv, true);
  if (st != SA_OK) return st;
  st = check_decode_shape(kv, batch, q_tokens, n_q_heads, mode);
  if (st != SA_OK) return st;
  if (!q || !page_lists || !page_counts || !out)
    return fail(SA_ERR_INVALID_ARGUMENT, "q, page_lists, page_counts and out must be set");
  if (list_stride <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "list_stride must be positive");
  if ((critical_counts == nullptr) != (ambient_head_mask == nullptr))
    return fail(SA_ERR_INVALID_ARGUMENT, "critical_counts and ambient_head_mask go together");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  if (num_splits < 0 || num_splits > 64) return fail(SA_ERR_INVALID_ARGUMENT, "num_splits must be in 0..64");
  const int n_sel = n_sel_of(kv, n_q_heads, mode);
  const int splits = num_splits > 0 ? num_splits : choose_splits(kv, batch, n_sel, list_stride, q_tokens, n_q_heads);
  *splits_out = splits;
  *need_out = decode_partials_bytes(kv, batch, q_tokens, n_q_heads, splits);
  return SA_OK;
}

// Debug validation of a decode call's device data (lengths, block table,
// counts, list entries, critical counts).
static sa_status decode_check_device(const sa_paged_kv* kv, int32_t batch, int32_t n_q_heads, sa_sel_mode mode,
                                     const int32_t* page_lists, const int32_t* page_counts, int32_t list_stride,
                                     const int32_t* critical_counts, hipStream_t stream) {
  if (!validate_on()) return SA_OK;
  Validator v(stream);
  v.kv(kv, 0, batch);
  v.lists(kv, batch, n_sel_of(kv, n_q_heads, mode), page_lists, page_counts, critical_counts, list_stride);
  return v.finish(kv, list_stride);
}

// Launches of a validated decode call; `workspace` holds at least the bytes
// decode_validate reported.
static sa_status decode_launch(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                               int32_t n_q_heads, const int32_t* page_lists, const int32_t* page_counts,
                               int32_t list_stride, sa_sel_mode mode, const int32_t* critical_counts,
                               const uint32_t* ambient_head_mask, float sm_scale, int splits, void* out,
                               float* out_lse, void* workspace, hipStream_t stream) {
  sa::DecodeParams p{};
  p.q = q;
  p.k_pool = kv->k_pool;
  p.v_pool = kv->v_pool;
  p.block_table = kv->block_table;
  p.seq_lens = kv->seq_lens;
  p.lists = page_lists;
  p.counts = page_counts;
  p.ccounts = critical_counts;
  p.amask = ambient_head_mask;
  p.out = out;
  p.out_lse = out_lse;
  const size_t rows = (size_t)batch * q_tokens * n_q_heads;
  if (splits > 1) {
    p.part_o = reinterpret_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                          align_up(rows * splits * kv->d_v * partial_elem_bytes(kv)));
    p.part_bf16 = is_latent(kv) ? 1 : 0;
  }
  p.B = batch;
  p.T = q_tokens;
  p.Hq = n_q_heads;
  p.Hkv = kv->n_kv_heads;
  p.G = n_q_heads / kv->n_kv_heads;
  p.n_sel = n_sel_of(kv, n_q_heads, mode);
  p.per_q = mode == SA_SEL_PER_Q_HEAD;
  p.list_stride = list_stride;
  p.max_pages = kv->max_pages;
  p.mask_words = (n_q_heads + 31) / 32;
  p.P = kv->page_size;
  p.d_qk = kv->d_qk;
  p.d_v = kv->d_v;
  p.splits = splits;
  p.scale_log2 = sm_scale * sa::kLog2e;
  p.fp8 = kv->dtype == SA_DTYPE_FP8_E4M3 ? 1 : 0;
  p.k_scale = kv->k_scale;
  p.v_scale = kv->v_scale;
  hipError_t e = is_latent(kv) ? sa::launch_mla_decode(p, stream)
                               : sa::launch_decode(p, kv->dtype != SA_DTYPE_FP32, stream);
  if (e != hipSuccess) return device_status(e, "decode launch");
  if (splits > 1) {
    sa::MergeParams mp{};
    mp.part_o = p.part_o;
    mp.part_lse = p.part_lse;
    mp.out = out;
    mp.out_lse = out_lse;
    mp.rows = (int)rows;
    mp.splits = splits;
    mp.d_v = kv->d_v;
    mp.out_fp32 = kv->dtype == SA_DTYPE_FP32;
    mp.part_bf16 = p.part_bf16;
    e = sa::launch_merge(mp, stream);
    if (e != hipSuccess) return device_status(e, "merge launch");
  }
  return ok();
}

sa_status sa_sparse_decode(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                           int32_t n_q_heads, const int32_t* page_lists, const int32_t* page_counts,
                           int32_t list_stride, sa_sel_mode mode, const int32_t* critical_counts,
                           const uint32_t* ambient_head_mask, float sm_scale, int32_t num_splits, void* out,
                           float* out_lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int splits = 1;
  size_t need = 0;
  sa_status st = decode_validate(kv, batch, q, q_tokens, n_q_heads, page_lists, page_counts, list_stride, mode,
                                 critical_counts, ambient_head_mask, sm_scale, num_splits, out, &splits, &need);
  if (st != SA_OK) return st;
  if (workspace_bytes < need || (need && !workspace))
    return fail(SA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  st = decode_check_device(kv, batch, n_q_heads, mode, page_lists, page_counts, list_stride, critical_counts, stream);
  if (st != SA_OK) return st;
  return decode_launch(kv, batch, q, q_tokens, n_q_heads, page_lists, page_counts, list_stride, mode,
                       critical_counts, ambient_head_mask, sm_scale, splits, out, out_lse, workspace, stream);
}

// ------------------------------------------------- decode without allocation
// Split partials of sa_sparse_decode_noalloc live in this file-scope device
// array.  Its name is a host-side stand-in in host code: the device address of
// each GPU's copy comes from hipGetSymbolAddress (taken once per device, with
// that device current) and only that address is ever handed to a kernel.
__device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxScratchDevices = 256;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxScratchDevices];   // device address of `scratch`, per device

static sa_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(SA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
    if (!addr) return fail(SA_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = addr;
  }
  *ptr = g_scratch_dev[dev];
  return SA_OK;
}

sa_status sa_sparse_decode_noalloc(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                                   int32_t n_q_heads, const int32_t* page_lists, const int32_t* page_counts,
                                   int32_t list_stride, sa_sel_mode mode, const int32_t* critical_counts,
                                   const uint32_t* ambient_head_mask, float sm_scale, int32_t num_splits,
                                   void* out, float* out_lse, hipStream_t stream) {
  int splits = 1;
  size_t need = 0;
  sa_status st = decode_validate(kv, batch, q, q_tokens, n_q_heads, page_lists, page_counts, list_stride, mode,
                                 critical_counts, ambient_head_mask, sm_scale, num_splits, out, &splits, &need);
  if (st != SA_OK) return st;
  if (need > (size_t)SA_NOALLOC_SCRATCH_BYTES)
    return fail(SA_ERR_WORKSPACE_TOO_SMALL,
                "%d splits need %zu bytes of partials; the static scratch holds %zu (use fewer splits, or "
                "sa_sparse_decode with a workspace)", splits, need, (size_t)SA_NOALLOC_SCRATCH_BYTES);
  st = decode_check_device(kv, batch, n_q_heads, mode, page_lists, page_counts, list_stride, critical_counts, stream);
  if (st != SA_OK) return st;
  void* ws = nullptr;
  if (need) {
    st = scratch_for_current_device(&ws);
    if (st != SA_OK) return st;
  }
  return decode_launch(kv, batch, q, q_tokens, n_q_heads, page_lists, page_counts, list_stride, mode,
                       critical_counts, ambient_head_mask, sm_scale, splits, out, out_lse, ws, stream);
}

// ---------------------------------------------------------- select + decode
sa_status sa_select_decode(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                           int32_t n_q_heads, float* page_summary, int32_t refresh_newest_page, int32_t sink_pages,
                           int32_t window_pages, int32_t top_k, int32_t* page_lists, int32_t list_stride,
                           int32_t* page_counts, float sm_scale, void* out, float* out_lse, hipStream_t stream) {
  sa_status st = check_kv(kv, true);
  if (st != SA_OK) return st;
  st = check_decode_shape(kv, batch, q_tokens, n_q_heads, SA_SEL_PER_KV_HEAD);
  if (st != SA_OK) return st;
  if (kv->dtype != SA_DTYPE_BF16 || is_latent(kv) || kv->d_qk != 128 || kv->page_size != 64)
    return fail(SA_ERR_UNSUPPORTED, "select+decode needs bf16, a V pool, d 128 and page_size 64");
  if (q_tokens * (n_q_heads / kv->n_kv_heads) > sa::kScoreInlineRows)
    return fail(SA_ERR_UNSUPPORTED, "select+decode pools at most %d query rows", sa::kScoreInlineRows);
  if (!q || !page_summary || !page_lists || !page_counts || !out)
    return fail(SA_ERR_INVALID_ARGUMENT, "q, page_summary, page_lists, page_counts and out must be set");
  if (sink_pages < 0 || window_pages < 0 || top_k < 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "sink_pages, window_pages and top_k must be >= 0");
  const long need_stride = std::min<long>(kv->max_pages, (long)sink_pages + window_pages + top_k);
  if (list_stride < need_stride || list_stride <= 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "list_stride %d < min(max_pages, sink+window+top_k) = %ld", list_stride,
                need_stride);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  // the keys and the list sit in LDS beside the decode's 128 KiB of staging
  const size_t lds_max = sa::select_decode_lds_limit();
  if (sa::select_decode_lds_bytes(kv->max_pages, list_stride) > lds_max)
    return fail(SA_ERR_UNSUPPORTED, "select+decode holds max_pages + list_stride <= %zu entries in LDS",
                lds_max / sizeof(uint32_t));
  const int n_sel = kv->n_kv_heads;

  sa::ScoreParams sp{};
  sp.q = q;
  sp.mu = page_summary;
  sp.block_table = kv->block_table;
  sp.seq_lens = kv->seq_lens;
  sp.scores = nullptr;
  sp.B = batch;
  sp.T = q_tokens;
  sp.Hq = n_q_heads;
  sp.Hkv = kv->n_kv_heads;
  sp.G = n_q_heads / kv->n_kv_heads;
  sp.n_sel = n_sel;
  sp.d = kv->d_qk;
  sp.P = kv->page_size;
  sp.max_pages = kv->max_pages;
  sp.per_q = 0;
  sp.refresh = refresh_newest_page ? 1 : 0;
  sp.k_pool = kv->k_pool;
  sp.mu_out = page_summary;

  sa::SelectParams p{};
  p.seq_lens = kv->seq_lens;
  p.lists = page_lists;
  p.counts = page_counts;
  p.ccounts = nullptr;
  p.n_sel = n_sel;
  p.P = kv->page_size;
  p.list_stride = list_stride;
  p.sink = sink_pages;
  p.window = window_pages;
  p.top_k = top_k;
  p.critical_k = 0;
  p.tiered = 0;

  sa::DecodeParams dp{};
  dp.q = q;
  dp.k_pool = kv->k_pool;
  dp.v_pool = kv->v_pool;
  dp.block_table = kv->block_table;
  dp.seq_lens = kv->seq_lens;
  dp.lists = page_lists;
  dp.counts = page_counts;
  dp.out = out;
  dp.out_lse = out_lse;
  dp.B = batch;
  dp.T = q_tokens;
  dp.Hq = n_q_heads;
  dp.Hkv = kv->n_kv_heads;
  dp.G = n_q_heads / kv->n_kv_heads;
  dp.n_sel = n_sel;
  dp.per_q = 0;
  dp.list_stride = list_stride;
  dp.max_pages = kv->max_pages;
  dp.mask_words = (n_q_heads + 31) / 32;
  dp.P = kv->page_size;
  dp.d_qk = kv->d_qk;
  dp.d_v = kv->d_v;
  dp.splits = 1;
  dp.scale_log2 = sm_scale * sa::kLog2e;
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, 0, batch);
    st = v.finish(kv, list_stride);
    if (st != SA_OK) return st;
  }
  return device_status(sa::launch_select_decode(sp, p, dp, batch, stream), "select+decode launch");
}

// ------------------------------------------------------------------ prefill
size_t sa_block_sparse_prefill_workspace_size(const sa_paged_kv* kv, int32_t q_len, int32_t n_q_heads,
                                              int32_t n_kv_blocks) {
  (void)kv; (void)q_len; (void)n_q_heads; (void)n_kv_blocks;
  return 0;
}

sa_status sa_block_sparse_prefill(const sa_paged_kv* kv, int32_t seq, const void* q, int32_t q_len,
                                  int32_t q_start, int32_t n_q_heads, const uint8_t* block_mask, int32_t block_q,
                                  int32_t n_kv_blocks, int32_t* block_table_out, int32_t* block_counts_out,
                                  float sm_scale, void* out, float* out_lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  (void)workspace; (void)workspace_bytes;
  sa_status st = check_kv(kv, true);
  if (st != SA_OK) return st;
  if (kv->dtype != SA_DTYPE_BF16 || is_latent(kv) || kv->d_qk != 128 || kv->page_size != 64)
    return fail(SA_ERR_UNSUPPORTED, "prefill needs bf16, a V pool, d 128 and page_size 64");
  if (seq < 0) return fail(SA_ERR_INVALID_ARGUMENT, "seq must be >= 0");
  if (!q || !block_mask || !block_table_out || !block_counts_out || !out)
    return fail(SA_ERR_INVALID_ARGUMENT, "q, block_mask, block_table_out, block_counts_out and out must be set");
  if (q_len <= 0 || q_start < 0 || block_q <= 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "q_len and block_q must be positive, q_start >= 0");
  if (n_q_heads <= 0 || n_q_heads % kv->n_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_q_heads must be a positive multiple of n_kv_heads");
  const long need_blocks = ((long)q_start + q_len + kv->page_size - 1) / kv->page_size;
  if (n_kv_blocks > 4096)
    return fail(SA_ERR_UNSUPPORTED, "prefill supports up to 4096 KV blocks (got %d)", n_kv_blocks);
  if (n_kv_blocks < need_blocks || n_kv_blocks > kv->max_pages)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_kv_blocks %d must cover q_start+q_len (%ld) and be <= max_pages %d",
                n_kv_blocks, need_blocks, kv->max_pages);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  const int G = n_q_heads / kv->n_kv_heads;
  if (G > 8) return fail(SA_ERR_UNSUPPORTED, "prefill supports up to 8 query heads per KV head");

  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, seq, 1);
    st = v.finish(kv, 0);
    if (st != SA_OK) return st;
  }

  sa::UnionParams up{};
  up.mask = block_mask;
  up.table = block_table_out;
  up.counts = block_counts_out;
  up.Hq = n_q_heads;
  up.Hkv = kv->n_kv_heads;
  up.G = G;
  up.nqb = (q_len + block_q - 1) / block_q;
  up.nkb = n_kv_blocks;
  hipError_t e = sa::launch_union(up, stream);
  if (e != hipSuccess) return device_status(e, "union launch");

  sa::PrefillParams p{};
  p.q = q;
  p.k_pool = kv->k_pool;
  p.v_pool = kv->v_pool;
  p.bt_row = kv->block_table + (size_t)seq * kv->max_pages;
  p.seq_len = kv->seq_lens + seq;
  p.table = block_table_out;
  p.counts = block_counts_out;
  p.out = out;
  p.out_lse = out_lse;
  p.q_len = q_len;
  p.q_start = q_start;
  p.Hq = n_q_heads;
  p.Hkv = kv->n_kv_heads;
  p.G = G;
  p.nkb = n_kv_blocks;
  p.P = kv->page_size;
  p.scale_log2 = sm_scale * sa::kLog2e;
  e = sa::launch_prefill(p, stream);
  if (e != hipSuccess) return device_status(e, "prefill launch");
  return ok();
}

// -------------------------------------------------------- mean correction
size_t sa_prefill_mean_correction_workspace_size(const sa_paged_kv* kv, int32_t n_kv_blocks) {
  if (!kv || kv->n_kv_heads <= 0 || n_kv_blocks <= 0) return 0;
  return sa::mean_correct_workspace(kv->n_kv_heads, n_kv_blocks, nullptr, nullptr);
}

sa_status sa_prefill_mean_correction(const sa_paged_kv* kv, int32_t seq, const void* q, int32_t q_len,
                                     int32_t q_start, int32_t n_q_heads, const int32_t* block_table,
                                     const int32_t* block_counts, int32_t n_kv_blocks, const float* page_summary,
                                     const float* value_summary, float sm_scale, void* out, float* out_lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  sa_status st = check_kv(kv, false);
  if (st != SA_OK) return st;
  if (kv->dtype != SA_DTYPE_BF16 || is_latent(kv) || kv->d_qk != 128 || kv->page_size != 64)
    return fail(SA_ERR_UNSUPPORTED, "mean correction needs bf16, a V pool, d 128 and page_size 64");
  if (seq < 0) return fail(SA_ERR_INVALID_ARGUMENT, "seq must be >= 0");
  if (!q || !block_table || !block_counts || !page_summary || !value_summary || !out || !out_lse)
    return fail(SA_ERR_INVALID_ARGUMENT,
                "q, block_table, block_counts, page_summary, value_summary, out and out_lse must be set");
  if (q_len <= 0 || q_start < 0) return fail(SA_ERR_INVALID_ARGUMENT, "q_len must be positive, q_start >= 0");
  if (n_q_heads <= 0 || n_q_heads % kv->n_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_q_heads must be a positive multiple of n_kv_heads");
  const long need_blocks = ((long)q_start + q_len + kv->page_size - 1) / kv->page_size;
  if (n_kv_blocks > sa::kPrefillMaxBlocks)
    return fail(SA_ERR_UNSUPPORTED, "mean correction supports up to %d KV blocks (got %d)", sa::kPrefillMaxBlocks,
                n_kv_blocks);
  if (n_kv_blocks < need_blocks || n_kv_blocks > kv->max_pages)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_kv_blocks %d must cover q_start+q_len (%ld) and be <= max_pages %d",
                n_kv_blocks, need_blocks, kv->max_pages);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  if (n_q_heads / kv->n_kv_heads > 8)
    return fail(SA_ERR_UNSUPPORTED, "mean correction supports up to 8 query heads per KV head");
  const size_t need = sa::mean_correct_workspace(kv->n_kv_heads, n_kv_blocks, nullptr, nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(SA_ERR_WORKSPACE_TOO_SMALL, "mean correction needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, seq, 1);
    st = v.finish(kv, 0);
    if (st != SA_OK) return st;
  }
  sa::MeanCorrParams p{};
  sa::mean_correct_workspace(kv->n_kv_heads, n_kv_blocks, workspace, &p);
  p.q = q;
  p.mu = page_summary;
  p.nu = value_summary;
  p.bt_row = kv->block_table + (size_t)seq * kv->max_pages;
  p.seq_len = kv->seq_lens + seq;
  p.table = block_table;
  p.counts = block_counts;
  p.out = out;
  p.out_lse = out_lse;
  p.q_len = q_len;
  p.q_start = q_start;
  p.Hq = n_q_heads;
  p.Hkv = kv->n_kv_heads;
  p.G = n_q_heads / kv->n_kv_heads;
  p.nkb = n_kv_blocks;
  p.P = kv->page_size;
  p.scale_log2 = sm_scale * sa::kLog2e;
  return device_status(sa::launch_mean_correct(p, stream), "mean correction launch");
}

// --------------------------------------------------------------- autotuner
static size_t mass_stride(const sa_paged_kv* kv) { return (size_t)(kv->max_pages + 3) / 4 * 4; }

size_t sa_head_page_mass_workspace_size(const sa_paged_kv* kv, int32_t batch, int32_t q_tokens,
                                        int32_t n_q_heads) {
  if (!kv || batch <= 0 || q_tokens <= 0 || n_q_heads <= 0 || kv->max_pages <= 0) return 0;
  return align_up((size_t)batch * q_tokens * n_q_heads * mass_stride(kv) * sizeof(float));
}

static sa_status check_tuner_heads(const sa_paged_kv* kv, int32_t n_q_heads) {
  if (n_q_heads <= 0 || n_q_heads % kv->n_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_q_heads must be a positive multiple of n_kv_heads");
  if (n_q_heads / kv->n_kv_heads > sa::kTuneMaxGroup)
    return fail(SA_ERR_UNSUPPORTED, "at most %d query heads per KV head", sa::kTuneMaxGroup);
  if (kv->max_pages > sa::kTuneMaxPages)
    return fail(SA_ERR_UNSUPPORTED, "max_pages %d exceeds %d", kv->max_pages, sa::kTuneMaxPages);
  return SA_OK;
}

sa_status sa_head_page_mass(const sa_paged_kv* kv, int32_t batch, const void* q, int32_t q_tokens,
                            int32_t n_q_heads, const float* page_summary, float sm_scale, float* head_mass,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  sa_status st = check_kv(kv, false);
  if (st != SA_OK) return st;
  if ((st = check_tuner_heads(kv, n_q_heads)) != SA_OK) return st;
  if (kv->dtype == SA_DTYPE_FP32) return fail(SA_ERR_UNSUPPORTED, "the mass estimate needs bf16 queries");
  if (kv->d_qk != 64 && kv->d_qk != 128 && kv->d_qk != 576)
    return fail(SA_ERR_UNSUPPORTED, "d_qk %d unsupported (64, 128 or 576)", kv->d_qk);
  if (batch <= 0 || q_tokens <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "batch and q_tokens must be positive");
  if (!q || !page_summary || !head_mass)
    return fail(SA_ERR_INVALID_ARGUMENT, "q, page_summary and head_mass must be set");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(SA_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  const size_t need = sa_head_page_mass_workspace_size(kv, batch, q_tokens, n_q_heads);
  if (!workspace || workspace_bytes < need)
    return fail(SA_ERR_WORKSPACE_TOO_SMALL, "head mass needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, 0, batch);
    st = v.finish(kv, 0);
    if (st != SA_OK) return st;
  }
  sa::MassParams p{};
  p.q = q;
  p.mu = page_summary;
  p.block_table = kv->block_table;
  p.seq_lens = kv->seq_lens;
  p.est = static_cast<float*>(workspace);
  p.mass = head_mass;
  p.B = batch;
  p.T = q_tokens;
  p.Hq = n_q_heads;
  p.Hkv = kv->n_kv_heads;
  p.G = n_q_heads / kv->n_kv_heads;
  p.d = kv->d_qk;
  p.P = kv->page_size;
  p.max_pages = kv->max_pages;
  p.stride = (int)mass_stride(kv);
  p.sm_scale = sm_scale;
  return device_status(sa::launch_head_mass(p, stream), "head mass launch");
}

size_t sa_autotune_tiers_workspace_size(const sa_paged_kv* kv, int32_t batch, int32_t n_heads) {
  if (!kv || batch <= 0 || n_heads <= 0 || kv->n_kv_heads <= 0 || kv->max_pages <= 0) return 0;
  const size_t rows = (size_t)batch * kv->n_kv_heads;
  return align_up(rows * kv->max_pages * sizeof(float)) +
         align_up(rows * kv->max_pages * n_heads * sizeof(float)) +
         align_up(rows * sa::autotune_chunks(kv->max_pages) * sa::kTuneMaxGrid * sa::kTuneMaxGrid * sizeof(float));
}

sa_status sa_autotune_tiers(const sa_paged_kv* kv, int32_t batch, int32_t q_tokens, int32_t n_q_heads,
                            const float* head_mass, const float* scores, int32_t scores_stride,
                            int32_t sink_pages, int32_t window_pages, int32_t budget, const int32_t* alphas,
                            int32_t n_alphas, const int32_t* ambient_heads, int32_t n_heads, float* coverage_out,
                            int32_t* choice_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  sa_status st = check_kv(kv, false);
  if (st != SA_OK) return st;
  if ((st = check_tuner_heads(kv, n_q_heads)) != SA_OK) return st;
  if (batch <= 0 || q_tokens <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "batch and q_tokens must be positive");
  if (!head_mass || !scores || !alphas || !ambient_heads || !coverage_out || !choice_out)
    return fail(SA_ERR_INVALID_ARGUMENT, "head_mass, scores, alphas, ambient_heads, coverage_out and choice_out "
                                         "must be set");
  if (scores_stride < kv->max_pages)
    return fail(SA_ERR_INVALID_ARGUMENT, "scores_stride %d must be >= max_pages %d", scores_stride, kv->max_pages);
  if (sink_pages < 0 || window_pages < 0 || budget < 0)
    return fail(SA_ERR_INVALID_ARGUMENT, "sink_pages, window_pages and budget must be >= 0");
  if (n_alphas < 1 || n_alphas > sa::kTuneMaxGrid || n_heads < 1 || n_heads > sa::kTuneMaxGrid)
    return fail(SA_ERR_INVALID_ARGUMENT, "n_alphas and n_heads must be in [1, %d]", sa::kTuneMaxGrid);
  const int G = n_q_heads / kv->n_kv_heads;
  sa::TuneParams p{};
  for (int i = 0; i < n_alphas; ++i) {
    if (alphas[i] < 0) return fail(SA_ERR_INVALID_ARGUMENT, "alphas[%d] = %d < 0", i, alphas[i]);
    p.alpha[i] = alphas[i];
  }
  for (int k = 0; k < n_heads; ++k) {
    if (ambient_heads[k] < 1) return fail(SA_ERR_INVALID_ARGUMENT, "ambient_heads[%d] = %d < 1", k, ambient_heads[k]);
    p.heads[k] = ambient_heads[k];
  }
  for (int i = 0; i < n_alphas; ++i)
    for (int k = 0; k < n_heads; ++k) {
      const long rest = (long)budget - (long)alphas[i] * G;
      p.beta[i * n_heads + k] = rest < 0 ? -1 : (int)std::min<long>(rest / ambient_heads[k], INT32_MAX);
    }
  const size_t need = sa_autotune_tiers_workspace_size(kv, batch, n_heads);
  if (!workspace || workspace_bytes < need)
    return fail(SA_ERR_WORKSPACE_TOO_SMALL, "autotune needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, 0, batch);
    st = v.finish(kv, 0);
    if (st != SA_OK) return st;
  }
  const size_t rows = (size_t)batch * kv->n_kv_heads;
  char* w = static_cast<char*>(workspace);
  p.mall = reinterpret_cast<float*>(w);
  w += align_up(rows * kv->max_pages * sizeof(float));
  p.tsum = reinterpret_cast<float*>(w);
  w += align_up(rows * kv->max_pages * n_heads * sizeof(float));
  p.part = reinterpret_cast<float*>(w);
  p.mass = head_mass;
  p.scores = scores;
  p.seq_lens = kv->seq_lens;
  p.coverage = coverage_out;
  p.choice = choice_out;
  p.B = batch;
  p.T = q_tokens;
  p.Hq = n_q_heads;
  p.Hkv = kv->n_kv_heads;
  p.G = G;
  p.P = kv->page_size;
  p.max_pages = kv->max_pages;
  p.scores_stride = scores_stride;
  p.sink = sink_pages;
  p.window = window_pages;
  p.n_a = n_alphas;
  p.n_h = n_heads;
  return device_status(sa::launch_autotune(p, stream), "autotune launch");
}

sa_status sa_ambient_head_mask(const sa_paged_kv* kv, int32_t batch, int32_t n_q_heads, const float* head_mass,
                               const int32_t* page_lists, int32_t list_stride, const int32_t* page_counts,
                               const int32_t* critical_counts, int32_t ambient_heads, uint32_t* ambient_mask_out,
                               hipStream_t stream) {
  sa_status st = check_kv(kv, false);
  if (st != SA_OK) return st;
  if ((st = check_tuner_heads(kv, n_q_heads)) != SA_OK) return st;
  if (batch <= 0 || list_stride <= 0) return fail(SA_ERR_INVALID_ARGUMENT, "batch and list_stride must be positive");
  if (!head_mass || !page_lists || !page_counts || !critical_counts || !ambient_mask_out)
    return fail(SA_ERR_INVALID_ARGUMENT, "head_mass, page_lists, page_counts, critical_counts and "
                                         "ambient_mask_out must be set");
  if (ambient_heads < 0) return fail(SA_ERR_INVALID_ARGUMENT, "ambient_heads must be >= 0");
  if (validate_on()) {
    Validator v(stream);
    v.kv(kv, 0, batch);
    v.lists(kv, batch, kv->n_kv_heads, page_lists, page_counts, critical_counts, list_stride);
    st = v.finish(kv, list_stride);
    if (st != SA_OK) return st;
  }
  sa::AmbientMaskParams p{};
  p.mass = head_mass;
  p.lists = page_lists;
  p.counts = page_counts;
  p.ccounts = critical_counts;
  p.mask = ambient_mask_out;
  p.B = batch;
  p.Hq = n_q_heads;
  p.Hkv = kv->n_kv_heads;
  p.G = n_q_heads / kv->n_kv_heads;
  p.max_pages = kv->max_pages;
  p.list_stride = list_stride;
  p.words = (n_q_heads + 31) / 32;
  p.h = ambient_heads;
  return device_status(sa::launch_ambient_mask(p, stream), "ambient mask launch");
}

}  // extern "C"
