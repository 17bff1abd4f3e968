// Host side of the C ABI declared in include/lcs.h: argument validation, workspace
// sizing and kernel launch.  Every check runs before anything touches the device,
// so an invalid call returns a status without a launch (and without a GPU).
#include "../../include/lcs.h"
#include "lcs_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

namespace {

thread_local char g_err[512] = "";

lcs_status fail(lcs_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

lcs_status check_kv(const lcs_paged_kv* kv) {
  if (kv == nullptr) return fail(LCS_E_ARG, "kv is NULL");
  if (kv->k == nullptr || kv->v == nullptr || kv->block_table == nullptr)
    return fail(LCS_E_ARG, "kv->k, kv->v and kv->block_table must be non-NULL");
  if (kv->d != 64 && kv->d != 128) return fail(LCS_E_UNSUPPORTED, "head dim %d not in {64, 128}", kv->d);
  if (!is_pow2(kv->page_size) || kv->page_size > 1024)
    return fail(LCS_E_UNSUPPORTED, "page_size %d is not a power of two in [1, 1024]", kv->page_size);
  if (kv->num_pages < 1 || kv->max_pages < 1 || kv->Hkv < 1)
    return fail(LCS_E_SHAPE, "num_pages (%d), max_pages (%d) and Hkv (%d) must be >= 1",
                kv->num_pages, kv->max_pages, kv->Hkv);
  if ((long long)kv->num_pages * kv->Hkv * kv->page_size >= (1ll << 31))
    return fail(LCS_E_UNSUPPORTED, "num_pages*Hkv*page_size must stay below 2^31 rows");
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return fail(LCS_E_ARG, "kv->k and kv->v must be 16-byte aligned");
  return LCS_OK;
}

lcs_status check_heads(int32_t Hq, int32_t Hkv) {
  if (Hq < 1) return fail(LCS_E_SHAPE, "Hq must be >= 1");
  if (Hq % Hkv != 0) return fail(LCS_E_SHAPE, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
  return LCS_OK;
}

lcs_status hip_status(hipError_t e) {
  if (e == hipSuccess) return LCS_OK;
  return fail(LCS_E_HIP, "HIP launch failed: %s", hipGetErrorString(e));
}

}  // namespace

// Device scratch of lcs_sparse_draft_attn_noalloc: its split-K partials and block-union
// plan live here instead of in a caller workspace.  Every GPU the library runs on holds
// one copy for the life of the process.  Host code never uses this name as an address:
// it takes the device address from hipGetSymbolAddress (scratch_ptr) once per device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of the current device's scratch, looked up on its first use there
// (with that device current) and kept per device.
lcs_status scratch_ptr(void** out) {
  static std::atomic<void*> ptrs[kMaxDevices] = {};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LCS_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LCS_E_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = ptrs[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(LCS_E_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      ptrs[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LCS_OK;
}

}  // namespace

namespace lcs {

int32_t device_cus() {
  static std::atomic<int32_t> cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  int32_t n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) {
    (void)hipGetLastError();
    v = kDefaultCUs;
  }
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace lcs

extern "C" {

const char* lcs_last_error(void) { return g_err; }

const char* lcs_version(void) { return "lcs 0.1 gfx950"; }

size_t lcs_verify_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq, const lcs_paged_kv* kv,
                                  int32_t max_prefix_len) {
  if (kv == nullptr || kv->Hkv < 1 || Hq < 1 || n_q < 1 || B < 0 || max_prefix_len < 0) return 0;
  if (Hq % kv->Hkv != 0 || (kv->d != 64 && kv->d != 128)) return 0;
  return lcs::attn_plan(lcs::MODE_DENSE, B, n_q, Hq, kv->Hkv, kv->d, kv->page_size, max_prefix_len, 0, 0,
                         lcs::device_cus())
      .total_bytes;
}

}  // extern "C"

namespace {

// Shared body of the two verify entry points; the collected rows arrive as the
// kernel's (cmask, n_cl, cswap, cdup) encoding, already validated against n_q.
lcs_status verify_impl(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q, int32_t Hq,
                       const int32_t* prefix_len, int32_t max_prefix_len, const uint64_t* tree_mask,
                       float scale, uint64_t cmask, int32_t n_cl, int32_t cswap, int32_t cdup, float* out,
                       float* logits, int64_t logits_ld, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream, float* scores = nullptr, int64_t scores_ld = 0) {
  if (B == 0) return LCS_OK;   // empty batch: nothing is read or written, pointers may be NULL
  if (q == nullptr || prefix_len == nullptr || out == nullptr)
    return fail(LCS_E_ARG, "q, prefix_len and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(LCS_E_ARG, "q and out must be 16-byte aligned");
  if (!isfinite(scale) || !(scale > 0.f)) return fail(LCS_E_ARG, "scale must be finite and positive");
  if (logits != nullptr && logits_ld < max_prefix_len)
    return fail(LCS_E_SHAPE, "logits_ld %lld < max_prefix_len %d", (long long)logits_ld, max_prefix_len);
  if ((long long)max_prefix_len + n_q > (long long)kv->max_pages * kv->page_size)
    return fail(LCS_E_SHAPE, "max_prefix_len + n_q exceeds max_pages * page_size");
  const lcs::AttnPlan plan = lcs::attn_plan(lcs::MODE_DENSE, B, n_q, Hq, kv->Hkv, kv->d, kv->page_size,
                                            max_prefix_len, 0, 0, lcs::device_cus());
  if (workspace_bytes < plan.total_bytes || (plan.part_bytes > 0 && workspace == nullptr))
    return fail(LCS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, plan.total_bytes);
  lcs::AttnArgs a{};
  a.k = static_cast<const uint16_t*>(kv->k);
  a.v = static_cast<const uint16_t*>(kv->v);
  a.bt = kv->block_table;
  a.num_pages = kv->num_pages;
  a.lg_page = ilog2(kv->page_size);
  a.max_pages = kv->max_pages;
  a.Hkv = kv->Hkv;
  a.q = static_cast<const uint16_t*>(q);
  a.B = B;
  a.n_q = n_q;
  a.Hq = Hq;
  a.G = Hq / kv->Hkv;
  a.mode = lcs::MODE_DENSE;
  a.prefix_len = prefix_len;
  a.max_prefix_len = max_prefix_len;
  a.rowmask = tree_mask;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.cmask = (logits != nullptr) ? cmask : 0;
  a.n_cl = n_cl;
  a.cswap = cswap;
  a.cdup = cdup;
  a.logits = logits;
  a.logits_ld = logits_ld;
  a.lvec4 = (logits != nullptr && aligned(logits, 16) && logits_ld % 4 == 0) ? 1 : 0;
  a.scores = scores;
  a.scores_ld = scores_ld;
  if (scores != nullptr) {
    // the partial sums need both collected rows of every head of a group in one
    // workgroup, and their staging area (the Q tile) must hold 2G x 32 floats per wave
    if (plan.n_rc != 1)
      return fail(LCS_E_UNSUPPORTED, "partial scores need n_q * Hq / Hkv <= %d rows (have %d)", lcs::kMaxRowsPerWG,
                  plan.rows);
    if (256LL * a.G > 8LL * plan.QT * kv->d)
      return fail(LCS_E_UNSUPPORTED, "partial scores need Hq / Hkv <= %d at %d rows and d = %d",
                  plan.QT * kv->d / 32, plan.rows, kv->d);
    a.cmask = cmask;
    a.logits = nullptr;
  }
  a.out = out;
  a.lse = lse;
  return hip_status(lcs::attn_launch(plan, a, workspace, static_cast<hipStream_t>(stream)));
}

lcs_status verify_checks(const lcs_paged_kv* kv, int32_t B, int32_t n_q, int32_t Hq, int32_t max_prefix_len) {
  lcs_status st = check_kv(kv);
  if (st != LCS_OK) return st;
  if ((st = check_heads(Hq, kv->Hkv)) != LCS_OK) return st;
  if (B < 0) return fail(LCS_E_SHAPE, "B must be >= 0");
  if (n_q < 1) return fail(LCS_E_SHAPE, "n_q must be >= 1");
  if (n_q > 64) return fail(LCS_E_UNSUPPORTED, "n_q %d > 64 verifier rows", n_q);
  if (Hq / kv->Hkv > 64) return fail(LCS_E_UNSUPPORTED, "Hq / Hkv = %d > 64 query heads per KV head", Hq / kv->Hkv);
  if (max_prefix_len < 0) return fail(LCS_E_SHAPE, "max_prefix_len must be >= 0");
  return LCS_OK;
}

}  // namespace

extern "C" {

lcs_status lcs_verify_attn(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q, int32_t Hq,
                           const int32_t* prefix_len, int32_t max_prefix_len, const uint64_t* tree_mask,
                           float scale, int32_t collect_row0, int32_t collect_row1, float* out,
                           float* logits, int64_t logits_ld, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  lcs_status st = verify_checks(kv, B, n_q, Hq, max_prefix_len);
  if (st != LCS_OK) return st;
  if (collect_row0 < 0 || collect_row0 >= n_q || collect_row1 < 0 || collect_row1 >= n_q)
    return fail(LCS_E_ARG, "collect rows (%d, %d) outside [0, %d)", collect_row0, collect_row1, n_q);
  const uint64_t cmask = (1ull << collect_row0) | (1ull << collect_row1);
  return verify_impl(kv, q, B, n_q, Hq, prefix_len, max_prefix_len, tree_mask, scale, cmask, 2,
                     collect_row0 > collect_row1 ? 1 : 0, collect_row0 == collect_row1 ? 1 : 0, out, logits,
                     logits_ld, lse, workspace, workspace_bytes, stream);
}

lcs_status lcs_verify_attn_scores(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q, int32_t Hq,
                                  const int32_t* prefix_len, int32_t max_prefix_len, const uint64_t* tree_mask,
                                  float scale, int32_t collect_row0, int32_t collect_row1, float* out,
                                  float* scores, int64_t scores_ld, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  lcs_status st = verify_checks(kv, B, n_q, Hq, max_prefix_len);
  if (st != LCS_OK) return st;
  if (collect_row0 < 0 || collect_row0 >= n_q || collect_row1 < 0 || collect_row1 >= n_q)
    return fail(LCS_E_ARG, "collect rows (%d, %d) outside [0, %d)", collect_row0, collect_row1, n_q);
  if (B > 0 && scores == nullptr) return fail(LCS_E_ARG, "scores must be non-NULL");
  if (B > 0 && scores_ld < max_prefix_len)
    return fail(LCS_E_SHAPE, "scores_ld %lld < max_prefix_len %d", (long long)scores_ld, max_prefix_len);
  const uint64_t cmask = (1ull << collect_row0) | (1ull << collect_row1);
  return verify_impl(kv, q, B, n_q, Hq, prefix_len, max_prefix_len, tree_mask, scale, cmask, 2,
                     collect_row0 > collect_row1 ? 1 : 0, collect_row0 == collect_row1 ? 1 : 0, out, nullptr, 0,
                     lse, workspace, workspace_bytes, stream, scores, scores_ld);
}

lcs_status lcs_verify_attn_rows(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q, int32_t Hq,
                                const int32_t* prefix_len, int32_t max_prefix_len, const uint64_t* tree_mask,
                                float scale, uint64_t collect_mask, float* out, float* logits,
                                int64_t logits_ld, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  lcs_status st = verify_checks(kv, B, n_q, Hq, max_prefix_len);
  if (st != LCS_OK) return st;
  if (logits != nullptr) {
    if (collect_mask == 0) return fail(LCS_E_ARG, "collect_mask is empty but logits is not NULL");
    if (n_q < 64 && (collect_mask >> n_q) != 0)
      return fail(LCS_E_ARG, "collect_mask 0x%llx names rows at or above n_q = %d",
                  (unsigned long long)collect_mask, n_q);
  }
  return verify_impl(kv, q, B, n_q, Hq, prefix_len, max_prefix_len, tree_mask, scale, collect_mask,
                     __builtin_popcountll(collect_mask), 0, 0, out, logits, logits_ld, lse, workspace,
                     workspace_bytes, stream);
}

size_t lcs_select_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, lcs_set_mode mode,
                                  int32_t max_prefix_len, int32_t block_size) {
  if (B < 0 || Hkv < 1 || Hq < 1 || max_prefix_len < 0) return 0;
  if (mode == LCS_SET_BLOCK && (!is_pow2(block_size) || block_size < 4 || block_size > lcs::kScorePos)) return 0;
  return lcs::select_plan(B, Hq, Hkv, (int32_t)mode, max_prefix_len, block_size).total_bytes;
}

}  // extern "C"

namespace {

lcs_status select_impl(const float* logits, int64_t logits_ld, int32_t n_rows, int32_t kind, const float* lse,
                       int32_t n_q, uint64_t rows_mask, int32_t B, int32_t Hq, int32_t Hkv,
                       const int32_t* prefix_len, int32_t max_prefix_len, lcs_set_mode mode, int32_t top_k,
                       int32_t n_sink, int32_t n_recent, int32_t block_size, int32_t* indices, int32_t* counts,
                       int32_t cap, void* workspace, size_t workspace_bytes, void* stream, int32_t block_lse = 0,
                       const lcs_paged_kv* phys_kv = nullptr) {
  if (Hkv < 1) return fail(LCS_E_SHAPE, "Hkv must be >= 1");
  lcs_status st = check_heads(Hq, Hkv);
  if (st != LCS_OK) return st;
  if (mode != LCS_SET_SHARED && mode != LCS_SET_PER_KV_HEAD && mode != LCS_SET_BLOCK)
    return fail(LCS_E_ARG, "unknown set mode %d", (int)mode);
  if (B < 0) return fail(LCS_E_SHAPE, "B must be >= 0");
  if (B == 0) return LCS_OK;   // empty batch: nothing is read or written, pointers may be NULL
  if (logits == nullptr || prefix_len == nullptr || indices == nullptr || counts == nullptr)
    return fail(LCS_E_ARG, "logits, prefix_len, indices and counts must be non-NULL");
  if (kind == lcs::SCORE_SOFTMAX_WT && lse == nullptr) return fail(LCS_E_ARG, "softmax-weight scores need lse");
  if (top_k < 0 || n_sink < 0 || n_recent < 0) return fail(LCS_E_ARG, "top_k, n_sink, n_recent must be >= 0");
  if (max_prefix_len < 0) return fail(LCS_E_SHAPE, "max_prefix_len must be >= 0");
  if (max_prefix_len >= (1 << 24)) return fail(LCS_E_UNSUPPORTED, "max_prefix_len must be < 2^24");
  if (logits_ld < max_prefix_len) return fail(LCS_E_SHAPE, "logits_ld %lld < max_prefix_len %d",
                                              (long long)logits_ld, max_prefix_len);
  long long items = max_prefix_len, need;
  if (mode == LCS_SET_BLOCK) {
    if (!is_pow2(block_size) || block_size < 4 || block_size > lcs::kScorePos)
      return fail(LCS_E_UNSUPPORTED, "block_size %d is not a power of two in [4, %d]", block_size, lcs::kScorePos);
    items = (max_prefix_len + block_size - 1) / block_size;
    need = ((long long)n_sink + block_size - 1) / block_size + (long long)top_k +
           ((long long)n_recent + block_size - 1) / block_size + 1;
  } else {
    need = (long long)n_sink + top_k + n_recent;
  }
  if (need > items) need = items;
  if (cap < need) return fail(LCS_E_SHAPE, "cap %d < %lld entries the selection can produce", cap, need);
  const int32_t reads = (mode == LCS_SET_SHARED ? Hq : Hq / Hkv) * n_rows;   // values per position
  const lcs::SelPlan plan = lcs::select_plan(B, Hq, Hkv, (int32_t)mode, max_prefix_len, block_size,
                                             lcs::device_cus(), reads);
  if (workspace == nullptr || workspace_bytes < plan.total_bytes)
    return fail(LCS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, plan.total_bytes);
  lcs::SelArgs a{};
  a.logits = logits;
  a.ld = logits_ld;
  a.n_rows = n_rows;
  a.kind = kind;
  a.lse = lse;
  a.n_q = n_q;
  a.rows_mask = rows_mask;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.mode = (int32_t)mode;
  a.prefix_len = prefix_len;
  a.max_len = max_prefix_len;
  // The kernels add the window sizes in 32-bit arithmetic.  A size at or beyond the
  // longest prefix (items in block mode) keeps every item either way, so clamping to it
  // changes no result and keeps those sums far from overflow.
  a.top_k = (int32_t)(top_k < items ? top_k : items);
  a.n_sink = n_sink < max_prefix_len ? n_sink : max_prefix_len;
  a.n_recent = n_recent < max_prefix_len ? n_recent : max_prefix_len;
  a.lg_bs = (mode == LCS_SET_BLOCK) ? ilog2(block_size) : 0;
  a.vec4 = (aligned(logits, 16) && logits_ld % 4 == 0) ? 1 : 0;
  a.block_lse = block_lse;
  if (phys_kv != nullptr) {
    // physical slots: page * page_size + slot through the sequence's block table
    if (mode == LCS_SET_BLOCK) return fail(LCS_E_UNSUPPORTED, "physical slots are for token sets, not blocks");
    if ((st = check_kv(phys_kv)) != LCS_OK) return st;
    if ((long long)max_prefix_len > (long long)phys_kv->max_pages * phys_kv->page_size)
      return fail(LCS_E_SHAPE, "max_prefix_len exceeds max_pages * page_size");
    if ((long long)phys_kv->num_pages * phys_kv->page_size >= (1ll << 31))
      return fail(LCS_E_UNSUPPORTED, "num_pages * page_size must stay below 2^31 slots");
    a.bt = phys_kv->block_table;
    a.max_pages = phys_kv->max_pages;
    a.lg_page = ilog2(phys_kv->page_size);
  }
  a.indices = indices;
  a.counts = counts;
  a.cap = cap;
  return hip_status(lcs::select_launch(plan, a, workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

lcs_status lcs_select_topk(const float* logits, int64_t logits_ld, int32_t B, int32_t Hq, int32_t Hkv,
                           const int32_t* prefix_len, int32_t max_prefix_len, lcs_set_mode mode,
                           int32_t top_k, int32_t n_sink, int32_t n_recent, int32_t block_size,
                           int32_t* indices, int32_t* counts, int32_t cap, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return select_impl(logits, logits_ld, 2, lcs::SCORE_LOGIT_SUM, nullptr, 0, 0, B, Hq, Hkv, prefix_len,
                     max_prefix_len, mode, top_k, n_sink, n_recent, block_size, indices, counts, cap, workspace,
                     workspace_bytes, stream);
}

lcs_status lcs_select_topk_physical(const float* logits, int64_t logits_ld, int32_t B, int32_t Hq, int32_t Hkv,
                                    const int32_t* prefix_len, int32_t max_prefix_len, lcs_set_mode mode,
                                    int32_t top_k, int32_t n_sink, int32_t n_recent, const lcs_paged_kv* kv,
                                    int32_t* indices, int32_t* counts, int32_t cap, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (kv == nullptr) return fail(LCS_E_ARG, "kv is NULL");
  return select_impl(logits, logits_ld, 2, lcs::SCORE_LOGIT_SUM, nullptr, 0, 0, B, Hq, Hkv, prefix_len,
                     max_prefix_len, mode, top_k, n_sink, n_recent, 0, indices, counts, cap, workspace,
                     workspace_bytes, stream, 0, kv);
}

lcs_status lcs_select_topk_blocks(const float* logits, int64_t logits_ld, int32_t B, int32_t Hq, int32_t Hkv,
                                  const int32_t* prefix_len, int32_t max_prefix_len, lcs_block_score block_score,
                                  int32_t top_k, int32_t n_sink, int32_t n_recent, int32_t block_size,
                                  int32_t* indices, int32_t* counts, int32_t cap, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (block_score != LCS_BLOCK_MAX && block_score != LCS_BLOCK_LSE)
    return fail(LCS_E_ARG, "unknown block score %d", (int)block_score);
  return select_impl(logits, logits_ld, 2, lcs::SCORE_LOGIT_SUM, nullptr, 0, 0, B, Hq, Hkv, prefix_len,
                     max_prefix_len, LCS_SET_BLOCK, top_k, n_sink, n_recent, block_size, indices, counts, cap,
                     workspace, workspace_bytes, stream, block_score == LCS_BLOCK_LSE ? 1 : 0);
}

lcs_status lcs_select_topk_scores(const float* scores, int64_t scores_ld, int32_t B, int32_t Hkv,
                                  const int32_t* prefix_len, int32_t max_prefix_len, lcs_set_mode mode,
                                  int32_t top_k, int32_t n_sink, int32_t n_recent, int32_t block_size,
                                  int32_t* indices, int32_t* counts, int32_t cap, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  // one score row per KV head: the selector's head loop runs over KV heads, one row each
  return select_impl(scores, scores_ld, 1, lcs::SCORE_LOGIT_SUM, nullptr, 0, 0, B, Hkv, Hkv, prefix_len,
                     max_prefix_len, mode, top_k, n_sink, n_recent, block_size, indices, counts, cap, workspace,
                     workspace_bytes, stream);
}

lcs_status lcs_select_topk_rows(const float* logits, int64_t logits_ld, int32_t n_rows, lcs_score_kind kind,
                                const float* lse, int32_t n_q, uint64_t rows_mask, int32_t B, int32_t Hq,
                                int32_t Hkv, const int32_t* prefix_len, int32_t max_prefix_len,
                                lcs_set_mode mode, int32_t top_k, int32_t n_sink, int32_t n_recent,
                                int32_t block_size, int32_t* indices, int32_t* counts, int32_t cap,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (n_rows < 1 || n_rows > 64) return fail(LCS_E_ARG, "n_rows %d outside [1, 64]", n_rows);
  if (kind != LCS_SCORE_LOGIT_SUM && kind != LCS_SCORE_SOFTMAX_WEIGHT)
    return fail(LCS_E_ARG, "unknown score kind %d", (int)kind);
  if (kind == LCS_SCORE_SOFTMAX_WEIGHT) {
    if (n_q < 1 || n_q > 64) return fail(LCS_E_ARG, "n_q %d outside [1, 64]", n_q);
    if (__builtin_popcountll(rows_mask) != n_rows || (n_q < 64 && (rows_mask >> n_q) != 0))
      return fail(LCS_E_ARG, "rows_mask 0x%llx must name n_rows = %d rows below n_q = %d",
                  (unsigned long long)rows_mask, n_rows, n_q);
  }
  return select_impl(logits, logits_ld, n_rows,
                     kind == LCS_SCORE_SOFTMAX_WEIGHT ? lcs::SCORE_SOFTMAX_WT : lcs::SCORE_LOGIT_SUM, lse, n_q,
                     rows_mask, B, Hq, Hkv, prefix_len, max_prefix_len, mode, top_k, n_sink, n_recent, block_size,
                     indices, counts, cap, workspace, workspace_bytes, stream);
}

size_t lcs_sparse_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq, const lcs_paged_kv* kv,
                                  lcs_set_mode mode, int32_t cap, int32_t max_tail_len) {
  if (kv == nullptr || kv->Hkv < 1 || Hq < 1 || n_q < 1 || B < 0 || cap < 0 || max_tail_len < 0) return 0;
  if (Hq % kv->Hkv != 0 || (kv->d != 64 && kv->d != 128)) return 0;
  const int32_t m = (mode == LCS_SET_BLOCK) ? lcs::MODE_BLOCK
                    : (mode == LCS_SET_SHARED) ? lcs::MODE_LIST_SHARED : lcs::MODE_LIST_PER_HEAD;
  return lcs::attn_plan(m, B, n_q, Hq, kv->Hkv, kv->d, kv->page_size, 0, cap, max_tail_len,
                         lcs::device_cus()).total_bytes;
}

}  // extern "C"

namespace {

// Shared body of the two sparse entry points.  use_scratch: the workspace is the
// library's static device scratch of the current device instead of the caller's.
lcs_status sparse_impl(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q, int32_t Hq,
                       lcs_set_mode mode, const int32_t* indices, const int32_t* counts, int32_t cap,
                       const int32_t* tail_begin, const int32_t* tail_len, int32_t max_tail_len,
                       const uint64_t* tail_mask, float scale, float* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream, bool use_scratch, bool phys = false) {
  lcs_status st = check_kv(kv);
  if (st != LCS_OK) return st;
  if ((st = check_heads(Hq, kv->Hkv)) != LCS_OK) return st;
  if (mode != LCS_SET_SHARED && mode != LCS_SET_PER_KV_HEAD && mode != LCS_SET_BLOCK)
    return fail(LCS_E_ARG, "unknown set mode %d", (int)mode);
  if (B < 0) return fail(LCS_E_SHAPE, "B must be >= 0");
  if (n_q < 1) return fail(LCS_E_SHAPE, "n_q must be >= 1");
  if (n_q > 64) return fail(LCS_E_UNSUPPORTED, "n_q %d > 64 rows", n_q);
  if (cap < 0 || max_tail_len < 0) return fail(LCS_E_SHAPE, "cap and max_tail_len must be >= 0");
  if (B == 0) return LCS_OK;   // empty batch: nothing is read or written, pointers may be NULL
  if (q == nullptr || out == nullptr || tail_begin == nullptr || tail_len == nullptr)
    return fail(LCS_E_ARG, "q, out, tail_begin and tail_len must be non-NULL");
  if (cap > 0 && (indices == nullptr || counts == nullptr))
    return fail(LCS_E_ARG, "indices and counts must be non-NULL when cap > 0");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(LCS_E_ARG, "q and out must be 16-byte aligned");
  if (!isfinite(scale) || !(scale > 0.f)) return fail(LCS_E_ARG, "scale must be finite and positive");
  if (tail_mask != nullptr && max_tail_len > 64)
    return fail(LCS_E_UNSUPPORTED, "a tail mask covers at most 64 tail slots (max_tail_len %d)", max_tail_len);
  if (mode == LCS_SET_BLOCK && kv->page_size % lcs::kStepTokens != 0)
    return fail(LCS_E_UNSUPPORTED, "block mode needs page_size %% %d == 0 (page_size %d)", lcs::kStepTokens,
                kv->page_size);
  const int32_t m = (mode == LCS_SET_BLOCK) ? lcs::MODE_BLOCK
                    : (mode == LCS_SET_SHARED) ? lcs::MODE_LIST_SHARED : lcs::MODE_LIST_PER_HEAD;
  const lcs::AttnPlan plan =
      lcs::attn_plan(m, B, n_q, Hq, kv->Hkv, kv->d, kv->page_size, 0, cap, max_tail_len, lcs::device_cus());
  if (use_scratch) {
    if (plan.total_bytes > kStaticScratchBytes)
      return fail(LCS_E_WORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                  plan.total_bytes, kStaticScratchBytes);
    if ((st = scratch_ptr(&workspace)) != LCS_OK) return st;
    workspace_bytes = kStaticScratchBytes;
  }
  if (workspace_bytes < plan.total_bytes ||
      ((plan.part_bytes > 0 || m == lcs::MODE_BLOCK) && workspace == nullptr))
    return fail(LCS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, plan.total_bytes);
  lcs::AttnArgs a{};
  a.k = static_cast<const uint16_t*>(kv->k);
  a.v = static_cast<const uint16_t*>(kv->v);
  a.bt = kv->block_table;
  a.num_pages = kv->num_pages;
  a.lg_page = ilog2(kv->page_size);
  a.max_pages = kv->max_pages;
  a.Hkv = kv->Hkv;
  a.q = static_cast<const uint16_t*>(q);
  a.B = B;
  a.n_q = n_q;
  a.Hq = Hq;
  a.G = Hq / kv->Hkv;
  a.mode = m;
  a.rowmask = tail_mask;
  a.indices = indices;
  a.counts = counts;
  a.cap = cap;
  a.max_tail_len = max_tail_len;
  a.tail_begin = tail_begin;
  a.tail_len = tail_len;
  a.phys = phys ? 1 : 0;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  return hip_status(lcs::attn_launch(plan, a, workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

lcs_status lcs_sparse_draft_attn(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q, int32_t Hq,
                                 lcs_set_mode mode, const int32_t* indices, const int32_t* counts,
                                 int32_t cap, const int32_t* tail_begin, const int32_t* tail_len,
                                 int32_t max_tail_len, const uint64_t* tail_mask, float scale, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_impl(kv, q, B, n_q, Hq, mode, indices, counts, cap, tail_begin, tail_len, max_tail_len, tail_mask,
                     scale, out, lse, workspace, workspace_bytes, stream, false);
}

lcs_status lcs_sparse_draft_attn_physical(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                                          int32_t Hq, lcs_set_mode mode, const int32_t* indices,
                                          const int32_t* counts, int32_t cap, const int32_t* tail_begin,
                                          const int32_t* tail_len, int32_t max_tail_len, const uint64_t* tail_mask,
                                          float scale, float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (mode == LCS_SET_BLOCK) return fail(LCS_E_UNSUPPORTED, "physical slots are for token sets, not blocks");
  if (kv != nullptr && (long long)kv->num_pages * kv->page_size >= (1ll << 31))
    return fail(LCS_E_UNSUPPORTED, "num_pages * page_size must stay below 2^31 slots");
  return sparse_impl(kv, q, B, n_q, Hq, mode, indices, counts, cap, tail_begin, tail_len, max_tail_len, tail_mask,
                     scale, out, lse, workspace, workspace_bytes, stream, false, true);
}

lcs_status lcs_sparse_draft_attn_noalloc(const lcs_paged_kv* kv, const void* q, int32_t B, int32_t n_q,
                                         int32_t Hq, lcs_set_mode mode, const int32_t* indices,
                                         const int32_t* counts, int32_t cap, const int32_t* tail_begin,
                                         const int32_t* tail_len, int32_t max_tail_len,
                                         const uint64_t* tail_mask, float scale, float* out, float* lse,
                                         void* stream) {
  return sparse_impl(kv, q, B, n_q, Hq, mode, indices, counts, cap, tail_begin, tail_len, max_tail_len, tail_mask,
                     scale, out, lse, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {

lcs::AttnArgs kv_args(const lcs_paged_kv* kv) {
  lcs::AttnArgs a{};
  a.k = static_cast<const uint16_t*>(kv->k);
  a.v = static_cast<const uint16_t*>(kv->v);
  a.bt = kv->block_table;
  a.num_pages = kv->num_pages;
  a.lg_page = ilog2(kv->page_size);
  a.max_pages = kv->max_pages;
  a.Hkv = kv->Hkv;
  return a;
}

lcs_status check_compression(int32_t cmp_len, int32_t cmp_stride, int32_t max_cmp) {
  if (!is_pow2(cmp_len) || cmp_len > 1024)
    return fail(LCS_E_UNSUPPORTED, "cmp_len %d is not a power of two in [1, 1024]", cmp_len);
  if (cmp_stride < 1 || cmp_stride > cmp_len)
    return fail(LCS_E_ARG, "cmp_stride %d outside [1, cmp_len = %d]", cmp_stride, cmp_len);
  if (max_cmp < 1) return fail(LCS_E_SHAPE, "max_cmp must be >= 1");
  return LCS_OK;
}

}  // namespace

extern "C" {

lcs_status lcs_nsa_compress(const lcs_paged_kv* kv, int32_t B, const int32_t* prefix_len, int32_t max_prefix_len,
                            int32_t cmp_len, int32_t cmp_stride, void* k_cmp, void* v_cmp, int32_t max_cmp,
                            void* stream) {
  lcs_status st = check_kv(kv);
  if (st != LCS_OK) return st;
  if ((st = check_compression(cmp_len, cmp_stride, max_cmp)) != LCS_OK) return st;
  if (B < 0 || max_prefix_len < 0) return fail(LCS_E_SHAPE, "B and max_prefix_len must be >= 0");
  if ((long long)max_prefix_len > (long long)kv->max_pages * kv->page_size)
    return fail(LCS_E_SHAPE, "max_prefix_len exceeds max_pages * page_size");
  if ((long long)B * kv->Hkv * max_cmp >= (1ll << 31))
    return fail(LCS_E_UNSUPPORTED, "B * Hkv * max_cmp must stay below 2^31 rows");
  if (B == 0) return LCS_OK;
  if (prefix_len == nullptr || k_cmp == nullptr || v_cmp == nullptr)
    return fail(LCS_E_ARG, "prefix_len, k_cmp and v_cmp must be non-NULL");
  if (!aligned(k_cmp, 16) || !aligned(v_cmp, 16)) return fail(LCS_E_ARG, "k_cmp and v_cmp must be 16-byte aligned");
  lcs::AttnArgs a = kv_args(kv);
  a.max_prefix_len = max_prefix_len;
  a.cmp_len = cmp_len;
  a.cmp_stride = cmp_stride;
  a.max_cmp = max_cmp;
  return hip_status(lcs::compress_launch(a, kv->d, B, prefix_len, static_cast<uint16_t*>(k_cmp),
                                         static_cast<uint16_t*>(v_cmp), static_cast<hipStream_t>(stream)));
}

size_t lcs_nsa_plan_bytes(int32_t B, int32_t n_q, int32_t Hkv, int32_t cap) {
  if (B < 0 || n_q < 1 || Hkv < 1 || cap < 0) return 0;
  return lcs::union_layout(B, Hkv, n_q, cap).total_bytes;
}

lcs_status lcs_nsa_plan(const lcs_paged_kv* kv, int32_t B, int32_t n_q, const int32_t* indices,
                        const int32_t* counts, int32_t cap, lcs_group_mode group, void* plan, size_t plan_bytes,
                        void* stream) {
  lcs_status st = check_kv(kv);
  if (st != LCS_OK) return st;
  if (group != LCS_GROUP_EXACT && group != LCS_GROUP_APPROXIMATE)
    return fail(LCS_E_ARG, "unknown group mode %d", (int)group);
  if (B < 0 || cap < 0) return fail(LCS_E_SHAPE, "B and cap must be >= 0");
  if (n_q < 1) return fail(LCS_E_SHAPE, "n_q must be >= 1");
  if (n_q > 64) return fail(LCS_E_UNSUPPORTED, "n_q %d > 64 rows", n_q);
  const lcs::UnionLayout u = lcs::union_layout(B, kv->Hkv, n_q, cap);
  if (B == 0) return LCS_OK;
  if (plan == nullptr || plan_bytes < u.total_bytes)
    return fail(LCS_E_WORKSPACE, "plan of %zu bytes, %zu needed", plan_bytes, u.total_bytes);
  if (cap > 0 && (indices == nullptr || counts == nullptr))
    return fail(LCS_E_ARG, "indices and counts must be non-NULL when cap > 0");
  lcs::AttnArgs a = kv_args(kv);
  a.B = B;
  a.n_q = n_q;
  a.indices = indices;
  a.counts = counts;
  a.cap = cap;
  a.ucap = n_q * cap;
  char* pb = static_cast<char*>(plan);
  a.ublk = reinterpret_cast<const int32_t*>(pb);
  a.umask = reinterpret_cast<const uint64_t*>(pb + u.ublk_bytes);
  a.ucount = reinterpret_cast<const int32_t*>(pb + u.ublk_bytes + u.umask_bytes);
  a.approx = (group == LCS_GROUP_APPROXIMATE) ? 1 : 0;
  return hip_status(lcs::union_launch(a, static_cast<hipStream_t>(stream)));
}

size_t lcs_nsa_workspace_bytes(int32_t B, int32_t n_q, int32_t Hq, const lcs_paged_kv* kv, int32_t cap,
                               int32_t max_tail_len, int32_t max_cmp, int32_t window) {
  if (kv == nullptr || kv->Hkv < 1 || Hq < 1 || n_q < 1 || B < 0 || cap < 0 || max_tail_len < 0 || max_cmp < 1 ||
      window < 0)
    return 0;
  if (Hq % kv->Hkv != 0 || (kv->d != 64 && kv->d != 128)) return 0;
  return lcs::attn_plan_nsa(B, n_q, Hq, kv->Hkv, kv->d, kv->page_size, cap, max_tail_len, max_cmp, window,
                            lcs::device_cus())
      .total_bytes;
}

lcs_status lcs_nsa_attn(const lcs_paged_kv* kv, const void* k_cmp, const void* v_cmp, int32_t max_cmp,
                        int32_t cmp_len, int32_t cmp_stride, int32_t window, const void* q, int32_t B, int32_t n_q,
                        int32_t Hq, const void* plan, size_t plan_bytes, int32_t cap, const int32_t* tail_begin,
                        const int32_t* tail_len, int32_t max_tail_len, const uint64_t* tail_mask,
                        const float* gates, float scale, float* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  lcs_status st = check_kv(kv);
  if (st != LCS_OK) return st;
  if ((st = check_heads(Hq, kv->Hkv)) != LCS_OK) return st;
  if ((st = check_compression(cmp_len, cmp_stride, max_cmp)) != LCS_OK) return st;
  if (B < 0 || cap < 0 || max_tail_len < 0 || window < 0)
    return fail(LCS_E_SHAPE, "B, cap, max_tail_len and window must be >= 0");
  if (n_q < 1) return fail(LCS_E_SHAPE, "n_q must be >= 1");
  if (n_q > 64) return fail(LCS_E_UNSUPPORTED, "n_q %d > 64 rows", n_q);
  if (Hq / kv->Hkv > 64) return fail(LCS_E_UNSUPPORTED, "Hq / Hkv = %d > 64 query heads per KV head", Hq / kv->Hkv);
  if (kv->page_size % lcs::kStepTokens != 0)
    return fail(LCS_E_UNSUPPORTED, "NSA selection needs page_size %% %d == 0 (page_size %d)", lcs::kStepTokens,
                kv->page_size);
  if (tail_mask != nullptr && max_tail_len > 64)
    return fail(LCS_E_UNSUPPORTED, "a tail mask covers at most 64 tail slots (max_tail_len %d)", max_tail_len);
  if ((long long)B * kv->Hkv * max_cmp >= (1ll << 31))
    return fail(LCS_E_UNSUPPORTED, "B * Hkv * max_cmp must stay below 2^31 rows");
  if (B == 0) return LCS_OK;
  if (q == nullptr || out == nullptr || tail_begin == nullptr || tail_len == nullptr || gates == nullptr ||
      plan == nullptr || k_cmp == nullptr || v_cmp == nullptr)
    return fail(LCS_E_ARG, "q, out, tail_begin, tail_len, gates, plan, k_cmp and v_cmp must be non-NULL");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cmp, 16) || !aligned(v_cmp, 16))
    return fail(LCS_E_ARG, "q, out, k_cmp and v_cmp must be 16-byte aligned");
  if (!isfinite(scale) || !(scale > 0.f)) return fail(LCS_E_ARG, "scale must be finite and positive");
  const lcs::UnionLayout u = lcs::union_layout(B, kv->Hkv, n_q, cap);
  if (plan_bytes < u.total_bytes) return fail(LCS_E_WORKSPACE, "plan of %zu bytes, %zu needed", plan_bytes,
                                              u.total_bytes);
  const lcs::AttnPlan p = lcs::attn_plan_nsa(B, n_q, Hq, kv->Hkv, kv->d, kv->page_size, cap, max_tail_len, max_cmp,
                                             window, lcs::device_cus());
  if (workspace == nullptr || workspace_bytes < p.total_bytes)
    return fail(LCS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, p.total_bytes);
  lcs::AttnArgs a = kv_args(kv);
  a.q = static_cast<const uint16_t*>(q);
  a.B = B;
  a.n_q = n_q;
  a.Hq = Hq;
  a.G = Hq / kv->Hkv;
  a.mode = lcs::MODE_NSA;
  a.rowmask = tail_mask;
  a.cap = cap;
  a.tail_begin = tail_begin;
  a.tail_len = tail_len;
  a.max_tail_len = max_tail_len;
  const char* pb = static_cast<const char*>(plan);
  a.ublk = reinterpret_cast<const int32_t*>(pb);
  a.umask = reinterpret_cast<const uint64_t*>(pb + u.ublk_bytes);
  a.ucount = reinterpret_cast<const int32_t*>(pb + u.ublk_bytes + u.umask_bytes);
  a.ucap = n_q * cap;
  a.ck = static_cast<const uint16_t*>(k_cmp);
  a.cv = static_cast<const uint16_t*>(v_cmp);
  a.max_cmp = max_cmp;
  a.cmp_len = cmp_len;
  a.cmp_stride = cmp_stride;
  a.window = window;
  a.gates = gates;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;
  return hip_status(lcs::attn_launch(p, a, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
