// Host half of the paged KV-cache attention library: error state, metadata
// validation, the planner (inspector) and the argument checking of run /
// append / merge before their kernels are launched.
//
// Sources: "Deep Dive - FlashInfer" (length contract, causal rule, plan/run,
// split-KV trade-offs), "FlashInfer 中的 KV-Cache 布局" (CSR page table,
// NHD/HND, MLA cache), "GPU attention backends: FlashInfer and
// FlashAttention" (plan once per batch, pinned staging reuse).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "internal.h"

using pkv::Item;
using pkv::MergeItem;

namespace pkv {

LaunchEvents& armed_launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}

}  // namespace pkv

namespace {

thread_local std::string g_error;
thread_local int32_t g_reason = PKV_META_NONE;

pkv_status fail(pkv_status code, const std::string& msg, int32_t reason = PKV_META_NONE) {
  g_error = msg;
  g_reason = reason;
  return code;
}

pkv_status meta_fail(int32_t reason, const std::string& msg) {
  return fail(PKV_ERR_METADATA, msg, reason);
}

pkv_status ok() {
  g_error.clear();
  g_reason = PKV_META_NONE;
  return PKV_OK;
}

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Copies a host table; an empty one may have a null data pointer, which
// memcpy must not be given even for zero bytes.
template <typename T>
void copy_table(void* dst, const std::vector<T>& v) {
  if (!v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(T));
}

int page_shift_of(int32_t p) {
  if (p <= 0 || (p & (p - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < p) ++s;
  return s;
}

size_t dtype_size(int32_t dt) { return dt == PKV_F32 ? 4 : (dt == PKV_FP8_E4M3 ? 1 : 2); }

// ------------------------------------------------------------- validation --

// Checks one indptr: starts at 0, never decreases.
pkv_status check_indptr(const char* name, const int32_t* indptr, int32_t batch) {
  if (indptr[0] != 0)
    return meta_fail(PKV_META_INDPTR_START, std::string(name) + fmt("[0] = %lld, expected 0", indptr[0]));
  for (int32_t i = 0; i < batch; ++i)
    if (indptr[i + 1] < indptr[i])
      return meta_fail(PKV_META_INDPTR_ORDER, std::string(name) + fmt(" decreases at %lld", i));
  return PKV_OK;
}

// The rule order mirrors the statement of the metadata contract: batch, page
// size, heads, qo_indptr, kv_indptr, index count, then per request its pages
// and tail, then per request qo_len against kv_len.
pkv_status validate_impl(const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_indices, int64_t num_indices,
                         const int32_t* last, int32_t batch, int32_t page_size,
                         int32_t max_num_pages, int32_t hq, int32_t hkv, bool decode,
                         std::vector<int32_t>* kv_len_out, bool check_qo_kv = true) {
  if (batch < 0) return meta_fail(PKV_META_BATCH_SIZE, "negative batch size");
  if (page_size < 1) return meta_fail(PKV_META_PAGE_SIZE, fmt("page_size %lld < 1", page_size));
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return meta_fail(PKV_META_HEAD_GROUP, fmt("%lld qo heads do not group over %lld kv heads", hq, hkv));
  if (!kv_indptr || (batch > 0 && !last)) return fail(PKV_ERR_INVALID_ARG, "null metadata pointer");
  if (qo_indptr) {
    pkv_status s = check_indptr("qo_indptr", qo_indptr, batch);
    if (s) return s;
  }
  pkv_status s = check_indptr("kv_indptr", kv_indptr, batch);
  if (s) return s;
  if (kv_indices && kv_indptr[batch] > num_indices)
    return meta_fail(PKV_META_INDICES_LENGTH,
                     fmt("kv_indptr[B] = %lld > %lld indices", kv_indptr[batch], num_indices));
  if (kv_len_out) kv_len_out->assign(batch, 0);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = kv_indptr[b + 1] - kv_indptr[b];
    if (n < 1) return meta_fail(PKV_META_EMPTY_PAGE_LIST, fmt("request %lld owns no page", b));
    if (kv_indices) {
      for (int32_t i = kv_indptr[b]; i < kv_indptr[b + 1]; ++i) {
        const int32_t p = kv_indices[i];
        if (p < 0 || p >= max_num_pages)
          return meta_fail(PKV_META_PAGE_INDEX,
                           fmt("request %lld: page %lld outside [0, %lld)", b, p, max_num_pages));
      }
    }
    if (last[b] < 1 || last[b] > page_size)
      return meta_fail(PKV_META_LAST_PAGE_LEN,
                       fmt("request %lld: tail %lld outside 1..%lld", b, last[b], page_size));
    const int64_t len = int64_t(page_size) * (n - 1) + last[b];
    if (len > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, fmt("request %lld: kv_len overflows int32", b));
    if (kv_len_out) (*kv_len_out)[b] = int32_t(len);
  }
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t q = qo_indptr ? int64_t(qo_indptr[b + 1]) - qo_indptr[b] : 1;
    const int64_t len = int64_t(page_size) * (kv_indptr[b + 1] - kv_indptr[b] - 1) + last[b];
    if (decode && q != 1)
      return meta_fail(PKV_META_DECODE_QO_LEN, fmt("request %lld: decode needs qo_len 1, got %lld", b, q));
    if (check_qo_kv && q > len)
      return meta_fail(PKV_META_QO_EXCEEDS_KV, fmt("request %lld: qo_len %lld > kv_len %lld", b, q, len));
  }
  return PKV_OK;
}

// ---------------------------------------------------------------- planner --

constexpr int32_t kMinSplitTokens = 256;
constexpr int64_t kMaxChunkPages = 1024;   // kernels stage one chunk's page ids on chip
constexpr int32_t kMfmaTileRows = 256;   // prefill tile height in (row, head) pairs

int32_t default_target(int32_t mode) {
  return mode == PKV_MODE_MLA_DECODE ? 1 : (mode == PKV_MODE_DECODE ? 3 : 4);
}
int32_t default_tail_split(int32_t mode) { return mode == PKV_MODE_DECODE ? 2 : 1; }
// The default tail split applies only while the kept chunks times the head
// slices number at most this many per CU: beyond that the longest-first order
// already ends on small items, and the extra items and merge rows only cost
// (2048 decode requests of 1-96 keys: 188 us unsplit against 349 us split).
constexpr int64_t kTailSplitMaxPerCu = 5;
// Decode plans run one-wave workgroups by default when their items average at
// most kOneWaveMaxKeys keys and number (times the kv heads) at least
// kOneWaveMinPerCu per CU.  Measured, attention + merge with 4-wave / one-wave
// workgroups (items x kv heads per CU, mean keys per item): 2048 requests of
// 1-96 keys (64, 47) 196 / 95 us; 1024 of 16-256 (32, 136) 144 / 110 us; 512
// of 64-512 (16, 291) 107 / 106 us; 384 of 128-1024 (12, 589) 146 / 169 us;
// the skewed batch (3.75, 355) 43 / 50 us; 64 of 512-4096 (5.9, 734) 94 / 123 us.
constexpr int64_t kOneWaveMaxKeys = 384;
constexpr int64_t kOneWaveMinPerCu = 24;
// MLA head groups: the kernel runs groups of 128 heads (one wave per 32
// heads) or of 64 heads (two waves per 32 heads).  By default the heads form
// groups of 128 when their count allows it, else groups of 64.
int32_t mla_head_groups(const pkv_plan_params* p) {
  if (p->mla_head_groups > 0) return p->mla_head_groups;
  return p->num_qo_heads % 128 == 0 ? p->num_qo_heads / 128 : p->num_qo_heads / 64;
}
bool mla_groups_ok(const pkv_plan_params* p, int64_t groups) {
  if (groups < 1 || p->num_qo_heads % groups != 0) return false;
  const int64_t width = p->num_qo_heads / groups;
  return width == 128 || width == 64;
}
constexpr int32_t kCascadeTargetPerCu = 1;

constexpr int32_t kRaggedPage = 16;   // ragged keys are chunked as if in pages of this many tokens
constexpr int32_t kMfmaHeadDim = 128;  // the head dim the MFMA prefill kernel is built for

// Query rows per work item.  Prefill over a bf16 or fp8 cache at the MFMA
// kernel's head dim gets a tile of 256 (row, head) pairs; every other case is
// one row per item, because the row kernel that runs it streams an item's
// keys once per row (a tall tile would serialise its rows in one workgroup).
int32_t rows_per_tile(int32_t mode, int32_t group, int32_t kv_dtype, int32_t mask_mode, int32_t head_dim) {
  if (mode != PKV_MODE_PREFILL || (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3)) return 1;
  if (head_dim != kMfmaHeadDim) return 1;
  if (mask_mode == PKV_MASK_CUSTOM && group < 2) return 1;   // masked tiles need a head group of 2+
  return std::max<int32_t>(1, kMfmaTileRows / group);
}

struct PlanResult {
  std::vector<Item> items;
  std::vector<MergeItem> merges;
  std::vector<pkv::MaskRow> mask_rows;   // custom-masked plans: one per request
  std::vector<int32_t> tile_merge;       // decode plans: merge item of request b's tile, or -1
  pkv_plan_info info;
};

// Paged decode plans carry the tables of the split merge inside the
// attention launch: per request its merge item (int32), and per (merge item,
// kv head) a counter of finished chunks (int32, zero between launches).
bool has_merge_tables(const pkv_plan_params* p) {
  return p->mode == PKV_MODE_DECODE && p->kv_format == PKV_KV_PAGED && p->mask_mode == PKV_MASK_NONE;
}

// Ragged metadata, in the oracle's order: heads, qo_indptr, kv_indptr, then
// qo_len <= kv_len per request.
pkv_status validate_ragged(const int32_t* qo_indptr, const int32_t* kv_indptr, int32_t batch, int32_t hq,
                           int32_t hkv) {
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return meta_fail(PKV_META_HEAD_GROUP, fmt("%lld qo heads do not group over %lld kv heads", hq, hkv));
  if (batch < 0) return meta_fail(PKV_META_BATCH_SIZE, "negative batch size");
  if (!qo_indptr || !kv_indptr) return fail(PKV_ERR_INVALID_ARG, "null metadata pointer");
  pkv_status s = check_indptr("qo_indptr", qo_indptr, batch);
  if (!s) s = check_indptr("kv_indptr", kv_indptr, batch);
  if (s) return s;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t q = int64_t(qo_indptr[b + 1]) - qo_indptr[b], k = int64_t(kv_indptr[b + 1]) - kv_indptr[b];
    if (q > k) return meta_fail(PKV_META_QO_EXCEEDS_KV, fmt("request %lld: qo_len %lld > kv_len %lld", b, q, k));
  }
  return PKV_OK;
}

uint64_t fnv1a(uint64_t h, const void* data, size_t bytes) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < bytes; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

uint64_t fingerprint(const pkv_plan_params& prm, const int32_t* qo, const int32_t* kv_indptr,
                     const int32_t* kv_indices, int64_t num_indices, const int32_t* last) {
  uint64_t h = 1469598103934665603ull;
  h = fnv1a(h, &prm, sizeof prm);
  const int32_t b = prm.batch_size;
  if (qo) h = fnv1a(h, qo, sizeof(int32_t) * (b + 1));
  h = fnv1a(h, kv_indptr, sizeof(int32_t) * (b + 1));
  if (b > 0 && last) h = fnv1a(h, last, sizeof(int32_t) * b);
  if (kv_indices) {
    const int64_t n = std::min<int64_t>(num_indices, kv_indptr[b]);
    h = fnv1a(h, kv_indices, sizeof(int32_t) * n);
  }
  return h;
}

pkv_status check_params(const pkv_plan_params* p) {
  if (!p) return fail(PKV_ERR_INVALID_ARG, "null params");
  if (p->mode < PKV_MODE_DECODE || p->mode > PKV_MODE_MLA_DECODE)
    return fail(PKV_ERR_INVALID_ARG, fmt("unknown mode %lld", p->mode));
  const bool fp8 = p->kv_dtype == PKV_FP8_E4M3;
  if (fp8 ? p->q_dtype != PKV_BF16 : p->q_dtype != p->kv_dtype)
    return fail(PKV_ERR_UNSUPPORTED, "q_dtype must equal kv_dtype (bf16 queries over an fp8 cache)");
  if (p->kv_dtype != PKV_F32 && p->kv_dtype != PKV_BF16 && !fp8)
    return fail(PKV_ERR_UNSUPPORTED, fmt("dtype %lld", p->kv_dtype));
  if (fp8 && p->mode == PKV_MODE_MLA_DECODE) return fail(PKV_ERR_UNSUPPORTED, "MLA runs on bf16 caches");
  if (p->head_dim_qk < 1 || p->head_dim_vo < 1) return fail(PKV_ERR_INVALID_ARG, "head dims must be >= 1");
  if (p->mode == PKV_MODE_MLA_DECODE) {
    if (p->num_kv_heads != 1 || p->head_dim_qk != 576 || p->head_dim_vo != 512 || p->kv_dtype != PKV_BF16)
      return fail(PKV_ERR_UNSUPPORTED, "MLA decode needs 1 kv head, dims 576/512, bf16");
  } else if (p->head_dim_qk != p->head_dim_vo) {
    return fail(PKV_ERR_UNSUPPORTED, "head_dim_qk must equal head_dim_vo outside MLA");
  }
  if (p->fixed_split_pages < 0 || p->target_per_cu < 0 || p->mla_head_groups < 0 || p->tail_split < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative planner knob");
  if (p->kv_format != PKV_KV_PAGED && p->kv_format != PKV_KV_RAGGED)
    return fail(PKV_ERR_INVALID_ARG, fmt("unknown kv_format %lld", p->kv_format));
  if (p->mask_mode != PKV_MASK_NONE && p->mask_mode != PKV_MASK_CUSTOM)
    return fail(PKV_ERR_INVALID_ARG, fmt("unknown mask_mode %lld", p->mask_mode));
  if (p->merge_in_launch != 0 && p->merge_in_launch != 1)
    return fail(PKV_ERR_INVALID_ARG, "merge_in_launch must be 0 or 1");
  if (p->row_waves != 0 && p->row_waves != 1 && p->row_waves != 4)
    return fail(PKV_ERR_INVALID_ARG, "row_waves must be 0, 1 or 4");
  if (p->row_waves == 1 && p->mode != PKV_MODE_DECODE)
    return fail(PKV_ERR_UNSUPPORTED, "one-wave row workgroups run decode plans only");
  if ((p->kv_format == PKV_KV_RAGGED || p->mask_mode == PKV_MASK_CUSTOM) && p->mode != PKV_MODE_PREFILL)
    return fail(PKV_ERR_UNSUPPORTED, "ragged KV and custom masks need prefill mode");
  if (p->mask_mode == PKV_MASK_CUSTOM && p->causal)
    return fail(PKV_ERR_INVALID_ARG, "a custom mask replaces the causal rule: set causal to 0");
  return PKV_OK;
}

// all_partial: every tile writes partial rows (a cascade merges them later);
// check_qo_kv = false drops the qo_len <= kv_len rule (a cascade's shared
// levels may hold fewer keys than their subtree has query rows).
pkv_status plan_impl(const pkv_plan_params* prm, const int32_t* qo_indptr, const int32_t* kv_indptr,
                     const int32_t* kv_indices, int64_t num_indices, const int32_t* last,
                     PlanResult* out, bool all_partial = false, bool check_qo_kv = true) {
  pkv_status s = check_params(prm);
  if (s) return s;
  const bool prefill = prm->mode == PKV_MODE_PREFILL;
  const bool mla = prm->mode == PKV_MODE_MLA_DECODE;
  if (!prefill && qo_indptr) return fail(PKV_ERR_INVALID_ARG, "decode modes take no qo_indptr");
  if (prefill && !qo_indptr) return fail(PKV_ERR_INVALID_ARG, "prefill needs qo_indptr");
  const int32_t batch = prm->batch_size;
  const int32_t max_pages = prm->max_num_pages > 0 ? prm->max_num_pages : INT32_MAX;
  const bool ragged = prm->kv_format == PKV_KV_RAGGED;
  std::vector<int32_t> kv_len;
  // Ragged keys are planned over a virtual page table of kRaggedPage-token
  // pages; items then address request b's keys from entry b of kv_indptr.
  std::vector<int32_t> v_indptr, v_last;
  int32_t page_size = prm->page_size;
  const int32_t* const user_kv_indptr = kv_indptr;
  const int32_t* const user_last = last;
  if (ragged) {
    s = validate_ragged(qo_indptr, kv_indptr, batch, prm->num_qo_heads, prm->num_kv_heads);
    if (s) return s;
    page_size = kRaggedPage;
    v_indptr.assign(size_t(batch) + 1, 0);
    v_last.assign(size_t(batch), 0);
    kv_len.assign(size_t(batch), 0);
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t k = kv_indptr[b + 1] - kv_indptr[b];
      const int32_t n = int32_t(cdiv(k, kRaggedPage));
      kv_len[b] = k;
      v_indptr[b + 1] = v_indptr[b] + n;
      v_last[b] = n ? k - kRaggedPage * (n - 1) : 0;
    }
    kv_indptr = v_indptr.data();
    last = v_last.data();
  } else {
    s = validate_impl(qo_indptr, kv_indptr, kv_indices, num_indices, last, batch, prm->page_size,
                      max_pages, prm->num_qo_heads, prm->num_kv_heads, !prefill, &kv_len, check_qo_kv);
    if (s) return s;
  }

  int32_t num_cus = prm->num_cus;
  if (num_cus <= 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "querying the compute-unit count");
  }
  const int32_t group = prm->num_qo_heads / prm->num_kv_heads;
  const int32_t rows = rows_per_tile(prm->mode, group, prm->kv_dtype, prm->mask_mode, prm->head_dim_qk);
  int32_t heads_y = prm->num_kv_heads;
  if (mla) {
    heads_y = mla_head_groups(prm);
    if (!mla_groups_ok(prm, heads_y)) return fail(PKV_ERR_UNSUPPORTED, "MLA decode runs head groups of 64 or 128 heads");
  }
  const int32_t target_per_cu = prm->target_per_cu > 0 ? prm->target_per_cu : default_target(prm->mode);
  int32_t tail_split = prm->tail_split > 0 ? prm->tail_split : default_tail_split(prm->mode);
  const bool causal = prefill ? prm->causal != 0 : true;

  // Step 1-3: tiles, page work, chunk size.
  std::vector<int64_t> q_len(batch), n_pages(batch), tiles(batch);
  int64_t work = 0;
  int64_t total_rows = 0;
  for (int32_t b = 0; b < batch; ++b) {
    q_len[b] = prefill ? int64_t(qo_indptr[b + 1]) - qo_indptr[b] : 1;
    n_pages[b] = kv_indptr[b + 1] - kv_indptr[b];
    tiles[b] = cdiv(q_len[b], rows);
    work += tiles[b] * n_pages[b] * heads_y;
    total_rows += q_len[b];
  }
  const int64_t target = int64_t(target_per_cu) * num_cus;
  int64_t chunk = prm->fixed_split_pages > 0
                      ? prm->fixed_split_pages
                      : std::max<int64_t>(cdiv(kMinSplitTokens, page_size), cdiv(work, target));
  chunk = std::min(chunk, kMaxChunkPages);
  if (mla && prm->fixed_split_pages <= 0) {
    // The MLA kernel holds one workgroup per CU: grow the chunk to the
    // smallest size whose workgroup count fits the target, so the rounding of
    // every request to whole chunks does not spill into a second round.
    auto units = [&](int64_t c) {
      int64_t u = 0;
      for (int32_t b = 0; b < batch; ++b) u += tiles[b] * cdiv(n_pages[b], c);
      return u * heads_y;
    };
    if (units(kMaxChunkPages) <= target) {
      int64_t lo = chunk, hi = kMaxChunkPages;
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (units(mid) <= target) hi = mid;
        else lo = mid + 1;
      }
      chunk = lo;
    } else {
      chunk = kMaxChunkPages;
    }
  }
  const int64_t chunk_tokens = chunk * page_size;
  // Keys of tile t of request b that some row of the tile sees: [0, limit).
  auto tile_limit = [&](int32_t b, int64_t t) {
    const int64_t k = kv_len[b];
    const int64_t l0 = t * rows;
    const int64_t diag = causal ? k - q_len[b] + l0 : k;
    return std::min<int64_t>(k, diag + std::min<int64_t>(rows, q_len[b] - l0));
  };
  if (prm->tail_split <= 0 && tail_split > 1) {
    int64_t units = 0;   // kept chunks of every tile (step 5) before any tail split
    for (int32_t b = 0; b < batch; ++b)
      for (int64_t t = 0; t < tiles[b]; ++t)
        units += std::min(cdiv(n_pages[b], chunk), std::max<int64_t>(0, cdiv(tile_limit(b, t), chunk_tokens)));
    if (units * heads_y > kTailSplitMaxPerCu * num_cus) tail_split = 1;
  }

  // Step 4-6: chunks per tile, causal pruning, partial-row assignment.
  struct Raw {
    int64_t cost;
    int32_t b, t, c;
    Item it;
  };
  std::vector<Raw> raw;
  out->merges.clear();
  int64_t slot = 0;
  bool split_any = false;
  std::vector<std::pair<int32_t, int32_t>> kept;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t k = kv_len[b];
    for (int64_t t = 0; t < tiles[b]; ++t) {
      const int64_t l0 = t * rows;
      const int64_t n_rows = std::min<int64_t>(rows, q_len[b] - l0);
      const int64_t diag = causal ? k - q_len[b] + l0 : k;
      const int64_t limit = std::min<int64_t>(k, diag + n_rows);
      kept.clear();
      const int64_t n_chunks = cdiv(n_pages[b], chunk);
      for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t lo = c * chunk_tokens;
        if (lo >= limit) break;
        const int64_t hi = std::min<int64_t>(std::min<int64_t>(lo + chunk_tokens, k), limit);
        kept.emplace_back(int32_t(lo), int32_t(hi));
      }
      // Tail split: the tile's final chunk, if longer than one page, becomes
      // tail_split page-aligned pieces, so the end of the longest-first order
      // is made of small items.
      if (tail_split > 1 && !kept.empty()) {
        const int64_t lo = kept.back().first, hi = kept.back().second;
        const int64_t pages = cdiv(hi - lo, page_size);
        if (pages > 1) {
          kept.pop_back();
          const int64_t step = cdiv(pages, tail_split) * page_size;
          for (int64_t s0 = lo; s0 < hi; s0 += step)
            kept.emplace_back(int32_t(s0), int32_t(std::min<int64_t>(hi, s0 + step)));
        }
      }
      const int32_t q_row0 = int32_t((prefill ? qo_indptr[b] : b) + l0);
      if (kept.size() == 1 && !all_partial) {
        Item it{q_row0, int32_t(n_rows), kept[0].first, kept[0].second, int32_t(diag), kv_indptr[b], -1, b};
        raw.push_back({int64_t(kept[0].second - kept[0].first), b, int32_t(t), 0, it});
        continue;
      }
      split_any = true;
      if (slot + int64_t(kept.size()) * n_rows > INT32_MAX)
        return fail(PKV_ERR_INVALID_ARG, "too many partial rows");
      out->merges.push_back({q_row0, int32_t(n_rows), int32_t(slot), int32_t(kept.size())});
      for (size_t ci = 0; ci < kept.size(); ++ci) {
        Item it{q_row0, int32_t(n_rows), kept[ci].first, kept[ci].second, int32_t(diag), kv_indptr[b],
                int32_t(slot + int64_t(ci) * n_rows), b};
        raw.push_back({int64_t(kept[ci].second - kept[ci].first), b, int32_t(t), int32_t(ci), it});
      }
      slot += int64_t(kept.size()) * n_rows;
    }
  }
  // Step 7: most keys first (a tile's kernel time follows its key count, not
  // its row count); (b, t, c) breaks ties, so the order is unique.
  std::sort(raw.begin(), raw.end(), [](const Raw& x, const Raw& y) {
    if (x.cost != y.cost) return x.cost > y.cost;
    if (x.b != y.b) return x.b < y.b;
    if (x.t != y.t) return x.t < y.t;
    return x.c < y.c;
  });
  if (raw.size() > size_t(INT32_MAX)) return fail(PKV_ERR_INVALID_ARG, "too many work items");
  out->items.resize(raw.size());
  for (size_t i = 0; i < raw.size(); ++i) out->items[i] = raw[i].it;
  if (ragged)
    for (Item& it : out->items) it.page_base = it.batch;   // entry b of kv_indptr: request b's first key
  // Custom mask: where each request's rows start in the packed mask.
  out->mask_rows.clear();
  int64_t mask_bits = 0;
  if (prm->mask_mode == PKV_MASK_CUSTOM) {
    out->mask_rows.resize(size_t(batch));
    for (int32_t b = 0; b < batch; ++b) {
      out->mask_rows[b] = {mask_bits, qo_indptr[b], kv_len[b]};
      mask_bits += q_len[b] * int64_t(kv_len[b]);
    }
  }

  out->tile_merge.clear();
  if (has_merge_tables(prm)) {   // a decode tile is one request: merge item q_row0 == b
    out->tile_merge.assign(size_t(batch), -1);
    for (size_t m = 0; m < out->merges.size(); ++m) out->tile_merge[size_t(out->merges[m].q_row0)] = int32_t(m);
  }

  pkv_plan_info& in = out->info;
  std::memset(&in, 0, sizeof in);
  in.mode = prm->mode;
  in.batch_size = batch;
  in.num_items = int32_t(out->items.size());
  in.num_merges = int32_t(out->merges.size());
  in.num_partial_rows = int32_t(slot);
  in.chunk_pages = int32_t(std::min<int64_t>(chunk, INT32_MAX));
  in.split = split_any ? 1 : 0;
  in.rows_per_tile = rows;
  in.heads_y = heads_y;
  in.num_cus = num_cus;
  in.target = int32_t(std::min<int64_t>(target, INT32_MAX));
  in.total_rows = int32_t(total_rows);
  in.row_waves = 4;
  if (prm->row_waves > 0) {
    in.row_waves = prm->row_waves;
  } else if (prm->mode == PKV_MODE_DECODE && !out->items.empty()) {
    int64_t keys = 0;
    for (const Item& it : out->items) keys += int64_t(it.kv_end) - it.kv_start;
    const int64_t n = int64_t(out->items.size());
    if (keys <= kOneWaveMaxKeys * n && n * heads_y >= kOneWaveMinPerCu * num_cus) in.row_waves = 1;
  }
  const int64_t hq = prm->num_qo_heads;
  in.mask_bits = mask_bits;
  const int64_t merge_ctrs = out->tile_merge.empty() ? 0 : int64_t(out->merges.size()) * prm->num_kv_heads;
  const int64_t staging = align256(int64_t(out->items.size()) * sizeof(Item)) +
                          align256(int64_t(out->merges.size()) * sizeof(MergeItem)) +
                          align256(int64_t(out->mask_rows.size()) * sizeof(pkv::MaskRow)) +
                          align256(int64_t(out->tile_merge.size()) * 4) + align256(merge_ctrs * 4);
  in.staging_bytes = staging;
  in.workspace_bytes = staging + align256(slot * hq * 4) + align256(slot * hq * prm->head_dim_vo * 4);
  in.fingerprint = fingerprint(*prm, qo_indptr, user_kv_indptr, kv_indices, num_indices, user_last);
  return PKV_OK;
}

// ---------------------------------------------------------------- cascade --

struct CascadeResult {
  std::vector<Item> items;
  std::vector<int32_t> row_ptr, slots;
  std::vector<pkv_plan_info> level_info;
  std::vector<int32_t> level_mode, level_item_off;
  pkv_cascade_info info;
};

// Level checks in the oracle's order: every level's page-table rules (a
// shared level without qo_len <= kv_len, its qo_indptr checked after its
// pages), then equal row counts, then nesting.
pkv_status cascade_validate(const pkv_plan_params* prm, int32_t num_levels, const pkv_cascade_level* lv) {
  if (num_levels < 1 || !lv) return meta_fail(PKV_META_CASCADE_ROWS, "a cascade needs at least one level");
  const int32_t max_pages = prm->max_num_pages > 0 ? prm->max_num_pages : INT32_MAX;
  for (int32_t l = 0; l < num_levels; ++l) {
    const pkv_cascade_level& L = lv[l];
    if (L.num_nodes < 0) return meta_fail(PKV_META_BATCH_SIZE, fmt("level %lld: negative node count", l));
    if (!L.qo_indptr) return fail(PKV_ERR_INVALID_ARG, fmt("level %lld: null qo_indptr", l));
    pkv_status s;
    if (l == num_levels - 1) {
      s = validate_impl(L.qo_indptr, L.kv_indptr, L.kv_indices, L.num_indices, L.kv_last_page_len, L.num_nodes,
                        prm->page_size, max_pages, prm->num_qo_heads, prm->num_kv_heads, false, nullptr);
    } else {
      s = validate_impl(nullptr, L.kv_indptr, L.kv_indices, L.num_indices, L.kv_last_page_len, L.num_nodes,
                        prm->page_size, max_pages, prm->num_qo_heads, prm->num_kv_heads, false, nullptr);
      if (!s) s = check_indptr("qo_indptr", L.qo_indptr, L.num_nodes);
    }
    if (s) return s;
  }
  const int32_t rows = lv[0].qo_indptr[lv[0].num_nodes];
  for (int32_t l = 1; l < num_levels; ++l)
    if (lv[l].qo_indptr[lv[l].num_nodes] != rows)
      return meta_fail(PKV_META_CASCADE_ROWS, fmt("level %lld covers %lld query rows, level 0 %lld", l,
                                                  lv[l].qo_indptr[lv[l].num_nodes], rows));
  for (int32_t l = 0; l + 1 < num_levels; ++l) {
    const pkv_cascade_level& up = lv[l];
    const pkv_cascade_level& dn = lv[l + 1];
    // Both indptrs are non-decreasing: walk them together.
    int32_t j = 0;
    for (int32_t i = 0; i <= up.num_nodes; ++i) {
      const int32_t b = up.qo_indptr[i];
      while (j <= dn.num_nodes && dn.qo_indptr[j] < b) ++j;
      if (j > dn.num_nodes || dn.qo_indptr[j] != b)
        return meta_fail(PKV_META_CASCADE_NESTING,
                         fmt("level %lld has node boundary %lld that level %lld does not", l, b, l + 1));
    }
  }
  return PKV_OK;
}

pkv_status cascade_impl(const pkv_plan_params* prm, int32_t num_levels, const pkv_cascade_level* lv,
                        CascadeResult* out) {
  if (prm->kv_format != PKV_KV_PAGED || prm->mask_mode != PKV_MASK_NONE)
    return fail(PKV_ERR_UNSUPPORTED, "cascades run on paged caches without custom masks");
  pkv_status s = cascade_validate(prm, num_levels, lv);
  if (s) return s;
  const int32_t rows = lv[0].qo_indptr[lv[0].num_nodes];
  std::vector<std::vector<int32_t>> per_row(static_cast<size_t>(rows));
  out->items.clear();
  out->level_info.clear();
  out->level_mode.clear();
  out->level_item_off.clear();
  int64_t slot_base = 0, page_base = 0;
  uint64_t h = 1469598103934665603ull;
  for (int32_t l = 0; l < num_levels; ++l) {
    const pkv_cascade_level& L = lv[l];
    bool one_row = L.num_nodes > 0;
    for (int32_t n = 0; n < L.num_nodes && one_row; ++n) one_row = L.qo_indptr[n + 1] - L.qo_indptr[n] == 1;
    pkv_plan_params p = *prm;
    p.mode = one_row ? PKV_MODE_DECODE : PKV_MODE_PREFILL;
    p.batch_size = L.num_nodes;
    p.causal = (prm->causal && l == num_levels - 1) ? 1 : 0;
    // A level is one launch of its own: by default one item per CU (larger
    // chunks also leave fewer partial states to merge).
    if (p.target_per_cu <= 0) p.target_per_cu = kCascadeTargetPerCu;
    PlanResult r;
    s = plan_impl(&p, one_row ? nullptr : L.qo_indptr, L.kv_indptr, L.kv_indices, L.num_indices,
                  L.kv_last_page_len, &r, true, l == num_levels - 1);
    if (s) return s;
    if (slot_base + r.info.num_partial_rows > INT32_MAX || page_base + L.kv_indptr[L.num_nodes] > INT32_MAX)
      return fail(PKV_ERR_INVALID_ARG, "cascade too large for int32 slots or page offsets");
    out->level_item_off.push_back(int32_t(out->items.size()));
    for (Item it : r.items) {
      it.page_base += int32_t(page_base);
      it.out_slot += int32_t(slot_base);
      out->items.push_back(it);
    }
    for (const MergeItem& m : r.merges)
      for (int32_t rr = 0; rr < m.num_rows; ++rr)
        for (int32_t c = 0; c < m.num_chunks; ++c)
          per_row[size_t(m.q_row0 + rr)].push_back(int32_t(slot_base + m.slot0 + int64_t(c) * m.num_rows + rr));
    out->level_info.push_back(r.info);
    out->level_mode.push_back(p.mode);
    h = fnv1a(h, &r.info.fingerprint, sizeof(uint64_t));
    h = fnv1a(h, L.qo_indptr, sizeof(int32_t) * (L.num_nodes + 1));   // decode levels do not hash it
    slot_base += r.info.num_partial_rows;
    page_base += L.kv_indptr[L.num_nodes];
  }
  out->row_ptr.assign(size_t(rows) + 1, 0);
  out->slots.clear();
  out->slots.reserve(size_t(slot_base));
  for (int32_t r = 0; r < rows; ++r) {
    out->slots.insert(out->slots.end(), per_row[size_t(r)].begin(), per_row[size_t(r)].end());
    out->row_ptr[size_t(r) + 1] = int32_t(out->slots.size());
  }
  pkv_cascade_info& in = out->info;
  std::memset(&in, 0, sizeof in);
  in.num_levels = num_levels;
  in.total_rows = rows;
  in.num_items = int32_t(out->items.size());
  in.num_partial_rows = int32_t(slot_base);
  in.num_merge_slots = int32_t(out->slots.size());
  const int64_t hq = prm->num_qo_heads;
  in.staging_bytes = align256(int64_t(out->items.size()) * sizeof(Item)) + align256(int64_t(rows + 1) * 4) +
                     align256(int64_t(out->slots.size()) * 4);
  in.workspace_bytes = in.staging_bytes + align256(slot_base * hq * 4) + align256(slot_base * hq * prm->head_dim_vo * 4);
  in.fingerprint = h;
  return PKV_OK;
}

// Pinned staging buffers remember the event of the last upload made from
// them and the plan that made it, so a later plan does not overwrite bytes
// still being copied.  An entry lives as long as that plan: destroying the
// plan waits for its upload and drops the entry (and its event) unless a
// later plan has reused the buffer since.  A buffer whose address is reused
// after its last plan is gone therefore starts without a stale event.
struct StagingSlot {
  hipEvent_t event;
  const void* owner;   // the plan whose upload the event records
};
std::mutex g_staging_mu;
std::unordered_map<void*, StagingSlot> g_staging;

// Copies a plan's host-built tables to the start of the device workspace.
// With a pinned staging buffer the copy is asynchronous; the buffer's event
// records it, and a later upload from the same buffer first waits for that
// event.  Without one, the bytes go through a temporary host vector and the
// stream is synchronised before it is freed.
hipError_t upload_staging(void* h_staging, void* ws, int64_t bytes, hipStream_t st, const void* owner,
                          const std::function<void(char*)>& fill) {
  hipError_t e;
  if (h_staging) {
    std::lock_guard<std::mutex> lock(g_staging_mu);
    auto it = g_staging.find(h_staging);
    if (it == g_staging.end()) {
      hipEvent_t ev;
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
      it = g_staging.emplace(h_staging, StagingSlot{ev, owner}).first;
    } else {
      e = hipEventSynchronize(it->second.event);   // the previous upload from this buffer
      if (e != hipSuccess) return e;
    }
    it->second.owner = owner;
    char* hs = static_cast<char*>(h_staging);
    std::memset(hs, 0, size_t(bytes));
    fill(hs);
    e = hipMemcpyAsync(ws, hs, size_t(bytes), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipEventRecord(it->second.event, st);
    return e;
  }
  std::vector<char> tmp(size_t(bytes), 0);
  fill(tmp.data());
  e = hipMemcpyAsync(ws, tmp.data(), tmp.size(), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return e;
}

// Called when `owner` is destroyed: if it made the last upload from
// h_staging, wait for that upload and release the buffer's event.
void release_staging(void* h_staging, const void* owner) {
  if (!h_staging) return;
  std::lock_guard<std::mutex> lock(g_staging_mu);
  auto it = g_staging.find(h_staging);
  if (it == g_staging.end() || it->second.owner != owner) return;
  (void)hipEventSynchronize(it->second.event);
  (void)hipEventDestroy(it->second.event);
  g_staging.erase(it);
}

// Plans that lead to a run must bound the page ids they will dereference.
// The MLA run takes raw cache pointers without a descriptor, so its plan
// carries the pool size.
// Whether workgroups i and i + 8 of a launch run on one XCD on `device`
// (the order in which the command processor hands workgroups to the XCDs),
// checked once per device with a small probe launch: the split merge inside
// the decode launch relies on it.  A failed check (or PKV_MERGE_IN_ATTENTION=0)
// leaves the merge to its own launch.
bool xcd_groups_ok(int device) {
  static std::mutex mu;
  static std::unordered_map<int, bool> known;
  std::lock_guard<std::mutex> lock(mu);
  auto f = known.find(device);
  if (f != known.end()) return f->second;
  bool ok = false;
  const char* env = std::getenv("PKV_MERGE_IN_ATTENTION");
  if (!(env && env[0] == '0')) {
    constexpr int32_t kBlocks = 1024;
    int32_t* d = nullptr;
    std::vector<int32_t> h(kBlocks, -1);
    if (hipMalloc(&d, kBlocks * sizeof(int32_t)) == hipSuccess) {
      if (pkv::launch_xcd_probe(d, kBlocks, nullptr) == hipSuccess &&
          hipMemcpy(h.data(), d, kBlocks * sizeof(int32_t), hipMemcpyDeviceToHost) == hipSuccess) {
        ok = true;
        for (int32_t i = 0; i < kBlocks; ++i) ok = ok && h[i] >= 0 && h[i] == h[i % 8];
      }
      (void)hipFree(d);
    }
    (void)hipGetLastError();   // a failed probe only turns the fused merge off
  }
  known[device] = ok;
  return ok;
}

// Whether run() folds a plan's split rows inside the attention launch: a
// paged decode plan (one row per tile, each chunk of it one workgroup per kv
// head: workgroup item * Hkv + j serves head (j + b) mod Hkv of request b),
// kv heads a multiple of 8 so that every chunk of one (request, kv head)
// lands on the same XCD.
constexpr int32_t kMergeInMaxChunks = 16;   // plans whose rows have more chunks merge in their own launch

bool merge_in_launch_ok(const pkv_plan_params* p, int device) {
  return p->merge_in_launch == 1 && has_merge_tables(p) && p->num_kv_heads % 8 == 0 && xcd_groups_ok(device);
}

pkv_status check_runnable(const pkv_plan_params* p) {
  if (p && p->mode == PKV_MODE_MLA_DECODE && p->max_num_pages <= 0)
    return fail(PKV_ERR_INVALID_ARG, "MLA plans need max_num_pages (the pool size): pkv_run_mla has no "
                                     "cache descriptor to bound page ids by");
  return PKV_OK;
}

}  // namespace

struct pkv_plan {
  pkv_plan_params params;
  pkv_plan_info info;
  Item* d_items;
  MergeItem* d_merges;
  pkv::MaskRow* d_mask_rows = nullptr;   // custom-masked plans
  float* d_part_lse;
  float* d_part_o;
  int device;
  // Split merge inside the attention launch (decode plans whose kv heads
  // are a multiple of 8 on a device that runs workgroups i and i + 8 on one
  // XCD): the tables, and whether run() uses them.
  int32_t* d_tile_merge = nullptr;
  int32_t* d_merge_ctr = nullptr;
  bool merge_in = false;
  // Fixed-capacity plans (pkv_graph_plan_create): every run launches grids
  // sized by the capacities and the kernels read the live counts from
  // d_counts, so one captured graph serves every later update.
  bool graph = false;
  pkv_graph_caps caps{};
  int32_t* d_counts = nullptr;   // [0] live items, [1] live merge items
  char* d_ws = nullptr;
  void* h_staging = nullptr;   // pinned staging of the uploads (fixed-capacity plans: also of updates)
  int64_t staging_bytes = 0;

  int32_t grid_items() const { return graph ? caps.max_items : info.num_items; }
  int32_t grid_merges() const { return graph ? caps.max_merges : info.num_merges; }
  const int32_t* live_items() const { return graph ? d_counts : nullptr; }
  const int32_t* live_merges() const { return graph ? d_counts + 1 : nullptr; }
};

extern "C" {

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }
const char* pkv_last_error(void) { return g_error.c_str(); }
int32_t pkv_last_meta_reason(void) { return g_reason; }

pkv_status pkv_device_num_cus(int32_t* out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "null output");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  return ok();
}

pkv_status pkv_validate(const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                        int64_t num_indices, const int32_t* kv_last_page_len, int32_t batch_size,
                        int32_t page_size, int32_t max_num_pages, int32_t num_qo_heads,
                        int32_t num_kv_heads, int32_t decode, int32_t* kv_len_out) {
  std::vector<int32_t> lens;
  pkv_status s = validate_impl(qo_indptr, kv_indptr, kv_indices, num_indices, kv_last_page_len,
                               batch_size, page_size, max_num_pages, num_qo_heads, num_kv_heads,
                               decode != 0, &lens);
  if (s) return s;
  if (kv_len_out) std::copy(lens.begin(), lens.end(), kv_len_out);
  return ok();
}

pkv_status pkv_validate_append(const int32_t* append_indptr, const int32_t* kv_indptr,
                               const int32_t* kv_indices, int64_t num_indices,
                               const int32_t* kv_last_page_len, int32_t batch_size, int32_t page_size,
                               int32_t max_num_pages) {
  if (!append_indptr || !kv_indices) return fail(PKV_ERR_INVALID_ARG, "null metadata pointer");
  std::vector<int32_t> lens;
  pkv_status s = validate_impl(append_indptr, kv_indptr, kv_indices, num_indices, kv_last_page_len,
                               batch_size, page_size, max_num_pages, 1, 1, false, &lens);
  if (s) return s;
  std::unordered_set<int64_t> seen;
  for (int32_t b = 0; b < batch_size; ++b) {
    const int32_t n = append_indptr[b + 1] - append_indptr[b];
    for (int32_t t = 0; t < n; ++t) {
      const int64_t pos = int64_t(lens[b]) - n + t;
      const int64_t page = kv_indices[kv_indptr[b] + pos / page_size];
      const int64_t key = page * page_size + pos % page_size;
      if (!seen.insert(key).second)
        return meta_fail(PKV_META_APPEND_COLLISION,
                         fmt("page %lld slot %lld written twice", page, pos % page_size));
    }
  }
  return ok();
}

pkv_status pkv_plan_compute(const pkv_plan_params* params, const int32_t* qo_indptr,
                            const int32_t* kv_indptr, const int32_t* kv_indices, int64_t num_indices,
                            const int32_t* kv_last_page_len, int32_t* items_out, int64_t items_capacity,
                            int32_t* merges_out, int64_t merges_capacity, pkv_plan_info* info) {
  PlanResult r;
  pkv_status s = plan_impl(params, qo_indptr, kv_indptr, kv_indices, num_indices, kv_last_page_len, &r);
  if (s) return s;
  if (info) *info = r.info;
  if (items_out) {
    if (items_capacity < int64_t(r.items.size()) * PKV_ITEM_WORDS)
      return fail(PKV_ERR_WORKSPACE, "work-item buffer too small");
    copy_table(items_out, r.items);
  }
  if (merges_out) {
    if (merges_capacity < int64_t(r.merges.size()) * PKV_MERGE_WORDS)
      return fail(PKV_ERR_WORKSPACE, "merge buffer too small");
    copy_table(merges_out, r.merges);
  }
  return ok();
}

pkv_status pkv_plan_create(const pkv_plan_params* params, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, const int32_t* kv_indices, int64_t num_indices,
                           const int32_t* kv_last_page_len, void* d_workspace, size_t ws_bytes,
                           void* h_staging, size_t staging_bytes, void* stream, pkv_plan** plan_out) {
  if (!plan_out) return fail(PKV_ERR_INVALID_ARG, "null plan_out");
  *plan_out = nullptr;
  PlanResult r;
  pkv_status s = plan_impl(params, qo_indptr, kv_indptr, kv_indices, num_indices, kv_last_page_len, &r);
  if (!s) s = check_runnable(params);
  if (s) return s;
  const pkv_plan_info& in = r.info;
  if (in.workspace_bytes > 0 && (!d_workspace || int64_t(ws_bytes) < in.workspace_bytes))
    return fail(PKV_ERR_WORKSPACE, fmt("workspace %lld bytes < %lld needed", int64_t(ws_bytes),
                                       in.workspace_bytes));
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256 != 0)
    return fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (h_staging && int64_t(staging_bytes) < in.staging_bytes)
    return fail(PKV_ERR_WORKSPACE, fmt("staging %lld bytes < %lld needed", int64_t(staging_bytes),
                                       in.staging_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(d_workspace);
  const int64_t items_bytes = align256(int64_t(r.items.size()) * sizeof(Item));
  const int64_t merges_bytes = align256(int64_t(r.merges.size()) * sizeof(MergeItem));
  const int64_t lse_bytes = align256(int64_t(in.num_partial_rows) * params->num_qo_heads * 4);

  pkv_plan* plan = new pkv_plan;
  plan->params = *params;
  plan->info = in;
  plan->d_items = reinterpret_cast<Item*>(ws);
  plan->d_merges = reinterpret_cast<MergeItem*>(ws + items_bytes);
  plan->d_mask_rows = reinterpret_cast<pkv::MaskRow*>(ws + items_bytes + merges_bytes);
  plan->d_part_lse = reinterpret_cast<float*>(ws + in.staging_bytes);
  plan->d_part_o = reinterpret_cast<float*>(ws + in.staging_bytes + lse_bytes);
  const int64_t tm_off = items_bytes + merges_bytes + align256(int64_t(r.mask_rows.size()) * sizeof(pkv::MaskRow));
  const int64_t ctr_off = tm_off + align256(int64_t(r.tile_merge.size()) * 4);
  const int64_t ctr_bytes = r.tile_merge.empty() ? 0 : int64_t(r.merges.size()) * params->num_kv_heads * 4;
  hipError_t e = hipGetDevice(&plan->device);
  if (e != hipSuccess) {
    delete plan;
    return hip_fail(e, "hipGetDevice");
  }
  if (!r.tile_merge.empty()) {
    plan->d_tile_merge = reinterpret_cast<int32_t*>(ws + tm_off);
    plan->d_merge_ctr = reinterpret_cast<int32_t*>(ws + ctr_off);
    // One workgroup merges a row's chunks at the end of the launch: with
    // many chunks (one long request split many ways) that serial tail costs
    // more than a merge launch of its own.
    int32_t most = 0;
    for (const MergeItem& mi : r.merges) most = std::max(most, mi.num_chunks);
    // One-wave workgroups fold no merge inside the launch.
    plan->merge_in = r.info.row_waves == 4 && !r.merges.empty() && most <= kMergeInMaxChunks &&
                     merge_in_launch_ok(params, plan->device);
  }
  plan->info.merge_in_launch = plan->merge_in ? 1 : 0;
  plan->h_staging = h_staging;
  if (in.staging_bytes > 0) {
    e = upload_staging(h_staging, ws, in.staging_bytes, st, plan, [&](char* hs) {
      copy_table(hs, r.items);
      copy_table(hs + items_bytes, r.merges);
      copy_table(hs + items_bytes + merges_bytes, r.mask_rows);
      copy_table(hs + tm_off, r.tile_merge);
      std::memset(hs + ctr_off, 0, size_t(ctr_bytes));   // counters start at zero
    });
    if (e != hipSuccess) {
      release_staging(h_staging, plan);
      delete plan;
      return hip_fail(e, "uploading the plan");
    }
  }
  if (const char* lg = std::getenv("PKV_LOG")) {
    if (lg[0] == '1')
      std::fprintf(stderr, "[pkv] plan mode=%d B=%d items=%d merges=%d chunk_pages=%d split=%d ws=%lld\n",
                   in.mode, in.batch_size, in.num_items, in.num_merges, in.chunk_pages, in.split,
                   (long long)in.workspace_bytes);
  }
  *plan_out = plan;
  return ok();
}

pkv_status pkv_plan_get_info(const pkv_plan* plan, pkv_plan_info* info) {
  if (!plan || !info) return fail(PKV_ERR_INVALID_ARG, "null argument");
  *info = plan->info;
  return ok();
}

pkv_status pkv_plan_check(const pkv_plan* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_indices, int64_t num_indices,
                          const int32_t* kv_last_page_len) {
  if (!plan || !kv_indptr) return fail(PKV_ERR_INVALID_ARG, "null argument");
  const uint64_t h = fingerprint(plan->params, qo_indptr, kv_indptr, kv_indices, num_indices,
                                 kv_last_page_len);
  if (h != plan->info.fingerprint)
    return fail(PKV_ERR_STALE_PLAN, "metadata differs from the batch the plan was built for");
  return ok();
}

pkv_status pkv_plan_destroy(pkv_plan* plan) {
  if (plan) release_staging(plan->h_staging, plan);
  delete plan;
  return ok();
}

// ------------------------------------------------------------------- run --

static pkv_status check_ptr16(const void* p, const char* what) {
  if (!p) return fail(PKV_ERR_INVALID_ARG, std::string("null ") + what);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, std::string(what) + " must be 16-byte aligned");
  return PKV_OK;
}

static bool stride_ok(int64_t stride, size_t esize) { return stride >= 0 && (stride * int64_t(esize)) % 16 == 0; }

}  // extern "C"

namespace {

// Argument checks shared by pkv_run_attention and pkv_cascade_run; fills
// every AttnArgs field except the work list and the partial buffers.
pkv_status prepare_attn(const pkv_plan_params& p, int plan_device, bool has_items, const void* q,
                        int64_t q_stride_token, int64_t q_stride_head, const pkv_cache_desc* cache,
                        const int32_t* d_kv_indices, void* o, int64_t o_stride_token, int64_t o_stride_head,
                        float* lse, float sm_scale, pkv::AttnArgs* a) {
  if (!cache) return fail(PKV_ERR_INVALID_ARG, "null cache");
  if (cache->page_size != p.page_size || cache->num_kv_heads != p.num_kv_heads ||
      cache->head_dim != p.head_dim_qk || cache->dtype != p.kv_dtype)
    return fail(PKV_ERR_INVALID_ARG, "cache descriptor does not match the plan");
  if (p.max_num_pages > 0 && cache->max_num_pages != p.max_num_pages)
    return fail(PKV_ERR_INVALID_ARG, "cache page count does not match the plan");
  const size_t es = dtype_size(p.q_dtype), es_kv = dtype_size(p.kv_dtype);
  pkv_status s;
  if ((s = check_ptr16(q, "q")) || (s = check_ptr16(o, "o")) || (s = check_ptr16(cache->k, "cache k")) ||
      (s = check_ptr16(cache->v, "cache v")))
    return s;
  if (!d_kv_indices && has_items) return fail(PKV_ERR_INVALID_ARG, "null kv_indices");
  if (!stride_ok(q_stride_token, es) || !stride_ok(q_stride_head, es) || !stride_ok(o_stride_token, es) ||
      !stride_ok(o_stride_head, es) || !stride_ok(cache->page_stride, es_kv) ||
      !stride_ok(cache->token_stride, es_kv) || !stride_ok(cache->head_stride, es_kv))
    return fail(PKV_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan_device)
    return fail(PKV_ERR_INVALID_ARG, "plan was built on another device");
  a->items = nullptr;
  a->num_items = 0;
  a->live_items = nullptr;
  a->num_kv_heads = p.num_kv_heads;
  a->num_qo_heads = p.num_qo_heads;
  a->q = q;
  a->q_stride_token = q_stride_token;
  a->q_stride_head = q_stride_head;
  a->k = cache->k;
  a->v = cache->v;
  a->page_stride = cache->page_stride;
  a->token_stride = cache->token_stride;
  a->head_stride = cache->head_stride;
  a->page_size = cache->page_size;
  a->page_shift = page_shift_of(cache->page_size);
  a->max_num_pages = cache->max_num_pages;
  a->kv_indices = d_kv_indices;
  a->o = o;
  a->o_stride_token = o_stride_token;
  a->o_stride_head = o_stride_head;
  a->lse = lse;
  a->part_o = nullptr;
  a->part_lse = nullptr;
  a->mask = nullptr;
  a->mask_rows = nullptr;
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt(float(p.head_dim_qk));
  a->scale_log2 = scale * 1.4426950408889634f;
  a->v_scale = 1.f;
  a->k_new = nullptr;
  a->v_new = nullptr;
  a->new_stride_token = 0;
  a->new_stride_head = 0;
  a->append_indptr = nullptr;
  a->kv_indptr = nullptr;
  a->kv_last = nullptr;
  a->nnz_new = 0;
  a->merges = nullptr;
  a->tile_merge = nullptr;
  a->merge_ctr = nullptr;
  if (p.kv_dtype == PKV_FP8_E4M3) {   // the key scale multiplies every logit
    if (cache->k_scale > 0.f) a->scale_log2 *= cache->k_scale;
    if (cache->v_scale > 0.f) a->v_scale = cache->v_scale;
  }
  return PKV_OK;
}

// The attention kernel for a plan's mode: the MFMA tile kernel for bf16
// prefill, the row kernel otherwise.
pkv_status launch_attn_mode(int32_t mode, const pkv_plan_params& p, const pkv::AttnArgs& a, hipStream_t st,
                            int32_t row_waves = 4) {
  const int32_t group = p.num_qo_heads / p.num_kv_heads;
  bool supported = false;
  hipError_t e;
  if (mode == PKV_MODE_PREFILL && (p.kv_dtype == PKV_BF16 || p.kv_dtype == PKV_FP8_E4M3))
    e = pkv::launch_prefill_mfma(p.kv_dtype, p.head_dim_qk, group, a, st, &supported);
  else if (row_waves == 1)
    e = pkv::launch_attn_rows_one_wave(p.kv_dtype, p.head_dim_qk, group, a, st, &supported);
  else
    e = pkv::launch_attn_rows(p.kv_dtype, p.head_dim_qk, group, a, st, &supported);
  if (!supported)
    return fail(PKV_ERR_UNSUPPORTED, fmt("no kernel for head_dim %lld, group %lld, dtype %lld",
                                         p.head_dim_qk, group, p.kv_dtype));
  if (e != hipSuccess) return hip_fail(e, "launching attention");
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_run_attention(const pkv_plan* plan, const void* q, int64_t q_stride_token,
                             int64_t q_stride_head, const pkv_cache_desc* cache, const int32_t* d_kv_indices,
                             void* o, int64_t o_stride_token, int64_t o_stride_head, float* lse, float sm_scale,
                             void* stream) {
  if (!plan || !cache) return fail(PKV_ERR_INVALID_ARG, "null plan or cache");
  const pkv_plan_params& p = plan->params;
  if (p.mode == PKV_MODE_MLA_DECODE) return fail(PKV_ERR_INVALID_ARG, "MLA plans run through pkv_run_mla");
  if (p.kv_format == PKV_KV_RAGGED) return fail(PKV_ERR_INVALID_ARG, "ragged plans run through pkv_run_ragged");
  if (p.mask_mode == PKV_MASK_CUSTOM) return fail(PKV_ERR_INVALID_ARG, "custom-masked plans run through pkv_run_masked");
  pkv::AttnArgs a;
  const int32_t grid_items = plan->grid_items();
  pkv_status s = prepare_attn(p, plan->device, grid_items > 0, q, q_stride_token, q_stride_head, cache,
                              d_kv_indices, o, o_stride_token, o_stride_head, lse, sm_scale, &a);
  if (s) return s;
  if (grid_items == 0) return ok();
  a.items = plan->d_items;
  a.num_items = grid_items;
  a.live_items = plan->live_items();
  a.part_o = plan->d_part_o;
  a.part_lse = plan->d_part_lse;
  s = launch_attn_mode(p.mode, p, a, static_cast<hipStream_t>(stream), plan->info.row_waves);
  if (s) return s;
  return ok();
}

pkv_status pkv_run_merge(const pkv_plan* plan, void* o, int64_t o_stride_token, int64_t o_stride_head,
                         float* lse, void* stream) {
  if (!plan) return fail(PKV_ERR_INVALID_ARG, "null plan");
  if (plan->grid_merges() == 0) return ok();
  const pkv_plan_params& p = plan->params;
  const size_t es = dtype_size(p.q_dtype);
  pkv_status s = check_ptr16(o, "o");
  if (s) return s;
  if (!stride_ok(o_stride_token, es) || !stride_ok(o_stride_head, es))
    return fail(PKV_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  pkv::MergePartialArgs m;
  m.merges = plan->d_merges;
  m.num_merges = plan->grid_merges();
  m.live_merges = plan->live_merges();
  m.max_rows = plan->info.rows_per_tile;
  m.num_heads = p.num_qo_heads;
  m.head_dim = p.head_dim_vo;
  m.part_o = plan->d_part_o;
  m.part_lse = plan->d_part_lse;
  m.o = o;
  m.o_stride_token = o_stride_token;
  m.o_stride_head = o_stride_head;
  m.lse = lse;
  hipError_t e = pkv::launch_merge_partials(p.q_dtype, m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the split merge");
  return ok();
}

pkv_status pkv_time_next_attention(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "pass both timing events or neither");
  pkv::LaunchEvents& ev = pkv::armed_launch_events();
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

pkv_status pkv_run(const pkv_plan* plan, const void* q, int64_t q_stride_token, int64_t q_stride_head,
                   const pkv_cache_desc* cache, const int32_t* d_kv_indices, void* o,
                   int64_t o_stride_token, int64_t o_stride_head, float* lse, float sm_scale,
                   void* stream) {
  if (plan && plan->merge_in)   // one launch: the split rows are folded inside it
    return pkv_run_append(plan, q, q_stride_token, q_stride_head, cache, d_kv_indices, nullptr, nullptr, 0, 0,
                          nullptr, nullptr, nullptr, 0, o, o_stride_token, o_stride_head, lse, sm_scale, 1, stream);
  pkv_status s = pkv_run_attention(plan, q, q_stride_token, q_stride_head, cache, d_kv_indices, o, o_stride_token,
                                   o_stride_head, lse, sm_scale, stream);
  if (s) return s;
  if (plan->params.mode == PKV_MODE_MLA_DECODE) return ok();
  return pkv_run_merge(plan, o, o_stride_token, o_stride_head, lse, stream);
}

pkv_status pkv_run_append(const pkv_plan* plan, const void* q, int64_t q_stride_token, int64_t q_stride_head,
                          const pkv_cache_desc* cache, const int32_t* d_kv_indices, const void* k_new,
                          const void* v_new, int64_t new_stride_token, int64_t new_stride_head,
                          const int32_t* d_append_indptr, const int32_t* d_kv_indptr,
                          const int32_t* d_kv_last_page_len, int32_t nnz, void* o, int64_t o_stride_token,
                          int64_t o_stride_head, float* lse, float sm_scale, int32_t with_merge, void* stream) {
  if (!plan || !cache) return fail(PKV_ERR_INVALID_ARG, "null plan or cache");
  const pkv_plan_params& p = plan->params;
  if (p.mode != PKV_MODE_DECODE || p.kv_format == PKV_KV_RAGGED || p.mask_mode == PKV_MASK_CUSTOM)
    return fail(PKV_ERR_UNSUPPORTED, "the fused append runs with paged decode plans without a custom mask");
  if (nnz < 0) return fail(PKV_ERR_INVALID_ARG, "negative nnz");
  pkv::AttnArgs a;
  const int32_t grid_items = plan->grid_items();
  pkv_status s = prepare_attn(p, plan->device, grid_items > 0, q, q_stride_token, q_stride_head, cache,
                              d_kv_indices, o, o_stride_token, o_stride_head, lse, sm_scale, &a);
  if (s) return s;
  if (nnz > 0) {
    const size_t es = dtype_size(p.kv_dtype);
    if ((s = check_ptr16(k_new, "k_new")) || (s = check_ptr16(v_new, "v_new"))) return s;
    if (!d_append_indptr || !d_kv_indptr || !d_kv_last_page_len)
      return fail(PKV_ERR_INVALID_ARG, "null append metadata");
    if (!stride_ok(new_stride_token, es) || !stride_ok(new_stride_head, es))
      return fail(PKV_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  }
  if (grid_items == 0) {
    // No attention work: the rows still go into the cache.
    if (nnz == 0) return ok();
    return pkv_append_paged_kv(k_new, v_new, new_stride_token, new_stride_head, d_append_indptr, d_kv_indptr,
                               d_kv_indices, d_kv_last_page_len, p.batch_size, nnz, cache, stream);
  }
  a.items = plan->d_items;
  a.num_items = grid_items;
  a.live_items = plan->live_items();
  a.part_o = plan->d_part_o;
  a.part_lse = plan->d_part_lse;
  if (nnz > 0) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.new_stride_token = new_stride_token;
    a.new_stride_head = new_stride_head;
    a.append_indptr = d_append_indptr;
    a.kv_indptr = d_kv_indptr;
    a.kv_last = d_kv_last_page_len;
    a.nnz_new = nnz;
  }
  const bool merge_in = with_merge && plan->merge_in;
  if (merge_in) {
    a.merges = plan->d_merges;
    a.tile_merge = plan->d_tile_merge;
    a.merge_ctr = plan->d_merge_ctr;
  }
  s = launch_attn_mode(p.mode, p, a, static_cast<hipStream_t>(stream), plan->info.row_waves);
  if (s) return s;
  if (!with_merge || merge_in) return ok();
  return pkv_run_merge(plan, o, o_stride_token, o_stride_head, lse, stream);
}

}  // extern "C"

namespace {

// Attention then split merge for an AttnArgs whose data fields are filled.
pkv_status run_with_args(const pkv_plan* plan, pkv::AttnArgs& a, void* o, int64_t o_stride_token,
                         int64_t o_stride_head, float* lse, void* stream) {
  const int32_t grid_items = plan->grid_items();
  if (grid_items > 0) {
    a.items = plan->d_items;
    a.num_items = grid_items;
    a.live_items = plan->live_items();
    a.part_o = plan->d_part_o;
    a.part_lse = plan->d_part_lse;
    pkv_status s = launch_attn_mode(plan->params.mode, plan->params, a, static_cast<hipStream_t>(stream),
                                    plan->info.row_waves);
    if (s) return s;
  }
  return pkv_run_merge(plan, o, o_stride_token, o_stride_head, lse, stream);
}

pkv_status check_mask_arg(const pkv_plan* plan, const uint8_t* d_mask, pkv::AttnArgs* a) {
  if (plan->params.mask_mode != PKV_MASK_CUSTOM) {
    if (d_mask) return fail(PKV_ERR_INVALID_ARG, "the plan was made without a custom mask");
    return PKV_OK;
  }
  if (!d_mask && plan->grid_items() > 0) return fail(PKV_ERR_INVALID_ARG, "null custom mask");
  if (reinterpret_cast<uintptr_t>(d_mask) % 16 != 0) return fail(PKV_ERR_INVALID_ARG, "mask must be 16-byte aligned");
  a->mask = reinterpret_cast<const uint32_t*>(d_mask);
  a->mask_rows = plan->d_mask_rows;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_run_masked(const pkv_plan* plan, const void* q, int64_t q_stride_token, int64_t q_stride_head,
                          const pkv_cache_desc* cache, const int32_t* d_kv_indices, const uint8_t* d_mask,
                          void* o, int64_t o_stride_token, int64_t o_stride_head, float* lse, float sm_scale,
                          void* stream) {
  if (!plan || !cache) return fail(PKV_ERR_INVALID_ARG, "null plan or cache");
  const pkv_plan_params& p = plan->params;
  if (p.mask_mode != PKV_MASK_CUSTOM) return fail(PKV_ERR_INVALID_ARG, "the plan was made without a custom mask");
  if (p.kv_format == PKV_KV_RAGGED) return fail(PKV_ERR_INVALID_ARG, "ragged plans run through pkv_run_ragged");
  pkv::AttnArgs a;
  pkv_status s = prepare_attn(p, plan->device, plan->grid_items() > 0, q, q_stride_token, q_stride_head, cache,
                              d_kv_indices, o, o_stride_token, o_stride_head, lse, sm_scale, &a);
  if (!s) s = check_mask_arg(plan, d_mask, &a);
  if (s) return s;
  s = run_with_args(plan, a, o, o_stride_token, o_stride_head, lse, stream);
  return s ? s : ok();
}

pkv_status pkv_run_ragged(const pkv_plan* plan, const void* q, int64_t q_stride_token, int64_t q_stride_head,
                          const void* k, const void* v, int64_t kv_stride_token, int64_t kv_stride_head,
                          const int32_t* d_kv_indptr, const uint8_t* d_mask, void* o, int64_t o_stride_token,
                          int64_t o_stride_head, float* lse, float sm_scale, void* stream) {
  if (!plan) return fail(PKV_ERR_INVALID_ARG, "null plan");
  const pkv_plan_params& p = plan->params;
  if (p.kv_format != PKV_KV_RAGGED) return fail(PKV_ERR_INVALID_ARG, "not a ragged plan");
  // The ragged tensors as a cache of one unbounded page per request: page b
  // starts at token kv_indptr[b] (page stride = token stride), so key j is
  // slot j of that page.  Scales stay at zero, i.e. 1 (an fp8 ragged run
  // takes unit scales).
  pkv_cache_desc desc{};
  desc.k = const_cast<void*>(k);
  desc.v = const_cast<void*>(v);
  desc.page_stride = kv_stride_token;
  desc.token_stride = kv_stride_token;
  desc.head_stride = kv_stride_head;
  desc.max_num_pages = p.max_num_pages;
  desc.page_size = p.page_size;
  desc.num_kv_heads = p.num_kv_heads;
  desc.head_dim = p.head_dim_qk;
  desc.dtype = p.kv_dtype;
  desc.layout = PKV_NHD;
  pkv::AttnArgs a;
  pkv_status s = prepare_attn(p, plan->device, plan->grid_items() > 0, q, q_stride_token, q_stride_head, &desc,
                              d_kv_indptr, o, o_stride_token, o_stride_head, lse, sm_scale, &a);
  if (!s) s = check_mask_arg(plan, d_mask, &a);
  if (s) return s;
  a.page_size = 1 << 30;
  a.page_shift = 30;
  a.max_num_pages = INT32_MAX;
  s = run_with_args(plan, a, o, o_stride_token, o_stride_head, lse, stream);
  return s ? s : ok();
}

pkv_status pkv_packbits(const uint8_t* d_bool, int64_t n, uint8_t* d_packed, void* stream) {
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (n == 0) return ok();
  if (!d_bool || !d_packed) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(d_packed) % 4 != 0) return fail(PKV_ERR_INVALID_ARG, "output must be 4-byte aligned");
  hipError_t e = pkv::launch_packbits(d_bool, n, reinterpret_cast<uint32_t*>(d_packed), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching packbits");
  return ok();
}

pkv_status pkv_run_mla(const pkv_plan* plan, const void* q_ckv, const void* q_kpe, const void* ckv,
                       const void* kpe, int64_t page_stride, int64_t token_stride,
                       const int32_t* d_kv_indices, void* o, float* lse, float sm_scale, void* stream) {
  if (!plan) return fail(PKV_ERR_INVALID_ARG, "null plan");
  const pkv_plan_params& p = plan->params;
  if (p.mode != PKV_MODE_MLA_DECODE) return fail(PKV_ERR_INVALID_ARG, "not an MLA plan");
  pkv_status s;
  if ((s = check_ptr16(q_ckv, "q_ckv")) || (s = check_ptr16(q_kpe, "q_kpe")) || (s = check_ptr16(ckv, "ckv")) ||
      (s = check_ptr16(kpe, "kpe")) || (s = check_ptr16(o, "o")))
    return s;
  if (!stride_ok(page_stride, 2) || !stride_ok(token_stride, 2))
    return fail(PKV_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  if (token_stride >= pkv::kMlaMaxTokenStride)
    return fail(PKV_ERR_UNSUPPORTED, "MLA token_stride must stay below 2^26 elements");
  if (!d_kv_indices && plan->grid_items() > 0) return fail(PKV_ERR_INVALID_ARG, "null kv_indices");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return fail(PKV_ERR_INVALID_ARG, "plan was built on another device");
  if (plan->grid_items() == 0) return ok();
  pkv::MlaArgs a;
  a.items = plan->d_items;
  a.num_items = plan->grid_items();
  a.live_items = plan->live_items();
  a.num_heads = p.num_qo_heads;
  a.head_groups = plan->info.heads_y;
  a.q_ckv = q_ckv;
  a.q_kpe = q_kpe;
  a.ckv = ckv;
  a.kpe = kpe;
  a.page_stride = page_stride;
  a.token_stride = token_stride;
  a.page_size = p.page_size;
  a.page_shift = page_shift_of(p.page_size);
  a.max_num_pages = p.max_num_pages;   // > 0: check_runnable at plan creation
  a.kv_indices = d_kv_indices;
  a.o = o;
  a.lse = lse;
  a.part_o = plan->d_part_o;
  a.part_lse = plan->d_part_lse;
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt(576.0f);
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = pkv::launch_mla_decode(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching MLA decode");
  if (plan->grid_merges() > 0) {
    pkv::MergePartialArgs m;
    m.merges = plan->d_merges;
    m.num_merges = plan->grid_merges();
    m.live_merges = plan->live_merges();
    m.max_rows = plan->info.rows_per_tile;
    m.num_heads = p.num_qo_heads;
    m.head_dim = 512;
    m.part_o = plan->d_part_o;
    m.part_lse = plan->d_part_lse;
    m.o = o;
    m.o_stride_token = int64_t(p.num_qo_heads) * 512;
    m.o_stride_head = 512;
    m.lse = lse;
    e = pkv::launch_mla_merge(m, st);
    if (e != hipSuccess) return hip_fail(e, "launching the MLA split merge");
  }
  return ok();
}

// --------------------------------------------------------- append, merge --

pkv_status pkv_append_paged_kv(const void* k_new, const void* v_new, int64_t new_stride_token,
                               int64_t new_stride_head, const int32_t* d_append_indptr,
                               const int32_t* d_kv_indptr, const int32_t* d_kv_indices,
                               const int32_t* d_kv_last_page_len, int32_t batch_size, int32_t nnz,
                               const pkv_cache_desc* cache, void* stream) {
  if (!cache) return fail(PKV_ERR_INVALID_ARG, "null cache");
  if (batch_size < 0 || nnz < 0) return fail(PKV_ERR_INVALID_ARG, "negative batch or nnz");
  if (nnz == 0) return ok();
  if (cache->dtype != PKV_F32 && cache->dtype != PKV_BF16 && cache->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "cache dtype");
  if (cache->page_size < 1 || cache->num_kv_heads < 1 || cache->head_dim < 1)
    return fail(PKV_ERR_INVALID_ARG, "cache shape");
  const size_t es = dtype_size(cache->dtype);
  pkv_status s;
  if ((s = check_ptr16(k_new, "k_new")) || (s = check_ptr16(v_new, "v_new")) ||
      (s = check_ptr16(cache->k, "cache k")) || (s = check_ptr16(cache->v, "cache v")))
    return s;
  if (!d_append_indptr || !d_kv_indptr || !d_kv_indices || !d_kv_last_page_len || batch_size == 0)
    return fail(PKV_ERR_INVALID_ARG, "null metadata pointer or empty batch");
  if ((cache->head_dim * es) % 16 != 0) return fail(PKV_ERR_UNSUPPORTED, "head_dim * dtype size must be a multiple of 16 bytes");
  if (!stride_ok(new_stride_token, es) || !stride_ok(new_stride_head, es) || !stride_ok(cache->page_stride, es) ||
      !stride_ok(cache->token_stride, es) || !stride_ok(cache->head_stride, es))
    return fail(PKV_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  hipError_t e = pkv::launch_append(cache->dtype, k_new, v_new, new_stride_token, new_stride_head,
                                    d_append_indptr, d_kv_indptr, d_kv_indices, d_kv_last_page_len,
                                    batch_size, nnz, cache->k, cache->v, cache->page_stride,
                                    cache->token_stride, cache->head_stride, cache->page_size,
                                    cache->num_kv_heads, cache->head_dim, cache->max_num_pages,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching append");
  return ok();
}

pkv_status pkv_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b, void* v_out,
                           float* s_out, int64_t num_rows, int32_t num_heads, int32_t head_dim, int32_t dtype,
                           void* stream) {
  if (num_rows < 0 || num_heads < 0 || head_dim < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "dtype");
  if (num_rows == 0 || num_heads == 0 || head_dim == 0) return ok();
  if (!v_a || !s_a || !v_b || !s_b || !v_out || !s_out) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  hipError_t e = pkv::launch_merge_pair(dtype, v_a, s_a, v_b, s_b, v_out, s_out, num_rows, num_heads, head_dim,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching merge_state");
  return ok();
}

pkv_status pkv_merge_states(const void* v, const float* s, void* v_out, float* s_out, int64_t num_rows,
                            int32_t num_states, int32_t num_heads, int32_t head_dim, int32_t dtype,
                            void* stream) {
  if (num_rows < 0 || num_states < 0 || num_heads < 0 || head_dim < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "dtype");
  if (num_rows == 0 || num_heads == 0 || head_dim == 0) return ok();
  if (!v_out || !s_out || (num_states > 0 && (!v || !s))) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  hipError_t e = pkv::launch_merge_many(dtype, v, s, v_out, s_out, num_rows, num_states, num_heads, head_dim,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching merge_states");
  return ok();
}

}  // extern "C"

// ------------------------------------------------ run without allocation --

// The device memory of pkv_run_noalloc: one array per device, part of this
// library's code object (loading the library on a device reserves it until
// the process ends).  Host code never takes the array's name as a device
// address: the first call on each device asks the runtime for the array's
// address on that device (hipGetSymbolAddress, with that device current) and
// every later use -- the work-list copy and the kernel arguments -- goes
// through that pointer.
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxScratchDevices] = {};

hipError_t scratch_on_device(int dev, char** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

pkv_status pkv_run_noalloc(const pkv_plan_params* params, const int32_t* qo_indptr, const int32_t* kv_indptr,
                           const int32_t* kv_indices, int64_t num_indices, const int32_t* kv_last_page_len,
                           const void* q, int64_t q_stride_token, int64_t q_stride_head, const pkv_cache_desc* cache,
                           const int32_t* d_kv_indices, void* o, int64_t o_stride_token, int64_t o_stride_head,
                           float* lse, float sm_scale, void* stream) {
  pkv_status s = check_params(params);
  if (s) return s;
  if (params->mode == PKV_MODE_MLA_DECODE || params->kv_format != PKV_KV_PAGED ||
      params->mask_mode != PKV_MASK_NONE)
    return fail(PKV_ERR_INVALID_ARG, "pkv_run_noalloc runs paged decode and prefill without a custom mask");
  PlanResult r;
  s = plan_impl(params, qo_indptr, kv_indptr, kv_indices, num_indices, kv_last_page_len, &r);
  if (s) return s;
  const pkv_plan_info& in = r.info;
  if (in.workspace_bytes > int64_t(PKV_NOALLOC_SCRATCH_BYTES))
    return fail(PKV_ERR_WORKSPACE, fmt("the batch needs %lld bytes of work list and partial states; "
                                       "pkv_run_noalloc has %lld (use pkv_plan_create with a workspace)",
                                       in.workspace_bytes, int64_t(PKV_NOALLOC_SCRATCH_BYTES)));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  pkv::AttnArgs a;
  s = prepare_attn(*params, dev, in.num_items > 0, q, q_stride_token, q_stride_head, cache, d_kv_indices, o,
                   o_stride_token, o_stride_head, lse, sm_scale, &a);
  if (s) return s;
  if (in.num_items == 0) return ok();
  char* ws = nullptr;
  e = scratch_on_device(dev, &ws);
  if (e != hipSuccess) return hip_fail(e, "locating the scratch array");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The work list and merge list go to the start of the array, the partial
  // states after them, in the layout of a plan's workspace.  The copy is
  // from ordinary (pageable) host memory, which the runtime has consumed
  // when hipMemcpyAsync returns; it is ordered after earlier work on `stream`.
  const int64_t items_bytes = align256(int64_t(r.items.size()) * sizeof(Item));
  const int64_t lse_bytes = align256(int64_t(in.num_partial_rows) * params->num_qo_heads * 4);
  std::vector<char> tables(size_t(in.staging_bytes), 0);
  copy_table(tables.data(), r.items);
  copy_table(tables.data() + items_bytes, r.merges);
  e = hipMemcpyAsync(ws, tables.data(), tables.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "copying the work list");
  a.items = reinterpret_cast<const Item*>(ws);
  a.num_items = in.num_items;
  a.live_items = nullptr;
  a.part_lse = reinterpret_cast<float*>(ws + in.staging_bytes);
  a.part_o = reinterpret_cast<float*>(ws + in.staging_bytes + lse_bytes);
  s = launch_attn_mode(params->mode, *params, a, st, in.row_waves);
  if (s) return s;
  if (in.num_merges > 0) {
    pkv::MergePartialArgs m;
    m.merges = reinterpret_cast<const MergeItem*>(ws + items_bytes);
    m.num_merges = in.num_merges;
    m.live_merges = nullptr;
    m.max_rows = in.rows_per_tile;
    m.num_heads = params->num_qo_heads;
    m.head_dim = params->head_dim_vo;
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.o = o;
    m.o_stride_token = o_stride_token;
    m.o_stride_head = o_stride_head;
    m.lse = lse;
    e = pkv::launch_merge_partials(params->q_dtype, m, st);
    if (e != hipSuccess) return hip_fail(e, "launching the split merge");
  }
  return ok();
}

}  // extern "C"

// ------------------------------------------------- fixed-capacity plans --

namespace {

struct GraphLayout {
  pkv_graph_caps caps;
  int32_t rows_per_tile;
  int64_t items_off, merges_off, mask_off, tm_off, ctr_off, ctr_bytes, staging_bytes, lse_off, o_off,
      workspace_bytes;
};

pkv_status graph_layout(const pkv_plan_params* prm, const pkv_graph_caps* in, GraphLayout* g) {
  pkv_status s = check_params(prm);
  if (s) return s;
  if (!in) return fail(PKV_ERR_INVALID_ARG, "null capacities");
  if (prm->batch_size < 0) return meta_fail(PKV_META_BATCH_SIZE, "negative batch size");
  if (prm->page_size < 1) return meta_fail(PKV_META_PAGE_SIZE, "page_size < 1");
  if (prm->num_qo_heads < 1 || prm->num_kv_heads < 1 || prm->num_qo_heads % prm->num_kv_heads != 0)
    return meta_fail(PKV_META_HEAD_GROUP, "qo heads do not group over kv heads");
  if (in->max_total_pages < 0 || in->max_total_rows < 0 || in->max_items < 0 || in->max_merges < 0 ||
      in->max_partial_rows < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative capacity");
  const bool prefill = prm->mode == PKV_MODE_PREFILL;
  const bool mla = prm->mode == PKV_MODE_MLA_DECODE;
  const int32_t group = prm->num_qo_heads / prm->num_kv_heads;
  if (prm->kv_format == PKV_KV_RAGGED)
    return fail(PKV_ERR_UNSUPPORTED, "fixed-capacity plans are built for paged caches");
  const int64_t R = rows_per_tile(prm->mode, group, prm->kv_dtype, prm->mask_mode, prm->head_dim_qk);
  int64_t hy = prm->num_kv_heads;
  if (mla) {
    hy = mla_head_groups(prm);
    if (!mla_groups_ok(prm, hy)) return fail(PKV_ERR_UNSUPPORTED, "MLA decode runs head groups of 64 or 128 heads");
  }
  int32_t num_cus = prm->num_cus;
  if (num_cus <= 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "querying the compute-unit count");
  }
  const int64_t B = prm->batch_size;
  const int64_t tiles = prefill ? cdiv(in->max_total_rows, R) + B : B;
  const int64_t S = prm->tail_split > 0 ? prm->tail_split : default_tail_split(prm->mode);
  const int64_t T = int64_t(prm->target_per_cu > 0 ? prm->target_per_cu : default_target(prm->mode)) * num_cus;
  const int64_t N = in->max_total_pages;
  const int64_t items = tiles * S + (prm->fixed_split_pages > 0 ? cdiv(tiles * N, prm->fixed_split_pages)
                                                               : cdiv(T, hy) + cdiv(tiles * N, kMaxChunkPages));
  pkv_graph_caps c = *in;
  if (c.max_items == 0) c.max_items = int32_t(std::min<int64_t>(items, INT32_MAX));
  if (c.max_merges == 0) c.max_merges = int32_t(std::min<int64_t>(tiles, INT32_MAX));
  if (c.max_partial_rows == 0) c.max_partial_rows = int32_t(std::min<int64_t>(int64_t(c.max_items) * R, INT32_MAX));
  c.reserved = 0;
  g->caps = c;
  g->rows_per_tile = int32_t(R);
  g->items_off = 256;   // the two counters
  g->merges_off = g->items_off + align256(int64_t(c.max_items) * sizeof(Item));
  g->mask_off = g->merges_off + align256(int64_t(c.max_merges) * sizeof(MergeItem));
  g->tm_off = g->mask_off + (prm->mask_mode == PKV_MASK_CUSTOM ? align256(B * sizeof(pkv::MaskRow)) : 0);
  const bool tables = has_merge_tables(prm);
  g->ctr_off = g->tm_off + (tables ? align256(B * 4) : 0);
  g->ctr_bytes = tables ? int64_t(c.max_merges) * prm->num_kv_heads * 4 : 0;
  g->staging_bytes = g->ctr_off + align256(g->ctr_bytes);
  g->lse_off = g->staging_bytes;
  g->o_off = g->lse_off + align256(int64_t(c.max_partial_rows) * prm->num_qo_heads * 4);
  g->workspace_bytes = g->o_off + align256(int64_t(c.max_partial_rows) * prm->num_qo_heads * prm->head_dim_vo * 4);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_graph_plan_size(const pkv_plan_params* params, const pkv_graph_caps* caps,
                               pkv_graph_caps* caps_out, int64_t* workspace_bytes, int64_t* staging_bytes) {
  GraphLayout g;
  pkv_status s = graph_layout(params, caps, &g);
  if (s) return s;
  if (caps_out) *caps_out = g.caps;
  if (workspace_bytes) *workspace_bytes = g.workspace_bytes;
  if (staging_bytes) *staging_bytes = g.staging_bytes;
  return ok();
}

pkv_status pkv_graph_plan_create(const pkv_plan_params* params, const pkv_graph_caps* caps, void* d_workspace,
                                 size_t ws_bytes, void* h_staging, size_t staging_bytes, void* stream,
                                 pkv_plan** plan_out) {
  if (!plan_out) return fail(PKV_ERR_INVALID_ARG, "null plan_out");
  *plan_out = nullptr;
  GraphLayout g;
  pkv_status s = graph_layout(params, caps, &g);
  if (!s) s = check_runnable(params);
  if (s) return s;
  if (params->row_waves == 1)
    return fail(PKV_ERR_UNSUPPORTED, "fixed-capacity plans run 4-wave row workgroups (row_waves 0 or 4)");
  if (!d_workspace || int64_t(ws_bytes) < g.workspace_bytes)
    return fail(PKV_ERR_WORKSPACE, fmt("workspace %lld bytes < %lld needed", int64_t(ws_bytes), g.workspace_bytes));
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256 != 0)
    return fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (!h_staging) return fail(PKV_ERR_INVALID_ARG, "a fixed-capacity plan needs a pinned staging buffer");
  if (int64_t(staging_bytes) < g.staging_bytes)
    return fail(PKV_ERR_WORKSPACE, fmt("staging %lld bytes < %lld needed", int64_t(staging_bytes), g.staging_bytes));
  char* ws = static_cast<char*>(d_workspace);
  pkv_plan* plan = new pkv_plan;
  plan->params = *params;
  std::memset(&plan->info, 0, sizeof plan->info);
  plan->info.mode = params->mode;
  plan->info.batch_size = params->batch_size;
  plan->info.rows_per_tile = g.rows_per_tile;
  plan->info.workspace_bytes = g.workspace_bytes;
  plan->info.staging_bytes = g.staging_bytes;
  plan->graph = true;
  plan->caps = g.caps;
  plan->d_ws = ws;
  plan->d_counts = reinterpret_cast<int32_t*>(ws);
  plan->d_items = reinterpret_cast<Item*>(ws + g.items_off);
  plan->d_merges = reinterpret_cast<MergeItem*>(ws + g.merges_off);
  plan->d_mask_rows = reinterpret_cast<pkv::MaskRow*>(ws + g.mask_off);
  plan->d_part_lse = reinterpret_cast<float*>(ws + g.lse_off);
  plan->d_part_o = reinterpret_cast<float*>(ws + g.o_off);
  plan->h_staging = h_staging;
  plan->staging_bytes = g.staging_bytes;
  hipError_t e = hipGetDevice(&plan->device);
  if (e == hipSuccess && has_merge_tables(params)) {
    plan->d_tile_merge = reinterpret_cast<int32_t*>(ws + g.tm_off);
    plan->d_merge_ctr = reinterpret_cast<int32_t*>(ws + g.ctr_off);
    plan->merge_in = g.caps.max_merges > 0 && merge_in_launch_ok(params, plan->device);
  }
  plan->info.merge_in_launch = plan->merge_in ? 1 : 0;
  plan->info.row_waves = 4;   // the captured launch keeps one kernel for every later batch
  // The live counts (and the merge counters) start at zero: a run before the
  // first update does nothing.
  if (e == hipSuccess)
    e = upload_staging(h_staging, ws, g.ctr_bytes > 0 ? g.ctr_off + g.ctr_bytes : 256,
                       static_cast<hipStream_t>(stream), plan, [](char*) {});
  if (e != hipSuccess) {
    release_staging(h_staging, plan);
    delete plan;
    return hip_fail(e, "initialising the fixed-capacity plan");
  }
  *plan_out = plan;
  return ok();
}

pkv_status pkv_plan_update(pkv_plan* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                           const int32_t* kv_indices, int64_t num_indices, const int32_t* kv_last_page_len,
                           void* stream) {
  if (!plan) return fail(PKV_ERR_INVALID_ARG, "null plan");
  if (!plan->graph) return fail(PKV_ERR_INVALID_ARG, "pkv_plan_update needs a fixed-capacity plan");
  PlanResult r;
  pkv_status s = plan_impl(&plan->params, qo_indptr, kv_indptr, kv_indices, num_indices, kv_last_page_len, &r);
  if (s) return s;
  const pkv_graph_caps& c = plan->caps;
  const int32_t B = plan->params.batch_size;
  if (plan->params.mode == PKV_MODE_PREFILL && r.info.total_rows > c.max_total_rows)
    return fail(PKV_ERR_WORKSPACE, fmt("%lld query rows > capacity %lld", r.info.total_rows, c.max_total_rows));
  if (kv_indptr[B] > c.max_total_pages)
    return fail(PKV_ERR_WORKSPACE, fmt("%lld pages > capacity %lld", kv_indptr[B], c.max_total_pages));
  if (r.info.num_items > c.max_items || r.info.num_merges > c.max_merges ||
      r.info.num_partial_rows > c.max_partial_rows)
    return fail(PKV_ERR_WORKSPACE, fmt("plan needs %lld items / %lld merges / %lld partial rows", r.info.num_items,
                                       r.info.num_merges, r.info.num_partial_rows) +
                                       fmt(" (capacity %lld / %lld / %lld)", c.max_items, c.max_merges,
                                           c.max_partial_rows));
  const int64_t items_off = 256;
  const int64_t merges_off = items_off + align256(int64_t(c.max_items) * sizeof(Item));
  const int64_t mask_off = merges_off + align256(int64_t(c.max_merges) * sizeof(MergeItem));
  GraphLayout g;
  pkv_status gs = graph_layout(&plan->params, &plan->caps, &g);
  if (gs) return gs;
  int64_t upload = r.mask_rows.empty() ? merges_off + int64_t(r.merges.size()) * sizeof(MergeItem)
                                       : mask_off + int64_t(r.mask_rows.size()) * sizeof(pkv::MaskRow);
  // Decode plans: the merge table of the live batch, and the counters zeroed
  // again (a run that failed part-way must not leave counts behind).
  if (!r.tile_merge.empty()) upload = g.ctr_off + g.ctr_bytes;
  hipError_t e = upload_staging(plan->h_staging, plan->d_ws, upload, static_cast<hipStream_t>(stream), plan,
                                [&](char* hs) {
                                  int32_t* counts = reinterpret_cast<int32_t*>(hs);
                                  counts[0] = r.info.num_items;
                                  counts[1] = r.info.num_merges;
                                  copy_table(hs + items_off, r.items);
                                  copy_table(hs + merges_off, r.merges);
                                  copy_table(hs + mask_off, r.mask_rows);
                                  copy_table(hs + g.tm_off, r.tile_merge);
                                });
  if (e != hipSuccess) return hip_fail(e, "uploading the plan");
  const int64_t ws_bytes = plan->info.workspace_bytes, st_bytes = plan->info.staging_bytes;
  const int32_t merge_in = plan->info.merge_in_launch;
  plan->info = r.info;
  plan->info.workspace_bytes = ws_bytes;
  plan->info.staging_bytes = st_bytes;
  plan->info.merge_in_launch = merge_in;
  plan->info.row_waves = 4;
  return ok();
}

}  // extern "C"

// --------------------------------------------------------------- cascade --

struct pkv_cascade_plan {
  pkv_plan_params params;
  pkv_cascade_info info;
  std::vector<pkv_plan_info> level_info;
  std::vector<int32_t> level_mode, level_item_off;
  Item* d_items;
  int32_t* d_row_ptr;
  int32_t* d_slots;
  float* d_part_lse;
  float* d_part_o;
  int device;
  void* h_staging = nullptr;
};

extern "C" {

pkv_status pkv_cascade_plan_compute(const pkv_plan_params* params, int32_t num_levels,
                                    const pkv_cascade_level* levels, pkv_cascade_info* info,
                                    pkv_plan_info* level_info, int32_t* items_out, int64_t items_capacity,
                                    int32_t* row_ptr_out, int64_t row_ptr_capacity, int32_t* slots_out,
                                    int64_t slots_capacity) {
  pkv_status s = check_params(params);
  if (s) return s;
  CascadeResult r;
  s = cascade_impl(params, num_levels, levels, &r);
  if (s) return s;
  if (info) *info = r.info;
  if (level_info) std::copy(r.level_info.begin(), r.level_info.end(), level_info);
  if (items_out) {
    if (items_capacity < int64_t(r.items.size()) * PKV_ITEM_WORDS)
      return fail(PKV_ERR_WORKSPACE, "work-item buffer too small");
    copy_table(items_out, r.items);
  }
  if (row_ptr_out) {
    if (row_ptr_capacity < int64_t(r.row_ptr.size())) return fail(PKV_ERR_WORKSPACE, "row pointer buffer too small");
    copy_table(row_ptr_out, r.row_ptr);
  }
  if (slots_out) {
    if (slots_capacity < int64_t(r.slots.size())) return fail(PKV_ERR_WORKSPACE, "slot buffer too small");
    copy_table(slots_out, r.slots);
  }
  return ok();
}

pkv_status pkv_cascade_plan_create(const pkv_plan_params* params, int32_t num_levels,
                                   const pkv_cascade_level* levels, void* d_workspace, size_t ws_bytes,
                                   void* h_staging, size_t staging_bytes, void* stream,
                                   pkv_cascade_plan** plan_out) {
  if (!plan_out) return fail(PKV_ERR_INVALID_ARG, "null plan_out");
  *plan_out = nullptr;
  pkv_status s = check_params(params);
  if (s) return s;
  CascadeResult r;
  s = cascade_impl(params, num_levels, levels, &r);
  if (s) return s;
  const pkv_cascade_info& in = r.info;
  if (in.workspace_bytes > 0 && (!d_workspace || int64_t(ws_bytes) < in.workspace_bytes))
    return fail(PKV_ERR_WORKSPACE, fmt("workspace %lld bytes < %lld needed", int64_t(ws_bytes), in.workspace_bytes));
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256 != 0)
    return fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (h_staging && int64_t(staging_bytes) < in.staging_bytes)
    return fail(PKV_ERR_WORKSPACE, fmt("staging %lld bytes < %lld needed", int64_t(staging_bytes), in.staging_bytes));
  char* ws = static_cast<char*>(d_workspace);
  const int64_t items_bytes = align256(int64_t(r.items.size()) * sizeof(Item));
  const int64_t rp_bytes = align256(int64_t(r.row_ptr.size()) * 4);
  const int64_t lse_bytes = align256(int64_t(in.num_partial_rows) * params->num_qo_heads * 4);
  pkv_cascade_plan* plan = new pkv_cascade_plan;
  plan->params = *params;
  plan->info = in;
  plan->level_info = r.level_info;
  plan->level_mode = r.level_mode;
  plan->level_item_off = r.level_item_off;
  plan->d_items = reinterpret_cast<Item*>(ws);
  plan->d_row_ptr = reinterpret_cast<int32_t*>(ws + items_bytes);
  plan->d_slots = reinterpret_cast<int32_t*>(ws + items_bytes + rp_bytes);
  plan->d_part_lse = reinterpret_cast<float*>(ws + in.staging_bytes);
  plan->d_part_o = reinterpret_cast<float*>(ws + in.staging_bytes + lse_bytes);
  plan->h_staging = h_staging;
  hipError_t e = hipGetDevice(&plan->device);
  if (e == hipSuccess && in.staging_bytes > 0)
    e = upload_staging(h_staging, ws, in.staging_bytes, static_cast<hipStream_t>(stream), plan, [&](char* hs) {
      copy_table(hs, r.items);
      copy_table(hs + items_bytes, r.row_ptr);
      copy_table(hs + items_bytes + rp_bytes, r.slots);
    });
  if (e != hipSuccess) {
    release_staging(h_staging, plan);
    delete plan;
    return hip_fail(e, "uploading the cascade plan");
  }
  *plan_out = plan;
  return ok();
}

pkv_status pkv_cascade_plan_get_info(const pkv_cascade_plan* plan, pkv_cascade_info* info) {
  if (!plan || !info) return fail(PKV_ERR_INVALID_ARG, "null argument");
  *info = plan->info;
  return ok();
}

pkv_status pkv_cascade_run(const pkv_cascade_plan* plan, const void* q, int64_t q_stride_token,
                           int64_t q_stride_head, const pkv_cache_desc* cache, const int32_t* d_kv_indices,
                           void* o, int64_t o_stride_token, int64_t o_stride_head, float* lse,
                           float sm_scale, void* stream) {
  if (!plan || !cache) return fail(PKV_ERR_INVALID_ARG, "null plan or cache");
  const pkv_plan_params& p = plan->params;
  pkv::AttnArgs a;
  pkv_status s = prepare_attn(p, plan->device, plan->info.num_items > 0, q, q_stride_token, q_stride_head, cache,
                              d_kv_indices, o, o_stride_token, o_stride_head, lse, sm_scale, &a);
  if (s) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  a.part_o = plan->d_part_o;
  a.part_lse = plan->d_part_lse;
  for (size_t l = 0; l < plan->level_info.size(); ++l) {
    const int32_t n = plan->level_info[l].num_items;
    if (n == 0) continue;
    a.items = plan->d_items + plan->level_item_off[l];
    a.num_items = n;
    s = launch_attn_mode(plan->level_mode[l], p, a, st);
    if (s) return s;
  }
  if (plan->info.total_rows > 0) {
    pkv::MergeRowsArgs m;
    m.row_ptr = plan->d_row_ptr;
    m.slots = plan->d_slots;
    m.num_rows = plan->info.total_rows;
    m.num_heads = p.num_qo_heads;
    m.head_dim = p.head_dim_vo;
    m.part_o = plan->d_part_o;
    m.part_lse = plan->d_part_lse;
    m.o = o;
    m.o_stride_token = o_stride_token;
    m.o_stride_head = o_stride_head;
    m.lse = lse;
    hipError_t e = pkv::launch_merge_rows(p.q_dtype, m, st);
    if (e != hipSuccess) return hip_fail(e, "launching the cascade merge");
  }
  return ok();
}

pkv_status pkv_cascade_plan_destroy(pkv_cascade_plan* plan) {
  if (plan) release_staging(plan->h_staging, plan);
  delete plan;
  return ok();
}

}  // extern "C"
