// Internal declarations shared by the host library and the HIP kernels.
// Not part of the C ABI (include/pkv.h is).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Timing events armed for the next attention kernel launched from this host
// thread (pkv_time_next_attention); null when none are armed.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchEvents& armed_launch_events();

// Launches an attention kernel.  With events armed, the dispatch itself
// records them at the kernel's start and end (hipExtLaunchKernelGGL), and
// they are disarmed; otherwise a plain launch.
template <typename Kernel, typename... Args>
void launch_attention_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  LaunchEvents& ev = armed_launch_events();
  if (ev.start || ev.stop) {
    const LaunchEvents use = ev;
    ev = LaunchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, use.start, use.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  }
}

// One unit of attention work: a tile of query rows of one request against one
// chunk of its keys.  The device replicates it over kv heads (or MLA head
// groups).  Row r of the tile sees key j when kv_start <= j < kv_end and
// j <= diag + r.
struct Item {
  int32_t q_row0;     // first global query row
  int32_t num_rows;   // rows in the tile
  int32_t kv_start;   // first key of the chunk
  int32_t kv_end;     // one past the last key any row of the tile sees in the chunk
  int32_t diag;       // causal limit of the tile's first row
  int32_t page_base;  // kv_indptr[b]
  int32_t out_slot;   // -1: final output; else first partial row
  int32_t batch;      // request index
};
static_assert(sizeof(Item) == 32, "work item is eight int32");

// One split tile: its chunks' partial states are rows slot0 + c*num_rows + r.
struct MergeItem {
  int32_t q_row0;
  int32_t num_rows;
  int32_t slot0;
  int32_t num_chunks;
};
static_assert(sizeof(MergeItem) == 16, "merge item is four int32");

enum DType : int32_t { kF32 = 0, kBF16 = 1, kFP8 = 2 };   // kFP8: E4M3 codes (K/V storage only)

// Custom mask of one request: bit (q_start + i, j) of the packed mask is
// bit0 + i * kv_len + j.
struct MaskRow {
  int64_t bit0;
  int32_t q_start;
  int32_t kv_len;
};
static_assert(sizeof(MaskRow) == 16, "mask row is 16 bytes");

struct AttnArgs {
  const Item* items;
  int32_t num_items;       // items the grid covers
  const int32_t* live_items;  // null, or a device count: items at or past it exit at once
  int32_t num_kv_heads;
  int32_t num_qo_heads;
  const void* q;
  int64_t q_stride_token, q_stride_head;
  const void* k;
  const void* v;
  int64_t page_stride, token_stride, head_stride;
  int32_t page_size;
  int32_t page_shift;  // log2(page_size) if a power of two, else -1
  int32_t max_num_pages;  // page ids outside [0, max_num_pages) are never dereferenced
  const int32_t* kv_indices;
  void* o;
  int64_t o_stride_token, o_stride_head;
  float* lse;          // [rows, Hq] or null
  float* part_o;       // [partial rows, Hq, Dvo]
  float* part_lse;     // [partial rows, Hq]
  float scale_log2;    // sm_scale * log2(e)
  const uint32_t* mask;        // packed custom mask (little-endian bits), or null
  const MaskRow* mask_rows;    // per request, when mask is set
  float v_scale;               // fp8 caches: factor applied to the normalised output
  // Append fused into a decode launch (null append_indptr: none).  Request b's
  // new rows k_new/v_new[append_indptr[b] .. append_indptr[b+1]) are its last
  // keys (kv_len from kv_indptr and kv_last): the kernel reads them from there
  // and the workgroup whose chunk holds them also writes them into the cache.
  const void* k_new;
  const void* v_new;
  int64_t new_stride_token, new_stride_head;   // elements
  const int32_t* append_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_last;
  int32_t nnz_new;             // rows of k_new / v_new
  // Split merge inside the decode launch (null merge_ctr: a separate merge
  // launch folds the partial states).  tile_merge[b]: merge item of request
  // b's tile or -1; merge_ctr[m * num_kv_heads + h]: chunks of merge item m
  // finished for kv head h (zero between launches).  Every chunk of one
  // (merge item, kv head) runs on one XCD (workgroup order), so their
  // partial states meet in that XCD's L2.
  const MergeItem* merges;
  const int32_t* tile_merge;
  int32_t* merge_ctr;
};

struct MergePartialArgs {
  const MergeItem* merges;
  int32_t num_merges;      // merge items the grid covers
  const int32_t* live_merges;  // null, or a device count: merge items at or past it exit at once
  int32_t max_rows;    // largest num_rows over the merge items
  int32_t num_heads;
  int32_t head_dim;
  const float* part_o;
  const float* part_lse;
  void* o;
  int64_t o_stride_token, o_stride_head;
  float* lse;
};

// Row-indexed merge (cascades): query row r folds the partial rows
// slots[row_ptr[r] .. row_ptr[r+1]) into o / lse.
struct MergeRowsArgs {
  const int32_t* row_ptr;   // [num_rows + 1]
  const int32_t* slots;
  int32_t num_rows;
  int32_t num_heads;
  int32_t head_dim;
  const float* part_o;
  const float* part_lse;
  void* o;
  int64_t o_stride_token, o_stride_head;
  float* lse;
};

struct MlaArgs {
  const Item* items;
  int32_t num_items;       // items the grid covers
  const int32_t* live_items;  // null, or a device count: items at or past it exit at once
  int32_t num_heads;
  int32_t head_groups;
  const void* q_ckv;   // [B, H, 512]
  const void* q_kpe;   // [B, H, 64]
  const void* ckv;
  const void* kpe;
  int64_t page_stride, token_stride;
  int32_t page_size;
  int32_t page_shift;
  int32_t max_num_pages;
  const int32_t* kv_indices;
  void* o;             // [B, H, 512]
  float* lse;          // [B, H] or null
  float* part_o;       // [partial rows, H, 512] as bf16 (the fp32-sized region holds them)
  float* part_lse;     // [partial rows, H]
  float scale_log2;
};

// Kernel launchers (each returns the launch error, if any).
hipError_t launch_attn_rows(int32_t dtype, int32_t head_dim, int32_t group, const AttnArgs& a,
                            hipStream_t stream, bool* supported);
// The same row kernel with one wave per workgroup (decode plans of many short
// items; plain runs and fused appends only).
hipError_t launch_attn_rows_one_wave(int32_t dtype, int32_t head_dim, int32_t group, const AttnArgs& a,
                                     hipStream_t stream, bool* supported);
hipError_t launch_prefill_mfma(int32_t kv_dtype, int32_t head_dim, int32_t group, const AttnArgs& a,
                               hipStream_t stream, bool* supported);
// The MLA kernel addresses the 8 rows one wave loads with 32-bit offsets:
// token_stride (elements) must stay below this.
constexpr int64_t kMlaMaxTokenStride = int64_t(1) << 26;
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream);
// Merge of MLA partial rows (bf16 rows of 512 dims, float LSE) into o (bf16).
hipError_t launch_mla_merge(const MergePartialArgs& a, hipStream_t stream);
hipError_t launch_merge_partials(int32_t dtype, const MergePartialArgs& a, hipStream_t stream);
hipError_t launch_merge_rows(int32_t dtype, const MergeRowsArgs& a, hipStream_t stream);
// out[i] = the XCD that ran workgroup i, for i < blocks (64 threads each).
hipError_t launch_xcd_probe(int32_t* d_out, int32_t blocks, hipStream_t st);
hipError_t launch_append(int32_t dtype, const void* k_new, const void* v_new, int64_t new_st,
                         int64_t new_sh, const int32_t* append_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_indices, const int32_t* last_page_len, int32_t batch,
                         int32_t nnz, void* k, void* v, int64_t page_stride, int64_t token_stride,
                         int64_t head_stride, int32_t page_size, int32_t num_heads, int32_t head_dim,
                         int32_t max_num_pages, hipStream_t stream);
hipError_t launch_merge_pair(int32_t dtype, const void* va, const float* sa, const void* vb,
                             const float* sb, void* vo, float* so, int64_t rows, int32_t heads,
                             int32_t dim, hipStream_t stream);
hipError_t launch_packbits(const uint8_t* in, int64_t n, uint32_t* out, hipStream_t stream);
hipError_t launch_merge_many(int32_t dtype, const void* v, const float* s, void* vo, float* so,
                             int64_t rows, int32_t states, int32_t heads, int32_t dim,
                             hipStream_t stream);

}  // namespace pkv
