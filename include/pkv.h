/*
 * pkv.h -- C ABI of the paged KV-cache attention library for AMD MI355X (gfx950).
 *
 * Batched attention of ragged queries against a paged KV cache described by a
 * CSR page table.  The calls follow the problem statement of three web pages:
 *   [DD]  "Deep Dive - FlashInfer" (leetllm.com)
 *   [KVL] "FlashInfer 中的 KV-Cache 布局" (KV-cache layouts, docs.flashinfer.cn)
 *   [GAB] "GPU attention backends: FlashInfer and FlashAttention"
 *         (mini-sglang from Scratch, Stage 4)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Plain C types only.  "host" pointers are ordinary CPU memory; "device"
 *   pointers are HIP device memory of the current device.  `stream` is a
 *   hipStream_t passed as void* (NULL = the null stream).
 * - Every call returns a pkv_status; nothing throws across the ABI.  On error
 *   pkv_last_error() returns a thread-local message; for PKV_ERR_METADATA,
 *   pkv_last_meta_reason() names the broken rule (pkv_meta_reason).
 * - All metadata arrays are int32 ([KVL] "Ragged Tensor" and "页表布局":
 *   indptr, page-index and tail-length arrays are 32-bit).
 * - Element strides are counted in elements of the payload dtype.
 * - The library never allocates device memory: the caller owns the caches,
 *   Q/O/LSE buffers, the plan workspace and the pinned staging buffer, and
 *   keeps them alive until the last queued call that uses them has finished
 *   ([DD] "Where FlashInfer sits in a serving stack": the engine owns pages
 *   and their lifetime).
 * - LSE values are base 2: lse = log2(sum_j exp(s_j)) with s_j the scaled
 *   logits; the empty state is (zero vector, -inf) ([DD] "Core mechanism:
 *   schedule work around state", "A worked split-KV example").
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,  /* null pointer, bad size/stride/alignment, plan/call mismatch */
  PKV_ERR_METADATA = 2,     /* page-table metadata breaks a rule (see pkv_meta_reason) */
  PKV_ERR_UNSUPPORTED = 3,  /* a head dim, group size, dtype or mode the library has no kernel for */
  PKV_ERR_WORKSPACE = 4,    /* workspace or staging buffer too small */
  PKV_ERR_STALE_PLAN = 5,   /* pkv_plan_check: metadata differs from what the plan was built on */
  PKV_ERR_HIP = 6           /* a HIP runtime call failed (message has the HIP error string) */
};

/* Metadata rules.  [DD] "Why inference attention becomes irregular" (length
 * contract and its rejections) and [KVL] "Ragged Tensor" / "页表布局" state
 * the first ones; the ones marked "completion" are our plainest reading. */
typedef enum {
  PKV_META_NONE = 0,
  PKV_META_BATCH_SIZE = 1,       /* batch_size < 0 */
  PKV_META_PAGE_SIZE = 2,        /* page_size < 1 */
  PKV_META_INDPTR_START = 3,     /* an indptr does not start at 0 */
  PKV_META_INDPTR_ORDER = 4,     /* an indptr decreases */
  PKV_META_EMPTY_PAGE_LIST = 5,  /* a request owns no page */
  PKV_META_LAST_PAGE_LEN = 6,    /* last_page_len outside 1..page_size */
  PKV_META_PAGE_INDEX = 7,       /* page id outside [0, max_num_pages) */
  PKV_META_INDICES_LENGTH = 8,   /* kv_indptr[B] > number of kv_indices */
  PKV_META_QO_EXCEEDS_KV = 9,    /* completion: qo_len > kv_len (kv_len counts the new tokens) */
  PKV_META_HEAD_GROUP = 10,      /* completion: num_qo_heads not a multiple of num_kv_heads */
  PKV_META_DECODE_QO_LEN = 11,   /* completion: decode mode needs qo_len == 1 */
  PKV_META_APPEND_COLLISION = 12, /* completion: two appended tokens target one slot */
  PKV_META_CASCADE_ROWS = 13,    /* completion: no cascade level, or levels cover different row counts */
  PKV_META_CASCADE_NESTING = 14  /* completion: a cascade level's node boundary is not one of the next level's */
} pkv_meta_reason;

/* PKV_FP8_E4M3: 8-bit E4M3 codes (the OCP fp8 format: bias 7, no infinity,
 * largest finite 448), for the K/V cache only, with bf16 queries and outputs
 * ([KVL] "布局：NHD/HND" notes low-precision fp8 caches and that HND suits
 * them).  Stored value x stands for x * k_scale (keys) or x * v_scale
 * (values), one scale per tensor (pkv_cache_desc). */
typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* [KVL] "布局：NHD/HND": the last three dims of a page are
 * (page_size, heads, head_dim) for NHD and (heads, page_size, head_dim) for HND. */
typedef enum { PKV_NHD = 0, PKV_HND = 1 } pkv_layout;

/* Key/value storage ([KVL] "页表布局" and "Ragged Tensor"). */
typedef enum {
  PKV_KV_PAGED = 0,   /* CSR page table over a page pool (pkv_run, pkv_run_masked) */
  PKV_KV_RAGGED = 1   /* request b's keys are data[kv_indptr[b] .. kv_indptr[b+1]) (pkv_run_ragged) */
} pkv_kv_format;

/* Visibility ([KVL] "掩码布局（2D Ragged Tensor）"). */
typedef enum {
  PKV_MASK_NONE = 0,   /* all keys, or the bottom-right causal rule when params.causal */
  PKV_MASK_CUSTOM = 1  /* a bit-packed per-request mask decides; params.causal must be 0 */
} pkv_mask_mode;

typedef enum {
  PKV_MODE_DECODE = 0,     /* one query row per request; no qo_indptr ([DD] "Plan then run") */
  PKV_MODE_PREFILL = 1,    /* ragged query rows (chunked prefill / append), optional causal mask */
  PKV_MODE_MLA_DECODE = 2  /* MLA latent cache, one query row per request ([KVL] MLA page layout) */
} pkv_mode;

const char* pkv_version(void);
const char* pkv_last_error(void);
int32_t pkv_last_meta_reason(void);

/* Number of compute units of the current device (HIP call). */
pkv_status pkv_device_num_cus(int32_t* num_cus_out);

/*
 * Paged cache descriptor.  k and v point at element (page 0, slot 0, head 0,
 * dim 0) of the K and V pools.  Element (page, slot, head, dim) of K is at
 *   k + page*page_stride + slot*token_stride + head*head_stride + dim.
 * The dim stride is 1.  This covers both storage forms of [KVL] "页表布局":
 *   5-D single tensor [pages, 2, ...]: v = k + (page_stride / 2),
 *                                      page_stride = 2 * page_size * heads * head_dim;
 *   (k, v) tuple of 4-D tensors:       page_stride = page_size * heads * head_dim;
 * and both layouts: NHD token_stride = heads*head_dim, head_stride = head_dim;
 *                   HND token_stride = head_dim, head_stride = page_size*head_dim.
 * `layout` is informational (the strides decide the addressing).
 */
typedef struct pkv_cache_desc {
  void* k;
  void* v;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  int32_t max_num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;   /* pkv_dtype */
  int32_t layout;  /* pkv_layout */
  float k_scale;   /* fp8 caches: dequantisation factor of every key (<= 0: 1) */
  float v_scale;   /* fp8 caches: dequantisation factor of every value (<= 0: 1) */
} pkv_cache_desc;

/*
 * Host-side metadata check.  [DD] "Why inference attention becomes
 * irregular": kv_len = page_size*(num_pages-1) + last_page_len with
 * 1 <= last_page_len <= page_size and a nonempty list of nonnegative page ids;
 * [KVL] "Ragged Tensor": indptr arrays have B+1 entries starting at 0.
 * Rules are checked in pkv_meta_reason order of the oracle's statement:
 * batch, page size, heads, qo_indptr, kv_indptr, indices length, per-request
 * pages and tail, then qo_len vs kv_len (and decode's qo_len == 1).
 *   qo_indptr        host, B+1 entries, or NULL (one row per request)
 *   kv_indptr        host, B+1 entries, counts pages
 *   kv_indices       host, num_indices entries (page ids in logical order)
 *   kv_last_page_len host, B entries
 *   kv_len_out       host, B entries, or NULL
 * Returns PKV_OK or PKV_ERR_METADATA (reason via pkv_last_meta_reason()).
 */
pkv_status pkv_validate(const int32_t* qo_indptr, const int32_t* kv_indptr,
                        const int32_t* kv_indices, int64_t num_indices,
                        const int32_t* kv_last_page_len, int32_t batch_size,
                        int32_t page_size, int32_t max_num_pages, int32_t num_qo_heads,
                        int32_t num_kv_heads, int32_t decode, int32_t* kv_len_out);

/*
 * Host-side check of an append batch: the metadata is valid, every request
 * appends at most kv_len tokens, and no two appended tokens map to the same
 * (page, slot) (which would be a write race).  All pointers host.
 */
pkv_status pkv_validate_append(const int32_t* append_indptr, const int32_t* kv_indptr,
                               const int32_t* kv_indices, int64_t num_indices,
                               const int32_t* kv_last_page_len, int32_t batch_size,
                               int32_t page_size, int32_t max_num_pages);

/*
 * append_paged_kv: scatter a ragged batch of new K/V rows into the paged
 * cache.  [KVL], FlashInfer API note under the MLA page layout: the caller
 * allocates the pages before appending.  The metadata is post-append: kv_len
 * already counts the new tokens ([DD] "Why inference attention becomes
 * irregular"), so the n_b new rows of request b land at logical positions
 * kv_len_b - n_b + t, i.e. page kv_indices[kv_indptr[b] + pos / page_size],
 * slot pos % page_size.  The copy is bit-exact.
 *   k_new, v_new      device, [nnz, num_kv_heads, head_dim] with the given
 *                     token / head strides (elements), dtype of the cache
 *   d_append_indptr   device, B+1 entries (new rows per request, prefix sums)
 *   d_kv_indptr, d_kv_indices, d_kv_last_page_len   device page table
 *   cache             host descriptor of the pools being written
 * Asynchronous on `stream`.  Shapes are checked on the host; the metadata
 * itself is read only on the device (use pkv_validate_append on the host
 * copy to check it).  Rows whose request lookup fails are skipped.
 */
pkv_status pkv_append_paged_kv(const void* k_new, const void* v_new, int64_t new_stride_token,
                               int64_t new_stride_head, const int32_t* d_append_indptr,
                               const int32_t* d_kv_indptr, const int32_t* d_kv_indices,
                               const int32_t* d_kv_last_page_len, int32_t batch_size, int32_t nnz,
                               const pkv_cache_desc* cache, void* stream);

/* ------------------------------------------------------------------ plan -- */

/*
 * plan(): the inspector half of plan/run ([DD] "Plan then run:
 * inspector-executor for GPU kernels"; [GAB] "FlashInfer: plan and run").
 * Runs once per batch on the host, turns the metadata into a work list of
 * (query tile, key chunk) items plus a merge list for split tiles, and copies
 * them to the caller's device workspace with one asynchronous copy through
 * the caller's pinned staging buffer.  Every layer of the batch then calls
 * run() with the same plan.
 *
 * Split policy ([DD] "Load balancing and split-KV decisions" gives the
 * trade-off, not an algorithm; this is our rule): chunk pages
 * C = fixed_split_pages if > 0, else max(ceil(256/page_size), ceil(W/T)) with
 * W = sum_b tiles_b * pages_b * heads_y and T = target_per_cu * num_cus; C is
 * capped at 1024 pages (a kernel stages one chunk's page ids on chip).
 * Chunks are page-aligned and disjoint; causal tiles drop chunks they cannot
 * see.  With tail_split S > 1, the final chunk of each tile, if longer than
 * one page, is cut into S page-aligned pieces of ceil(pages/S) pages.  Items
 * run most keys first (ties: request, tile, chunk), so the schedule ends on
 * small items.
 */
typedef struct pkv_plan pkv_plan;

typedef struct pkv_plan_params {
  int32_t mode;              /* pkv_mode */
  int32_t batch_size;
  int32_t num_qo_heads;      /* MLA: query heads */
  int32_t num_kv_heads;      /* MLA: must be 1 */
  int32_t head_dim_qk;       /* MLA: 576 (512 ckv + 64 kpe) */
  int32_t head_dim_vo;       /* MLA: 512 */
  int32_t page_size;
  int32_t causal;            /* prefill: bottom-right causal mask ([DD] "Causality uses
                                logical positions, not page numbers"); ignored by decode */
  int32_t q_dtype;           /* pkv_dtype of q and o; equals kv_dtype, or bf16 over an fp8 cache */
  int32_t kv_dtype;          /* pkv_dtype of the cache (fp8: E4M3 codes, bf16 queries) */
  int32_t num_cus;           /* 0: query the current device */
  int32_t fixed_split_pages; /* > 0 forces this chunk size in pages */
  int32_t target_per_cu;     /* 0: default (decode 3, prefill 4, MLA 1) */
  int32_t mla_head_groups;   /* MLA only: head groups of 64 or 128 heads each; 0: groups of 128 when
                                the head count allows, else of 64 */
  int32_t max_num_pages;     /* pool size, for the page-id range check */
  int32_t tail_split;        /* 0: default (decode 2, prefill 1, MLA 1); 1: off */
  int32_t kv_format;         /* pkv_kv_format; ragged needs PKV_MODE_PREFILL */
  int32_t mask_mode;         /* pkv_mask_mode; custom needs PKV_MODE_PREFILL and causal == 0 */
  int32_t merge_in_launch;   /* 1: fold the split merge into the attention launch where the plan
                                allows it (see pkv_run); 0: a merge launch of its own */
  int32_t row_waves;         /* decode only: waves per workgroup of the row kernel, 4 or 1; 0: the
                                plan picks 1 when its work items average at most 384 keys and,
                                times the kv heads, number at least 24 per CU (many short
                                requests: one-wave workgroups put four times as many items on a
                                CU), else 4.  One-wave plans fold no merge into the launch;
                                fixed-capacity plans run 4. */
} pkv_plan_params;

typedef struct pkv_plan_info {
  int32_t mode;
  int32_t batch_size;
  int32_t num_items;         /* work items (each replicated over heads_y on the device) */
  int32_t num_merges;
  int32_t num_partial_rows;
  int32_t chunk_pages;
  int32_t split;             /* 1 if any tile is split over several chunks */
  int32_t rows_per_tile;
  int32_t heads_y;           /* kv heads (decode/prefill) or head groups (MLA) */
  int32_t num_cus;
  int32_t target;            /* target_per_cu * num_cus */
  int32_t total_rows;        /* query rows (nnz) */
  int64_t workspace_bytes;   /* device workspace this plan needs */
  int64_t staging_bytes;     /* pinned staging this plan needs */
  uint64_t fingerprint;      /* hash of params + metadata (staleness check) */
  int64_t mask_bits;         /* custom mask: sum over requests of qo_len * kv_len */
  int32_t merge_in_launch;   /* 1: pkv_run / pkv_run_append fold split rows inside the
                                attention launch (set by plan creation, see pkv_run) */
  int32_t row_waves;         /* waves per workgroup of the row kernel (4, or 1: see row_waves in
                                pkv_plan_params); the MFMA and MLA kernels ignore it */
} pkv_plan_info;

/* Work item / merge item sizes in int32 words (layout documented in the
 * planner source; exposed for pkv_plan_compute's output buffers). */
#define PKV_ITEM_WORDS 8
#define PKV_MERGE_WORDS 4

/*
 * Host-only planning pass (no HIP call unless params->num_cus == 0): fills
 * info and, when the buffers are large enough, the work list
 * (info.num_items * PKV_ITEM_WORDS int32) and merge list
 * (info.num_merges * PKV_MERGE_WORDS int32).  Pass NULL buffers to query
 * sizes.  kv_indices may be NULL (the page-id range check is then skipped).
 * Returns PKV_ERR_WORKSPACE if a non-NULL buffer is too small.
 */
pkv_status pkv_plan_compute(const pkv_plan_params* params, const int32_t* qo_indptr,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            int64_t num_indices, const int32_t* kv_last_page_len,
                            int32_t* items_out, int64_t items_capacity, int32_t* merges_out,
                            int64_t merges_capacity, pkv_plan_info* info);

/*
 * Build a plan and upload it.  Host arrays as for pkv_validate (qo_indptr
 * NULL in decode/MLA modes).  d_workspace: device buffer of ws_bytes >=
 * info.workspace_bytes; h_staging: pinned host buffer (hipHostMalloc) of
 * staging_bytes >= info.staging_bytes, or NULL for a synchronous upload.  If
 * the same staging buffer was used by an earlier plan, this call first waits
 * for that plan's copy to finish ([GAB] "FlashInfer: plan and run": pinned
 * staging is reused, so the previous copy must complete first).  The plan
 * (host memory, owned by the library) stays valid only for this exact batch
 * ([DD] "Plan then run"; a plan reused after the page table changes gives
 * plausible output for the wrong sequence) and until pkv_plan_destroy.
 * The first split decode plan made with merge_in_launch = 1 on a device
 * (here or by pkv_graph_plan_create) also checks, once per device and
 * process, which
 * XCD runs each workgroup: a 1024-workgroup probe launch on the null stream,
 * a 4 KiB device buffer and a synchronous copy back.  The answer decides
 * merge_in_launch (PKV_MERGE_IN_ATTENTION=0 in the environment: never).
 */
pkv_status pkv_plan_create(const pkv_plan_params* params, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           int64_t num_indices, const int32_t* kv_last_page_len,
                           void* d_workspace, size_t ws_bytes, void* h_staging,
                           size_t staging_bytes, void* stream, pkv_plan** plan_out);

pkv_status pkv_plan_get_info(const pkv_plan* plan, pkv_plan_info* info);

/* PKV_OK if the metadata hashes to the plan's fingerprint, else
 * PKV_ERR_STALE_PLAN.  Host arrays as for pkv_plan_create. */
pkv_status pkv_plan_check(const pkv_plan* plan, const int32_t* qo_indptr,
                          const int32_t* kv_indptr, const int32_t* kv_indices,
                          int64_t num_indices, const int32_t* kv_last_page_len);

pkv_status pkv_plan_destroy(pkv_plan* plan);

/* ------------------------------------------------ fixed-capacity plans -- */

/*
 * Plans for captured runs ([DD] "Plan then run": plan does host work and
 * device copies, so it cannot be captured; compatible run calls can, and
 * graph-mode plans reserve their metadata buffers, fix the batch size and
 * bound the total query rows and page-index capacity -- stable addresses do
 * not make stale contents correct).
 *
 * pkv_graph_plan_create reserves, inside the caller's workspace, a work list,
 * a merge list and partial-state buffers of fixed capacity, plus two device
 * counters (zero until the first update).  pkv_plan_update -- host work plus
 * one asynchronous copy on `stream`, not capturable -- plans a batch of
 * exactly params->batch_size requests with the ordinary planner and writes
 * its lists and counts to those fixed addresses.  Runs on such a plan
 * (pkv_run, pkv_run_attention, pkv_run_merge, pkv_run_mla) launch grids sized
 * by the capacities; workgroups past the live counts exit at once.  Launch
 * shapes and pointers are therefore the same after every update, so a run
 * captured once replays correctly for every later batch within the
 * capacities, as long as the caller keeps q, the caches, kv_indices, o and
 * lse at fixed addresses and refreshes their contents.  The update's copy is
 * ordered on `stream`: runs of the previous batch must be ordered before it.
 *
 * Derived capacities (used for a field left 0).  With R the plan's rows per
 * tile, tiles = B (decode, MLA) or ceil(max_total_rows / R) + B (prefill),
 * S the tail split, T = target_per_cu * num_cus, hy the kv heads or MLA head
 * groups and N = max_total_pages:
 *   max_items        = tiles*S + (fixed_split_pages > 0 ? ceil(tiles*N / fixed_split_pages)
 *                                                       : ceil(T / hy) + ceil(tiles*N / 1024))
 *   max_merges       = tiles
 *   max_partial_rows = max_items * R
 * These bound every plan the planner can make within max_total_rows and N.
 */
typedef struct pkv_graph_caps {
  int32_t max_total_rows;    /* prefill: bound on qo_indptr[B]; decode and MLA: ignored (B rows) */
  int32_t max_total_pages;   /* bound on kv_indptr[B] */
  int32_t max_items;         /* 0: derived */
  int32_t max_merges;        /* 0: derived */
  int32_t max_partial_rows;  /* 0: derived */
  int32_t reserved;
} pkv_graph_caps;

/* Resolve the capacities (caps_out, derived fields filled in) and the
 * workspace / pinned staging sizes of a fixed-capacity plan.  Host only
 * (queries the device only if params->num_cus == 0). */
pkv_status pkv_graph_plan_size(const pkv_plan_params* params, const pkv_graph_caps* caps,
                               pkv_graph_caps* caps_out, int64_t* workspace_bytes, int64_t* staging_bytes);

/* Create a fixed-capacity plan.  d_workspace (256-byte aligned) and the
 * pinned h_staging (required) must hold the sizes pkv_graph_plan_size
 * reports and stay owned by this plan until pkv_plan_destroy.  Zeroes the
 * counters with one asynchronous copy on `stream`. */
pkv_status pkv_graph_plan_create(const pkv_plan_params* params, const pkv_graph_caps* caps, void* d_workspace,
                                 size_t ws_bytes, void* h_staging, size_t staging_bytes, void* stream,
                                 pkv_plan** plan_out);

/* Plan a new batch into a fixed-capacity plan (host arrays as for
 * pkv_plan_create).  PKV_ERR_INVALID_ARG for an ordinary plan; the metadata
 * errors of pkv_plan_create; PKV_ERR_WORKSPACE if the batch exceeds a
 * capacity (the plan then keeps its previous batch). */
pkv_status pkv_plan_update(pkv_plan* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                           const int32_t* kv_indices, int64_t num_indices, const int32_t* kv_last_page_len,
                           void* stream);

/* ------------------------------------------------------------------- run -- */

/*
 * run(): the executor half.  For every query row i of request b and query
 * head h, attention over the keys that row sees: key j with j < kv_len_b and,
 * when causal, j <= kv_len_b - qo_len_b + i ([DD] "Causality uses logical
 * positions, not page numbers").  Head h reads kv head h / (Hq/Hkv) ([DD]
 * "Plan then run", GQA grouping).  Key j of request b lives at page
 * kv_indices[kv_indptr[b] + j / page_size], slot j % page_size.
 *   q      device [nnz, Hq, head_dim_qk], strides in elements, dtype of the plan
 *   cache  host descriptor; must match the plan (page size, heads, dim, dtype)
 *   d_kv_indices device page ids (the same values the plan was built on)
 *   o      device [nnz, Hq, head_dim_vo], dtype of q, strides in elements
 *   lse    device float [nnz, Hq] (contiguous), base-2, or NULL
 *   sm_scale  logit scale; <= 0 selects 1/sqrt(head_dim_qk)
 * Enqueues one attention kernel and, if the plan split any tile, one merge
 * kernel on `stream`, unless the plan folds the split rows inside the
 * attention launch (pkv_plan_info.merge_in_launch): plans made with
 * params.merge_in_launch = 1 in paged decode mode whose kv heads are a
 * multiple of 8, on a device that runs workgroups i and i + 8 on one XCD,
 * where the last workgroup to finish a row's chunks merges them ([DD] "A
 * worked split-KV example"); plans from pkv_plan_create only when no row has
 * more than 16 chunks (one workgroup merging many chunks at the end of the
 * launch costs more than a merge launch).  No host synchronisation, no
 * allocation, no host copy.  Runs of one plan must not overlap in time: they
 * share its workspace (partial states and merge counters).
 */
pkv_status pkv_run(const pkv_plan* plan, const void* q, int64_t q_stride_token,
                   int64_t q_stride_head, const pkv_cache_desc* cache,
                   const int32_t* d_kv_indices, void* o, int64_t o_stride_token,
                   int64_t o_stride_head, float* lse, float sm_scale, void* stream);

/*
 * The two launches of pkv_run, separately: pkv_run_attention enqueues only
 * the attention kernel (rows of split tiles then hold fp32 partial states in
 * the plan's workspace, not in o/lse); pkv_run_merge enqueues only the merge
 * of those partial states into o/lse ([DD] "A worked split-KV example") and
 * is a no-op for a plan without splits.  pkv_run == attention then merge on
 * one stream.  Splitting them lets a caller place other work between the two
 * (for instance an exchange of partial states across devices, which the same
 * merge then combines, [DD] "Core mechanism: schedule work around state") or
 * time each kernel.  Arguments as for pkv_run.
 */
pkv_status pkv_run_attention(const pkv_plan* plan, const void* q, int64_t q_stride_token,
                             int64_t q_stride_head, const pkv_cache_desc* cache,
                             const int32_t* d_kv_indices, void* o, int64_t o_stride_token,
                             int64_t o_stride_head, float* lse, float sm_scale, void* stream);
pkv_status pkv_run_merge(const pkv_plan* plan, void* o, int64_t o_stride_token,
                         int64_t o_stride_head, float* lse, void* stream);

/*
 * append_paged_kv fused into a decode run: the result of
 * pkv_append_paged_kv(k_new, v_new, ..., d_kv_indptr, d_kv_indices,
 * d_kv_last_page_len, batch_size, nnz, cache) followed by pkv_run (with_merge
 * != 0) or pkv_run_attention (with_merge == 0) with one launch fewer: the
 * cache bit for bit, o and lse up to fp32 rounding (the block holding the
 * new keys is summed first).  [KVL], FlashInfer API note under the MLA page
 * layout (pages allocated first, then appended) and [DD] "Why inference
 * attention becomes irregular" (kv_len counts the new rows): the n_b new rows
 * of request b are its keys [kv_len_b - n_b, kv_len_b).  The attention kernel
 * reads those keys from k_new / v_new, and the workgroup whose key chunk holds
 * them stores them into the cache for its kv head.
 *   plan              a paged decode plan (one query row per request) without
 *                     a custom mask; other plans: PKV_ERR_UNSUPPORTED
 *   q ... sm_scale    as for pkv_run; cache is written (the new rows) and read
 *   k_new, v_new      device [nnz, num_kv_heads, head_dim], cache dtype,
 *                     strides in elements as for pkv_append_paged_kv
 *   d_append_indptr, d_kv_indptr, d_kv_last_page_len   device, B+1, B+1 and B
 *                     entries: the post-append metadata the plan was built on
 *   nnz               rows of k_new / v_new (0: a plain run)
 * Asynchronous on `stream`, no allocation.  The metadata is read only on the
 * device: inconsistent values give undefined rows, never an access outside
 * k_new, v_new or the pool (page ids outside it are skipped).
 */
pkv_status pkv_run_append(const pkv_plan* plan, const void* q, int64_t q_stride_token,
                          int64_t q_stride_head, const pkv_cache_desc* cache,
                          const int32_t* d_kv_indices, const void* k_new, const void* v_new,
                          int64_t new_stride_token, int64_t new_stride_head,
                          const int32_t* d_append_indptr, const int32_t* d_kv_indptr,
                          const int32_t* d_kv_last_page_len, int32_t nnz, void* o,
                          int64_t o_stride_token, int64_t o_stride_head, float* lse,
                          float sm_scale, int32_t with_merge, void* stream);

/*
 * Kernel timing (measurement support, not an operation of the method): arms
 * two events for the next attention kernel that this library launches from
 * the calling host thread (pkv_run, pkv_run_attention, pkv_run_masked,
 * pkv_run_ragged, pkv_run_mla, or a cascade level).  That launch passes them
 * to hipExtLaunchKernel, so the dispatch itself records start_event when the
 * kernel starts and stop_event when it ends: hipEventElapsedTime then gives
 * the kernel's own duration, with no separate event packets in the stream
 * around it.  The events are disarmed by that launch (one launch per arming;
 * a run that launches no attention kernel leaves them armed).
 *   start_event, stop_event  hipEvent_t handles created by the caller with
 *                            timing enabled, or both NULL to disarm
 * The library does not take ownership of the events.  Returns
 * PKV_ERR_INVALID_ARG when exactly one of them is NULL.
 */
pkv_status pkv_time_next_attention(void* start_event, void* stop_event);

/*
 * MLA decode run ([KVL] "多头潜在注意力页布局"): one latent row per token,
 * ckv (512) and kpe (64), shared by every query head; score =
 * sm_scale * (q_ckv . ckv + q_kpe . kpe); output = softmax-weighted ckv.
 *   q_ckv  device bf16 [B, H, 512] contiguous;  q_kpe device bf16 [B, H, 64] contiguous
 *   ckv    device bf16, element (page, slot, d) at ckv + page*page_stride + slot*token_stride + d
 *   kpe    device bf16, same strides (zero-copy slices of one [pages, P, 576] tensor work)
 *   o      device bf16 [B, H, 512] contiguous; lse device float [B, H] or NULL
 *   sm_scale <= 0 selects 1/sqrt(576)
 * token_stride must stay below 2^26 elements (PKV_ERR_UNSUPPORTED otherwise).
 */
pkv_status pkv_run_mla(const pkv_plan* plan, const void* q_ckv, const void* q_kpe,
                       const void* ckv, const void* kpe, int64_t page_stride,
                       int64_t token_stride, const int32_t* d_kv_indices, void* o, float* lse,
                       float sm_scale, void* stream);

/* ------------------------------------------------ run without allocation -- */

/* Bytes of the per-device array that pkv_run_noalloc works in. */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): pkv_run
 * without a plan object, workspace or staging buffer.  One call plans the
 * batch on the host (as pkv_plan_create does, same work list), copies the
 * work list into a device array that the library holds (one array of
 * PKV_NOALLOC_SCRATCH_BYTES per device, for the life of the process), and
 * runs attention and the split merge with the partial states in that array.  It calls no device or
 * pinned-host allocation routine; planning uses ordinary host memory only.
 *   params, host metadata        as for pkv_plan_create (paged decode or
 *                                prefill; MLA, ragged and custom-masked
 *                                plans are PKV_ERR_INVALID_ARG)
 *   q, cache, d_kv_indices, o, lse, sm_scale, stream   as for pkv_run
 * The array is shared by every call on a device and keeps the last call's
 * contents (nothing in it has to start at zero: each call writes the work
 * list and every partial state before reading them).  Calls on one device
 * must therefore not overlap: two calls on different streams of one device
 * race on the array, and a call on a stream is ordered after the earlier
 * ones only on that stream.  Returns PKV_ERR_WORKSPACE, with the size needed,
 * for a batch whose work list and partial states exceed the array (plan it
 * with pkv_plan_create and a workspace instead); the metadata and argument
 * errors of pkv_plan_create and pkv_run otherwise.
 */
pkv_status pkv_run_noalloc(const pkv_plan_params* params, const int32_t* qo_indptr, const int32_t* kv_indptr,
                           const int32_t* kv_indices, int64_t num_indices, const int32_t* kv_last_page_len,
                           const void* q, int64_t q_stride_token, int64_t q_stride_head,
                           const pkv_cache_desc* cache, const int32_t* d_kv_indices, void* o,
                           int64_t o_stride_token, int64_t o_stride_head, float* lse, float sm_scale,
                           void* stream);

/* --------------------------------------------------------------- cascade -- */

/*
 * Multi-level cascade attention ([KVL] "多级级联推理数据布局"): the queries
 * and outputs stay one ragged tensor and every level's keys live in the one
 * paged cache; level l views them through its own qo_indptr (query rows of
 * each node, i.e. of each subtree of the request tree) and its own page table
 * (kv_indptr, kv_indices, kv_last_page_len as in pkv_run).  Row i's output is
 * attention over the keys of all nodes on its path, level 0 first: the merge
 * of its per-level states ([DD] "Core mechanism: schedule work around state":
 * output plus base-2 LSE composes across shared prefixes).
 *
 * Readings (the layout page leaves them open): every level covers all rows
 * and the levels nest (each node's rows are whole nodes of the next level);
 * the keys of a shared level precede every query token below it, so only the
 * last level, whose nodes are requests, applies the bottom-right causal mask
 * (params->causal); the per-request metadata rules of pkv_validate hold per
 * level, except that a shared node may hold fewer keys than rows.
 *
 * Schedule (ours): each level is planned like pkv_plan_create -- as decode
 * when every node has one row, else as prefill, so a node shared by many
 * rows runs the MFMA tile kernel and its keys are read once for all of them
 * -- except that every tile writes fp32 partial states and that, unless
 * params->target_per_cu is set, every level targets one item per CU (each
 * level is a launch of its own).  A row-indexed merge
 * then folds, per query row, the partial states of all its levels and
 * chunks.  pkv_cascade_run enqueues one attention launch per level and one
 * merge.
 */
typedef struct pkv_cascade_level {
  int32_t num_nodes;
  const int32_t* qo_indptr;        /* host, num_nodes+1: query rows of each node */
  const int32_t* kv_indptr;        /* host, num_nodes+1: pages of each node */
  const int32_t* kv_indices;       /* host page ids of the level, or NULL (range check skipped) */
  int64_t num_indices;
  const int32_t* kv_last_page_len; /* host, num_nodes */
} pkv_cascade_level;

typedef struct pkv_cascade_info {
  int32_t num_levels;
  int32_t total_rows;        /* query rows (every level's qo_indptr[num_nodes]) */
  int32_t num_items;         /* work items over all levels */
  int32_t num_partial_rows;  /* partial states per head (every item writes some) */
  int32_t num_merge_slots;   /* entries of the row-indexed merge list (= num_partial_rows) */
  int32_t reserved;
  int64_t workspace_bytes;
  int64_t staging_bytes;
  uint64_t fingerprint;
} pkv_cascade_info;

typedef struct pkv_cascade_plan pkv_cascade_plan;

/*
 * Host-only cascade planning.  params: heads, dims, page size, dtypes, causal,
 * num_cus, max_num_pages and the split knobs apply to every level; mode and
 * batch_size are ignored (each level's mode follows from its node row counts,
 * its batch is its node count).  levels[0 .. num_levels) are host structs.
 * Metadata is checked level by level (pkv_meta_reason; PKV_META_CASCADE_* for
 * the cross-level rules).  Fills info and, when given, level_info
 * (num_levels entries: each level's plan as pkv_plan_get_info reports it),
 * the work list (info.num_items * PKV_ITEM_WORDS int32, levels back to back;
 * page_base counts into the concatenated page ids of all levels, out_slot
 * into the shared partial rows), the merge row pointers (total_rows + 1
 * int32) and the merge slot list (num_merge_slots int32).  Pass NULL buffers
 * to query sizes; PKV_ERR_WORKSPACE if a non-NULL buffer is too small.
 */
pkv_status pkv_cascade_plan_compute(const pkv_plan_params* params, int32_t num_levels,
                                    const pkv_cascade_level* levels, pkv_cascade_info* info,
                                    pkv_plan_info* level_info, int32_t* items_out, int64_t items_capacity,
                                    int32_t* row_ptr_out, int64_t row_ptr_capacity, int32_t* slots_out,
                                    int64_t slots_capacity);

/*
 * Build a cascade plan and upload it (workspace and staging rules as for
 * pkv_plan_create; ws_bytes >= info.workspace_bytes, staging_bytes >=
 * info.staging_bytes).  The plan (library-owned host memory) is valid for
 * this exact batch until pkv_cascade_plan_destroy.
 */
pkv_status pkv_cascade_plan_create(const pkv_plan_params* params, int32_t num_levels,
                                   const pkv_cascade_level* levels, void* d_workspace, size_t ws_bytes,
                                   void* h_staging, size_t staging_bytes, void* stream,
                                   pkv_cascade_plan** plan_out);

pkv_status pkv_cascade_plan_get_info(const pkv_cascade_plan* plan, pkv_cascade_info* info);

/*
 * Run a cascade: one attention launch per level (levels in order), then the
 * row-indexed merge into o / lse, all on `stream`; no allocation, no host
 * synchronisation.
 *   q, cache, o, lse, sm_scale   as for pkv_run (q/o hold every query row)
 *   d_kv_indices  device int32: the page ids of level 0 (kv_indptr[num_nodes]
 *                 of them), then those of level 1, and so on -- the same
 *                 values the plan was built on
 */
pkv_status pkv_cascade_run(const pkv_cascade_plan* plan, const void* q, int64_t q_stride_token,
                           int64_t q_stride_head, const pkv_cache_desc* cache, const int32_t* d_kv_indices,
                           void* o, int64_t o_stride_token, int64_t o_stride_head, float* lse,
                           float sm_scale, void* stream);

pkv_status pkv_cascade_plan_destroy(pkv_cascade_plan* plan);

/* ----------------------------------------------- ragged KV, custom masks -- */

/*
 * Custom-mask run ([KVL] "掩码布局（2D Ragged Tensor）"): as pkv_run, for a
 * plan made with mask_mode = PKV_MASK_CUSTOM.  Request b's mask is a qo_len x
 * kv_len boolean matrix, query-major; the matrices of all requests are
 * concatenated (request b starts at element sum_{c<b} qo_len_c * kv_len_c)
 * and bit-packed little-endian: element e is bit e % 8 of byte e / 8 (numpy
 * packbits order, which is what pkv_packbits writes).  Row i of request b
 * sees key j iff its element is 1; a row that sees no key gets (0, -inf).
 *   d_mask  device, 16-byte aligned, at least ceil(info.mask_bits / 8) + 32
 *           bytes (the kernels read aligned words and 32-byte row windows
 *           that may run past the last mask bit)
 * bf16 plans with head_dim 128 and at least 2 query heads per kv head run
 * the MFMA tile kernel (each tile's mask bits move into LDS with its keys);
 * the others run one query row per work item on the row kernel.
 */
pkv_status pkv_run_masked(const pkv_plan* plan, const void* q, int64_t q_stride_token, int64_t q_stride_head,
                          const pkv_cache_desc* cache, const int32_t* d_kv_indices, const uint8_t* d_mask,
                          void* o, int64_t o_stride_token, int64_t o_stride_head, float* lse, float sm_scale,
                          void* stream);

/*
 * Ragged-KV run ([KVL] "Ragged Tensor"): for a plan made with kv_format =
 * PKV_KV_RAGGED (kv_indptr counts tokens; kv_indices and kv_last_page_len are
 * not used by the planner and may be NULL).  Key j of request b is row
 * kv_indptr[b] + j of the data tensors.
 *   k, v         device, element (token t, kv head h, dim d) at
 *                k + t*kv_stride_token + h*kv_stride_head + d (NHD: strides
 *                Hkv*D and D), the plan's kv_dtype (an fp8 plan reads E4M3
 *                codes with unit scales: fold a K scale into sm_scale and
 *                apply a V scale to the output)
 *   d_kv_indptr  device int32, B+1 entries, the same values the plan was built on
 *   d_mask       device bit-packed custom mask (as for pkv_run_masked) for a
 *                custom-masked plan, else NULL
 * Other arguments as for pkv_run.
 */
pkv_status pkv_run_ragged(const pkv_plan* plan, const void* q, int64_t q_stride_token, int64_t q_stride_head,
                          const void* k, const void* v, int64_t kv_stride_token, int64_t kv_stride_head,
                          const int32_t* d_kv_indptr, const uint8_t* d_mask, void* o, int64_t o_stride_token,
                          int64_t o_stride_head, float* lse, float sm_scale, void* stream);

/*
 * Pack n device bytes (0 = false, anything else = true) into the
 * little-endian bit layout above: d_packed receives ceil(n / 32) 32-bit words
 * (ceil(n/32)*4 bytes; bits past n are 0; allocate the 32 extra bytes that
 * pkv_run_masked reads and zero them).  Asynchronous on `stream`.
 */
pkv_status pkv_packbits(const uint8_t* d_bool, int64_t n, uint8_t* d_packed, void* stream);

/* ----------------------------------------------------------------- merge -- */

/*
 * merge_state ([DD] "A worked split-KV example"): combine two attention
 * states over disjoint key sets, per (row, head):
 *   m = max(s_a, s_b); w_x = 2^(s_x - m); v = (w_a v_a + w_b v_b)/(w_a + w_b);
 *   s = m + log2(w_a + w_b); a -inf side passes the other side through.
 *   v_a, v_b, v_out  device [num_rows, num_heads, head_dim], dtype f32 or bf16
 *   s_a, s_b, s_out  device float [num_rows, num_heads]
 * v_out may alias v_a or v_b (and s_out s_a or s_b): each element is read
 * before it is written by the same thread.
 */
pkv_status pkv_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                           void* v_out, float* s_out, int64_t num_rows, int32_t num_heads,
                           int32_t head_dim, int32_t dtype, void* stream);

/*
 * Merge num_states states per (row, head) (associative in exact arithmetic,
 * [DD] "Core mechanism: schedule work around state").
 *   v      device [num_rows, num_states, num_heads, head_dim] (f32 or bf16)
 *   s      device float [num_rows, num_states, num_heads]
 *   v_out  device [num_rows, num_heads, head_dim] (dtype of v); s_out float [num_rows, num_heads]
 * num_states == 0 yields the empty state (0, -inf).
 */
pkv_status pkv_merge_states(const void* v, const float* s, void* v_out, float* s_out,
                            int64_t num_rows, int32_t num_states, int32_t num_heads,
                            int32_t head_dim, int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
