// Append (ragged -> paged scatter) and the attention-state merges.
//
// append_paged_kv: "FlashInfer 中的 KV-Cache 布局", FlashInfer API note under
// the MLA page layout (pages are allocated by the caller first); the new rows
// are the last n_b logical positions of each request because kv_len already
// counts them ("Deep Dive - FlashInfer", "Why inference attention becomes
// irregular").  A bit-exact copy, bound by HBM bandwidth.
//
// Merges: "Deep Dive - FlashInfer", "A worked split-KV example": shift by the
// largest base-2 statistic, normalise the weights 2^(s - shift) to scales,
// combine, and keep shift + log2(sum); an empty state (-inf) contributes
// nothing and two empty states stay empty.

#include <algorithm>

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

// Append: workgroup w copies the new rows of tokens [w*tpb, w*tpb + tpb)
// (tpb = tokens per block, chosen by the launcher).  Three phases, two
// barriers, both reached by every thread:
//   1. every thread issues the loads of its 16-byte chunks of those rows
//      (they do not depend on where the rows go), then scans requests
//      r = tid, tid + 256, ...: request r owns tokens [append_indptr[r],
//      append_indptr[r+1]); a request that owns some of the block's tokens
//      computes their logical positions kv_len_r - n_r + i, reads their page
//      ids and stores each token's destination offset in LDS (its page-table
//      entries are loaded with append_indptr, before the test, so the scan
//      costs one dependent load plus the page-id load);
//   2. every thread stores its chunks at their token's destination (rows
//      wider than 8 chunks per thread, one token per block then, copy the
//      rest in a loop).
// A token no request owns, or whose page id lies outside the pool, is
// skipped.
constexpr int kAppendThreads = 256;
constexpr int kAppendMaxTok = 16;     // tokens per block at most
constexpr int kAppendMaxChunks = 8;   // 16-byte chunks per thread at most

__global__ __launch_bounds__(kAppendThreads) void append_kernel(const char* k_new, const char* v_new, int64_t new_st_b,
                                                                int64_t new_sh_b, const int32_t* append_indptr,
                                                                const int32_t* kv_indptr, const int32_t* kv_indices,
                                                                const int32_t* last, int32_t batch, int32_t nnz,
                                                                int32_t tpb, char* k, char* v, int64_t page_b,
                                                                int64_t tok_b, int64_t head_b, int32_t page_size,
                                                                int32_t heads, int32_t row_chunks, int32_t max_pages) {
  __shared__ int64_t s_dst[kAppendMaxTok];   // byte offset of each token's slot, -1: skip
  const int tid = threadIdx.x;
  const int32_t t0 = int32_t(blockIdx.x) * tpb;
  const int32_t n = min(tpb, nnz - t0);
  const int32_t per = heads * row_chunks;    // chunks of one K (or V) row
  const int32_t total = n * 2 * per;
  // Chunk i: token i / (2 per); then K or V; then head and 16-byte chunk.
  auto locate = [&](int32_t i, int32_t& j, int32_t& which, int64_t& inner_src, int64_t& inner_dst) {
    j = i / (2 * per);
    const int32_t rem = i - j * 2 * per;
    which = rem >= per;
    const int32_t q = rem - which * per;
    const int32_t h = q / row_chunks, c = q - (q / row_chunks) * row_chunks;
    inner_src = int64_t(h) * new_sh_b + int64_t(c) * 16;
    inner_dst = int64_t(h) * head_b + int64_t(c) * 16;
  };
  uint4 data[kAppendMaxChunks];
#pragma unroll
  for (int x = 0; x < kAppendMaxChunks; ++x) {
    const int32_t i = tid + x * kAppendThreads;
    if (i < total) {
      int32_t j, which;
      int64_t is, id;
      locate(i, j, which, is, id);
      data[x] = dev::load16<true>((which ? v_new : k_new) + int64_t(t0 + j) * new_st_b + is);   // read once: nt
    }
  }
  if (tid < kAppendMaxTok) s_dst[tid] = -1;
  __syncthreads();
  for (int32_t r = tid; r < batch; r += kAppendThreads) {
    const int32_t a0 = append_indptr[r], a1 = append_indptr[r + 1];
    const int32_t p0 = kv_indptr[r], p1 = kv_indptr[r + 1], lst = last[r];
    const int32_t lo = max(a0, t0), hi = min(a1, t0 + n);
    if (lo >= hi) continue;
    const int32_t n_pages = p1 - p0;
    const int32_t kv_len = page_size * (n_pages - 1) + lst;
    for (int32_t t = lo; t < hi; ++t) {
      const int32_t pos = kv_len - (a1 - a0) + (t - a0);
      int64_t dst = -1;
      if (n_pages >= 1 && pos >= 0 && pos < kv_len) {
        const int32_t page = kv_indices[p0 + pos / page_size];
        if (page >= 0 && page < max_pages) dst = int64_t(page) * page_b + int64_t(pos % page_size) * tok_b;
      }
      s_dst[t - t0] = dst;
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < kAppendMaxChunks; ++x) {
    const int32_t i = tid + x * kAppendThreads;
    if (i < total) {
      int32_t j, which;
      int64_t is, id;
      locate(i, j, which, is, id);
      const int64_t dst = s_dst[j];
      if (dst >= 0) *reinterpret_cast<uint4*>((which ? v : k) + dst + id) = data[x];
    }
  }
  // Rows wider than the preloaded chunks (one token per block then): the rest.
  for (int32_t i = tid + kAppendMaxChunks * kAppendThreads; i < total; i += kAppendThreads) {
    int32_t j, which;
    int64_t is, id;
    locate(i, j, which, is, id);
    const int64_t dst = s_dst[j];
    if (dst >= 0)
      *reinterpret_cast<uint4*>((which ? v : k) + dst + id) =
          dev::load16<true>((which ? v_new : k_new) + int64_t(t0 + j) * new_st_b + is);
  }
}

template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
}
template <typename T>
__device__ __forceinline__ void store_f(T* p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_f<float>(float* p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_f<uint16_t>(uint16_t* p, int64_t i, float x) { p[i] = dev::f32_to_bf16(x); }

// Split-KV merge: workgroup (merge item, head, block of kMergeRows rows); the
// chunk states of row r are partial rows slot0 + c*num_rows + r.
//   * Up to 64 chunks (the usual case): each row of the block is merged by
//     one, two or four waves (a block with fewer rows splits each row's dims).
//     Lane c holds chunk c's statistic, so the shift (largest statistic) and
//     the weight sum are wave reductions; then every lane accumulates its dims
//     over the chunks, reading each chunk's scale from the lane that owns it.
//   * More chunks (one long row split many ways): the workgroup merges its
//     rows one at a time.  Up to 256 chunks, thread c loads chunk c's
//     statistic once, and every thread starts loading its share of the
//     partial values before the reductions; beyond that, the shift
//     and the weight sum are block reductions, the normalised scales of up to
//     kMergeSeg chunks at a time are staged in LDS, and groups of threads
//     accumulate disjoint chunk subsets of the output row (4 dims per thread)
//     whose sums are added at the end.
constexpr int kMergeThreads = 256;
constexpr int kMergeRows = kMergeThreads / 64;   // rows per workgroup
constexpr int kMergeWaveChunks = 64;            // chunk count up to which one wave merges a row
constexpr int kMergeSeg = 512;
constexpr int kMergePre = 8;   // chunks of partial values per thread loaded ahead (long rows)

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float block_reduce(float x, float* s_red, bool is_max) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  __syncthreads();   // s_red free (previous reduction fully read)
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = s_red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) r = is_max ? fmaxf(r, s_red[w]) : r + s_red[w];
  return r;
}

template <typename T, bool kVec4>
__global__ __launch_bounds__(kMergeThreads) void merge_partials_kernel(const MergePartialArgs a) {
  __shared__ float s_w[kMergeSeg];
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ float4 s_acc[kMergeThreads];
  if (a.live_merges && int32_t(blockIdx.x) >= *a.live_merges) return;   // fixed-capacity grid
  const MergeItem mi = a.merges[blockIdx.x];
  const int32_t h = blockIdx.y;
  const int tid = threadIdx.x;
  const int32_t hq = a.num_heads, d_all = a.head_dim;
  const int32_t r_lo = int32_t(blockIdx.z) * kMergeRows;
  const int32_t r_hi = min(mi.num_rows, r_lo + kMergeRows);
  if (r_lo >= r_hi) return;   // uniform over the workgroup
  const int32_t n = mi.num_chunks;

  if (n <= kMergeWaveChunks) {
    // Waves per row: all four share one row (each a quarter of its dims) when
    // the block has one row, two share a row when it has two.
    const int32_t rows_here = r_hi - r_lo;
    // Waves per row: up to four (one row) or two (two rows), at most one per
    // 128 dims (a wave covers 128 dims with two per lane).
    const int32_t by_dims = max(1, d_all / 128);
    const int32_t wpr = rows_here == 1 ? min(4, by_dims) : (rows_here == 2 ? min(2, by_dims) : 1);
    const int32_t w = tid >> 6;
    const int32_t r = r_lo + w / wpr;
    const int32_t slice = w - (w / wpr) * wpr;
    const int lane = tid & 63;
    if (r >= r_hi) return;
    const int32_t d_lo = slice * d_all / wpr, d_hi = (slice + 1) * d_all / wpr;
    const int64_t row_base = int64_t(mi.slot0) + r;
    const float* pbase = a.part_o + (row_base * hq + h) * d_all;
    const int64_t chunk_stride = int64_t(mi.num_rows) * hq * d_all;
    // Up to 8 chunks and one 128-dim pass (split decode and MLA rows): the
    // partial values are loaded together with the statistics, so the two
    // memory latencies overlap.
    const bool fast = kVec4 && n <= 8 && (d_hi - d_lo) <= 128 && ((d_hi - d_lo) & 1) == 0;
    float2 pre[8];
    if (fast) {
      const int32_t d = d_lo + 2 * lane;
      const float* src = pbase + (d < d_hi ? d : d_lo);
      // Only the row's own chunks are loaded (n is uniform over the wave).
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pre[j] = j < n ? *reinterpret_cast<const float2*>(src + int64_t(j) * chunk_stride) : make_float2(0.f, 0.f);
    }
    const float sc = lane < n ? a.part_lse[(row_base + int64_t(lane) * mi.num_rows) * hq + h] : -INFINITY;
    const float mx = wave_max(sc);
    const float wl = sc == -INFINITY ? 0.f : dev::fast_exp2(sc - mx);   // mx finite whenever sc is
    const float z = wave_sum(wl);
    const float scale = z > 0.f ? wl / z : 0.f;
    const int32_t row = mi.q_row0 + r;
    T* orow = static_cast<T*>(a.o) + int64_t(row) * a.o_stride_token + int64_t(h) * a.o_stride_head;
    // Every lane stays active through the chunk loop: the scale of chunk c
    // lives in lane c.  With an even slice width each lane owns two
    // consecutive dims (8-byte loads); chunks go four at a time so four loads
    // are in flight, the steps past the last chunk re-reading it with weight 0.
    // Lanes past the slice end read dim d_lo and store nothing.
    if (fast) {
      const int32_t d = d_lo + 2 * lane;
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float w = j < n ? __shfl(scale, j) : 0.f;
        acc0 = fmaf(w, pre[j].x, acc0);
        acc1 = fmaf(w, pre[j].y, acc1);
      }
      if (d < d_hi) {
        store_f<T>(orow, d, acc0);
        store_f<T>(orow, d + 1, acc1);
      }
    } else if (kVec4 && ((d_hi - d_lo) & 1) == 0) {
      for (int32_t d0 = d_lo; d0 < d_hi; d0 += 128) {
        const int32_t d = d0 + 2 * lane;
        const bool own = d < d_hi;
        const float* src = pbase + (own ? d : d_lo);
        float acc0 = 0.f, acc1 = 0.f;
        for (int32_t c = 0; c < n; c += 4) {
          float2 x[4];
          float w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int32_t cc = min(c + j, n - 1);
            w[j] = c + j < n ? __shfl(scale, cc) : 0.f;
            x[j] = *reinterpret_cast<const float2*>(src + int64_t(cc) * chunk_stride);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc0 = fmaf(w[j], x[j].x, acc0);
            acc1 = fmaf(w[j], x[j].y, acc1);
          }
        }
        if (own) {
          store_f<T>(orow, d, acc0);
          store_f<T>(orow, d + 1, acc1);
        }
      }
    } else {
      for (int32_t d0 = d_lo; d0 < d_hi; d0 += 64) {
        const int32_t d = d0 + lane;
        const bool own = d < d_hi;
        float acc = 0.f;
        for (int32_t c = 0; c < n; ++c) {
          const float w = __shfl(scale, c);
          if (own && w != 0.f) acc = fmaf(w, pbase[int64_t(c) * chunk_stride + d], acc);
        }
        if (own) store_f<T>(orow, d, acc);
      }
    }
    if (slice == 0 && lane == 0 && a.lse) a.lse[int64_t(row) * hq + h] = z > 0.f ? mx + __log2f(z) : -INFINITY;
    return;
  }

  constexpr int kVec = kVec4 ? 4 : 1;
  const int32_t nvec = d_all / kVec;
  const int32_t tpr = min(nvec, kMergeThreads);   // threads per group (one vector each)
  const int32_t groups = kMergeThreads / tpr;
  const int32_t grp = tid / tpr, lv = tid - (tid / tpr) * tpr;
  if (kVec4 && n <= kMergeThreads && nvec <= kMergeThreads) {
    // Up to 256 chunks, output rows of at most 1024 dims: thread c holds chunk
    // c's statistic (one load), and each group's first kMergePre chunks of
    // partial values are loaded before the reductions, so their memory
    // latency overlaps that of the statistics.
    for (int32_t r = r_lo; r < r_hi; ++r) {
      const int64_t row_base = int64_t(mi.slot0) + r;
      const float sc = tid < n ? a.part_lse[(row_base + int64_t(tid) * mi.num_rows) * hq + h] : -INFINITY;
      const bool own = lv < nvec;
      const int32_t v = own ? lv : 0;
      auto part = [&](int32_t c) {
        return *reinterpret_cast<const float4*>(a.part_o + ((row_base + int64_t(c) * mi.num_rows) * hq + h) * d_all +
                                                v * kVec);
      };
      float4 pre[kMergePre];
#pragma unroll
      for (int j = 0; j < kMergePre; ++j) pre[j] = part(min(grp + j * groups, n - 1));
      const float mx = block_reduce(sc, s_red, true);
      const float wl = sc == -INFINITY ? 0.f : dev::fast_exp2(sc - mx);   // mx finite whenever sc is
      const float z = block_reduce(wl, s_red, false);
      s_w[tid] = z > 0.f ? wl / z : 0.f;   // chunk tid's normalised scale (0 past n)
      __syncthreads();
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      auto add = [&](float w, const float4& x) {
        acc.x = fmaf(w, x.x, acc.x);
        acc.y = fmaf(w, x.y, acc.y);
        acc.z = fmaf(w, x.z, acc.z);
        acc.w = fmaf(w, x.w, acc.w);
      };
#pragma unroll
      for (int j = 0; j < kMergePre; ++j) {
        const int32_t c = grp + j * groups;
        if (c < n) add(s_w[c], pre[j]);
      }
      for (int32_t c = grp + kMergePre * groups; c < n; c += groups) add(s_w[c], part(c));
      s_acc[tid] = acc;
      __syncthreads();
      const int32_t row = mi.q_row0 + r;
      T* orow = static_cast<T*>(a.o) + int64_t(row) * a.o_stride_token + int64_t(h) * a.o_stride_head;
      if (grp == 0 && own) {
        float4 t = acc;
        for (int32_t g = 1; g < groups; ++g) {
          const float4 u = s_acc[g * tpr + lv];
          t.x += u.x;
          t.y += u.y;
          t.z += u.z;
          t.w += u.w;
        }
        store_f<T>(orow, v * kVec, t.x);
        store_f<T>(orow, v * kVec + 1, t.y);
        store_f<T>(orow, v * kVec + 2, t.z);
        store_f<T>(orow, v * kVec + 3, t.w);
      }
      if (tid == 0 && a.lse) a.lse[int64_t(row) * hq + h] = z > 0.f ? mx + __log2f(z) : -INFINITY;
      __syncthreads();   // s_w and s_acc are free for the next row
    }
    return;
  }
  for (int32_t r = r_lo; r < r_hi; ++r) {
    const int64_t row_base = int64_t(mi.slot0) + r;   // partial row of chunk c: row_base + c * num_rows
    float mx = -INFINITY;
    for (int32_t c = tid; c < n; c += kMergeThreads)
      mx = fmaxf(mx, a.part_lse[(row_base + int64_t(c) * mi.num_rows) * hq + h]);
    mx = block_reduce(mx, s_red, true);
    float zp = 0.f;
    if (mx != -INFINITY)
      for (int32_t c = tid; c < n; c += kMergeThreads) {
        const float sc = a.part_lse[(row_base + int64_t(c) * mi.num_rows) * hq + h];
        if (sc != -INFINITY) zp += dev::fast_exp2(sc - mx);
      }
    const float z = block_reduce(zp, s_red, false);
    const float inv_z = z > 0.f ? 1.f / z : 0.f;
    const int32_t row = mi.q_row0 + r;
    T* orow = static_cast<T*>(a.o) + int64_t(row) * a.o_stride_token + int64_t(h) * a.o_stride_head;
    for (int32_t v0 = 0; v0 < nvec; v0 += tpr) {
      const int32_t v = v0 + lv;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int32_t seg = 0; seg < n && z > 0.f; seg += kMergeSeg) {
        const int32_t m = min(kMergeSeg, n - seg);
        __syncthreads();   // s_w free
        for (int32_t i = tid; i < m; i += kMergeThreads) {
          const float sc = a.part_lse[(row_base + int64_t(seg + i) * mi.num_rows) * hq + h];
          s_w[i] = sc == -INFINITY ? 0.f : dev::fast_exp2(sc - mx) * inv_z;
        }
        __syncthreads();
        if (grp < groups && v < nvec) {
#pragma unroll 4
          for (int32_t i = grp; i < m; i += groups) {
            const float w = s_w[i];
            if (w != 0.f) {
              const float* src = a.part_o + ((row_base + int64_t(seg + i) * mi.num_rows) * hq + h) * d_all + v * kVec;
              if constexpr (kVec4) {
                const float4 x = *reinterpret_cast<const float4*>(src);
                acc.x = fmaf(w, x.x, acc.x);
                acc.y = fmaf(w, x.y, acc.y);
                acc.z = fmaf(w, x.z, acc.z);
                acc.w = fmaf(w, x.w, acc.w);
              } else {
                acc.x = fmaf(w, *src, acc.x);
              }
            }
          }
        }
      }
      __syncthreads();   // s_acc free
      s_acc[tid] = acc;
      __syncthreads();
      if (grp == 0 && v < nvec) {
        float4 t = acc;
        for (int32_t g = 1; g < groups; ++g) {
          const float4 u = s_acc[g * tpr + lv];
          t.x += u.x;
          t.y += u.y;
          t.z += u.z;
          t.w += u.w;
        }
        store_f<T>(orow, v * kVec, t.x);
        if constexpr (kVec4) {
          store_f<T>(orow, v * kVec + 1, t.y);
          store_f<T>(orow, v * kVec + 2, t.z);
          store_f<T>(orow, v * kVec + 3, t.w);
        }
      }
    }
    if (tid == 0 && a.lse) a.lse[int64_t(row) * hq + h] = z > 0.f ? mx + __log2f(z) : -INFINITY;
  }
}

// Row-indexed merge (cascades): one wave per (query row, head, slice of
// 64 * VW dims; lane l owns VW consecutive dims).  The row's states are the
// partial rows listed in slots[row_ptr[r] .. row_ptr[r+1]); they come from
// different levels and tiles, so no stride relates them.  Lanes take the
// states 64 at a time: the shift and the weight sum are wave reductions over
// all of them; then every lane accumulates its dims over the states, reading
// each state's partial row and normalised scale from the lane that loaded it,
// four states per step so that four loads are in flight.  Every listed
// partial row was written by the attention launches (empty ones as (0, -inf)),
// so a zero-weight state is read and multiplied by 0 rather than skipped.
template <typename T, int VW>
__global__ __launch_bounds__(256) void merge_rows_kernel(const MergeRowsArgs a, int32_t slices) {
  using V = typename std::conditional<VW == 2, float2, float>::type;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int32_t hq = a.num_heads, d_all = a.head_dim;
  if (unit >= int64_t(a.num_rows) * hq * slices) return;   // whole wave
  const int32_t slice = int32_t(unit % slices);
  const int64_t rh = unit / slices;
  const int32_t h = int32_t(rh % hq);
  const int32_t r = int32_t(rh / hq);
  const int32_t p0 = a.row_ptr[r];
  const int32_t n = a.row_ptr[r + 1] - p0;
  float mx = -INFINITY;
  for (int32_t c = lane; c < n; c += 64) mx = fmaxf(mx, a.part_lse[int64_t(a.slots[p0 + c]) * hq + h]);
  mx = wave_max(mx);
  float zl = 0.f;
  if (mx != -INFINITY)
    for (int32_t c = lane; c < n; c += 64) {
      const float sc = a.part_lse[int64_t(a.slots[p0 + c]) * hq + h];
      if (sc != -INFINITY) zl += dev::fast_exp2(sc - mx);
    }
  const float z = wave_sum(zl);
  const float inv_z = z > 0.f ? 1.f / z : 0.f;
  const int32_t d = (slice * 64 + lane) * VW;
  const bool own = d < d_all;
  const int32_t dd = own ? d : 0;   // lanes past the row's dims read dim 0 and store nothing
  float acc[VW];
#pragma unroll
  for (int v = 0; v < VW; ++v) acc[v] = 0.f;
  const float* po = a.part_o + int64_t(h) * d_all + dd;
  const int64_t row_stride = int64_t(hq) * d_all;
  for (int32_t cb = 0; cb < n && z > 0.f; cb += 64) {
    const int32_t c = cb + lane;
    int32_t slot_l = a.slots[p0 + min(c, n - 1)];
    float w_l = 0.f;
    if (c < n) {
      const float sc = a.part_lse[int64_t(slot_l) * hq + h];
      w_l = sc == -INFINITY ? 0.f : dev::fast_exp2(sc - mx) * inv_z;
    }
    const int32_t m = min(64, n - cb);
    for (int32_t i = 0; i < m; i += 4) {
      V x[4];
      float w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = min(i + j, m - 1);   // past the batch: the last state again, weight 0
        w[j] = i + j < m ? __shfl(w_l, src) : 0.f;
        const int32_t sl = __shfl(slot_l, src);
        x[j] = *reinterpret_cast<const V*>(po + int64_t(sl) * row_stride);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (VW == 2) {
          acc[0] = fmaf(w[j], x[j].x, acc[0]);
          acc[1] = fmaf(w[j], x[j].y, acc[1]);
        } else {
          acc[0] = fmaf(w[j], x[j], acc[0]);
        }
      }
    }
  }
  if (own) {
    T* orow = static_cast<T*>(a.o) + int64_t(r) * a.o_stride_token + int64_t(h) * a.o_stride_head;
#pragma unroll
    for (int v = 0; v < VW; ++v) store_f<T>(orow, d + v, acc[v]);
  }
  if (slice == 0 && lane == 0 && a.lse) a.lse[int64_t(r) * hq + h] = z > 0.f ? mx + __log2f(z) : -INFINITY;
}

// Bit packing of a boolean array: thread w packs elements [32w, 32w + 32)
// into word w, element 32w + i at bit i (little-endian bytes: element e at
// bit e % 8 of byte e / 8).
__global__ __launch_bounds__(256) void packbits_kernel(const uint8_t* in, int64_t n, uint32_t* out) {
  const int64_t w = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t e0 = w * 32;
  if (e0 >= n) return;
  uint32_t word = 0;
  for (int i = 0; i < 32; ++i)
    if (e0 + i < n && in[e0 + i] != 0) word |= 1u << i;
  out[w] = word;
}

// Pairwise merge: one wave per (row, head).  Each wave reads both statistics
// before any lane writes, so v_out / s_out may alias the inputs.
template <typename T>
__global__ __launch_bounds__(256) void merge_pair_kernel(const T* va, const float* sa, const T* vb, const float* sb,
                                                         T* vo, float* so, int64_t row_heads, int32_t dim) {
  const int64_t rh = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rh >= row_heads) return;
  const float a_s = sa[rh], b_s = sb[rh];
  const bool a_empty = a_s == -INFINITY, b_empty = b_s == -INFINITY;
  const float mx = fmaxf(a_s, b_s);
  const float wa = a_empty ? 0.f : dev::fast_exp2(a_s - mx);
  const float wb = b_empty ? 0.f : dev::fast_exp2(b_s - mx);
  const float z = wa + wb;
  const float ca = z > 0.f ? wa / z : 0.f, cb = z > 0.f ? wb / z : 0.f;
  for (int32_t d = lane; d < dim; d += 64) {
    const int64_t i = rh * dim + d;
    const float x = load_f<T>(va, i), y = load_f<T>(vb, i);
    float out;
    if (a_empty) out = y;
    else if (b_empty) out = x;
    else out = ca * x + cb * y;
    store_f<T>(vo, i, out);
  }
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) so[rh] = a_empty ? b_s : (b_empty ? a_s : mx + __log2f(z));
}

// Many-way merge: one wave per (row, head) over num_states states.
template <typename T>
__global__ __launch_bounds__(256) void merge_many_kernel(const T* v, const float* s, T* vo, float* so, int64_t rows,
                                                         int32_t states, int32_t heads, int32_t dim) {
  const int64_t rh = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rh >= rows * heads) return;
  const int64_t row = rh / heads;
  const int32_t h = int32_t(rh - row * heads);
  float mx = -INFINITY;
  for (int32_t k = 0; k < states; ++k) mx = fmaxf(mx, s[(row * states + k) * heads + h]);
  float z = 0.f;
  if (mx != -INFINITY)
    for (int32_t k = 0; k < states; ++k) {
      const float sk = s[(row * states + k) * heads + h];
      if (sk != -INFINITY) z += dev::fast_exp2(sk - mx);
    }
  for (int32_t d = lane; d < dim; d += 64) {
    float acc = 0.f;
    if (z > 0.f)
      for (int32_t k = 0; k < states; ++k) {
        const float sk = s[(row * states + k) * heads + h];
        if (sk != -INFINITY)
          acc = fmaf(dev::fast_exp2(sk - mx) / z, load_f<T>(v, ((row * states + k) * heads + h) * dim + d), acc);
      }
    store_f<T>(vo, rh * dim + d, acc);
  }
  if (lane == 0) so[rh] = z > 0.f ? mx + __log2f(z) : -INFINITY;
}

// The XCD (accelerator complex die) that runs each workgroup, from the
// hardware register that names it: the library checks once per device that
// workgroups i and i + 8 share one XCD before it relies on that for the
// split merge inside the decode launch.
__global__ void xcd_probe_kernel(int32_t* out) {
  int32_t id;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
  if (threadIdx.x == 0) out[blockIdx.x] = id & 0xf;
}

}  // namespace

hipError_t launch_xcd_probe(int32_t* d_out, int32_t blocks, hipStream_t st) {
  hipLaunchKernelGGL(xcd_probe_kernel, dim3(uint32_t(blocks)), dim3(64), 0, st, d_out);
  return hipGetLastError();
}

hipError_t launch_append(int32_t dtype, const void* k_new, const void* v_new, int64_t new_st, int64_t new_sh,
                         const int32_t* append_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* last_page_len, int32_t batch, int32_t nnz, void* k, void* v,
                         int64_t page_stride, int64_t token_stride, int64_t head_stride, int32_t page_size,
                         int32_t num_heads, int32_t head_dim, int32_t max_num_pages, hipStream_t st) {
  const int64_t es = dtype == kF32 ? 4 : (dtype == kFP8 ? 1 : 2);
  const int32_t row_chunks = int32_t(head_dim * es / 16);
  const int64_t token_chunks = 2 * int64_t(num_heads) * row_chunks;   // K and V rows of one token
  // Tokens per block: one.  Blocks of several tokens (up to what the
  // per-thread chunk registers hold) read all their rows before they write
  // any, and with every block resident at once the copy's reads and writes
  // then hardly overlap: on the prefill batch (9680 new tokens, 8 kv heads,
  // head_dim 128) one token per block took 23.2 us, two 24.6, four 27.2 and
  // eight 26.5.  The kernel keeps the general form (tpb tokens per block).
  const int64_t cap = std::max<int64_t>(1, int64_t(kAppendThreads) * kAppendMaxChunks / token_chunks);
  const int64_t tpb = std::min<int64_t>({cap, int64_t(kAppendMaxTok), int64_t(1)});
  const int64_t blocks = (nnz + tpb - 1) / tpb;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_kernel, dim3(uint32_t(blocks)), dim3(kAppendThreads), 0, st,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), new_st * es, new_sh * es,
                     append_indptr, kv_indptr, kv_indices, last_page_len, batch, nnz, int32_t(tpb),
                     static_cast<char*>(k), static_cast<char*>(v), page_stride * es, token_stride * es,
                     head_stride * es, page_size, num_heads, row_chunks, max_num_pages);
  return hipGetLastError();
}

hipError_t launch_merge_partials(int32_t dtype, const MergePartialArgs& a, hipStream_t st) {
  const int32_t row_blocks = (std::max(a.max_rows, 1) + kMergeRows - 1) / kMergeRows;
  if (row_blocks > 65535 || a.num_heads > 65535) return hipErrorInvalidValue;
  const dim3 grid(uint32_t(a.num_merges), uint32_t(a.num_heads), uint32_t(row_blocks));
  const dim3 block(kMergeThreads);
  const bool vec4 = a.head_dim % 4 == 0;
  if (dtype == kBF16) {
    if (vec4)
      hipLaunchKernelGGL((merge_partials_kernel<uint16_t, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((merge_partials_kernel<uint16_t, false>), grid, block, 0, st, a);
  } else {
    if (vec4)
      hipLaunchKernelGGL((merge_partials_kernel<float, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((merge_partials_kernel<float, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_merge_rows(int32_t dtype, const MergeRowsArgs& a, hipStream_t st) {
  if (a.num_rows <= 0 || a.num_heads <= 0 || a.head_dim <= 0) return hipSuccess;
  const bool pair = a.head_dim % 128 == 0;   // two dims per lane (8-byte loads)
  const int32_t slices = pair ? a.head_dim / 128 : (a.head_dim + 63) / 64;
  const int64_t blocks = (int64_t(a.num_rows) * a.num_heads * slices + 3) / 4;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid{static_cast<uint32_t>(blocks)}, block{256};
  if (dtype == kBF16) {
    if (pair)
      hipLaunchKernelGGL((merge_rows_kernel<uint16_t, 2>), grid, block, 0, st, a, slices);
    else
      hipLaunchKernelGGL((merge_rows_kernel<uint16_t, 1>), grid, block, 0, st, a, slices);
  } else {
    if (pair)
      hipLaunchKernelGGL((merge_rows_kernel<float, 2>), grid, block, 0, st, a, slices);
    else
      hipLaunchKernelGGL((merge_rows_kernel<float, 1>), grid, block, 0, st, a, slices);
  }
  return hipGetLastError();
}

hipError_t launch_packbits(const uint8_t* in, int64_t n, uint32_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t words = (n + 31) / 32;
  const int64_t blocks = (words + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(packbits_kernel, dim3(uint32_t(blocks)), dim3(256), 0, st, in, n, out);
  return hipGetLastError();
}

hipError_t launch_merge_pair(int32_t dtype, const void* va, const float* sa, const void* vb, const float* sb,
                             void* vo, float* so, int64_t rows, int32_t heads, int32_t dim, hipStream_t st) {
  const int64_t rh = rows * heads;
  const int64_t blocks = (rh + 3) / 4;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (dtype == kBF16)
    hipLaunchKernelGGL(merge_pair_kernel<uint16_t>, dim3(uint32_t(blocks)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(va), sa, static_cast<const uint16_t*>(vb), sb,
                       static_cast<uint16_t*>(vo), so, rh, dim);
  else
    hipLaunchKernelGGL(merge_pair_kernel<float>, dim3(uint32_t(blocks)), dim3(256), 0, st,
                       static_cast<const float*>(va), sa, static_cast<const float*>(vb), sb, static_cast<float*>(vo),
                       so, rh, dim);
  return hipGetLastError();
}

hipError_t launch_merge_many(int32_t dtype, const void* v, const float* s, void* vo, float* so, int64_t rows,
                             int32_t states, int32_t heads, int32_t dim, hipStream_t st) {
  const int64_t blocks = (rows * heads + 3) / 4;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (dtype == kBF16)
    hipLaunchKernelGGL(merge_many_kernel<uint16_t>, dim3(uint32_t(blocks)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(v), s, static_cast<uint16_t*>(vo), so, rows, states, heads, dim);
  else
    hipLaunchKernelGGL(merge_many_kernel<float>, dim3(uint32_t(blocks)), dim3(256), 0, st,
                       static_cast<const float*>(v), s, static_cast<float*>(vo), so, rows, states, heads, dim);
  return hipGetLastError();
}

}  // namespace pkv
