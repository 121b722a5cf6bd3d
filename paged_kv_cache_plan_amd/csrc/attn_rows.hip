// Paged attention, one query row at a time: the decode kernel.
//
// Decode reads a long history for very little arithmetic, so this kernel is
// built around HBM streaming ("Deep Dive - FlashInfer", "Ragged prefill and
// paged decode"): each workgroup takes one work item (a key chunk of one
// request) for one kv head and all G query heads that share it (GQA: query head
// h reads kv head h / G).  Every K and V row is fetched from HBM exactly once
// per kv head and used for all G heads.  The arithmetic is plain VALU work.
//
// Work split inside a workgroup (4 waves of 64 lanes): waves take interleaved
// blocks of 16 keys, and each wave keeps the loads of its next block in flight
// while it computes the current one (two register sets).
//   Score phase: a quad of 4 lanes owns one key; each lane loads a quarter of
//     the key row with 16-byte loads (4 lanes x 16 B = 64 contiguous bytes per
//     instruction) and forms partial dot products for the G heads (bf16 pairs
//     through v_dot2c_f32_bf16); two DPP quad exchanges finish them.
//   Softmax: the wave is cut into softmax groups (a 16-lane row, or half a row
//     for 64-wide heads).  A group's quads score exactly the keys its value
//     lanes consume, so the running max m, the rescale factor and the weights
//     stay inside the group: the block max is two DPP row rotations, with no
//     cross-row traffic.  Scores are pre-multiplied by sm_scale * log2 e and
//     exponentiated with exp2.
//   Value phase: 16 lanes own one value row (each lane 16 bytes), 4 rows per
//     load instruction.  For bf16, the weights of two keys are packed as a bf16
//     pair in LDS and the values of the same two keys are paired with v_perm,
//     so one v_dot2c accumulates two keys for one (head, dim).  The rescale of
//     the accumulator is skipped when no lane's max moved.
// At the end the groups and the 4 waves are merged and written either as the
// final output (dtype of Q, plus base-2 LSE) or as an fp32 partial state for
// the split merge ("Deep Dive - FlashInfer", "A worked split-KV example").
//
// One-wave workgroups: this file compiled with PKV_ROWS_WAVES = 1 (the
// translation unit attn_rows_one_wave.hip) gives the same kernel with one wave
// per workgroup, which takes every 16-key block of its item itself.  Batches
// of many short items (a few blocks each) leave most waves of a 4-wave
// workgroup idle and pay one workgroup start per (item, kv head); one-wave
// workgroups put up to four times as many items on a CU at once.  Plans pick
// it for decode batches of many short items (the rule and its measurements
// are in the host planner).
//
// Loads are branch-free: a key past the end of the row's range re-reads the
// last valid key (its weight is zero), and a page id outside the pool is
// replaced by page 0 so no access leaves the cache allocation (the host
// validates page ids; such rows would give undefined values, never a fault).
//
// Multi-row tiles (float32 prefill) loop over their rows; row r sees key j iff
// j <= diag + r ("Causality uses logical positions, not page numbers").
//
// An fp8 cache (E4M3 codes, "FlashInfer 中的 KV-Cache 布局" names fp8 caches)
// is read at one byte per element: a 16-byte load holds 16 codes, which
// v_cvt_scalef32_pk_bf16_fp8 expands (exactly) into two bf16 chunks, so the
// arithmetic is the bf16 path's.  The per-tensor K scale is folded into the
// logit scale and the V scale is applied to the normalised output.

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

// Waves per workgroup of this translation unit's kernels: 4, or 1 (see above).
#ifndef PKV_ROWS_WAVES
#define PKV_ROWS_WAVES 4
#endif
constexpr int kWaves = PKV_ROWS_WAVES;
static_assert(kWaves == 4 || kWaves == 1, "row kernel workgroups of 4 or 1 waves");
constexpr int kBlockKeys = 16;
constexpr int kSegPages = 1024;   // page ids staged in LDS per segment
// K and V rows are read once per launch: non-temporal loads (compile-time tunable).
#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1
#endif
constexpr bool kStreamKV = PKV_DECODE_NT != 0;
// Lanes that share one key row (16 or 8; compile-time tunable).  Each load
// instruction then covers whole 128-byte lines of VT = 64 / lanes key rows.
#ifndef PKV_DECODE_ROW_LANES
#define PKV_DECODE_ROW_LANES 16
#endif
constexpr int kRowLanes = PKV_DECODE_ROW_LANES;
// Key blocks in flight per wave (register sets): 2 or 3 (compile-time tunable;
// 3 applies to bf16 only, where the extra set still fits in 256 VGPRs).
#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 2
#endif
// Minimum waves per SIMD the register allocation must allow (compile-time tunable).
#ifndef PKV_ROWS_MIN_WAVES
#define PKV_ROWS_MIN_WAVES 2
#endif

template <typename T>
struct Elem {
  static constexpr int kPer16 = 16 / int(sizeof(T));
};

template <typename T>
__device__ __forceinline__ void dot_chunk(const uint4& q, const uint4& k, float& acc);

template <>
__device__ __forceinline__ void dot_chunk<uint16_t>(const uint4& q, const uint4& k, float& acc) {
  acc = dev::dot2_bf16(q.x, k.x, acc);
  acc = dev::dot2_bf16(q.y, k.y, acc);
  acc = dev::dot2_bf16(q.z, k.z, acc);
  acc = dev::dot2_bf16(q.w, k.w, acc);
}

template <>
__device__ __forceinline__ void dot_chunk<float>(const uint4& q, const uint4& k, float& acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
}

// Two floats as a bf16 pair (round to nearest even): lo in bits 0-15.
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
  dev::bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { *p = dev::f32_to_bf16(x); }
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }

// Sum over the L lanes that share one key row (L = 16: a DPP row; L = 8: half
// a row).  Every step pairs lanes symmetrically (x + partner), so all L lanes
// end with bitwise the same sum.
template <int L>
__device__ __forceinline__ float row_sum(float x) {
  x += dev::dpp<dev::kQuadSwap1>(x);
  x += dev::dpp<dev::kQuadSwap2>(x);
  x += dev::dpp<dev::kRowHalfMirror>(x);
  if constexpr (L == 16) x += dev::dpp<dev::kRowMirror>(x);
  return x;
}

// Rows with many (head, dim) accumulators and wide register sets (float32, or
// bf16 with 8 heads per group at head_dim 128) need more than 256 VGPRs; they
// run one wave per SIMD instead of spilling.
template <typename T, int D, int G>
constexpr int rows_min_waves() {
  return int(sizeof(T)) * D * G >= 2048 ? 1 : PKV_ROWS_MIN_WAVES;
}

// 16 fp8 codes -> two chunks of 8 bf16 values (exact conversion).
__device__ __forceinline__ void expand_fp8(const uint4& raw, uint4& lo, uint4& hi) {
  auto cv0 = [](uint32_t w) {   // codes in bytes 0, 1
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  };
  auto cv1 = [](uint32_t w) {   // codes in bytes 2, 3
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  };
  lo = make_uint4(cv0(raw.x), cv1(raw.x), cv0(raw.y), cv1(raw.y));
  hi = make_uint4(cv0(raw.z), cv1(raw.z), cv0(raw.w), cv1(raw.w));
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Split merge inside the decode launch ("Deep Dive - FlashInfer", "A worked
// split-KV example": shift by the largest base-2 statistic, weights
// 2^(s - shift) normalised by their sum, LSE = shift + log2 sum).  Called by
// every thread of a workgroup that has just written the partial state of one
// chunk of (row, kv head): it counts the chunk in merge_ctr, and the
// workgroup that finishes the last chunk folds all of them into o and lse.
// All chunks of one (merge item, kv head) run on the same XCD, so the partial
// states stored by the others are in its L2 once each writer has waited for
// its stores; the reader drops its own L1 lines first.  The arithmetic and
// its order are those of the separate merge kernel.
template <int W, typename T, int D, int G>
__device__ void merge_in_launch(const AttnArgs& a, int32_t m, const MergeItem& mi, int32_t row, int32_t kvh) {
  __shared__ int32_t s_last;
  const int32_t hq = a.num_qo_heads;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's partial stores are in L2
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t* ctr = a.merge_ctr + int64_t(m) * a.num_kv_heads + kvh;
    const int32_t done = atomicAdd(ctr, 1) + 1;
    const bool last = done == mi.num_chunks;
    if (last) atomicExch(ctr, 0);   // zero again for the next launch
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;   // uniform: another workgroup finishes this row
  asm volatile("buffer_inv sc0" ::: "memory");
  const int32_t n = mi.num_chunks, slot0 = mi.slot0;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int32_t hh = wave; hh < G; hh += W) {
    const int32_t head = kvh * G + hh;
    const float* pbase = a.part_o + (int64_t(slot0) * hq + head) * D;
    const int64_t cstride = int64_t(hq) * D;   // partial rows of one merge item's chunks are consecutive
    auto stat = [&](int32_t c) { return a.part_lse[(int64_t(slot0) + c) * hq + head]; };
    const bool pre = n <= 8 && D <= 128;
    float2 x8[8];
    const int32_t d_first = min(2 * lane, D - 2);
    if (pre) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x8[j] = j < n ? *reinterpret_cast<const float2*>(pbase + int64_t(j) * cstride + d_first)
                      : make_float2(0.f, 0.f);
    }
    const float sc = lane < n ? stat(lane) : -INFINITY;
    float mx = sc;
    for (int32_t c = lane + 64; c < n; c += 64) mx = fmaxf(mx, stat(c));
    mx = wave_max(mx);
    const float wl = sc == -INFINITY ? 0.f : dev::fast_exp2(sc - mx);   // mx finite whenever sc is
    float zp = wl;
    for (int32_t c = lane + 64; c < n; c += 64) {
      const float s2 = stat(c);
      zp += s2 == -INFINITY ? 0.f : dev::fast_exp2(s2 - mx);
    }
    const float z = wave_sum(zp);
    const float scale = z > 0.f ? wl / z : 0.f;
    auto weight = [&](int32_t c) {   // chunk c's normalised weight
      if (c < 64) return __shfl(scale, c);
      const float s2 = stat(c);
      return s2 == -INFINITY || !(z > 0.f) ? 0.f : dev::fast_exp2(s2 - mx) / z;
    };
    T* orow = static_cast<T*>(a.o) + int64_t(row) * a.o_stride_token + int64_t(head) * a.o_stride_head;
    if (pre) {
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float w = j < n ? __shfl(scale, j) : 0.f;
        acc0 = fmaf(w, x8[j].x, acc0);
        acc1 = fmaf(w, x8[j].y, acc1);
      }
      if (2 * lane < D) {
        store_out<T>(orow + 2 * lane, acc0);
        store_out<T>(orow + 2 * lane + 1, acc1);
      }
    } else {
      // Many chunks: the partial rows come in groups of kFold, the loads of
      // the next group issued before the current one is folded, so that the
      // row waits for about n / kFold L2 round trips (it waited for n / 4).
      // The fold keeps the chunk order.
      constexpr int kFold = 16;
      for (int32_t d0 = 0; d0 < D; d0 += 128) {
        const int32_t d = d0 + 2 * lane;
        const float* src = pbase + min(d, D - 2);
        float acc0 = 0.f, acc1 = 0.f;
        float2 x[kFold], y[kFold];
        auto fetch = [&](float2 (&dst)[kFold], int32_t c0) {   // chunks past the last re-read it
          const float* pj = src + int64_t(c0) * cstride;
#pragma unroll
          for (int j = 0; j < kFold; ++j) {
            dst[j] = *reinterpret_cast<const float2*>(pj);
            pj += c0 + j + 1 < n ? cstride : 0;
          }
        };
        auto fold = [&](const float2 (&xs)[kFold], int32_t c0) {
#pragma unroll
          for (int j = 0; j < kFold; ++j) {
            const float w = c0 + j < n ? weight(c0 + j) : 0.f;
            acc0 = fmaf(w, xs[j].x, acc0);
            acc1 = fmaf(w, xs[j].y, acc1);
          }
        };
        fetch(x, 0);
        for (int32_t c0 = 0; c0 < n; c0 += 2 * kFold) {
          if (c0 + kFold < n) fetch(y, c0 + kFold);
          fold(x, c0);
          if (c0 + kFold >= n) break;
          if (c0 + 2 * kFold < n) fetch(x, c0 + 2 * kFold);
          fold(y, c0 + kFold);
        }
        if (d < D) {
          store_out<T>(orow + d, acc0);
          store_out<T>(orow + d + 1, acc1);
        }
      }
    }
    if (lane == 0 && a.lse) a.lse[int64_t(row) * hq + head] = z > 0.f ? mx + __log2f(z) : -INFINITY;
  }
}

// W: waves per workgroup (4 or 1).  T: query / output elements (bf16 bits or
// float).  TK: stored K/V elements (T itself, or uint8_t E4M3 codes with T = bf16).
template <int W, typename T, typename TK, int D, int G, bool kAligned, bool kMask, bool kAppend, bool kMergeIn>
__global__ __launch_bounds__(64 * W, (rows_min_waves<T, D, G>())) void attn_rows_kernel(const AttnArgs a) {
  constexpr int kThreads = 64 * W;
  constexpr bool kBF16 = sizeof(T) == 2;
  constexpr bool kFp8 = sizeof(TK) == 1;
  static_assert(!kFp8 || kBF16, "fp8 caches compute on the bf16 path");
  constexpr int E = Elem<T>::kPer16;       // elements per (expanded) 16-byte chunk
  constexpr int RE = 16 / int(sizeof(TK)); // elements per 16-byte load of K or V
  constexpr int X = RE / E;                // expanded chunks per load (2 for fp8)
  constexpr int NCH = D / RE;              // loads per key row
  constexpr int VL = NCH < kRowLanes ? NCH : kRowLanes;  // lanes per key row = one softmax group
  constexpr int VCR = NCH / VL;            // loads per lane and key row
  constexpr int VC = VCR * X;              // expanded chunks per lane
  constexpr int VT = 64 / VL;              // key rows per load instruction = groups per wave
  constexpr int NU = kBlockKeys / VT;      // load instructions per block = keys per group per block
  static_assert(NCH % VL == 0 && (VL == 16 || VL == 8), "unsupported head_dim");
  static_assert(NU % 2 == 0, "keys of a group come in pairs");
  constexpr int kDepth = (kBF16 && G <= 4) ? PKV_DECODE_DEPTH : 2;

  __shared__ int32_t s_pages[kSegPages];
  __shared__ float s_m[W][G];
  __shared__ float s_l[W][G];
  __shared__ float s_acc[W][G][D];
  // Fused append: the first boundary block's K and V rows of each wave
  // (bf16 and fp8 rows; float32 rows load their boundary block after the loop).
  constexpr bool kPreBoundary = kBF16 && kDepth == 2;
  __shared__ uint4 s_new[(kAppend && kPreBoundary) ? W * NU * VCR * 128 : 1];

  const int32_t hkv = a.num_kv_heads;
  const int32_t item_idx = blockIdx.x / hkv;
  if (a.live_items && item_idx >= *a.live_items) return;   // fixed-capacity grid: whole workgroup
  const Item it = a.items[item_idx];
  // Workgroup item * Hkv + j takes kv head (j + b) mod Hkv of request b:
  // workgroups run on XCD (blockIdx mod 8), so every XCD serves a mix of kv
  // heads (heads whose rows sit at some offsets in the token rows stream
  // more slowly than others; on the decode batch this evens out the XCDs'
  // finish times and saves about 4% of the launch), while all chunks of one
  // (request, kv head) still share an XCD, as the merge inside the launch
  // needs.  (Rotating by the item instead measured slower than no rotation.)
  const int32_t kvh = (int32_t(blockIdx.x) - item_idx * hkv + it.batch % hkv) % hkv;
  // A chunk of a split decode row, with the merge inside the launch: its
  // merge item, read now so that the end of the workgroup waits on no load.
  int32_t merge_m = -1;
  MergeItem merge_item{0, 0, 0, 0};
  if (kMergeIn && it.out_slot >= 0) {
    merge_m = a.tile_merge[it.batch];
    merge_item = a.merges[merge_m];
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Group vg of the wave holds key u * VT + vg of each 16-key block (u < NU);
  // lane vi of the group holds chunks vi + VL * c of those rows.
  const int vg = lane / VL, vi = lane % VL;

  const TK* kbase = static_cast<const TK*>(a.k) + int64_t(kvh) * a.head_stride;
  const TK* vbase = static_cast<const TK*>(a.v) + int64_t(kvh) * a.head_stride;
  // Expanded chunk c = X * cr + x of lane vi covers dims dim_of(c) + [0, E).
  auto dim_of = [&](int c) { return (vi + VL * (c / X)) * RE + (c % X) * E; };
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t hq = a.num_qo_heads;
  const int32_t psz = a.page_size, pshift = a.page_shift;
  const uint32_t max_pages = uint32_t(a.max_num_pages);
  auto page_of = [&](int32_t j) { return kAligned ? (j >> pshift) : (pshift >= 0 ? (j >> pshift) : (j / psz)); };
  auto slot_of = [&](int32_t j) {
    return kAligned ? (j & (psz - 1)) : (pshift >= 0 ? (j & (psz - 1)) : (j - (j / psz) * psz));
  };

  // Fused append: the request's n_b new rows are its keys [kv_len - n_b,
  // kv_len) (kv_len already counts them), read from k_new / v_new and stored
  // into their cache slots for this kv head by the workgroup whose chunk
  // holds them, as the append kernel would (each key of a decode row lies in
  // one item).  Key j >= new_lo is row j + new_off of k_new (clamped into the
  // nnz_new rows, so that inconsistent metadata never reads outside them).
  int32_t new_lo = INT32_MAX, new_off = 0;
  const TK* knew = nullptr;
  const TK* vnew = nullptr;
  if constexpr (kAppend) {
    const int32_t b = it.batch;
    const int32_t a0 = a.append_indptr[b], a1 = a.append_indptr[b + 1];
    const int32_t np = a.kv_indptr[b + 1] - a.kv_indptr[b];
    const int32_t kvlen = np > 0 ? (np - 1) * psz + a.kv_last[b] : 0;
    new_lo = max(kvlen - (a1 - a0), 0);
    new_off = a1 - kvlen;
    knew = static_cast<const TK*>(a.k_new) + int64_t(kvh) * a.new_stride_head;
    vnew = static_cast<const TK*>(a.v_new) + int64_t(kvh) * a.new_stride_head;
  }

  for (int r = 0; r < it.num_rows; ++r) {
    const int32_t row = it.q_row0 + r;
    const int32_t lo = it.kv_start;
    const int32_t hi = min(it.kv_end, it.diag + r + 1);
    int64_t mask_bit0 = 0;   // bit of (row, key 0) in the packed custom mask
    if constexpr (kMask) {
      const MaskRow mr = a.mask_rows[it.batch];
      mask_bit0 = mr.bit0 + int64_t(row - mr.q_start) * mr.kv_len;
    }

    uint4 qreg[G][VC];
    const T* qrow = static_cast<const T*>(a.q) + int64_t(row) * a.q_stride_token +
                    int64_t(kvh * G) * a.q_stride_head;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < VC; ++c)
        qreg[h][c] = *reinterpret_cast<const uint4*>(qrow + int64_t(h) * a.q_stride_head + dim_of(c));

    float m[G], l[G], acc[G][VC * E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < VC * E; ++e) acc[h][e] = 0.f;
    }

    const int32_t p_lo = lo < hi ? page_of(lo) : 0;
    const int32_t p_hi = lo < hi ? page_of(hi - 1) + 1 : 0;
    for (int32_t sp = p_lo; sp < p_hi; sp += kSegPages) {
      // Stage this segment's page ids in LDS.
      const int32_t np = min(kSegPages, p_hi - sp);
      __syncthreads();
      for (int i = threadIdx.x; i < np; i += kThreads) {
        const int32_t pg = pages[sp + i];
        // Ids outside the pool read page 0; with a fused append they keep the
        // sign bit as a mark, so that no new row is stored through them.
        s_pages[i] = uint32_t(pg) < max_pages ? pg : (kAppend ? INT32_MIN : 0);
      }
      __syncthreads();
      auto page_id = [&](int32_t i) { return kAppend ? (s_pages[i] & INT32_MAX) : s_pages[i]; };
      const int32_t tlo = max(lo, sp * psz);
      int32_t thi = min(hi, (sp + np) * psz);   // lowered below past a fused append's new keys

      // Element offset of key j's row; keys at or past thi re-read key thi-1.
      auto row_off = [&](int32_t j) -> int64_t {
        j = min(j, thi - 1);
        return int64_t(page_id(page_of(j) - sp)) * a.page_stride + int64_t(slot_of(j)) * a.token_stride;
      };
      // K and V rows of one block: instruction u moves key rows u*VT + g, each
      // read by VL lanes as contiguous 16-byte chunks (whole rows per request).
      auto load = [&](int32_t blk, uint4 (&kr)[NU][VCR], uint4 (&vr)[NU][VCR]) {
        int64_t off[NU];
        if constexpr (kAligned) {
          // A 16-key block never crosses a page: one page id for the block.
          const int64_t base = int64_t(page_id((blk >> pshift) - sp)) * a.page_stride;
          const int32_t last = thi - 1 - blk;
          const int32_t s0 = blk & (psz - 1);
#pragma unroll
          for (int u = 0; u < NU; ++u) off[u] = base + int64_t(s0 + min(u * VT + vg, last)) * a.token_stride;
        } else {
#pragma unroll
          for (int u = 0; u < NU; ++u) off[u] = row_off(blk + u * VT + vg);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int c = 0; c < VCR; ++c) kr[u][c] = dev::load16<kStreamKV>(kbase + off[u] + (vi + VL * c) * RE);
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int c = 0; c < VCR; ++c) vr[u][c] = dev::load16<kStreamKV>(vbase + off[u] + (vi + VL * c) * RE);
      };

      auto compute = [&](int32_t blk, uint4 (&kraw)[NU][VCR], uint4 (&vraw)[NU][VCR]) __attribute__((always_inline)) {
        // K and V rows as bf16 / f32 chunks (fp8 codes expanded in registers).
        uint4 kr[NU][VC], vr[NU][VC];
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int c = 0; c < VCR; ++c) {
            if constexpr (kFp8) {
              expand_fp8(kraw[u][c], kr[u][2 * c], kr[u][2 * c + 1]);
              expand_fp8(vraw[u][c], vr[u][2 * c], vr[u][2 * c + 1]);
            } else {
              kr[u][c] = kraw[u][c];
              vr[u][c] = vraw[u][c];
            }
          }
        // Scores of the group's NU keys for the G heads; every lane of the
        // group ends with all of them, so the softmax below is in-lane.
        float p[NU][G];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int32_t key = blk + u * VT + vg;
          bool ok = key < thi;
          if constexpr (kMask) {   // custom mask: the key's bit in this row
            const int64_t bit = mask_bit0 + (ok ? key : 0);
            ok = ok && ((a.mask[bit >> 5] >> (bit & 31)) & 1u);
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < VC; ++c) dot_chunk<T>(qreg[h][c], kr[u][c], part);
            const float sc = row_sum<VL>(part) * a.scale_log2;
            p[u][h] = ok ? sc : -INFINITY;
          }
        }
        float scale[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float mx = p[0][h];
#pragma unroll
          for (int u = 1; u < NU; ++u) mx = fmaxf(mx, p[u][h]);
          const float m_new = fmaxf(m[h], mx);
          const bool live = m_new != -INFINITY;   // false only while every key so far was skipped
          scale[h] = live ? dev::fast_exp2(m[h] - m_new) : 1.f;
          float sum = 0.f;
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            p[u][h] = live ? dev::fast_exp2(p[u][h] - m_new) : 0.f;
            sum += p[u][h];
          }
          l[h] = l[h] * scale[h] + sum;
          m[h] = m_new;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (__any(scale[h] != 1.f)) {
#pragma unroll
            for (int e = 0; e < VC * E; ++e) acc[h][e] *= scale[h];
          }
        }
        if constexpr (kBF16) {
          // Two keys per v_dot2c: the weights as a bf16 pair, the values of
          // the same two keys paired per dim with v_perm.
#pragma unroll
          for (int w = 0; w < NU / 2; ++w) {
            uint32_t pp[G];
#pragma unroll
            for (int h = 0; h < G; ++h) pp[h] = pack_pair(p[2 * w][h], p[2 * w + 1][h]);
#pragma unroll
            for (int c = 0; c < VC; ++c) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t x0 = word(vr[2 * w][c], i), x1 = word(vr[2 * w + 1][c], i);
                const uint32_t even = __builtin_amdgcn_perm(x1, x0, 0x05040100u);  // dim 2i of both keys
                const uint32_t odd = __builtin_amdgcn_perm(x1, x0, 0x07060302u);   // dim 2i+1
#pragma unroll
                for (int h = 0; h < G; ++h) {
                  acc[h][c * E + 2 * i] = dev::dot2_bf16(even, pp[h], acc[h][c * E + 2 * i]);
                  acc[h][c * E + 2 * i + 1] = dev::dot2_bf16(odd, pp[h], acc[h][c * E + 2 * i + 1]);
                }
              }
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int c = 0; c < VC; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float x = __uint_as_float(word(vr[u][c], i));
#pragma unroll
                for (int h = 0; h < G; ++h) acc[h][c * E + i] = fmaf(p[u][h], x, acc[h][c * E + i]);
              }
        }
      };

      constexpr int32_t kStride = W * kBlockKeys;
      // Fused append: the blocks from the one holding the segment's first new
      // key nlo onward (the boundary blocks) mix cached keys (below nlo) and
      // rows of k_new / v_new.  Each goes to the wave that owns it in the
      // loop's interleave; the wave loads its first one here, ahead of the
      // loop's loads, and computes it first (the online softmax is
      // order-free, so only the fp32 rounding differs from the order without
      // the append).  The loop below covers the cached blocks [tlo, nb0).
      const int32_t thi_all = thi;
      int32_t nlo = thi, nb0 = thi, bb = thi, bb0 = thi;
      // The boundary block blk (cached keys through the page ids, new keys
      // from k_new / v_new) into the register set kx / vx.
      auto load_mixed = [&](int32_t blk, uint4 (&kx)[NU][VCR], uint4 (&vx)[NU][VCR]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int32_t key = min(blk + u * VT + vg, thi_all - 1);
          const int64_t row = min(max(int64_t(new_off) + key, int64_t(0)), int64_t(a.nnz_new) - 1);
          const bool fresh = key >= nlo;
          const int64_t off = fresh ? row * a.new_stride_token
                                    : int64_t(page_id(page_of(key) - sp)) * a.page_stride +
                                          int64_t(slot_of(key)) * a.token_stride;
          const TK* kp = (fresh ? knew : kbase) + off;
          const TK* vp = (fresh ? vnew : vbase) + off;
#pragma unroll
          for (int c = 0; c < VCR; ++c) {
            kx[u][c] = dev::load16<kStreamKV>(kp + (vi + VL * c) * RE);
            vx[u][c] = dev::load16<kStreamKV>(vp + (vi + VL * c) * RE);
          }
        }
      };
      if constexpr (kAppend) {
        nlo = max(tlo, new_lo);
        if (nlo < thi) {
          nb0 = tlo + (nlo - tlo) / kBlockKeys * kBlockKeys;
          const int32_t k0 = (nb0 - tlo) / kBlockKeys;
          bb = nb0 + ((wave - k0) % W + W) % W * kBlockKeys;
          bb0 = bb;
          thi = nb0;
        }
      }

      // Register sets: the loads of the next block(s) are in flight while a
      // block computes.  The prefetch is unconditional (past the end it
      // re-reads the last block, which the caches serve) so that every path
      // through the loop has the same loads outstanding and the wait before a
      // block's compute covers only that block's own loads.
      const int32_t blk_max = kAligned ? ((thi - 1) & ~(kBlockKeys - 1)) : thi - 1;
      int32_t blk = tlo + wave * kBlockKeys;
      // The new rows of boundary block blk (in kx / vx) into their cache
      // slots, first row only.  Issued after the wave's last load: a store
      // counts like a load in the wave's memory counter, and one between the
      // loop's loads would make every later wait cover it too.
      auto store_new = [&](int32_t blk, uint4 (&kx)[NU][VCR], uint4 (&vx)[NU][VCR]) __attribute__((always_inline)) {
        if (r != 0) return;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int32_t key = blk + u * VT + vg;
          const int32_t pg = key >= nlo && key < thi_all ? s_pages[page_of(key) - sp] : -1;
          if (pg >= 0) {   // a marked (outside the pool) page stores nothing
            // The cache is the caller's writable pool (const only for the plain run).
            const int64_t off = int64_t(pg) * a.page_stride + int64_t(slot_of(key)) * a.token_stride;
            TK* kd = const_cast<TK*>(kbase) + off;
            TK* vd = const_cast<TK*>(vbase) + off;
#pragma unroll
            for (int c = 0; c < VCR; ++c) {
              *reinterpret_cast<uint4*>(kd + (vi + VL * c) * RE) = kx[u][c];
              *reinterpret_cast<uint4*>(vd + (vi + VL * c) * RE) = vx[u][c];
            }
          }
        }
      };
      // Block bb against the segment's full key range.
      auto boundary = [&](uint4 (&kx)[NU][VCR], uint4 (&vx)[NU][VCR]) __attribute__((always_inline)) {
        const int32_t thi_loop = thi;
        thi = thi_all;
        compute(bb, kx, vx);
        thi = thi_loop;
      };
      // The first boundary block's rows wait in LDS (which takes no part in
      // the memory counter) from its compute, ahead of the loop, to their
      // stores after it.
      auto stash = [&](uint4 (&kx)[NU][VCR], uint4 (&vx)[NU][VCR], bool put) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int c = 0; c < VCR; ++c) {
            uint4* sk = &s_new[((wave * NU + u) * VCR + c) * 128 + lane];
            if (put) {
              sk[0] = kx[u][c];
              sk[64] = vx[u][c];
            } else {
              kx[u][c] = sk[0];
              vx[u][c] = sk[64];
            }
          }
      };
      bool first_done = false;   // the first boundary block is computed (rows in s_new)
      uint4 ka[NU][VCR], kb[NU][VCR], va[NU][VCR], vb[NU][VCR];
      if constexpr (kDepth == 3) {
        uint4 kc[NU][VCR], vc[NU][VCR];
        if (blk < thi) {
          load(blk, ka, va);
          load(min(blk + kStride, blk_max), kb, vb);
          while (true) {
            load(min(blk + 2 * kStride, blk_max), kc, vc);
            compute(blk, ka, va);
            blk += kStride;
            if (blk >= thi) break;
            load(min(blk + 2 * kStride, blk_max), ka, va);
            compute(blk, kb, vb);
            blk += kStride;
            if (blk >= thi) break;
            load(min(blk + 2 * kStride, blk_max), kb, vb);
            compute(blk, kc, vc);
            blk += kStride;
            if (blk >= thi) break;
          }
        }
      } else {
        // A wave that owns a boundary block loads it first, into kb (free
        // until the loop's first prefetch), and computes it while the loop's
        // first loads are in flight.
        if (kAppend && kPreBoundary && bb < thi_all) load_mixed(bb, kb, vb);
        if (blk < thi) {
          load(blk, ka, va);
          if constexpr (kAppend && kPreBoundary) {
            if (bb < thi_all) {
              boundary(kb, vb);
              stash(kb, vb, true);
              first_done = true;
            }
          }
          while (true) {
            load(min(blk + kStride, blk_max), kb, vb);
            compute(blk, ka, va);
            blk += kStride;
            if (blk >= thi) break;
            load(min(blk + kStride, blk_max), ka, va);
            compute(blk, kb, vb);
            blk += kStride;
            if (blk >= thi) break;
          }
        }
      }
      if constexpr (kAppend) {
        if (first_done) {
          stash(ka, va, false);
          store_new(bb, ka, va);
          bb += kStride;
        }
        // A wave without cached blocks takes its first boundary block here
        // (already in kb when prefetched); appends that reach past one block
        // per wave take the rest here.
        for (; bb < thi_all; bb += kStride) {
          if (!(kPreBoundary && kDepth == 2 && bb == bb0)) load_mixed(bb, kb, vb);
          boundary(kb, vb);
          store_new(bb, kb, vb);
        }
      }
    }

    // Wave state: rescale every group to the wave max, then sum l and acc
    // over the groups (l and m are the same on all lanes of a group).
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mw = m[h];
#pragma unroll
      for (int off = VL; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
      const float f = m[h] == -INFINITY ? 0.f : dev::fast_exp2(m[h] - mw);
      float lw = l[h] * f;
#pragma unroll
      for (int off = VL; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
      l[h] = lw;
      m[h] = mw;
#pragma unroll
      for (int e = 0; e < VC * E; ++e) {
        float x = acc[h][e] * f;
#pragma unroll
        for (int off = VL; off < 64; off <<= 1) x += __shfl_xor(x, off);
        acc[h][e] = x;
      }
    }
    if (lane < VL) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < VC; ++c)
#pragma unroll
          for (int e = 0; e < E; ++e) s_acc[wave][h][dim_of(c) + e] = acc[h][c * E + e];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
    __syncthreads();

    // Merge the waves' states and write the row.
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
      const int h = idx / D, d = idx - (idx / D) * D;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) mm = fmaxf(mm, s_m[w][h]);
      float ll = 0.f, oo = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = s_m[w][h] == -INFINITY ? 0.f : dev::fast_exp2(s_m[w][h] - mm);
        ll += f * s_l[w][h];
        oo += f * s_acc[w][h][d];
      }
      const bool empty = !(ll > 0.f);
      float out = empty ? 0.f : oo / ll;
      if constexpr (kFp8) out *= a.v_scale;
      const float lse2 = empty ? -INFINITY : mm + __log2f(ll);
      const int32_t head = kvh * G + h;
      if (it.out_slot < 0) {
        T* orow = static_cast<T*>(a.o) + int64_t(row) * a.o_stride_token + int64_t(head) * a.o_stride_head;
        store_out<T>(orow + d, out);
        if (d == 0 && a.lse) a.lse[int64_t(row) * hq + head] = lse2;
      } else {
        const int64_t prow = int64_t(it.out_slot + r) * hq + head;
        a.part_o[prow * D + d] = out;
        if (d == 0) a.part_lse[prow] = lse2;
      }
    }
    if constexpr (kMergeIn) {
      if (merge_m >= 0) merge_in_launch<W, T, D, G>(a, merge_m, merge_item, row, kvh);
    }
    __syncthreads();
  }
}

template <typename T, typename TK, int D, int G>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const int64_t blocks = int64_t(a.num_items) * a.num_kv_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const bool aligned = a.page_shift >= 4;   // a power-of-two page of at least 16 keys
  const dim3 grid{static_cast<uint32_t>(blocks)}, block{64 * kWaves};
  if (a.mask && (a.append_indptr || a.merge_ctr)) return hipErrorInvalidValue;   // masks run plain launches
  // Each variant is its own kernel, so that the plain decode launch carries
  // neither the append nor the in-launch merge code (their registers cost
  // the plain kernel about 1 us on the decode batch).
  auto go = [&](auto kernel) { launch_attention_kernel(kernel, grid, block, st, a); };
  if constexpr (kWaves == 1) {
    // One-wave workgroups serve decode plans only: plain runs and runs with a
    // fused append (no masks, no merge inside the launch).
    if (a.mask || a.merge_ctr) return hipErrorInvalidValue;
    if (a.append_indptr) {
      if (aligned) go(attn_rows_kernel<1, T, TK, D, G, true, false, true, false>);
      else go(attn_rows_kernel<1, T, TK, D, G, false, false, true, false>);
    } else {
      if (aligned) go(attn_rows_kernel<1, T, TK, D, G, true, false, false, false>);
      else go(attn_rows_kernel<1, T, TK, D, G, false, false, false, false>);
    }
  } else if (a.mask) {
    if (aligned) go(attn_rows_kernel<4, T, TK, D, G, true, true, false, false>);
    else go(attn_rows_kernel<4, T, TK, D, G, false, true, false, false>);
  } else if (a.append_indptr && a.merge_ctr) {
    if (aligned) go(attn_rows_kernel<4, T, TK, D, G, true, false, true, true>);
    else go(attn_rows_kernel<4, T, TK, D, G, false, false, true, true>);
  } else if (a.append_indptr) {
    if (aligned) go(attn_rows_kernel<4, T, TK, D, G, true, false, true, false>);
    else go(attn_rows_kernel<4, T, TK, D, G, false, false, true, false>);
  } else if (a.merge_ctr) {
    if (aligned) go(attn_rows_kernel<4, T, TK, D, G, true, false, false, true>);
    else go(attn_rows_kernel<4, T, TK, D, G, false, false, false, true>);
  } else {
    if (aligned) go(attn_rows_kernel<4, T, TK, D, G, true, false, false, false>);
    else go(attn_rows_kernel<4, T, TK, D, G, false, false, false, false>);
  }
  return hipGetLastError();
}

template <typename T, typename TK, int D>
hipError_t launch_g(int32_t group, const AttnArgs& a, hipStream_t st, bool* ok) {
  *ok = true;
  switch (group) {
    case 1: return launch_t<T, TK, D, 1>(a, st);
    case 2: return launch_t<T, TK, D, 2>(a, st);
    case 4: return launch_t<T, TK, D, 4>(a, st);
    case 8:
      if (sizeof(T) == 2) return launch_t<T, TK, D, 8>(a, st);
      break;
    default: break;
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

#if PKV_ROWS_WAVES == 1
hipError_t launch_attn_rows_one_wave(int32_t dtype, int32_t head_dim, int32_t group, const AttnArgs& a,
                                     hipStream_t st, bool* supported) {
#else
hipError_t launch_attn_rows(int32_t dtype, int32_t head_dim, int32_t group, const AttnArgs& a,
                            hipStream_t st, bool* supported) {
#endif
  *supported = false;
  if (dtype == kBF16) {
    if (head_dim == 128) return launch_g<uint16_t, uint16_t, 128>(group, a, st, supported);
    if (head_dim == 64) return launch_g<uint16_t, uint16_t, 64>(group, a, st, supported);
  } else if (dtype == kF32) {
    if (head_dim == 128) return launch_g<float, float, 128>(group, a, st, supported);
    if (head_dim == 64) return launch_g<float, float, 64>(group, a, st, supported);
  } else if (dtype == kFP8) {   // bf16 queries over an E4M3 cache
    if (head_dim == 128) return launch_g<uint16_t, uint8_t, 128>(group, a, st, supported);
  }
  return hipSuccess;
}

}  // namespace pkv
