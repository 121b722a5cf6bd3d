// Paged prefill / append attention for bf16 with MFMA tiles (gfx950).
//
// Prefill and append attention is a dense contraction once a tile of keys
// is gathered ("Deep Dive - FlashInfer", "Ragged prefill and paged decode"),
// so both products run on v_mfma_f32_32x32x16_bf16:
//
//   * A workgroup (8 waves, two per SIMD) owns one work item for one kv head:
//     up to 256 (query row, head) pairs -- 256/G rows times the G query heads
//     that share the kv head -- against one chunk of keys.  Wave w owns pairs
//     [32w, 32w + 32).  All eight waves consume the same K/V tiles, so each
//     tile brought on chip feeds 256 pairs.
//   * Keys stream through LDS in tiles of 64, in a ring of four K and four V
//     tiles filled by direct global->LDS loads (global_load_lds_dwordx4): no
//     staging registers and no LDS store instructions.  The loads of K(t+4) and
//     V(t+3) are issued right after the one barrier of tile t and have three
//     whole tiles to land; the barrier waits only for the loads issued three
//     tiles earlier.
//   * Page gather: on pages of >= 16 keys (a power of two) the 16 keys that one
//     load instruction covers share a page, so the page id is wave-uniform and
//     its 64-bit offset is scalar arithmetic; each lane adds a fixed 32-bit
//     offset.  Other page sizes and a chunk's partial last tile locate every
//     key through the page table per lane.
//   * Tiles are stored unpadded with an XOR swizzle of the 16-byte chunks of a
//     row (K: chunk ^ (row & 15); V: chunk ^ 4*(row & 3)), chosen so that the
//     K operand reads (16 rows, one chunk) and the transposed V reads (4 rows,
//     32 bytes each) hit distinct LDS banks.
//   * Scores are computed transposed, S^T = K Q^T (M = keys, N = pairs), so
//     each lane holds the scores of ONE pair: the row max and row sum are
//     in-lane over 32 keys plus one exchange with lane l^32.  Q stays in
//     registers as the B operand for the whole chunk.
//   * The weights P^T come out of that layout already shaped as the B operand
//     of O^T = V^T P^T (the key order inside an MFMA k-step is a permutation
//     shared by both operands, which the contraction does not see); V^T is read
//     from the row-major LDS tile with ds_read_b64_tr_b16.  O^T accumulates in
//     registers, one pair per lane, matching the row statistics.
//   * Online softmax in the log2 domain with a lazy max: the accumulator is
//     rescaled only when a row's max grows by more than 8 (so weights stay below
//     2^8); masking (causal diagonal, chunk end) is applied only on tiles that
//     need it ("Causality uses logical positions, not page numbers": row r of
//     the tile sees key j iff j <= diag + r).  The scores of tile t+1 are
//     issued on the matrix cores interleaved with the exponentials of tile t.
//
// The epilogue writes the normalised rows (bf16) and base-2 LSE, or fp32
// partial states for the split merge ("A worked split-KV example").
//
// fp8 caches ("FlashInfer 中的 KV-Cache 布局" names E4M3 caches): the kFp8
// variant moves K and V tiles of E4M3 codes (128-byte rows, half the bytes)
// through a ring of four fp8 slots by the same direct loads.  One tile step
// ahead of its use, the waves expand each landed tile exactly into bf16
// (v_cvt_scalef32_pk_bf16_fp8) and store it, with the bf16 swizzles, into one
// of two bf16 work tiles, which the unchanged MFMA phases then read.  The
// expansion of tile t+1 and the products of tile t share one barrier per step.
// The K scale is folded into the logit scale, the V scale into the final
// normalisation.
//
// Custom masks ("FlashInfer 中的 KV-Cache 布局", "掩码布局"): the kMask
// variant moves, with every K tile, the tile's mask bits of each of its rows
// into LDS by the same direct loads: 32 bytes per row, read from the 16-byte
// boundary at or below the row's first key bit, which covers the 64 bits of
// the tile.  The first waves issue these loads (one more per tile step, and a
// correspondingly larger wait count at their barriers); every lane then reads
// its row's 64 bits with a funnel shift and keeps the scores whose bit is 1.

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kD = 128;          // head dim
constexpr int kKeys = 64;        // keys per LDS tile
constexpr int kTile = kKeys * kD;  // elements of one K or V tile (16 KiB)
constexpr int kMaxChunkPages = 1024;   // the planner never makes a chunk longer than this
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazyMax = 8.f;  // rescale only when a row max grows by more than this (log2 units)

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// lane i supplies the address of 4 consecutive bf16 values C_i[0..3] and
// receives C_{4e + i/4}[i % 4] for e = 0..3.
__device__ __forceinline__ bf16x4_t tr_read(const uint16_t* lds_elem) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(const_cast<uint16_t*>(lds_elem)));
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// lds_wave_base + 16 l (the LDS address goes in M0, so it must be
// wave-uniform; a write of M0 needs one wait state, the s_nop, before a load
// that reads it).  Issued as inline assembly so that the compiler neither
// reorders it nor inserts waits for it: the kernel's own protocol orders these
// loads (each tile barrier waits until only the latest tile step's loads are
// outstanding, and the kernel drains them all before its epilogue).
__device__ __forceinline__ void dma16(const void* src, uint16_t* lds_wave_base) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "m0");
}

// Waits for every outstanding tile load of this wave.
__device__ __forceinline__ void dma_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes into LDS (any LDS byte address, wave-uniform base) -- mask rows.
__device__ __forceinline__ void dma16_bytes(const void* src, const void* lds_wave_base) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "m0");
}

// Pins a value in registers at this point of the instruction stream, so the
// compiler cannot sink its computation into a later block.
__device__ __forceinline__ void keep(const uint4& x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}

// Barrier for tiles filled by direct loads.  The loads count on vmcnt; a
// plain __syncthreads() carries a release fence that the compiler lowers to
// vmcnt(0) (the loads write LDS), which would drain every prefetch.  Instead
// each wave waits until at most 2 * kLoadsPerTile of its own loads -- those of
// the two most recent tile steps -- are outstanding and all its LDS reads have
// returned, then joins the barrier.  The memory clobber keeps the compiler
// from moving LDS accesses across it.
constexpr int kLoadsPerTile = 4;   // per thread and tile step: 2 for a K tile + 2 for a V tile
__device__ __forceinline__ void dma_barrier() {
  static_assert(kLoadsPerTile == 4, "the wait count below is written out");
  asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// fp8 tiles: one load per thread for each of K and V per step, and the slot
// expanded in step t was loaded in step t-2, so only the previous step's two
// loads may still be outstanding.
__device__ __forceinline__ void dma_barrier_fp8() {
  asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// ... and for the waves that also load mask rows (three loads per step).
__device__ __forceinline__ void dma_barrier_fp8_mask_wave() {
  asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 E4M3 codes -> two chunks of 8 bf16 values (exact conversion).
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

// Waves that also load mask rows issue kLoadsPerTile + 1 loads per step.
__device__ __forceinline__ void dma_barrier_mask_wave() {
  asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int G, bool kPow2, bool kMask, bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void prefill_mfma_kernel(const AttnArgs a) {
  constexpr int kTileRows = 256 / G;                 // query rows of a work item
  constexpr int kMaskInstr = kTileRows * 2 / 64;     // 16-byte mask pieces of a tile / 64 lanes
  static_assert(!kMask || (kMaskInstr >= 1 && kMaskInstr <= kWaves), "mask rows per tile");
  constexpr int kEs = kFp8 ? 1 : 2;                  // bytes per stored K/V element
  // Ring slot i holds K(t+1) (first half) and V(t) (second half) for the
  // tile steps t with t % 4 == i: exactly what step t reads, and what step
  // t-3 loads.  Four separate arrays, so the compiler can tell the slot being
  // read from the slots being loaded.  (kFp8: the ring holds E4M3 codes in
  // s_f<i>, and step t reads the bf16 work tile s_w<t % 2>.)
  __shared__ __attribute__((aligned(16))) uint16_t s_b0[kFp8 ? 8 : 2 * kTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_b1[kFp8 ? 8 : 2 * kTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_b2[kFp8 ? 8 : 2 * kTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_b3[kFp8 ? 8 : 2 * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t s_f0[kFp8 ? 2 * kTile : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_f1[kFp8 ? 2 * kTile : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_f2[kFp8 ? 2 * kTile : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_f3[kFp8 ? 2 * kTile : 16];
  __shared__ __attribute__((aligned(16))) uint16_t s_w0[kFp8 ? 2 * kTile : 8];
  __shared__ __attribute__((aligned(16))) uint16_t s_w1[kFp8 ? 2 * kTile : 8];
  __shared__ int32_t s_pages[kMaxChunkPages];
  // Mask ring (kMask): slot i holds, for the tile whose K is in s_b<i>, 32
  // bytes per tile row.
  __shared__ uint4 s_mask[kMask ? 4 * kTileRows * 2 : 1];

  const int32_t hkv = a.num_kv_heads;
  const int32_t item_idx = blockIdx.x / hkv;
  const int32_t kvh = blockIdx.x - item_idx * hkv;
  if (a.live_items && item_idx >= *a.live_items) return;   // fixed-capacity grid: whole workgroup
  const Item it = a.items[item_idx];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;          // lane half: which 8-element k slice of an MFMA operand
  const int col = lane & 31;        // MFMA column: the pair this lane scores

  // This lane's (row, head) pair.
  const int pair = wave * 32 + col;
  const int prow = pair / G, phead = pair - (pair / G) * G;
  const bool pair_ok = prow < it.num_rows;
  // Waves whose 32 pairs all lie past the tile's rows (short tiles: a
  // request's last rows, small cascade nodes) only load and synchronise.
  const bool wave_active = 32 * wave < it.num_rows * G;
  const int32_t qrow_idx = it.q_row0 + prow;
  const int32_t head = kvh * G + phead;
  const int32_t limit = pair_ok ? min(it.kv_end - 1, it.diag + prow) : -1;   // last visible key
  // Smallest row limit in the wave: tiles ending at or before it need no mask.
  const int32_t wave_limit_min = min(it.kv_end - 1, it.diag + (wave * 32) / G);
  // Custom mask: bit of (row, key 0) for this lane's row and for the row whose
  // mask pieces this lane loads (lane l of mask wave w: row (64w + l) / 2).
  int64_t mask_row_bit = 0, mask_dma_bit = 0;
  const char* const mask_bytes = reinterpret_cast<const char*>(a.mask);
  if constexpr (kMask) {
    const MaskRow mr = a.mask_rows[it.batch];
    const int32_t local0 = it.q_row0 - mr.q_start;
    mask_row_bit = mr.bit0 + int64_t(local0 + (pair_ok ? prow : 0)) * mr.kv_len;
    const int dma_r = (64 * min(wave, kMaskInstr - 1) + lane) >> 1;
    mask_dma_bit = mr.bit0 + int64_t(local0 + (dma_r < it.num_rows ? dma_r : 0)) * mr.kv_len;
  }

  const char* const kbase = static_cast<const char*>(a.k) + int64_t(kvh) * a.head_stride * kEs;
  const char* const vbase = static_cast<const char*>(a.v) + int64_t(kvh) * a.head_stride * kEs;
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t psz = a.page_size, pshift = a.page_shift;
  const uint32_t max_pages = uint32_t(a.max_num_pages);
  const int64_t page_bytes = a.page_stride * kEs;
  const uint32_t tok_bytes = uint32_t(a.token_stride) * kEs;   // the launcher bounds 16 rows of it below 2^31

  // Q^T as the B operand: k-step s covers dims [16s, 16s+16); this lane holds dims 16s + 8h + [0, 8).
  uint4 qreg[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + int64_t(qrow_idx) * a.q_stride_token +
                         int64_t(head) * a.q_stride_head;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qreg[s] = pair_ok ? *reinterpret_cast<const uint4*>(qp + 16 * s + 8 * h) : make_uint4(0, 0, 0, 0);
  }

  f32x16_t oacc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[n][v] = 0.f;
  float m_used = -INFINITY;   // running max in scaled log2 units
  float lsum = 0.f;           // this lane's share of the row sum (its half of every key block)

  const int32_t kv_lo = it.kv_start, kv_hi = it.kv_end;
  const int32_t ntiles = kv_hi > kv_lo ? (kv_hi - kv_lo + kKeys - 1) / kKeys : 0;

  // Page ids of the chunk (at most kMaxChunkPages, a planner guarantee) go to
  // LDS once; ids outside the pool read page 0 instead.
  const int32_t pg_lo = kv_hi > kv_lo ? (kPow2 ? kv_lo >> pshift : kv_lo / psz) : 0;
  const int32_t pg_n =
      kv_hi > kv_lo ? min(kMaxChunkPages, (kPow2 ? (kv_hi - 1) >> pshift : (kv_hi - 1) / psz) - pg_lo + 1) : 0;
  for (int i = tid; i < pg_n; i += kThreads) {
    const int32_t pg = pages[pg_lo + i];
    s_pages[i] = uint32_t(pg) < max_pages ? pg : 0;
  }
  // Q must have landed before the tile loop on every path: the compiler does
  // not count the tile loads (inline assembly), so a Q load still pending at
  // the loop would make it wait for every outstanding load before the first
  // score product of each tile step.
#pragma unroll
  for (int s = 0; s < 8; ++s) keep(qreg[s]);
  __syncthreads();

  // Tile loads.  A tile is four groups of 16 rows.  Load instruction i (0, 1)
  // of wave w fills rows 16g + 4(w%4) + [0, 4) of group g = 2i + w/4 (1 KiB);
  // lane l writes row 16g + 4(w%4) + l/16, stored chunk l%16, which holds
  // source chunk (l%16) ^ swizzle(row).  Keys past the chunk end (and whole
  // tiles past it) re-read the last key: their scores are masked to -inf or
  // never used, so their weights are exactly zero.
  const int w4 = wave & 3, gh = wave >> 2;
  const int dma_row = 4 * w4 + (lane >> 4);                      // row within each 16-row group
  const int ck = (lane & 15) ^ dma_row;                          // K: chunk ^ (row & 15)
  const int cv = (lane & 15) ^ ((lane >> 4) << 2);               // V: chunk ^ 4 (row & 3)
  const uint32_t lane_k = uint32_t(dma_row) * tok_bytes + uint32_t(ck) * 16;
  const uint32_t lane_v = uint32_t(dma_row) * tok_bytes + uint32_t(cv) * 16;
  const bool aligned = kPow2 && pshift >= 4;
  // A full tile on pages of >= 16 keys: each 16-row group covers keys
  // t0 + 16g + [0, 16), all on one page, so its page offset is uniform.
  auto tile_aligned = [&](int32_t t0) { return aligned && t0 + kKeys <= kv_hi; };
  // Byte offsets of this wave's two groups (g = gh, 2 + gh) of an aligned tile.
  auto page_offsets = [&](int32_t t0, int64_t (&off)[2]) {
    int32_t pg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) pg[i] = s_pages[((t0 + 16 * (2 * i + gh)) >> pshift) - pg_lo];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      off[i] = int64_t(__builtin_amdgcn_readfirstlane(pg[i])) * page_bytes +
               int64_t((t0 + 16 * (2 * i + gh)) & (psz - 1)) * tok_bytes;
  };
  auto dma_aligned = [&](const char* base, uint32_t lane_off, uint16_t* dst, const int64_t (&off)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(base + off[i] + lane_off, dst + (16 * (2 * i + gh) + 4 * w4) * kD);
  };
  auto dma_general = [&](const char* base, int chunk, uint16_t* dst, int32_t t0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = 2 * i + gh;
      const int32_t j = min(t0 + 16 * g + dma_row, kv_hi - 1);
      const int32_t pi = kPow2 ? (j >> pshift) : (j / psz);
      const int32_t sl = kPow2 ? (j & (psz - 1)) : (j - pi * psz);
      const int32_t pg = s_pages[min(pi - pg_lo, kMaxChunkPages - 1)];
      dma16(base + (int64_t(pg) * page_bytes + int64_t(sl) * tok_bytes + chunk * 16), dst + (16 * g + 4 * w4) * kD);
    }
  };
  // Every tile step issues exactly kLoadsPerTile loads per thread (tiles past
  // the chunk end load the last key), so the barrier's wait count is exact.
  // The K load of a tile computes its page offsets; its V load one step later
  // reuses them.
  int64_t off_next[2] = {0, 0};
  auto load_k = [&](uint16_t* dst, int32_t t0) {
    if (tile_aligned(t0)) {
      page_offsets(t0, off_next);
      dma_aligned(kbase, lane_k, dst, off_next);
    } else {
      dma_general(kbase, ck, dst, t0);
    }
  };
  auto load_v = [&](uint16_t* dst, int32_t t0) {   // after load_k of the same tile
    if (tile_aligned(t0)) dma_aligned(vbase, lane_v, dst, off_next);
    else dma_general(vbase, cv, dst, t0);
  };
  // Mask pieces of the tile starting at t0 (mask waves only): lane l of wave
  // w fetches half l & 1 of row (64w + l) / 2's 32 bytes.  Tiles past the
  // chunk end fetch the bits of its last key instead (never used).
  auto load_m = [&](uint4* slot, int32_t t0) {
    if constexpr (kMask) {
      if (wave < kMaskInstr) {
        const int64_t bit = mask_dma_bit + min(t0, kv_hi - 1);
        const char* src = mask_bytes + ((bit >> 3) & ~int64_t(15)) + 16 * (lane & 1);
        dma16_bytes(src, slot + 64 * wave);
      }
    }
  };
  auto barrier = [&]() {
    if (kMask && wave < kMaskInstr) dma_barrier_mask_wave();
    else dma_barrier();
  };

  // S^T of the K tile in kbuf: two 32-key blocks.  Lane (col, h) reads row
  // 32kb + col, source chunk 2st + h, stored at chunk (2st + h) ^ (col & 15).
  const int kx = h ^ (col & 15);
  auto scores = [&](const uint16_t* kbuf, f32x16_t (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 kv = *reinterpret_cast<const uint4*>(kbuf + (kb * 32 + col) * kD + ((2 * st) ^ kx) * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), as_bf16x8(qreg[st]), sacc[kb], 0, 0, 0);
      }
    }
  };

  // V^T reads: 16-lane group grp, lane gi reads row 4h + gi/4 (+16ks, +8 for
  // the upper half) at elements 32n + 16(grp&1) + 4(gi&3), i.e. source chunk
  // 4n + 2(grp&1) + (gi&3)/2, stored at chunk 4(n ^ gi/4) + 2(grp&1) + (gi&3)/2.
  const int grp = lane >> 4, gi = lane & 15;
  const int v_lane = (4 * h + (gi >> 2)) * kD + (2 * (grp & 1) + ((gi & 3) >> 1)) * 8 + 4 * (gi & 1);
  const int v_sw = gi >> 2;
  const float c = a.scale_log2;

  // Causal / chunk-end mask of a score tile whose first key is t0: the key of
  // value v in block kb is t0 + 32kb + 8(v/4) + 4h + v%4.  Tiles that end at
  // or before every row limit of the wave need none.
  auto mask_tile = [&](f32x16_t (&sc)[2], int32_t t0, const uint4* mslot) {
    if constexpr (kMask) {
      // This row's 64 bits for keys t0 .. t0 + 63: bit k of (lo, hi).
      const int64_t bit = mask_row_bit + t0;
      const int sh = int(bit & 127);
      const uint32_t* words = reinterpret_cast<const uint32_t*>(mslot + 2 * (pair_ok ? prow : 0));
      const int w0 = sh >> 5, s5 = sh & 31;
      const uint32_t d0 = words[w0], d1 = words[w0 + 1], d2 = words[w0 + 2];
      const uint32_t lo = __builtin_amdgcn_alignbit(d1, d0, s5);
      const uint32_t hi = __builtin_amdgcn_alignbit(d2, d1, s5);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int k = 8 * (v >> 2) + 4 * h + (v & 3);
          const int32_t j = t0 + 32 * kb + k;
          const bool on = (((kb ? hi : lo) >> k) & 1u) != 0;
          sc[kb][v] = (on && j <= limit) ? sc[kb][v] : -INFINITY;
        }
      return;
    }
    if (t0 + kKeys - 1 > wave_limit_min) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t j = t0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
          sc[kb][v] = j <= limit ? sc[kb][v] : -INFINITY;
        }
    }
  };
  auto tile_max = [&](const f32x16_t (&sc)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb][v]);
    return fmaxf(mx, __shfl_xor(mx, 32));
  };
  // Lazy running max: move to the tile max only when it exceeds the current
  // shift by more than kLazyMax (the accumulator and sum are rescaled then).
  auto update_max = [&](float mx) {
    const float m_cand = mx * c;
    const bool grow = m_cand > m_used + kLazyMax || (m_used == -INFINITY && m_cand != -INFINITY);
    if (__any(grow)) {
      const float m_new = grow ? m_cand : m_used;
      const float f = grow ? (m_used == -INFINITY ? 0.f : dev::fast_exp2(m_used - m_new)) : 1.f;
      m_used = m_new;
      lsum *= f;
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[n][v] *= f;
    }
  };
  // Weights of k-step ks (16 keys) of a tile as the bf16 B operand of the PV
  // product.  exp2(-inf) = 0 covers masked keys; a row with no visible key yet
  // has only -inf scores, so any finite shift works for it.  The row sum adds
  // the fp32 weights.
  auto weights = [&](const f32x16_t (&sc)[2], int ks, float shift, float& ls0, float& ls1) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = dev::fast_exp2(fmaf(sc[ks >> 1][8 * (ks & 1) + e], c, -shift));
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      ls0 += p[e];
      ls1 += p[e + 1];
    }
    return make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
  };
  // O^T += V^T P^T for k-step ks (16 keys), all four 32-dim blocks.  The
  // transposed read gives lane i of each 16-lane group the value rows of 4
  // keys at one dim.
  auto pv_step = [&](const uint16_t* vbuf, int ks, const uint4& pbk) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint16_t* base = vbuf + 16 * ks * kD + v_lane + 32 * (n ^ v_sw);
      const bf16x4_t lo = tr_read(base);
      const bf16x4_t hi = tr_read(base + 8 * kD);
      const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16x8(pbk), oacc[n], 0, 0, 0);
    }
  };

  // One tile step t, in phases: the weights of tile t (vector work), O +=
  // V(t) P(t) (16 MFMAs), then S(t+1) = K(t+1) Q^T (16 MFMAs) into the same
  // registers, then its mask and max.  One score tile is live at a time, which
  // leaves the registers to keep several LDS reads in flight ahead of the
  // MFMAs; the two waves that share a SIMD overlap one's vector phase with
  // the other's matrix phase.  On entry S(t) is in sc (masked, its max folded
  // into m_used) and K(t+1), V(t) are (being) loaded into kread / vread;
  // V(t+3) -> vdma and K(t+4) -> kdma are issued here.
  auto body = [&](int32_t t, const uint16_t* kread, const uint16_t* vread, uint16_t* kdma, uint16_t* vdma,
                  const uint4* mread, uint4* mdma, f32x16_t (&sc)[2]) {
    const int32_t t0 = kv_lo + t * kKeys;
    // K(t+1) and V(t) have landed for every wave, and every wave is done
    // reading the slot of step t-1, which now takes V(t+3) and K(t+4).
    barrier();
    load_v(vdma, t0 + 3 * kKeys);
    load_k(kdma, t0 + 4 * kKeys);
    load_m(mdma, t0 + 4 * kKeys);
    if (!wave_active) return;
    const float shift = m_used != -INFINITY ? m_used : 0.f;
    float ls0 = 0.f, ls1 = 0.f;
    uint4 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pb[ks] = weights(sc, ks, shift, ls0, ls1);
    lsum += ls0 + ls1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pv_step(vread, ks, pb[ks]);
    if (t + 1 < ntiles) {
      scores(kread, sc);
      mask_tile(sc, t0 + kKeys, mread);
      update_max(tile_max(sc));
    }
  };

  // fp8 tiles: 64 rows of 128 codes (8 KiB).  Wave w's single load
  // instruction of a tile fills rows 8w + l/8, chunk l%8 (lane l), unswizzled;
  // keys past the chunk end re-read the last key.  On pages of >= 8 keys (a
  // power of two) the 8 rows of an instruction share a page.
  const bool aligned8 = kPow2 && pshift >= 3;
  const uint32_t lane8 = uint32_t(lane >> 3) * tok_bytes + uint32_t(lane & 7) * 16;
  auto load8 = [&](const char* base, uint8_t* dst, int32_t t0) {
    if constexpr (kFp8) {
      const int32_t r0 = t0 + 8 * wave;
      const char* src;
      if (aligned8 && t0 + kKeys <= kv_hi) {
        const int32_t pg = __builtin_amdgcn_readfirstlane(s_pages[(r0 >> pshift) - pg_lo]);
        src = base + (int64_t(pg) * page_bytes + int64_t(r0 & (psz - 1)) * tok_bytes) + lane8;
      } else {
        const int32_t j = min(r0 + (lane >> 3), kv_hi - 1);
        const int32_t pi = kPow2 ? (j >> pshift) : (j / psz);
        const int32_t sl = kPow2 ? (j & (psz - 1)) : (j - pi * psz);
        const int32_t pg = s_pages[min(pi - pg_lo, kMaxChunkPages - 1)];
        src = base + (int64_t(pg) * page_bytes + int64_t(sl) * tok_bytes) + (lane & 7) * 16;
      }
      dma16_bytes(src, dst + 1024 * wave);
    }
  };
  // Expands an fp8 slot (K half, V half) into a bf16 work tile with the bf16
  // swizzles: thread c expands chunk c (row c/8, dims 16(c%8) + [0, 16)) of
  // each half into bf16 chunks 2(c%8) and 2(c%8) + 1 of that row.
  auto expand_tile = [&](const uint8_t* src, uint16_t* dst) {
    if constexpr (kFp8) {
      const int row = tid >> 3, c2 = 2 * (tid & 7);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint4 raw = *reinterpret_cast<const uint4*>(src + half * kTile + 16 * tid);
        uint4 lo, hi;
        expand_fp8(raw, lo, hi);
        const int swz = half == 0 ? (row & 15) : 4 * (row & 3);
        uint16_t* drow = dst + half * kTile + row * kD;
        *reinterpret_cast<uint4*>(drow + (c2 ^ swz) * 8) = lo;
        *reinterpret_cast<uint4*>(drow + ((c2 + 1) ^ swz) * 8) = hi;
      }
    }
  };
  // fp8 tile step t: fp8 slot (t+1) % 4 (K(t+2), V(t+1)) landed for every wave
  // and is expanded into work tile (t+1) % 2 for the next step; this step's
  // products read work tile t % 2 (K(t+1), V(t)), expanded during step t-1.
  // Slot (t+3) % 4, expanded during step t-2, takes V(t+3) and K(t+4).
  auto body8 = [&](int32_t t, uint8_t* fdma, const uint8_t* fexp, uint16_t* wexp, const uint16_t* wread,
                   const uint4* mread, uint4* mdma, f32x16_t (&sc)[2]) {
    const int32_t t0 = kv_lo + t * kKeys;
    if (kMask && wave < kMaskInstr) dma_barrier_fp8_mask_wave();
    else dma_barrier_fp8();
    load8(vbase, fdma + kTile, t0 + 3 * kKeys);
    load8(kbase, fdma, t0 + 4 * kKeys);
    load_m(mdma, t0 + 4 * kKeys);
    expand_tile(fexp, wexp);
    if (!wave_active) return;
    const float shift = m_used != -INFINITY ? m_used : 0.f;
    float ls0 = 0.f, ls1 = 0.f;
    uint4 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pb[ks] = weights(sc, ks, shift, ls0, ls1);
    lsum += ls0 + ls1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pv_step(wread + kTile, ks, pb[ks]);
    if (t + 1 < ntiles) {
      scores(wread, sc);
      mask_tile(sc, t0 + kKeys, mread);
      update_max(tile_max(sc));
    }
  };

  // The prologue loads K(0) (slot 3), then V(s) and K(s+1) into slot s for
  // s = 0, 1, 2, and waits for all but the last two steps.
  f32x16_t sc[2];
  // Mask slot i goes with K slot s_b<i> (K(j) and its mask bits sit in slot (j + 3) % 4).
  constexpr int kMaskSlot = kMask ? kTileRows * 2 : 0;
  uint4* const m0 = s_mask;
  uint4* const m1 = s_mask + kMaskSlot;
  uint4* const m2 = s_mask + 2 * kMaskSlot;
  uint4* const m3 = s_mask + 3 * kMaskSlot;
  if constexpr (kFp8) {
   if (ntiles > 0) {
    // fp8 prologue: K(0) -> slot 3, then V(s), K(s+1) -> slot s for s = 0, 1,
    // 2 (one load per thread each, plus the mask rows of each K on the mask
    // waves); K(0), V(0) and K(1) (and their masks) land while the loads of
    // slots 1 and 2 stay in flight, are expanded into work tiles 1 (K(0)) and
    // 0, and the scores of tile 0 come from work tile 1.
    load8(kbase, s_f3, kv_lo);
    load_m(m3, kv_lo);
    load8(vbase, s_f0 + kTile, kv_lo);
    load8(kbase, s_f0, kv_lo + kKeys);
    load_m(m0, kv_lo + kKeys);
    load8(vbase, s_f1 + kTile, kv_lo + kKeys);
    load8(kbase, s_f1, kv_lo + 2 * kKeys);
    load_m(m1, kv_lo + 2 * kKeys);
    load8(vbase, s_f2 + kTile, kv_lo + 2 * kKeys);
    load8(kbase, s_f2, kv_lo + 3 * kKeys);
    load_m(m2, kv_lo + 3 * kKeys);
    if (kMask && wave < kMaskInstr) asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    expand_tile(s_f3, s_w1);   // its V half is never read
    expand_tile(s_f0, s_w0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wave_active) {
      scores(s_w1, sc);
      mask_tile(sc, kv_lo, m3);
      update_max(tile_max(sc));
    }
    for (int32_t t = 0; t < ntiles; t += 4) {
      body8(t, s_f3, s_f1, s_w1, s_w0, m0, m3, sc);
      if (t + 1 >= ntiles) break;
      body8(t + 1, s_f0, s_f2, s_w0, s_w1, m1, m0, sc);
      if (t + 2 >= ntiles) break;
      body8(t + 2, s_f1, s_f3, s_w1, s_w0, m2, m1, sc);
      if (t + 3 >= ntiles) break;
      body8(t + 3, s_f2, s_f0, s_w0, s_w1, m3, m2, sc);
    }
    dma_drain();
   }
  } else if (ntiles > 0) {
    load_k(s_b3, kv_lo);
    load_m(m3, kv_lo);
    load_v(s_b0 + kTile, kv_lo);
    load_k(s_b0, kv_lo + kKeys);
    load_m(m0, kv_lo + kKeys);
    load_v(s_b1 + kTile, kv_lo + kKeys);
    load_k(s_b1, kv_lo + 2 * kKeys);
    load_m(m1, kv_lo + 2 * kKeys);
    load_v(s_b2 + kTile, kv_lo + 2 * kKeys);
    load_k(s_b2, kv_lo + 3 * kKeys);
    load_m(m2, kv_lo + 3 * kKeys);
    barrier();
    if (wave_active) {
      scores(s_b3, sc);
      mask_tile(sc, kv_lo, m3);
      update_max(tile_max(sc));
    }
    for (int32_t t = 0; t < ntiles; t += 4) {
      body(t, s_b0, s_b0 + kTile, s_b3, s_b3 + kTile, m0, m3, sc);
      if (t + 1 >= ntiles) break;
      body(t + 1, s_b1, s_b1 + kTile, s_b0, s_b0 + kTile, m1, m0, sc);
      if (t + 2 >= ntiles) break;
      body(t + 2, s_b2, s_b2 + kTile, s_b1, s_b1 + kTile, m2, m1, sc);
      if (t + 3 >= ntiles) break;
      body(t + 3, s_b3, s_b3 + kTile, s_b2, s_b2 + kTile, m3, m2, sc);
    }
    // The last steps loaded tiles past the chunk end; they must land before
    // the workgroup can exit and its LDS be reused.
    dma_drain();
  }

  // Epilogue: row sum over both lane halves, normalise, write.
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!pair_ok) return;
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : (kFp8 ? a.v_scale : 1.f) / ltot;
  const float lse2 = empty ? -INFINITY : m_used + __log2f(ltot);
  const int32_t hq = a.num_qo_heads;
  if (it.out_slot < 0) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + int64_t(qrow_idx) * a.o_stride_token + int64_t(head) * a.o_stride_head;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 32 * n + 8 * q + 4 * h;
        uint2 w;
        w.x = pack2(oacc[n][4 * q + 0] * inv, oacc[n][4 * q + 1] * inv);
        w.y = pack2(oacc[n][4 * q + 2] * inv, oacc[n][4 * q + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    if (h == 0 && a.lse) a.lse[int64_t(qrow_idx) * hq + head] = lse2;
  } else {
    const int64_t prow_idx = int64_t(it.out_slot + prow) * hq + head;
    float* po = a.part_o + prow_idx * kD;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 32 * n + 8 * q + 4 * h;
        *reinterpret_cast<float4*>(po + d) =
            make_float4(oacc[n][4 * q] * inv, oacc[n][4 * q + 1] * inv, oacc[n][4 * q + 2] * inv,
                        oacc[n][4 * q + 3] * inv);
      }
    if (h == 0) a.part_lse[prow_idx] = lse2;
  }
}

template <int G, bool kMask, bool kFp8>
hipError_t launch_gm(const AttnArgs& a, hipStream_t st) {
  const int64_t blocks = int64_t(a.num_items) * a.num_kv_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid{static_cast<uint32_t>(blocks)}, block{kThreads};
  if (a.page_shift >= 0)
    launch_attention_kernel(prefill_mfma_kernel<G, true, kMask, kFp8>, grid, block, st, a);
  else
    launch_attention_kernel(prefill_mfma_kernel<G, false, kMask, kFp8>, grid, block, st, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const AttnArgs& a, bool fp8, hipStream_t st) {
  if constexpr (G >= 2) {
    if (a.mask) return fp8 ? launch_gm<G, true, true>(a, st) : launch_gm<G, true, false>(a, st);
  }
  return fp8 ? launch_gm<G, false, true>(a, st) : launch_gm<G, false, false>(a, st);
}

}  // namespace

hipError_t launch_prefill_mfma(int32_t kv_dtype, int32_t head_dim, int32_t group, const AttnArgs& a,
                               hipStream_t st, bool* supported) {
  // The tile loader forms 16 rows of token stride as a 32-bit byte offset.
  const bool strides_ok = a.token_stride >= 0 && a.token_stride * 2 * 16 < (int64_t(1) << 31);
  const bool fp8 = kv_dtype == kFP8;
  // A custom mask runs here for head groups of 2 or more (the mask tiles of
  // 256 rows would not fit the LDS left over).
  const bool mask_ok = !a.mask || group >= 2;
  if (head_dim == kD && strides_ok && mask_ok && (fp8 || kv_dtype == kBF16)) {
    *supported = true;
    switch (group) {
      case 1: return launch_g<1>(a, fp8, st);
      case 2: return launch_g<2>(a, fp8, st);
      case 4: return launch_g<4>(a, fp8, st);
      case 8: return launch_g<8>(a, fp8, st);
      default: break;
    }
  }
  // Other shapes run the row kernel (same results, VALU arithmetic).
  return launch_attn_rows(kv_dtype, head_dim, group, a, st, supported);
}

}  // namespace pkv
