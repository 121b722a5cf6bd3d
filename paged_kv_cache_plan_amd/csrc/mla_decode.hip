// MLA paged decode ("FlashInfer 中的 KV-Cache 布局", section on the MLA page
// layout): the cache has no head dimension; each token stores one 576-wide
// latent row, ckv (512) followed by kpe (64).  Every query head h scores a
// token as sm_scale * (q_ckv[h] . ckv + q_kpe[h] . kpe) and the output is the
// softmax-weighted sum of the ckv rows.
//
// With one query row per request and every head sharing every latent row,
// both products are dense contractions, here on v_mfma_f32_32x32x16_bf16
// (32 keys x 32 heads per instruction: half the instructions and operand
// reads per flop of the 16x16 shape):
//
//   * One workgroup (4 waves, one per SIMD) owns a work item (a key chunk of
//     one request) for a group of 128 heads: wave w owns heads [32w, 32w+32)
//     outright, scores every key of a tile (all 576 dims) and accumulates
//     every output dim (512 dims x 32 heads fill the 256 acc registers), so
//     the waves never exchange maxima or weights and every latent row comes
//     on chip once per item.  Groups of 64 heads run the same kernel with two
//     waves per 32 heads, each accumulating half of the output dims (both
//     compute the scores).
//   * Tiles of 32 latent rows (36 KiB) stream through a ring of four LDS
//     slots filled by direct global->LDS loads (global_load_lds_dwordx4,
//     issued from inline assembly so the compiler neither reorders nor waits
//     on them): tile t+3 is issued while tile t is computed, and the one
//     barrier per tile waits only for tile t+1.  A slot holds the 32 ckv rows
//     (1 KiB each) followed by the 32 kpe rows (128 bytes each), so one load
//     instruction fills a ckv row, or the kpe parts of 8 rows.  On pages of
//     8+ keys (a power of two) the 8 rows a wave loads share a page: one
//     scalar base per tile and fixed per-lane offsets.
//   * The 16-byte chunks of ckv row r are XOR-swizzled by a 4-bit g(r)
//     (within each group of 16 chunks), the kpe chunks by g(r) % 8: the K
//     operand reads (16 rows, one chunk, per 256-byte pass) and the
//     transposed V reads (4 rows x 64 bytes per pass) then hit distinct LDS
//     banks (the kpe reads meet 2-way conflicts, 4 reads of 100 per tile).
//   * Scores S^T = K Q^T (M = 32 keys, N = 32 heads, 36 k-steps of 16 dims)
//     with the wave's Q^T in registers; each lane then holds 16 scores of one
//     head, so the row max is in-lane plus one swap of the wave halves
//     (v_permlane32_swap).  O^T = V^T P^T (M = 32 dims, N = 32 heads, K = 16
//     keys): P^T comes straight from the score registers (the key order inside
//     a k-step is a permutation shared by both operands); V^T is read with
//     ds_read_b64_tr_b16.
//   * Software pipeline inside the wave: step t runs the score MFMAs of tile
//     t+1 interleaved with the exponentials of tile t, then the value MFMAs of
//     tile t interleaved with the max of tile t+1.  With one wave per SIMD
//     nothing else would hide the latency of either.
//   * Online softmax in the log2 domain with a fixed shift: the max of the
//     chunk's first tile.  Later weights may exceed 1 (bf16 and fp32 keep
//     their relative precision at any magnitude), so the accumulators are
//     never rescaled.  A tile whose max exceeds the shift by more than 32
//     (weights up to 2^32) makes the workgroup start the chunk over with the
//     largest max seen as the shift, which then bounds every weight by 1 on
//     the tiles seen; each such restart raises the shift by more than 32.
//
// The epilogue writes bf16 rows and base-2 LSE; the rows of a split chunk
// become partial states (bf16 rows, as the output, with a float LSE) that a
// merge kernel combines ("Deep Dive - FlashInfer", "A worked split-KV
// example").  bf16 partial rows halve the bytes that the split costs: with
// 128 heads a chunk's partial state is a third of its latent rows in bf16.

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kDimCkv = 512;
constexpr int kDimKpe = 64;
constexpr int kKeys = 32;                          // latent rows per tile
constexpr int kCkvRow = 2 * kDimCkv;               // bytes of a ckv row in LDS
constexpr int kKpeRow = 2 * kDimKpe;               // bytes of a kpe row in LDS
constexpr int kKpeOff = kKeys * kCkvRow;           // the kpe rows follow the ckv rows
constexpr int kSlot = kKpeOff + kKeys * kKpeRow;   // 36 KiB per tile
constexpr int kRing = 4;
constexpr int kSteps = (kDimCkv + kDimKpe) / 16;   // 36 score k-steps
constexpr int kCkvSteps = kDimCkv / 16;            // 32 of them over ckv
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = kKeys / kWaves;       // 8 rows: 9 load instructions per wave and tile
constexpr int kLoadsPerTile = kRowsPerWave + 1;
constexpr int kXcds = 8;                           // MI355X: 8 XCDs of 32 CUs
constexpr int kMaxChunkPages = 1024;
constexpr int kAheadK = 2;                         // K operand reads issued this many k-steps ahead
constexpr int kAheadV = 2;                         // V operand reads issued this many steps ahead
constexpr float kMaxGap = 32.f;                 // weights stay below 2^kMaxGap
static_assert(4 * kRowsPerWave + 1 < kSteps, "a tile's loads are spread one per four score k-steps");

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }
// MFMAs from inline assembly, so that O stays in the acc registers it fills
// and S in arch registers (left to itself the compiler moves them between
// the files, and spills).  The compiler then knows neither their latency nor
// their hazards: a value an MFMA wrote is read by other instructions only
// after mfma_drain (more than the 18 wait states a 32x32 MFMA result needs).
// Reading its result as the accumulator of the next MFMA of the same shape
// needs none, and the operands are loads or values written long before.
__device__ __forceinline__ void mfma_acc(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_arch(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_arch0(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_drain(f32x16_t& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}
// Chunk swizzle of LDS row r (16 values; rows r and r + 16 share it, and
// g(r + 8) = g(r) ^ 2): with a = r % 4, b = (r / 4) % 4,
// g(r) = (4a + b) ^ (2 (a / 2)).
__device__ __forceinline__ int swz(int r) {
  const int a = r & 3, b = (r >> 2) & 3;
  return (4 * a + b) ^ (2 * (a >> 1));
}

// Transposed LDS read: within each 16-lane group lane i supplies the address
// of 4 consecutive bf16 values C_i[0..3] and receives C_{4e + i/4}[i % 4].
__device__ __forceinline__ bf16x4_t tr_read(const uint8_t* lds) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(const_cast<uint8_t*>(lds)));
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// The two wave halves swap x (lane l meets lane l ^ 32); max or sum of the pair.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct global->LDS loads: lane l of the wave writes 16 bytes to M0 + 16 l.
// M0 must hold a wave-uniform LDS address, and a write of M0 needs one wait
// state before a load that reads it (the s_nop).  Inline assembly: the kernel
// waits for these loads itself (vmcnt before each tile barrier and the exit).
// Every latent row is read once per launch, so the loads are non-temporal
// (nt): the MLA batch ran about 4 % faster than with cached loads.
//
// The wave's 8 ckv rows of a tile from one scalar base (row j at
// base + voff[j], stored 1 KiB apart from lds_ckv on), then the kpe parts of
// the 8 rows in one instruction (base_kpe + voff_kpe, to lds_kpe).
__device__ __forceinline__ void dma_rows(const void* base, const uint32_t (&voff)[kRowsPerWave],
                                         const void* base_kpe, uint32_t voff_kpe, uint32_t lds_ckv,
                                         uint32_t lds_kpe) {
  asm volatile(
      "s_mov_b32 m0, %10\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %8 nt\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %8 nt\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %8 nt\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %8 nt\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %8 nt\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %8 nt\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %8 nt\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %7, %8 nt\n\t"
      "s_mov_b32 m0, %11\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %9, %12 nt" ::"v"(voff[0]),
      "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]), "v"(voff[6]), "v"(voff[7]), "s"(base),
      "v"(voff_kpe), "s"(lds_ckv), "s"(lds_kpe), "s"(base_kpe)
      : "m0", "scc");
}
// One ckv row from a scalar base (rows on different pages).
__device__ __forceinline__ void dma_row(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds)
               : "m0");
}
// 16 bytes from a per-lane address.
__device__ __forceinline__ void dma_lane(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds) : "m0");
}
// At most N of this wave's tile loads still in flight and its LDS reads
// returned, then the workgroup barrier.  The memory clobber keeps LDS
// accesses on their side.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// kDimSplit: waves per 32 heads (1: groups of 128 heads; 2: groups of 64
// heads, each wave accumulating half of the output dims).
template <int kDimSplit, bool kPow2>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(const MlaArgs a) {
  constexpr int kHeadsPerGroup = 32 * kWaves / kDimSplit;
  constexpr int kDimBlocks = kDimCkv / 32 / kDimSplit;   // 32-dim output blocks per wave
  constexpr int kPvSteps = (kKeys / 16) * kDimBlocks;     // value MFMAs per tile
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kRing * kSlot];
  __shared__ int32_t s_pages[kMaxChunkPages];
  __shared__ int32_t s_restart;   // set by a wave that saw a tile max above its shift + kMaxGap

  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each with
  // its own L2: the k-th workgroup of XCD x takes item (k / head_groups) * 8 +
  // x, head group k % head_groups, so the head groups of an item share an L2.
  const int32_t xcd = int32_t(blockIdx.x & (kXcds - 1)), k_on_xcd = int32_t(blockIdx.x / kXcds);
  const int32_t item_idx = (k_on_xcd / a.head_groups) * kXcds + xcd;
  const int32_t hgrp = k_on_xcd - (k_on_xcd / a.head_groups) * a.head_groups;
  if (item_idx >= a.num_items) return;
  if (a.live_items && item_idx >= *a.live_items) return;   // fixed-capacity grid: whole workgroup
  const Item it = a.items[item_idx];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;   // score / output column: this lane's head
  const int hk = lane >> 5;  // 8-element k slice of an MFMA operand
  const int dsl = wave % kDimSplit;
  const int32_t b = it.q_row0;
  const int32_t head = hgrp * kHeadsPerGroup + (wave / kDimSplit) * 32 + n;
  const char* const ckv = static_cast<const char*>(a.ckv);
  const char* const kpe = static_cast<const char*>(a.kpe);
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t psz = a.page_size, pshift = a.page_shift;
  const uint32_t max_pages = uint32_t(a.max_num_pages);
  const int64_t page_bytes = a.page_stride * 2, tok_bytes = a.token_stride * 2;

  const int32_t kv_lo = it.kv_start, kv_hi = it.kv_end;
  const int32_t ntiles = kv_hi > kv_lo ? (kv_hi - kv_lo + kKeys - 1) / kKeys : 0;
  const int32_t pg_lo = kv_hi > kv_lo ? (kPow2 ? kv_lo >> pshift : kv_lo / psz) : 0;
  const int32_t pg_n =
      kv_hi > kv_lo ? min(kMaxChunkPages, (kPow2 ? (kv_hi - 1) >> pshift : (kv_hi - 1) / psz) - pg_lo + 1) : 0;

  // Tile loads: wave w fills rows [8w, 8w + 8) of a slot.  Row r's stored
  // chunk p holds source chunk p ^ s(r) (s(r) < 8: within its group of 8).
  // Lane l of a ckv row load writes stored chunk l; lane l of the kpe load
  // writes stored chunk l & 7 of row 8w + l / 8.  Keys past the chunk end
  // re-read the last key (their scores are masked to -inf).
  const uint32_t tokb = uint32_t(tok_bytes);   // the host keeps 8 rows of offsets below 2^31
  const uint32_t lane16 = uint32_t(lane * 16);
  const uint32_t kchunk = uint32_t(((lane & 7) ^ (swz(8 * wave + (lane >> 3)) & 7)) * 16);
  const uint32_t kvoff = uint32_t(lane >> 3) * tokb + kchunk;
  const uint32_t ring_lds = uint32_t(reinterpret_cast<uintptr_t>(s_ring));
  const int32_t r_w = kRowsPerWave * wave;
  auto page_of_key = [&](int32_t j) {   // page id of key j of the chunk (from the staged list)
    const int32_t pi = kPow2 ? (j >> pshift) : (j / psz);
    return s_pages[min(pi - pg_lo, kMaxChunkPages - 1)];
  };
  auto slot_of_key = [&](int32_t j) { return kPow2 ? (j & (psz - 1)) : (j - (j / psz) * psz); };
  // The page of the wave's first row of tile t (read ahead of load_tile, so
  // that the LDS latency of the lookup is hidden).
  auto first_page = [&](int32_t t) { return page_of_key(min(kv_lo + t * kKeys + r_w, kv_hi - 1)); };
  // The wave's 8 rows of tile t lie on one page (pages of 8+ keys; chunks
  // start on page boundaries and the 8 rows on an 8-key boundary within
  // them): one scalar base (tile_base) and fixed per-lane offsets (cvoff).
  auto one_page = [&](int32_t t) { return kPow2 && pshift >= 3 && kv_lo + t * kKeys + r_w + kRowsPerWave <= kv_hi; };
  auto tile_base = [&](int32_t t, int32_t page0) {
    return int64_t(__builtin_amdgcn_readfirstlane(page0)) * page_bytes +
           int64_t((kv_lo + t * kKeys + r_w) & (psz - 1)) * tok_bytes;
  };
  uint32_t cvoff[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) cvoff[j] = (lane16 ^ uint32_t(16 * swz(r_w + j))) + uint32_t(j) * tokb;
  auto lds_ckv_of = [&](int32_t t) { return ring_lds + uint32_t((t & (kRing - 1)) * kSlot + r_w * kCkvRow); };
  auto lds_kpe_of = [&](int32_t t) { return ring_lds + uint32_t((t & (kRing - 1)) * kSlot + kKpeOff + r_w * kKpeRow); };
  auto load_tile = [&](int32_t t, int32_t page0) {
    const uint32_t lds_ckv = lds_ckv_of(t), lds_kpe = lds_kpe_of(t);
    const int32_t j0 = kv_lo + t * kKeys + r_w;
    if (one_page(t)) {
      const int64_t off = tile_base(t, page0);
      dma_rows(ckv + off, cvoff, kpe + off, kvoff, lds_ckv, lds_kpe);
    } else {
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j) {
        const int32_t jk = min(j0 + j, kv_hi - 1);
        const int64_t off = int64_t(__builtin_amdgcn_readfirstlane(page_of_key(jk))) * page_bytes +
                            int64_t(slot_of_key(jk)) * tok_bytes;
        dma_row(ckv + off, lane16 ^ uint32_t(16 * swz(r_w + j)), lds_ckv + uint32_t(j * kCkvRow));
      }
      const int32_t jk = min(j0 + (lane >> 3), kv_hi - 1);
      dma_lane(kpe + int64_t(page_of_key(jk)) * page_bytes + int64_t(slot_of_key(jk)) * tok_bytes + kchunk,
               lds_kpe);
    }
  };

  // The chunk's page ids are staged in LDS; their loads go out first, then
  // those of Q, whose latency then overlaps the staging and the first tile
  // loads (loads complete in order, so the first tile barrier also covers Q).
  int32_t pg_first = 0;
  if (tid < pg_n) pg_first = pages[pg_lo + tid];
  asm volatile("" ::: "memory");

  // Q^T as the B operand: k-step s covers dims [16s, 16s+16); this lane holds
  // dims 16s + 8hk + [0, 8) of its head (ckv dims first, then kpe).
  bf16x8_t qreg[kSteps];
  {
    const int64_t qrow = int64_t(b) * a.num_heads + head;
    const uint16_t* qc = static_cast<const uint16_t*>(a.q_ckv) + qrow * kDimCkv;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_kpe) + qrow * kDimKpe;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int d = 16 * s + 8 * hk;
      qreg[s] = d < kDimCkv ? *reinterpret_cast<const bf16x8_t*>(qc + d)
                            : *reinterpret_cast<const bf16x8_t*>(qp + d - kDimCkv);
    }
  }
  asm volatile("" ::: "memory");

  if (tid < pg_n) s_pages[tid] = uint32_t(pg_first) < max_pages ? pg_first : 0;   // ids outside the pool read page 0
  for (int i = tid + kThreads; i < pg_n; i += kThreads) {
    const int32_t pg = pages[pg_lo + i];
    s_pages[i] = uint32_t(pg) < max_pages ? pg : 0;
  }
  if (tid == 0) s_restart = 0;
  __syncthreads();


  // K operand reads: lane (n, hk) reads row n, source chunk 2s + hk, stored
  // at (2s + hk) ^ g(n) = 16 (s / 8) + ((2 (s % 8) + hk) ^ g(n)).  Relative
  // to a slot (slots are 4 KiB aligned) the offset of k-step s is that of
  // s % 4 with bit 7 flipped when s % 8 >= 4, plus 256 (s / 8): four per-lane
  // bases.  The kpe k-step u reads row n of the kpe rows at chunk
  // (2u + hk) ^ (g(n) % 8): the ckv offset of k-step u plus a per-lane delta.
  int kbase[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kbase[u] = n * kCkvRow + 16 * ((2 * u + hk) ^ swz(n));
  const int kpdelta = kKpeOff + n * (kKpeRow - kCkvRow) - 128 * (swz(n) >> 3);
  // V^T reads (A operand of O^T = V^T P^T: 32 dims x 16 keys).  Value
  // k-step ks takes the keys 8 ks + [0, 8) and 8 ks + 16 + [0, 8) of the tile,
  // as the weights below are packed.  In 16-lane group G = 2 hh + dh, lane j
  // supplies row 8 ks + 4 hh + j / 4 (+ 16 for the upper 4 keys of its k
  // slice; rows 16 apart share the swizzle) at dims 32 db + 16 dh + 4 (j % 4),
  // and receives dim 32 db + 16 dh + j of 4 keys.  The stored chunk is
  // 16 (db / 4) + ((4 (db % 4) + 2 dh + (j % 4) / 2) ^ g(row)): four bases by
  // db % 4 for ks = 0; for ks = 1 (g ^ 2) the slot offset has bit 5 flipped,
  // plus 8 rows.  The wave's first block db0 is a multiple of 4.
  const int db0 = dsl * kDimBlocks;
  int vbase[4];
  {
    const int G = lane >> 4, j = lane & 15, hh = G >> 1, dh = G & 1;
    const int row = 4 * hh + (j >> 2);
    const int sr = swz(row);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      vbase[q] = row * kCkvRow + 16 * ((4 * q + 2 * dh + ((j & 3) >> 1)) ^ sr) + 8 * (j & 1) + 64 * db0;
  }

  f32x16_t oacc[kDimBlocks];
  float m_used = -INFINITY;   // the shift of this lane's head
  float m_seen = -INFINITY;   // the largest tile max seen (per head)
  float lsum = 0.f;
  const float c = a.scale_log2;

  // S^T of the tile in ring slot `slot_off` into acc (36 k-steps, K operands
  // read two steps ahead into a ring of three); piece(s) runs inside k-step
  // s.  A scheduling fence after each step keeps the compiler from hoisting
  // further reads (which would need more registers than the wave has).
  auto scores = [&](uint32_t slot_off, f32x16_t& acc, auto&& piece) {
    bf16x8_t kop[kAheadK + 1];
    auto kread = [&](int s) {
      const int off = s < kCkvSteps ? ((int(slot_off) + kbase[s & 3]) ^ (128 * ((s >> 2) & 1))) + 256 * (s >> 3)
                                    : int(slot_off) + kbase[s - kCkvSteps] + kpdelta;
      return *reinterpret_cast<const bf16x8_t*>(s_ring + off);
    };
#pragma unroll
    for (int s = 0; s < kAheadK; ++s) kop[s] = kread(s);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (s + kAheadK < kSteps) kop[(s + kAheadK) % (kAheadK + 1)] = kread(s + kAheadK);
      if (s == 0) mfma_arch0(acc, kop[0], qreg[0]);
      else mfma_arch(acc, kop[s % (kAheadK + 1)], qreg[s]);
      piece(s);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_drain(acc);
  };
  // O^T += V^T P^T over the tile in `slot_off` for this wave's dim blocks:
  // step v is k-step v / kDimBlocks, block db0 + v % kDimBlocks; its V^T
  // operand is read two steps ahead.  piece(v) runs inside step v.
  auto values = [&](uint32_t slot_off, const uint4 (&pb)[2], auto&& piece) {
    bf16x8_t vop[kAheadV + 1];
    auto vread = [&](int v) {
      const int ks = v / kDimBlocks, d = v % kDimBlocks;
      const int off = ((int(slot_off) + vbase[d & 3]) ^ (32 * ks)) + 8 * ks * kCkvRow + 256 * (d >> 2);
      const bf16x4_t lo = tr_read(s_ring + off);
      const bf16x4_t hi = tr_read(s_ring + off + 16 * kCkvRow);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int v = 0; v < kAheadV; ++v) vop[v] = vread(v);
#pragma unroll
    for (int v = 0; v < kPvSteps; ++v) {
      if (v + kAheadV < kPvSteps) vop[(v + kAheadV) % (kAheadV + 1)] = vread(v + kAheadV);
      const int ks = v / kDimBlocks, d = v % kDimBlocks;
      mfma_acc(oacc[d], vop[v % (kAheadV + 1)], as_bf16x8(pb[ks]));
      piece(v);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Score slot i of a tile (lane (n, hk)) is key 8 (i / 4) + 4 hk + i % 4.
  auto mask_tile = [&](f32x16_t& sc, int32_t t0) {
    if (t0 + kKeys > kv_hi) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = t0 + 8 * (i >> 2) + 4 * hk + (i & 3) < kv_hi ? sc[i] : -INFINITY;
    }
  };
  auto slot_of = [&](int32_t t) { return uint32_t((t & (kRing - 1)) * kSlot); };

  // One pass over the chunk with shift m_used.  The first pass takes the max
  // of tile 0 as the shift and notes whether a later tile's max exceeds it by
  // more than kMaxGap (its weights could then overflow); the rare second pass
  // runs with the largest max of the chunk, so every weight is at most 1.
  f32x16_t sc_cur, sc_nxt;
  bool over = false;
  auto pass = [&](auto first_pass) {
    constexpr bool kFirst = decltype(first_pass)::value;
    // Prologue: tiles 0-2 in flight, S(0) and its max.
    load_tile(0, first_page(0));
    if (ntiles > 1) load_tile(1, first_page(1));
    if (ntiles > 2) load_tile(2, first_page(2));
    if (ntiles > 2) tile_barrier<2 * kLoadsPerTile>();
    else if (ntiles > 1) tile_barrier<kLoadsPerTile>();
    else tile_barrier<0>();
    scores(slot_of(0), sc_cur, [](int) {});
    mask_tile(sc_cur, kv_lo);
    if (kFirst) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc_cur[i]);
      m_used = max_halves(mx) * c;   // finite: tile 0 holds a visible key
      m_seen = m_used;
    }
#pragma unroll
    for (int d = 0; d < kDimBlocks; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
    lsum = 0.f;

    // Step t: entering, S(t) is in sc_cur.  After the barrier every wave has
    // tile t+1 and is done with the slot of tile t-1, which takes tile t+3.
    // Then S(t+1) is computed while the weights of tile t are formed, and
    // O += V(t) P(t) while the max of S(t+1) is formed.
    int32_t page_next = first_page(3);   // page of tile t+3 (looked up one step ahead)
    for (int32_t t = 0; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      if (t + 2 < ntiles) tile_barrier<kLoadsPerTile>();
      else tile_barrier<0>();
      // Tile t+3's loads.  When the wave's rows lie on one page they are
      // spread over the score k-steps below, one load per four MFMAs: issued
      // back to back, each load waits for the CU's memory pipeline to take
      // the one before (a tile is 36 KiB per CU), and the wave stalls.
      const bool load_next = t + 3 < ntiles;
      const bool spread = load_next && more && one_page(t + 3);
      if (load_next && !spread) load_tile(t + 3, page_next);
      const int64_t off_next = spread ? tile_base(t + 3, page_next) : 0;
      const uint32_t ckv_next = lds_ckv_of(t + 3), kpe_next = lds_kpe_of(t + 3);
      page_next = first_page(t + 4);
      // Weights of tile t, one per k-step 0-15 (exp2(-inf) = 0 covers masked
      // keys), summed and packed in pairs two k-steps later (so that no
      // instruction waits on an exponential between the MFMAs) into the B
      // operands of the two value k-steps.
      uint4 pb[2];
      float e[16];
      auto weights = [&](int s) {
        if (s < 16) {
          e[s] = dev::fast_exp2(fmaf(sc_cur[s], c, -m_used));
          asm volatile("" : "+v"(e[s]));   // here, between the MFMAs (not sunk to its use)
        }
        const int u = s - 2;
        if (u >= 0 && u < 16) {
          lsum += e[u];
          if (u & 1) {
            // pair q = u / 2 holds keys 8 (q / 2) + 4 hk + 2 (q % 2) + {0, 1}:
            // value k-step (q / 2) % 2, lower or upper half by q / 4
            const uint32_t v = pack2(e[u - 1], e[u]);
            const int q = u >> 1, ks = (q >> 1) & 1, w = 2 * (q >> 2) + (q & 1);
            if (w == 0) pb[ks].x = v;
            if (w == 1) pb[ks].y = v;
            if (w == 2) pb[ks].z = v;
            if (w == 3) pb[ks].w = v;
          }
        }
      };
      auto weights_loads = [&](int s) {
        weights(s);
        if (spread && (s & 3) == 1) {
          const int j = s >> 2;
          if (j < kRowsPerWave) dma_row(ckv + off_next, cvoff[j], ckv_next + uint32_t(j * kCkvRow));
          else dma_row(kpe + off_next, kvoff, kpe_next);
        }
      };
      if (more) {
        scores(slot_of(t + 1), sc_nxt, weights_loads);
        mask_tile(sc_nxt, kv_lo + (t + 1) * kKeys);
      } else {
#pragma unroll
        for (int s = 0; s < 18; ++s) weights(s);
      }
      float mx = -INFINITY;
      auto tmax = [&](int v) {   // steps 4-11: two scores of S(t+1) each (unused on the last tile)
        if (kFirst && v >= 4 && v < 12) {
          mx = fmaxf(mx, fmaxf(sc_nxt[2 * (v - 4)], sc_nxt[2 * (v - 4) + 1]));
          asm volatile("" : "+v"(mx));
        }
      };
      values(slot_of(t), pb, tmax);
      if (more) {
        if (kFirst) {
          const float m_next = max_halves(mx) * c;
          m_seen = fmaxf(m_seen, m_next);
          over = over || __any(m_next > m_used + kMaxGap);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sc_cur[i] = sc_nxt[i];
      }
    }
  };
  if (ntiles == 0) {   // an empty chunk writes an empty state
#pragma unroll
    for (int d = 0; d < kDimBlocks; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  } else {
    pass(std::true_type{});
    // Every wave's loads have landed (the last steps wait for all of them).
    if (over && lane == 0) s_restart = 1;
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_restart)) {
      m_used = m_seen;
      pass(std::false_type{});
    }
  }
  // The last value MFMAs have finished before any accumulator is read.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int d = 0; d < kDimBlocks; ++d) asm volatile("" : "+a"(oacc[d]));

  // Epilogue: row sum over the two lanes of this head, normalise, write this
  // wave's dims.  oacc[d][i] is dim 32 (db0 + d) + 8 (i / 4) + 4 hk + i % 4 of
  // this lane's head.
  const float ltot = sum_halves(lsum);
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse2 = empty ? -INFINITY : m_used + __log2f(ltot);
  // Whole rows go to o, rows of a split chunk to its partial row (bf16, like
  // o, with a float LSE).  The rows pass through LDS (the ring is free now),
  // so that each store instruction writes one whole 1 KiB row: a lane holds
  // 8-byte pieces of 32 rows, which stored directly would scatter every
  // instruction over 32 rows.  Staged rows are 1040 bytes apart.
  constexpr int kStageRow = 2 * kDimCkv + 16;
  __syncthreads();   // every wave is done reading the ring
  {
    const int row = (wave / kDimSplit) * 32 + n;
#pragma unroll
    for (int d = 0; d < kDimBlocks; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 w;
        w.x = pack2(oacc[d][4 * q] * inv, oacc[d][4 * q + 1] * inv);
        w.y = pack2(oacc[d][4 * q + 2] * inv, oacc[d][4 * q + 3] * inv);
        *reinterpret_cast<uint2*>(s_ring + row * kStageRow + 2 * (32 * (db0 + d) + 8 * q + 4 * hk)) = w;
      }
  }
  __syncthreads();
  const bool direct = it.out_slot < 0;
  const int64_t row0 = (direct ? int64_t(b) : int64_t(it.out_slot)) * a.num_heads + int64_t(hgrp) * kHeadsPerGroup;
  uint16_t* obase = static_cast<uint16_t*>(direct ? a.o : static_cast<void*>(a.part_o)) + row0 * kDimCkv;
  constexpr int kRowsOut = kHeadsPerGroup / kWaves;
#pragma unroll 8
  for (int r = 0; r < kRowsOut; ++r) {
    const int row = wave * kRowsOut + r;
    const uint4 v = *reinterpret_cast<const uint4*>(s_ring + row * kStageRow + 16 * lane);
    *reinterpret_cast<uint4*>(obase + int64_t(row) * kDimCkv + 8 * lane) = v;
  }
  float* lse_dst = direct ? a.lse : a.part_lse;
  if (hk == 0 && dsl == 0 && lse_dst) lse_dst[row0 + (wave / kDimSplit) * 32 + n] = lse2;
}

// Split merge of MLA rows ("Deep Dive - FlashInfer", "A worked split-KV
// example"): partial row p holds a chunk's normalised output (bf16, 512 dims)
// and its base-2 LSE s_p; the row's output is sum_p w_p o_p with
// w_p = 2^(s_p - m) / sum_q 2^(s_q - m), m the largest s_p, and its LSE is
// m + log2 sum_q 2^(s_q - m).  One wave per (merge item, head): lane l owns
// dims 8l .. 8l + 7; the statistics are wave-uniform loads.  A row whose
// chunks are all empty (every s_p = -inf) gets zeros and -inf.
constexpr int kMergeWaves = 4;
__global__ __launch_bounds__(64 * kMergeWaves) void mla_merge_kernel(const MergePartialArgs a) {
  if (a.live_merges && int32_t(blockIdx.x) >= *a.live_merges) return;   // fixed-capacity grid
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int32_t h = int32_t(blockIdx.y) * kMergeWaves + wave;
  if (h >= a.num_heads) return;
  const int lane = threadIdx.x & 63;
  const MergeItem mi = a.merges[blockIdx.x];
  const int32_t hq = a.num_heads, n = mi.num_chunks;
  const uint16_t* part = reinterpret_cast<const uint16_t*>(a.part_o);
  for (int32_t r = 0; r < mi.num_rows; ++r) {
    const int64_t row0 = int64_t(mi.slot0) + r;
    auto stat = [&](int32_t c) { return a.part_lse[(row0 + int64_t(c) * mi.num_rows) * hq + h]; };
    auto row_of = [&](int32_t c) {
      return reinterpret_cast<const uint4*>(part + ((row0 + int64_t(c) * mi.num_rows) * hq + h) * kDimCkv + 8 * lane);
    };
    // The first eight chunks' rows and (lane c) chunk c's statistic are
    // loaded together, so their latencies overlap.
    uint4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = *row_of(min(j, n - 1));
    const float sc_lane = lane < n ? stat(lane) : -INFINITY;
    float mx = sc_lane;
    for (int32_t c = lane + 64; c < n; c += 64) mx = fmaxf(mx, stat(c));
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float wl_lane = sc_lane == -INFINITY ? 0.f : dev::fast_exp2(sc_lane - mx);   // mx finite whenever sc is
    float z = wl_lane;
    for (int32_t c = lane + 64; c < n; c += 64) {
      const float sc = stat(c);
      z += sc == -INFINITY ? 0.f : dev::fast_exp2(sc - mx);
    }
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    const float inv_z = z > 0.f ? 1.f / z : 0.f;
    const float w_lane = wl_lane * inv_z;
    auto weight = [&](int32_t c) {   // normalised weight of chunk c (0 past the last)
      if (c >= n) return 0.f;
      if (c < 64) return __shfl(w_lane, c);
      const float sc = stat(c);
      return sc == -INFINITY ? 0.f : dev::fast_exp2(sc - mx) * inv_z;
    };
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto fold = [&](const uint4 (&xs)[8], int32_t c0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float w = weight(c0 + j);
        const uint32_t u[4] = {xs[j].x, xs[j].y, xs[j].z, xs[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(w, dev::bf16_lo(u[e]), acc[2 * e]);
          acc[2 * e + 1] = fmaf(w, dev::bf16_hi(u[e]), acc[2 * e + 1]);
        }
      }
    };
    fold(x, 0);
    // Further chunks eight at a time (eight 16-byte loads per lane in
    // flight); steps past the last chunk re-read it with weight 0.
    for (int32_t c0 = 8; c0 < n; c0 += 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = *row_of(min(c0 + j, n - 1));
      fold(x, c0);
    }
    const int32_t row = mi.q_row0 + r;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + int64_t(row) * a.o_stride_token + int64_t(h) * a.o_stride_head;
    uint4 out;
    out.x = pack2(acc[0], acc[1]);
    out.y = pack2(acc[2], acc[3]);
    out.z = pack2(acc[4], acc[5]);
    out.w = pack2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(orow + 8 * lane) = out;
    if (lane == 0 && a.lse) a.lse[int64_t(row) * hq + h] = z > 0.f ? mx + __log2f(z) : -INFINITY;
  }
}

template <int kDimSplit>
void launch_split(const MlaArgs& a, dim3 grid, hipStream_t st) {
  if (a.page_shift >= 0)
    launch_attention_kernel(mla_decode_kernel<kDimSplit, true>, grid, dim3(kThreads), st, a);
  else
    launch_attention_kernel(mla_decode_kernel<kDimSplit, false>, grid, dim3(kThreads), st, a);
}

}  // namespace

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st) {
  if (a.head_groups <= 0 || a.num_heads % a.head_groups != 0) return hipErrorInvalidValue;
  const int32_t width = a.num_heads / a.head_groups;
  if (width != 128 && width != 64) return hipErrorInvalidValue;
  // One wave's 8 rows of per-lane offsets are 32-bit.
  if (a.token_stride < 0 || a.token_stride >= kMlaMaxTokenStride) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t(a.num_items) + kXcds - 1) / kXcds * kXcds * a.head_groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (width == 128) launch_split<1>(a, dim3(uint32_t(blocks)), st);
  else launch_split<2>(a, dim3(uint32_t(blocks)), st);
  return hipGetLastError();
}

hipError_t launch_mla_merge(const MergePartialArgs& a, hipStream_t st) {
  if (a.num_merges <= 0) return hipSuccess;
  if (a.head_dim != kDimCkv || a.num_heads <= 0) return hipErrorInvalidValue;
  const int32_t head_blocks = (a.num_heads + kMergeWaves - 1) / kMergeWaves;
  if (head_blocks > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(uint32_t(a.num_merges), uint32_t(head_blocks)), dim3(64 * kMergeWaves), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace pkv
