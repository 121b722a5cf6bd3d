// MLA paged decode ("FlashInfer 中的 KV-Cache 布局", section on the MLA page
// layout): the cache has no head dimension; each token stores one 576-wide
// latent row, ckv (512) followed by kpe (64).  Every query head h scores a
// token as sm_scale * (q_ckv[h] . ckv + q_kpe[h] . kpe) and the output is the
// softmax-weighted sum of the ckv rows.
//
// With one query row per request and every head sharing every latent row,
// both products are dense contractions on v_mfma_f32_16x16x32_bf16:
//
//   * One workgroup (4 waves, one per SIMD) owns a work item (a key chunk of
//     one request) for 64 heads; the head groups of an item run on one XCD,
//     so all but the first read the latent rows from L2.  Wave w owns heads
//     [16w, 16w + 16) of the group outright: it scores every key of a tile
//     (all 576 dims) and accumulates every output dim (all 512), so the waves
//     never exchange maxima or weights.  The only synchronisation is one
//     barrier per tile for the shared LDS tiles.  A wave holds Q^T (72
//     registers), the output accumulator (128) and a tile's scores (16), with
//     room left to keep LDS reads in flight ahead of the MFMAs.
//   * Tiles of 64 latent rows (72 KiB) are double buffered in LDS and filled by
//     direct global->LDS loads (global_load_lds_dwordx4, issued from inline
//     assembly): the loads of tile t+1 run while tile t is computed.  A row
//     takes two load instructions, its ckv part (64 lanes, 1 KiB) and its kpe
//     part (8 lanes, 128 bytes).  Each instruction reads from one row, so its
//     source address is the same for the whole wave: it sits in scalar
//     registers and each lane adds a fixed offset, with no per-lane address
//     arithmetic per load.
//   * Rows are stored unpadded (72 chunks of 16 bytes) with the chunks of row r
//     XOR-swizzled by r & 7 inside each group of 8: with it the K operand reads
//     (16 rows, one chunk) and the transposed V reads (4 rows x 32 bytes per
//     16-lane group) run without LDS bank conflicts.
//   * Scores S^T = K Q^T (M = 16 keys, N = 16 heads, K = 576 dims: 18 MFMA
//     k-steps per 16-key block) with the wave's Q^T held in registers; every
//     lane then holds 16 scores of one head, so the row max and sum are
//     in-lane plus two lane exchanges.  O^T = V^T P^T (M = 16 dims, N = 16
//     heads, K = 32 keys): 32 accumulator blocks per wave.  P^T comes straight
//     from the score registers (the key order inside a k-step is a
//     permutation shared by both operands); V^T is read with
//     ds_read_b64_tr_b16.
//   * Online softmax in the log2 domain with a lazy max (rescale only when the
//     running max grows by more than 8).
//
// The epilogue writes bf16 rows and base-2 LSE, or fp32 partial states for the
// split merge ("Deep Dive - FlashInfer", "A worked split-KV example").

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kDimCkv = 512;
constexpr int kDimKpe = 64;
constexpr int kDim = kDimCkv + kDimKpe;   // 576
constexpr int kKeys = 64;                 // latent rows per LDS tile
constexpr int kTile = kKeys * kDim;       // elements per tile (72 KiB)
constexpr int kSteps = kDim / 32;         // score k-steps per 16-key block
constexpr int kKeyBlocks = kKeys / 16;    // 16-key score blocks per tile
constexpr int kDimBlocks = kDimCkv / 16;  // 16-dim output blocks per wave (all 512 dims)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerGroup = kWaves * kHeadsPerWave;   // 64 heads per workgroup
constexpr int kXcds = 8;                  // MI355X: 8 XCDs of 32 CUs
constexpr int kMaxChunkPages = 1024;
constexpr float kLazyMax = 8.f;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Transposed LDS read: within each 16-lane group lane i supplies the address
// of 4 consecutive bf16 values C_i[0..3] and receives C_{4e + i/4}[i % 4].
__device__ __forceinline__ bf16x4_t tr_read(const uint16_t* lds_elem) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(const_cast<uint16_t*>(lds_elem)));
}

// x *= f for a value held in an acc register, without a copy of x in the
// arch registers outside this sequence.  The accumulators live in acc
// registers for the whole kernel; written as plain C++, the rare rescale
// makes the compiler keep arch-register copies of all 128 of them live across
// the tile, which leaves too few registers to keep LDS reads in flight.
__device__ __forceinline__ float scale_acc(float x, float f) {
  float t;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(t)
               : "v"(f));
  return x;
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// lds_wave_base + 16 l (M0 holds the LDS address, so it must be wave-uniform).
// Inline assembly, so the compiler neither reorders it nor inserts waits for
// it: the kernel waits for these loads itself (vmcnt(0) before each tile
// barrier and before exit).
__device__ __forceinline__ void dma16(const void* src, const uint16_t* lds_wave_base) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "m0");
}
// The same with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the saddr form of the instruction), for rows whose
// address is the same for the whole wave.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, const uint16_t* lds_wave_base) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "m0");
}
// All of this wave's tile loads have landed and its LDS reads returned; then
// the workgroup barrier.  The memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void dma_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <bool kPow2>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(const MlaArgs a) {
  constexpr int kRowsPerWave = kKeys / kWaves;   // rows (two loads each) per wave and tile
  __shared__ __attribute__((aligned(16))) uint16_t s_t0[kTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_t1[kTile];
  __shared__ int32_t s_pages[kMaxChunkPages];

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
  const int n = lane & 15;   // score column (head) / output column; also the tr-read source index
  const int g = lane >> 4;   // 8-element k slice of an MFMA operand
  const int32_t b = it.q_row0;
  const int32_t head = hgrp * kHeadsPerGroup + wave * kHeadsPerWave + n;
  const char* const ckv = static_cast<const char*>(a.ckv);
  const char* const kpe = static_cast<const char*>(a.kpe);
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t psz = a.page_size, pshift = a.page_shift;
  const uint32_t max_pages = uint32_t(a.max_num_pages);
  const int64_t page_bytes = a.page_stride * 2, tok_bytes = a.token_stride * 2;

  // Q^T as the B operand: k-step s covers dims [32s, 32s+32); this lane holds
  // dims 32s + 8g + [0, 8) of its head (ckv dims first, then kpe).
  uint4 qreg[kSteps];
  {
    const int64_t qrow = int64_t(b) * a.num_heads + head;
    const uint16_t* qc = static_cast<const uint16_t*>(a.q_ckv) + qrow * kDimCkv;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_kpe) + qrow * kDimKpe;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int d = 32 * s + 8 * g;
      qreg[s] = d < kDimCkv ? *reinterpret_cast<const uint4*>(qc + d)
                            : *reinterpret_cast<const uint4*>(qp + d - kDimCkv);
    }
    // Wait for Q here, before any tile load is in flight (otherwise the
    // compiler's wait before the first MFMA would also drain the tile loads).
#pragma unroll
    for (int s = 0; s < kSteps; ++s) asm volatile("" ::"v"(qreg[s].x), "v"(qreg[s].y), "v"(qreg[s].z), "v"(qreg[s].w));
  }

  const int32_t kv_lo = it.kv_start, kv_hi = it.kv_end;
  const int32_t ntiles = kv_hi > kv_lo ? (kv_hi - kv_lo + kKeys - 1) / kKeys : 0;
  const int32_t pg_lo = kv_hi > kv_lo ? (kPow2 ? kv_lo >> pshift : kv_lo / psz) : 0;
  const int32_t pg_n =
      kv_hi > kv_lo ? min(kMaxChunkPages, (kPow2 ? (kv_hi - 1) >> pshift : (kv_hi - 1) / psz) - pg_lo + 1) : 0;
  for (int i = tid; i < pg_n; i += kThreads) {
    const int32_t pg = pages[pg_lo + i];
    s_pages[i] = uint32_t(pg) < max_pages ? pg : 0;   // ids outside the pool read page 0
  }
  __syncthreads();

  // Tile loads: wave w fills rows [16w, 16w + 16) of the tile.  Row r's
  // stored chunk c holds source chunk c ^ (r & 7) (within its group of 8):
  // lane l of the ckv load writes stored chunk l, lane l < 8 of the kpe load
  // stored chunk 64 + l, and both read source chunk l ^ (r & 7) of their
  // part.  Keys past the chunk end re-read the last key (their scores are
  // masked to -inf).
  uint32_t xoff[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) xoff[k] = uint32_t((lane ^ k) * 16);
  const int32_t r_w = kRowsPerWave * wave;
  auto page_of_key = [&](int32_t j) {   // page id of key j of the chunk (from the staged list)
    const int32_t pi = kPow2 ? (j >> pshift) : (j / psz);
    return s_pages[min(pi - pg_lo, kMaxChunkPages - 1)];
  };
  auto slot_of_key = [&](int32_t j) { return kPow2 ? (j & (psz - 1)) : (j - (j / psz) * psz); };
  auto load_row = [&](uint16_t* dst, int r, int64_t row_off) {
    dma16_s(ckv + row_off, xoff[r & 7], dst + r * kDim);
    if (lane < 8) dma16_s(kpe + row_off, xoff[r & 7], dst + r * kDim + kDimCkv);
  };
  auto load_tile = [&](uint16_t* dst, int32_t t0) {
    if (kPow2 && pshift >= 4 && t0 + kKeys <= kv_hi) {
      // The wave's 16 rows lie on one page (pages of 16+ keys, tiles start
      // on 16-key boundaries).
      const int32_t j0 = t0 + r_w;
      const int64_t base = int64_t(__builtin_amdgcn_readfirstlane(page_of_key(j0))) * page_bytes +
                           int64_t(j0 & (psz - 1)) * tok_bytes;
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j) load_row(dst, r_w + j, base + int64_t(j) * tok_bytes);
    } else {
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j) {
        const int32_t jk = min(t0 + r_w + j, kv_hi - 1);
        load_row(dst, r_w + j,
                 int64_t(__builtin_amdgcn_readfirstlane(page_of_key(jk))) * page_bytes +
                     int64_t(slot_of_key(jk)) * tok_bytes);
      }
    }
  };

  // K operand reads: block kb, k-step s, lane (n, g) reads row 16kb + n,
  // source chunk 4s + g, stored at (4s + g) ^ (n & 7) = 4(s ^ bx) + cx: even
  // and odd s use one base each.
  const int kx = n & 7;
  const int bx = kx >> 2, cx = (g ^ kx) & 3;
  const int k_even = n * kDim + 8 * cx + 32 * bx;
  const int k_odd = n * kDim + 8 * cx - 32 * bx;
  // V^T reads: lane (n, g) supplies row 4g + n/4 (+16 for keys 4..7 of its k
  // slice, +32 per k-step) at dims 16db + 4(n%4); the stored chunk is
  // 2(db ^ z) + v1, i.e. four per-lane bases by db % 4 plus 64 db/4.
  int v_base[4];
  {
    const int xv = 4 * (g & 1) + (n >> 2);
    const int z = xv >> 1, v1 = (((n & 3) >> 1) ^ xv) & 1;
    const int rowoff = (4 * g + (n >> 2)) * kDim;
#pragma unroll
    for (int r = 0; r < 4; ++r) v_base[r] = rowoff + 16 * (r ^ z) + 8 * v1 + 4 * (n & 1);
  }

  f32x4_t oacc[kDimBlocks];
#pragma unroll
  for (int d = 0; d < kDimBlocks; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, lsum = 0.f;
  const float c = a.scale_log2;

  // A tile is two halves.  scores(): S^T of its 64 keys for this wave's 16
  // heads, masked past the chunk end, and the tile max (sc[kb][i] is the
  // score of key 16kb + 4g + i for this lane's head).  finish(): the weights
  // under the current shift and O^T += V^T P^T over the 64 keys for all 512
  // dims.  Both products read their LDS operands two steps ahead of the
  // MFMAs that use them, into a ring of three register sets; a scheduling
  // fence after each step keeps the compiler from hoisting further reads
  // (which would need more registers than the wave has).
  f32x4_t sc[kKeyBlocks];
  auto scores = [&](const uint16_t* buf, int32_t t0) {
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb) sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 kop[3][kKeyBlocks];
    auto kread = [&](int st, uint4 (&dst)[kKeyBlocks]) {
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
        dst[kb] = *reinterpret_cast<const uint4*>(buf + ((st & 1) ? k_odd : k_even) + 16 * kb * kDim + 32 * st);
    };
    kread(0, kop[0]);
    kread(1, kop[1]);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (st + 2 < kSteps) kread(st + 2, kop[(st + 2) % 3]);
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kop[st % 3][kb]), as_bf16x8(qreg[st]), sc[kb], 0,
                                                         0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t0 + kKeys > kv_hi) {
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = t0 + 16 * kb + 4 * g + i < kv_hi ? sc[kb][i] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    return fmaxf(mx, __shfl_xor(mx, 32)) * c;   // the four lanes of a head agree
  };
  auto finish = [&](const uint16_t* buf) {
    // exp2(-inf) = 0 covers masked keys; a head with no visible key yet has
    // only -inf scores, so any finite shift works for it.
    const float shift = m_used != -INFINITY ? m_used : 0.f;
    uint4 pb[kKeys / 32];   // B operand of k-step ks: keys 32ks + {4g + i, 16 + 4g + i}
#pragma unroll
    for (int ks = 0; ks < kKeys / 32; ++ks) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = dev::fast_exp2(fmaf(sc[2 * ks][e], c, -shift));
        p[4 + e] = dev::fast_exp2(fmaf(sc[2 * ks + 1][e], c, -shift));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) lsum += p[e];
      pb[ks] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    }
    // Values: step v covers k-step v / 8 and output blocks 4(v % 8) .. +3.
    constexpr int kPvGroup = 4;
    constexpr int kPvSteps = (kKeys / 32) * kDimBlocks / kPvGroup;
    bf16x8_t vop[3][kPvGroup];
    auto vread = [&](int v, bf16x8_t (&dst)[kPvGroup]) {
      const int ks = v / (kDimBlocks / kPvGroup), dd0 = (v % (kDimBlocks / kPvGroup)) * kPvGroup;
#pragma unroll
      for (int i = 0; i < kPvGroup; ++i) {
        const int dd = dd0 + i;
        const uint16_t* base = buf + v_base[dd & 3] + 32 * ks * kDim + 64 * (dd >> 2);
        const bf16x4_t lo = tr_read(base);
        const bf16x4_t hi = tr_read(base + 16 * kDim);
        dst[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    vread(0, vop[0]);
    vread(1, vop[1]);
#pragma unroll
    for (int v = 0; v < kPvSteps; ++v) {
      if (v + 2 < kPvSteps) vread(v + 2, vop[(v + 2) % 3]);
      const int ks = v / (kDimBlocks / kPvGroup), dd0 = (v % (kDimBlocks / kPvGroup)) * kPvGroup;
#pragma unroll
      for (int i = 0; i < kPvGroup; ++i)
        oacc[dd0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[v % 3][i], as_bf16x8(pb[ks]), oacc[dd0 + i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Lazy running max: a tile moves the shift only when its max exceeds the
  // current one by more than kLazyMax (weights stay below 2^kLazyMax); then
  // the accumulator and the sum are rescaled.
  auto needs_rescale = [&](float m_cand) {
    return m_cand > m_used + kLazyMax || (m_used == -INFINITY && m_cand != -INFINITY);
  };

  // Tile loop.  Tile t is in buffer t % 2; after the barrier of tile t every
  // wave is done with the other buffer (tile t-1), which then takes tile t+1.
  // The rescale, rare after the first tile, leaves the inner loop, so the
  // accumulators keep one register assignment through it (a rescale inside
  // the loop makes the compiler copy them at every iteration).
  if (ntiles > 0) load_tile(s_t0, kv_lo);
  int32_t t = 0;
  while (t < ntiles) {
    float m_cand = -INFINITY;
    for (; t < ntiles; ++t) {
      tile_barrier();
      if (t + 1 < ntiles) load_tile((t & 1) ? s_t0 : s_t1, kv_lo + (t + 1) * kKeys);
      m_cand = scores((t & 1) ? s_t1 : s_t0, kv_lo + t * kKeys);
      if (__any(needs_rescale(m_cand))) break;
      finish((t & 1) ? s_t1 : s_t0);
    }
    if (t >= ntiles) break;
    const bool grow = needs_rescale(m_cand);
    const float m_new = grow ? m_cand : m_used;
    const float f = grow ? (m_used == -INFINITY ? 0.f : dev::fast_exp2(m_used - m_new)) : 1.f;
    m_used = m_new;
    lsum *= f;
#pragma unroll
    for (int d = 0; d < kDimBlocks; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[d][i] = scale_acc(oacc[d][i], f);
    finish((t & 1) ? s_t1 : s_t0);
    ++t;
  }
  if (ntiles > 0) dma_drain();

  // Epilogue: row sum over the four lanes of this head, normalise, write all
  // 512 dims.  oacc[dd][i] is dim 16dd + 4g + i of this lane's head.
  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse2 = empty ? -INFINITY : m_used + __log2f(ltot);
  const int dim0 = 4 * g;
  if (it.out_slot < 0) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + (int64_t(b) * a.num_heads + head) * kDimCkv;
#pragma unroll
    for (int dd = 0; dd < kDimBlocks; ++dd) {
      uint2 w;
      w.x = pack2(oacc[dd][0] * inv, oacc[dd][1] * inv);
      w.y = pack2(oacc[dd][2] * inv, oacc[dd][3] * inv);
      *reinterpret_cast<uint2*>(orow + dim0 + 16 * dd) = w;
    }
    if (g == 0 && a.lse) a.lse[int64_t(b) * a.num_heads + head] = lse2;
  } else {
    const int64_t prow = int64_t(it.out_slot) * a.num_heads + head;
    float* po = a.part_o + prow * kDimCkv;
#pragma unroll
    for (int dd = 0; dd < kDimBlocks; ++dd)
      *reinterpret_cast<float4*>(po + dim0 + 16 * dd) =
          make_float4(oacc[dd][0] * inv, oacc[dd][1] * inv, oacc[dd][2] * inv, oacc[dd][3] * inv);
    if (g == 0) a.part_lse[prow] = lse2;
  }
}

}  // namespace

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st) {
  if (a.num_heads != a.head_groups * kHeadsPerGroup) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t(a.num_items) + kXcds - 1) / kXcds * kXcds * a.head_groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.page_shift >= 0)
    launch_attention_kernel(mla_decode_kernel<true>, dim3(uint32_t(blocks)), dim3(kThreads), st, a);
  else
    launch_attention_kernel(mla_decode_kernel<false>, dim3(uint32_t(blocks)), dim3(kThreads), st, a);
  return hipGetLastError();
}

}  // namespace pkv
