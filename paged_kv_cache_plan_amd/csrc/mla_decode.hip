// MLA paged decode ("FlashInfer 中的 KV-Cache 布局", section on the MLA page
// layout): the cache has no head dimension; each token stores one 576-wide
// latent row, ckv (512) followed by kpe (64).  Every query head h scores a
// token as sm_scale * (q_ckv[h] . ckv + q_kpe[h] . kpe) and the output is the
// softmax-weighted sum of the ckv rows.
//
// With one query row per request and every head sharing every latent row,
// both products are dense contractions on v_mfma_f32_16x16x32_bf16:
//
//   * One workgroup (8 waves) owns a work item (a key chunk of one request) for
//     64 heads; the head halves of an item run on one XCD, so the second
//     reads the latent rows from L2.  Waves 2i and 2i+1 share heads
//     [16i, 16i + 16): wave 2i + h scores keys [32h, 32h + 32) of each tile
//     (all 576 dims) and accumulates output dims [256h, 256h + 256) over all 64
//     keys.  The pair exchanges its tile max and its bf16 weights through LDS,
//     so no MFMA is duplicated and each wave holds Q (72 registers) plus half
//     the output (64 registers), which leaves room to keep LDS reads in
//     flight.
//   * Tiles of 64 latent rows (72 KiB) are double buffered in LDS and filled by
//     direct global->LDS loads (global_load_lds_dwordx4, issued from inline
//     assembly; the tile barrier waits for them explicitly).
//   * Rows are stored unpadded (72 chunks of 16 bytes) with the chunks of row r
//     XOR-swizzled by r & 7 inside each group of 8: with it the K operand reads
//     (16 rows, one chunk) and the transposed V reads (4 rows x 32 bytes per
//     16-lane group) run without LDS bank conflicts (measured with the bank
//     conflict counter; the unswizzled and other tried layouts conflict 2- to
//     4-way).
//   * Scores S^T = K Q^T (M = 16 keys, N = 16 heads, K = 576 dims: 18 MFMA
//     k-steps per 16-key block) with the wave's Q^T held in registers; every
//     lane then holds 8 scores of one head and the row max / sum are in-lane
//     plus two exchanges (and the partner's max).  O^T = V^T P^T (M = 16
//     dims, N = 16 heads, K = 32 keys): 16 accumulator blocks per wave.  P^T
//     comes straight from the score registers (the key order inside a k-step
//     is a permutation shared by both operands) or from the partner through
//     LDS; V^T is read with ds_read_b64_tr_b16.
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
constexpr int kChunks = kDim / 8;         // 16-byte chunks per latent row
constexpr int kKeys = 64;                 // latent rows per LDS tile
constexpr int kTile = kKeys * kDim;       // elements per tile (72 KiB)
constexpr int kSteps = kDim / 32;         // score k-steps per 16-key block
constexpr int kDimBlocks = kDimCkv / 32;  // output blocks of 16 dims per wave (half the dims)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerGroup = 64;        // heads per workgroup
constexpr int kXcds = 8;                  // MI355X: 8 XCDs of 32 CUs
constexpr int kMaxChunkPages = 1024;
constexpr float kLazyMax = 8.f;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Transposed LDS read: within each 16-lane group lane i supplies the address
// of 4 consecutive bf16 values C_i[0..3] and receives C_{4e + i/4}[i % 4].
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
// lds_wave_base + 16 l (M0 holds the LDS address, so it must be wave-uniform).
// Inline assembly, so the compiler neither reorders it nor inserts waits for
// it: the kernel waits for these loads itself (vmcnt(0) before each tile
// barrier and before exit).
__device__ __forceinline__ void dma16(const void* src, const uint16_t* lds_wave_base) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "m0");
}
// All of this wave's tile loads have landed and its LDS reads returned; then
// the workgroup barrier.  The memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void dma_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <bool kPow2>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(const MlaArgs a) {
  constexpr int kLoadsPerWave = kKeys * kChunks / 64 / kWaves;   // 1 KiB load instructions per wave per tile
  static_assert(kKeys * kChunks % (64 * kWaves) == 0, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint16_t s_t0[kTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_t1[kTile];
  __shared__ int32_t s_pages[kMaxChunkPages];
  __shared__ uint4 s_p[kWaves][64];        // each wave's bf16 weights of its 32 keys
  __shared__ float s_max[kWaves][16];      // each wave's tile max per head
  __shared__ float s_sum[kWaves][16];      // each wave's row sum per head (epilogue)

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
  const int kh = wave & 1;   // key half scored / dim half accumulated
  const int n = lane & 15;   // score column (head) / output column; also the tr-read source index
  const int g = lane >> 4;   // 8-element k slice of an MFMA operand
  const int32_t b = it.q_row0;
  const int32_t head = hgrp * kHeadsPerGroup + (wave >> 1) * 16 + n;
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

  // Tile loads.  Load instruction q (wave w issues q = w * kLoadsPerWave + j)
  // fills 16-byte slots 64q .. 64q + 63 of the tile; lane i's slot 64q + i is
  // row (64q + i) / 72, stored chunk (64q + i) % 72, which holds source chunk
  // stored ^ (row & 7).  Keys past the chunk end re-read the last key (their
  // scores are masked to -inf).
  const bool aligned = kPow2 && pshift >= 6;   // a tile starting on a page boundary lies on one page
  auto load_tile = [&](uint16_t* dst, int32_t t0) {
    // The per-lane address terms are recomputed at every tile (a few integer
    // operations) instead of being kept live across the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const bool one_page = aligned && t0 + kKeys <= kv_hi && (t0 & (psz - 1)) + kKeys <= psz;
    int64_t page_off = 0;
    if (one_page)
      page_off = int64_t(__builtin_amdgcn_readfirstlane(s_pages[(t0 >> pshift) - pg_lo])) * page_bytes +
                 int64_t(t0 & (psz - 1)) * tok_bytes;
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int q = wave * kLoadsPerWave + j;
      const int slot = 64 * q + ln;
      const int row = slot / kChunks, cst = slot - (slot / kChunks) * kChunks;
      const int csrc = cst ^ (row & 7);
      const char* base = csrc < kDimCkv / 8 ? ckv + csrc * 16 : kpe + (csrc - kDimCkv / 8) * 16;
      int64_t off;
      if (one_page) {
        off = page_off + int64_t(row) * tok_bytes;
      } else {
        const int32_t jk = min(t0 + row, kv_hi - 1);
        const int32_t pi = kPow2 ? (jk >> pshift) : (jk / psz);
        const int32_t sl = kPow2 ? (jk & (psz - 1)) : (jk - pi * psz);
        off = int64_t(s_pages[min(pi - pg_lo, kMaxChunkPages - 1)]) * page_bytes + int64_t(sl) * tok_bytes;
      }
      dma16(base + off, dst + 64 * 8 * q);
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

  // S^T of this wave's key half of the tile in buf: sc[j][i] is the score of
  // key 32kh + 16j + 4g + i for this lane's head.
  const int k_half = 32 * kh * kDim;
  auto scores = [&](const uint16_t* buf, f32x4_t (&sc)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) sc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 kv =
            *reinterpret_cast<const uint4*>(buf + k_half + ((s & 1) ? k_odd : k_even) + 16 * j * kDim + 32 * s);
        sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qreg[s]), sc[j], 0, 0, 0);
      }
    }
  };

  // One tile: own scores, mask, pair max, lazy rescale, own weights, exchange,
  // O^T += V^T P^T over all 64 keys for this wave's dims.
  auto tile = [&](const uint16_t* buf, int32_t t0) {
    f32x4_t sc[2];
    scores(buf, sc);
    const int32_t k0 = t0 + 32 * kh;
    if (k0 + 32 > kv_hi) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[j][i] = k0 + 16 * j + 4 * g + i < kv_hi ? sc[j][i] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[j][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (g == 0) s_max[wave][n] = mx;
    __syncthreads();   // the pair's maxima are visible
    mx = fmaxf(mx, s_max[wave ^ 1][n]);
    // Both waves of the pair see the same maxima, so they take the same
    // rescale decisions and keep the same shift.
    const float m_cand = mx * c;
    const bool grow = m_cand > m_used + kLazyMax || (m_used == -INFINITY && m_cand != -INFINITY);
    if (__any(grow)) {
      const float m_new = grow ? m_cand : m_used;
      const float f = grow ? (m_used == -INFINITY ? 0.f : dev::fast_exp2(m_used - m_new)) : 1.f;
      m_used = m_new;
      lsum *= f;
#pragma unroll
      for (int d = 0; d < kDimBlocks; ++d) oacc[d] *= f;
    }
    // exp2(-inf) = 0 covers masked keys; a head with no visible key yet has
    // only -inf scores, so any finite shift works for it.
    const float shift = m_used != -INFINITY ? m_used : 0.f;
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = dev::fast_exp2(fmaf(sc[0][e], c, -shift));
      p[4 + e] = dev::fast_exp2(fmaf(sc[1][e], c, -shift));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) lsum += p[e];
    // B operand of k-step kh (keys 32kh + [0, 32)); the partner's is k-step 1 - kh.
    const uint4 p_own = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    s_p[wave][lane] = p_own;
    __syncthreads();   // the pair's weights are visible
    const uint4 p_other = s_p[wave ^ 1][lane];
    uint4 pb[2];
    pb[0] = kh == 0 ? p_own : p_other;
    pb[1] = kh == 0 ? p_other : p_own;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dd = 0; dd < kDimBlocks; ++dd) {
        const uint16_t* base = buf + v_base[dd & 3] + 32 * ks * kDim + 64 * (4 * kh + (dd >> 2));
        const bf16x4_t lo = tr_read(base);
        const bf16x4_t hi = tr_read(base + 16 * kDim);
        const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[dd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, as_bf16x8(pb[ks]), oacc[dd], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) {
    load_tile(s_t0, kv_lo);
    for (int32_t t = 0; t < ntiles; t += 2) {
      // Tile t has landed in s_t0 for every wave, and every wave is done with
      // s_t1 (tile t-1).
      tile_barrier();
      if (t + 1 < ntiles) load_tile(s_t1, kv_lo + (t + 1) * kKeys);
      tile(s_t0, kv_lo + t * kKeys);
      if (t + 1 >= ntiles) break;
      tile_barrier();
      if (t + 2 < ntiles) load_tile(s_t0, kv_lo + (t + 2) * kKeys);
      tile(s_t1, kv_lo + (t + 1) * kKeys);
    }
    dma_drain();
  }

  // Epilogue: row sum over the four lanes of this head and the partner wave,
  // normalise, write this wave's 256 dims.  oacc[dd][i] is dim
  // 256kh + 16dd + 4g + i of this lane's head.
  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (g == 0) s_sum[wave][n] = ltot;
  __syncthreads();
  ltot += s_sum[wave ^ 1][n];
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse2 = empty ? -INFINITY : m_used + __log2f(ltot);
  const int dim0 = 256 * kh + 4 * g;
  if (it.out_slot < 0) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + (int64_t(b) * a.num_heads + head) * kDimCkv;
#pragma unroll
    for (int dd = 0; dd < kDimBlocks; ++dd) {
      uint2 w;
      w.x = pack2(oacc[dd][0] * inv, oacc[dd][1] * inv);
      w.y = pack2(oacc[dd][2] * inv, oacc[dd][3] * inv);
      *reinterpret_cast<uint2*>(orow + dim0 + 16 * dd) = w;
    }
    if (kh == 0 && g == 0 && a.lse) a.lse[int64_t(b) * a.num_heads + head] = lse2;
  } else {
    const int64_t prow = int64_t(it.out_slot) * a.num_heads + head;
    float* po = a.part_o + prow * kDimCkv;
#pragma unroll
    for (int dd = 0; dd < kDimBlocks; ++dd)
      *reinterpret_cast<float4*>(po + dim0 + 16 * dd) =
          make_float4(oacc[dd][0] * inv, oacc[dd][1] * inv, oacc[dd][2] * inv, oacc[dd][3] * inv);
    if (kh == 0 && g == 0) a.part_lse[prow] = lse2;
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
