// MLA paged decode ("FlashInfer 中的 KV-Cache 布局", section on the MLA page
// layout): the cache has no head dimension; each token stores one 576-wide
// latent row, ckv (512) followed by kpe (64).  Every query head h scores a
// token as sm_scale * (q_ckv[h] . ckv + q_kpe[h] . kpe) and the output is the
// softmax-weighted sum of the ckv rows.
//
// With one query row per request and 128 heads sharing every latent row, both
// products are dense contractions, so they run on v_mfma_f32_32x32x16_bf16.
// One workgroup (4 waves) owns a work item (a key chunk of one request) for a
// group of 32 heads; tiles of 32 latent rows are gathered through the page
// table into LDS (the next tile's loads are in flight while a tile is used).
//
//   Scores S^T = K Q^T (M = 32 keys, N = 32 heads) over 576 dims = 36 MFMA
//   k-steps, split across the 4 waves (9 k-steps each, the matching slice of
//   Q held in registers).  The four partial score tiles are summed through LDS,
//   after which every lane holds the 32 scores of one head over its half of the
//   keys: the softmax is in-lane plus one exchange with lane l^32.
//   Output O^T = V^T P^T with V = ckv: wave w owns output dims [128w, 128w+128)
//   for all 32 heads; V^T comes from the LDS tile with ds_read_b64_tr_b16 and
//   P^T straight from the score registers (the key order inside a k-step is a
//   permutation shared by both operands).
//
// The epilogue writes bf16 rows and base-2 LSE, or fp32 partial states for the
// split merge ("Deep Dive - FlashInfer", "A worked split-KV example").

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kHeadsPerGroup = 32;
constexpr int kKeys = 32;              // latent rows per LDS tile
constexpr int kDimCkv = 512;
constexpr int kDimKpe = 64;
constexpr int kDim = kDimCkv + kDimKpe;
constexpr int kPitch = kDim + 8;       // LDS row pitch (elements): 1168 bytes, 292 dwords
constexpr int kChunks = kDim / 8;      // 16-byte chunks per latent row
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStepsPerWave = kDim / 16 / kWaves;   // 9 score k-steps per wave
constexpr int kLoads = kKeys * kChunks / kThreads;  // 16-byte loads per thread per tile
constexpr int kMaxChunkPages = 1024;
constexpr float kLazyMax = 8.f;
constexpr int kXcds = 8;               // MI355X: 8 XCDs of 32 CUs
// Latent rows are shared by the head groups of a chunk through L2; the
// non-temporal hint is a compile-time choice.
#ifndef PKV_MLA_NT
#define PKV_MLA_NT 0
#endif
constexpr bool kStreamKV = PKV_MLA_NT != 0;
static_assert(kKeys * kChunks % kThreads == 0, "tile loads split evenly");

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

template <bool kPow2>
__global__ __launch_bounds__(kThreads, 2) void mla_decode_kernel(const MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_kv[kKeys * kPitch];
  __shared__ float s_part[kWaves][16][64];   // partial S^T per wave, [value][lane]
  __shared__ int32_t s_pages[kMaxChunkPages];

  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each with
  // its own L2.  The head groups of one item read the same latent rows, so
  // they are given consecutive slots on one XCD: the k-th workgroup of XCD x
  // takes item (k / head_groups) * 8 + x, head group k % head_groups.
  const int32_t xcd = int32_t(blockIdx.x & (kXcds - 1)), k_on_xcd = int32_t(blockIdx.x / kXcds);
  const int32_t item_idx = (k_on_xcd / a.head_groups) * kXcds + xcd;
  const int32_t grp = k_on_xcd - (k_on_xcd / a.head_groups) * a.head_groups;
  if (item_idx >= a.num_items) return;
  const Item it = a.items[item_idx];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int32_t b = it.q_row0;
  const int32_t head = grp * kHeadsPerGroup + col;
  const uint16_t* ckv = static_cast<const uint16_t*>(a.ckv);
  const uint16_t* kpe = static_cast<const uint16_t*>(a.kpe);
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t psz = a.page_size, pshift = a.page_shift;
  const uint32_t max_pages = uint32_t(a.max_num_pages);

  // Q^T slice of this wave (k-steps 9w .. 9w+8 of the 576 dims): lane holds
  // head `col`, dims 16s + 8h + [0, 8).
  uint4 qreg[kStepsPerWave];
  {
    const int64_t qrow = int64_t(b) * a.num_heads + head;
    const uint16_t* qc = static_cast<const uint16_t*>(a.q_ckv) + qrow * kDimCkv;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_kpe) + qrow * kDimKpe;
#pragma unroll
    for (int i = 0; i < kStepsPerWave; ++i) {
      const int d = 16 * (kStepsPerWave * wave + i) + 8 * h;
      qreg[i] = d < kDimCkv ? *reinterpret_cast<const uint4*>(qc + d)
                            : *reinterpret_cast<const uint4*>(qp + d - kDimCkv);
    }
  }

  const int32_t kv_lo = it.kv_start, kv_hi = it.kv_end;
  const int32_t ntiles = kv_hi > kv_lo ? (kv_hi - kv_lo + kKeys - 1) / kKeys : 0;
  const int32_t pg_lo = kv_hi > kv_lo ? (kPow2 ? kv_lo >> pshift : kv_lo / psz) : 0;
  const int32_t pg_n =
      kv_hi > kv_lo ? min(kMaxChunkPages, (kPow2 ? (kv_hi - 1) >> pshift : (kv_hi - 1) / psz) - pg_lo + 1) : 0;
  for (int i = tid; i < pg_n; i += kThreads) {
    const int32_t pg = pages[pg_lo + i];
    s_pages[i] = uint32_t(pg) < max_pages ? pg : 0;
  }
  __syncthreads();

  // Tile loader: load i of thread tid moves chunk c = tid + 256 i of the tile,
  // i.e. key c / 72, 16-byte chunk c % 72 (ckv for chunks < 64, kpe after).
  // Keys past the chunk end re-read the last key (their scores are masked).
  // The nine staging registers are named individually so they stay in VGPRs.
  auto src_of = [&](int32_t t0, int i) -> const void* {
    const int c = tid + kThreads * i;
    const int key = c / kChunks, part = c - (c / kChunks) * kChunks;
    const int32_t j = min(t0 + key, kv_hi - 1);
    const int32_t pi = kPow2 ? (j >> pshift) : (j / psz);
    const int32_t sl = kPow2 ? (j & (psz - 1)) : (j - pi * psz);
    const int64_t off =
        int64_t(s_pages[min(pi - pg_lo, kMaxChunkPages - 1)]) * a.page_stride + int64_t(sl) * a.token_stride;
    const uint16_t* base = part < kDimCkv / 8 ? ckv + part * 8 : kpe + (part - kDimCkv / 8) * 8;
    return base + off;
  };
  auto dst_of = [&](int i) -> uint4* {
    const int c = tid + kThreads * i;
    const int key = c / kChunks, part = c - (c / kChunks) * kChunks;
    return reinterpret_cast<uint4*>(&s_kv[key * kPitch + part * 8]);
  };
  static_assert(kLoads == 9, "nine staging registers");
  uint4 st0, st1, st2, st3, st4, st5, st6, st7, st8;
#define PKV_MLA_GLOAD(T0)      \
  do {                         \
    st0 = dev::load16<kStreamKV>(src_of((T0), 0));    \
    st1 = dev::load16<kStreamKV>(src_of((T0), 1));    \
    st2 = dev::load16<kStreamKV>(src_of((T0), 2));    \
    st3 = dev::load16<kStreamKV>(src_of((T0), 3));    \
    st4 = dev::load16<kStreamKV>(src_of((T0), 4));    \
    st5 = dev::load16<kStreamKV>(src_of((T0), 5));    \
    st6 = dev::load16<kStreamKV>(src_of((T0), 6));    \
    st7 = dev::load16<kStreamKV>(src_of((T0), 7));    \
    st8 = dev::load16<kStreamKV>(src_of((T0), 8));    \
  } while (0)
#define PKV_MLA_LSTORE()  \
  do {                    \
    *dst_of(0) = st0;     \
    *dst_of(1) = st1;     \
    *dst_of(2) = st2;     \
    *dst_of(3) = st3;     \
    *dst_of(4) = st4;     \
    *dst_of(5) = st5;     \
    *dst_of(6) = st6;     \
    *dst_of(7) = st7;     \
    *dst_of(8) = st8;     \
  } while (0)

  f32x16_t oacc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[n][v] = 0.f;
  float m_used = -INFINITY, lsum = 0.f;
  const float c = a.scale_log2;

  const uint16_t* const k_rd = &s_kv[col * kPitch + 16 * kStepsPerWave * wave + 8 * h];
  const int grp16 = lane >> 4, gi = lane & 15;
  const uint16_t* const v_rd =
      &s_kv[(4 * h + (gi >> 2)) * kPitch + 128 * wave + 16 * (grp16 & 1) + 4 * (gi & 3)];

  if (ntiles > 0) {
    PKV_MLA_GLOAD(kv_lo);
    PKV_MLA_LSTORE();
  }
  __syncthreads();

  for (int32_t t = 0; t < ntiles; ++t) {
    const int32_t t0 = kv_lo + t * kKeys;
    if (t + 1 < ntiles) PKV_MLA_GLOAD(t0 + kKeys);

    // Partial scores over this wave's 9 k-steps.
    f32x16_t sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int i = 0; i < kStepsPerWave; ++i) {
      const uint4 kv = *reinterpret_cast<const uint4*>(k_rd + 16 * i);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), as_bf16x8(qreg[i]), sacc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) s_part[wave][v][lane] = sacc[v];
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) x += s_part[w][v][lane];
      // key of value v: t0 + 8(v/4) + 4h + v%4
      const int32_t j = t0 + 8 * (v >> 2) + 4 * h + (v & 3);
      sacc[v] = j < kv_hi ? x : -INFINITY;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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
    const float shift = m_used != -INFINITY ? m_used : 0.f;
    uint4 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = dev::fast_exp2(fmaf(sacc[8 * ks + e], c, -shift));
        lsum += p[e];
      }
      pb[ks] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    }

    // O^T[128w + 32n + ., heads] += V^T P^T over the tile's 32 keys.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint16_t* base = v_rd + 16 * ks * kPitch + 32 * n;
        const bf16x4_t lo = tr_read(base);
        const bf16x4_t hi = tr_read(base + 8 * kPitch);
        const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16x8(pb[ks]), oacc[n], 0, 0, 0);
      }
    }

    __syncthreads();   // every wave is done with this tile and with s_part
    if (t + 1 < ntiles) PKV_MLA_LSTORE();
    __syncthreads();
  }

#undef PKV_MLA_GLOAD
#undef PKV_MLA_LSTORE

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse2 = empty ? -INFINITY : m_used + __log2f(ltot);
  if (it.out_slot < 0) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + (int64_t(b) * a.num_heads + head) * kDimCkv;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 128 * wave + 32 * n + 8 * q + 4 * h;
        uint2 w;
        w.x = pack2(oacc[n][4 * q + 0] * inv, oacc[n][4 * q + 1] * inv);
        w.y = pack2(oacc[n][4 * q + 2] * inv, oacc[n][4 * q + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    if (wave == 0 && h == 0 && a.lse) a.lse[int64_t(b) * a.num_heads + head] = lse2;
  } else {
    const int64_t prow = int64_t(it.out_slot) * a.num_heads + head;
    float* po = a.part_o + prow * kDimCkv;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 128 * wave + 32 * n + 8 * q + 4 * h;
        *reinterpret_cast<float4*>(po + d) = make_float4(oacc[n][4 * q] * inv, oacc[n][4 * q + 1] * inv,
                                                         oacc[n][4 * q + 2] * inv, oacc[n][4 * q + 3] * inv);
      }
    if (wave == 0 && h == 0) a.part_lse[prow] = lse2;
  }
}

}  // namespace

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st) {
  if (a.num_heads != a.head_groups * kHeadsPerGroup) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t(a.num_items) + kXcds - 1) / kXcds * kXcds * a.head_groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.page_shift >= 0)
    hipLaunchKernelGGL((mla_decode_kernel<true>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((mla_decode_kernel<false>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
