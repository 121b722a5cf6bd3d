// Paged prefill / append attention for bf16 with MFMA tiles (gfx950).
//
// Prefill and append attention is a dense contraction once a tile of keys
// is gathered ("Deep Dive - FlashInfer", "Ragged prefill and paged decode"),
// so both products run on v_mfma_f32_32x32x16_bf16:
//
//   * A workgroup (4 waves) owns one work item for one kv head: up to 128
//     (query row, head) pairs -- 128/G rows times the G query heads that share
//     the kv head -- against one chunk of keys.  Wave w owns pairs
//     [32w, 32w + 32).
//   * Keys stream through LDS in tiles of 64, double-buffered: the page-table
//     gather of tile t+1 (16-byte global loads, each row located through
//     kv_indices) is in flight while tile t is consumed.
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
//     the tile sees key j iff j <= diag + r).
//
// The epilogue writes the normalised rows (bf16) and base-2 LSE, or fp32
// partial states for the split merge ("A worked split-KV example").

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
// LDS row pitches (elements).  K rows are read 16 bytes per lane, 32 rows at
// one column: a pitch of 68 dwords spreads consecutive rows over distinct
// 4-bank groups.  V rows are read by the transposed load, 4 rows x 32 bytes
// per 16-lane group: a pitch of 72 dwords puts those 4 rows on disjoint banks.
constexpr int kPitchK = kD + 8;
constexpr int kPitchV = kD + 16;
constexpr int kMaxChunkPages = 1024;   // the planner never makes a chunk longer than this
constexpr int kWaves = 4;
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

template <int G, bool kPow2>
__global__ __launch_bounds__(kThreads, 2) void prefill_mfma_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kKeys * kPitchK];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kKeys * kPitchV];
  __shared__ int32_t s_pages[kMaxChunkPages];

  const int32_t hkv = a.num_kv_heads;
  const int32_t item_idx = blockIdx.x / hkv;
  const int32_t kvh = blockIdx.x - item_idx * hkv;
  const Item it = a.items[item_idx];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;          // lane half: which 8-element k slice of an MFMA operand
  const int col = lane & 31;        // MFMA column: the pair this lane scores

  // This lane's (row, head) pair.
  const int pair = wave * 32 + col;
  const int prow = pair / G, phead = pair - (pair / G) * G;
  const bool pair_ok = prow < it.num_rows;
  const int32_t qrow_idx = it.q_row0 + prow;
  const int32_t head = kvh * G + phead;
  const int32_t limit = pair_ok ? min(it.kv_end - 1, it.diag + prow) : -1;   // last visible key
  // Smallest row limit in the wave: tiles ending at or before it need no mask.
  const int32_t wave_limit_min = min(it.kv_end - 1, it.diag + (wave * 32) / G);

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + int64_t(kvh) * a.head_stride;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + int64_t(kvh) * a.head_stride;
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t psz = a.page_size, pshift = a.page_shift;
  const uint32_t max_pages = uint32_t(a.max_num_pages);

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

  // Page ids of the chunk (at most kMaxChunkPages, a planner guarantee) go to LDS once.
  const int32_t pg_lo = kv_hi > kv_lo ? (kPow2 ? kv_lo >> pshift : kv_lo / psz) : 0;
  const int32_t pg_n =
      kv_hi > kv_lo ? min(kMaxChunkPages, (kPow2 ? (kv_hi - 1) >> pshift : (kv_hi - 1) / psz) - pg_lo + 1) : 0;
  for (int i = tid; i < pg_n; i += kThreads) {
    const int32_t pg = pages[pg_lo + i];
    s_pages[i] = uint32_t(pg) < max_pages ? pg : 0;
  }
  __syncthreads();

  // Tile loader: thread tid moves 16 bytes of 4 keys (key tid/16 + 16i,
  // dims (tid%16)*8) of K or V.  Keys past the chunk end re-read the last key
  // (their scores are masked to -inf, so their weights are exactly zero).
  const int ld_key = tid >> 4, ld_chunk = tid & 15;
  // Full tiles on pages of at least 16 keys: a thread's four keys
  // t0 + ld_key + 16i sit on page (t0 + 16i) >> shift, the same page for the
  // whole workgroup, so only the slot depends on the thread.
  const bool aligned = kPow2 && pshift >= 4;
  const int64_t ld_lane_off = int64_t(ld_key) * a.token_stride + ld_chunk * 8;
  auto tile_offsets = [&](int32_t t0, int64_t (&off)[4]) {
    if (aligned && t0 + kKeys <= kv_hi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t j0 = t0 + 16 * i;
        off[i] = int64_t(s_pages[(j0 >> pshift) - pg_lo]) * a.page_stride + int64_t(j0 & (psz - 1)) * a.token_stride +
                 ld_lane_off;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t j = min(t0 + ld_key + 16 * i, kv_hi - 1);
        const int32_t pi = kPow2 ? (j >> pshift) : (j / psz);
        const int32_t sl = kPow2 ? (j & (psz - 1)) : (j - pi * psz);
        off[i] = int64_t(s_pages[min(pi - pg_lo, kMaxChunkPages - 1)]) * a.page_stride + int64_t(sl) * a.token_stride +
                 ld_chunk * 8;
      }
    }
  };
  uint4 kst0, kst1, kst2, kst3, vst0, vst1, vst2, vst3;
  auto gload_k = [&](int32_t t0) {
    int64_t off[4];
    tile_offsets(t0, off);
    kst0 = *reinterpret_cast<const uint4*>(kbase + off[0]);
    kst1 = *reinterpret_cast<const uint4*>(kbase + off[1]);
    kst2 = *reinterpret_cast<const uint4*>(kbase + off[2]);
    kst3 = *reinterpret_cast<const uint4*>(kbase + off[3]);
  };
  auto gload_v = [&](int32_t t0) {
    int64_t off[4];
    tile_offsets(t0, off);
    vst0 = *reinterpret_cast<const uint4*>(vbase + off[0]);
    vst1 = *reinterpret_cast<const uint4*>(vbase + off[1]);
    vst2 = *reinterpret_cast<const uint4*>(vbase + off[2]);
    vst3 = *reinterpret_cast<const uint4*>(vbase + off[3]);
  };
  uint16_t* const k_st = &s_k[ld_key * kPitchK + ld_chunk * 8];
  uint16_t* const v_st = &s_v[ld_key * kPitchV + ld_chunk * 8];
  auto lstore_k = [&]() {
    *reinterpret_cast<uint4*>(k_st) = kst0;
    *reinterpret_cast<uint4*>(k_st + 16 * kPitchK) = kst1;
    *reinterpret_cast<uint4*>(k_st + 32 * kPitchK) = kst2;
    *reinterpret_cast<uint4*>(k_st + 48 * kPitchK) = kst3;
  };
  auto lstore_v = [&]() {
    *reinterpret_cast<uint4*>(v_st) = vst0;
    *reinterpret_cast<uint4*>(v_st + 16 * kPitchV) = vst1;
    *reinterpret_cast<uint4*>(v_st + 32 * kPitchV) = vst2;
    *reinterpret_cast<uint4*>(v_st + 48 * kPitchV) = vst3;
  };

  // S^T of the K tile currently in LDS: two 32-key blocks.
  const uint16_t* const k_rd = &s_k[col * kPitchK + 8 * h];
  // The two 32-key blocks alternate so consecutive MFMAs are independent.
  auto scores = [&](f32x16_t (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 kv = *reinterpret_cast<const uint4*>(k_rd + kb * 32 * kPitchK + 16 * st);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), as_bf16x8(qreg[st]), sacc[kb], 0, 0, 0);
      }
    }
  };

  const int grp = lane >> 4, gi = lane & 15;
  const uint16_t* const v_rd = &s_v[(4 * h + (gi >> 2)) * kPitchV + 16 * (grp & 1) + 4 * (gi & 3)];
  const float c = a.scale_log2;

  // One tile: softmax of S(t) (in scur) and O += V(t) P(t), while the scores
  // S(t+1) of the K tile already in LDS are computed into snext.  On entry LDS
  // holds K(t+1) and V(t); on exit it holds K(t+2) and V(t+1).
  auto body = [&](int32_t t, f32x16_t (&scur)[2], f32x16_t (&snext)[2]) {
    const int32_t t0 = kv_lo + t * kKeys;
    if (t + 2 < ntiles) gload_k(t0 + 2 * kKeys);
    if (t + 1 < ntiles) gload_v(t0 + kKeys);

    // Masking: key of value v in block kb is t0 + 32kb + 8(v/4) + 4h + v%4.
    if (t0 + kKeys - 1 > wave_limit_min) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t j = t0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
          scur[kb][v] = j <= limit ? scur[kb][v] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, scur[kb][v]);
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

    // S(t+1) on the matrix cores while the weights of tile t are formed.
    scores(snext);
    // exp2(-inf) = 0 covers masked keys; a row with no visible key yet has
    // only -inf scores, so any finite shift works for it.
    const float shift = m_used != -INFINITY ? m_used : 0.f;
    uint4 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = dev::fast_exp2(fmaf(scur[ks >> 1][8 * (ks & 1) + e], c, -shift));
        lsum += p[e];
      }
      pb[ks] = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
    }

    // O^T += V^T P^T: d-block n, k-step ks (16 keys).  The transposed read
    // gives lane i of each 16-lane group the value rows of 4 keys at one dim.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint16_t* base = v_rd + 16 * ks * kPitchV + 32 * n;
        const bf16x4_t lo = tr_read(base);
        const bf16x4_t hi = tr_read(base + 8 * kPitchV);
        const bf16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16x8(pb[ks]), oacc[n], 0, 0, 0);
      }
    }

    __syncthreads();   // every wave is done with K(t+1) and V(t)
    if (t + 2 < ntiles) lstore_k();
    if (t + 1 < ntiles) lstore_v();
    __syncthreads();
  };

  f32x16_t sa[2], sb[2];
  if (ntiles > 0) {
    gload_k(kv_lo);
    gload_v(kv_lo);
    lstore_k();
    lstore_v();
    __syncthreads();
    scores(sa);
    if (ntiles > 1) gload_k(kv_lo + kKeys);
    __syncthreads();
    if (ntiles > 1) lstore_k();
    __syncthreads();
  }
  for (int32_t t = 0; t < ntiles; t += 2) {
    body(t, sa, sb);
    if (t + 1 >= ntiles) break;
    body(t + 1, sb, sa);
  }

  // Epilogue: row sum over both lane halves, normalise, write.
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!pair_ok) return;
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
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

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t st) {
  const int64_t blocks = int64_t(a.num_items) * a.num_kv_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.page_shift >= 0)
    hipLaunchKernelGGL((prefill_mfma_kernel<G, true>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<G, false>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_mfma(int32_t head_dim, int32_t group, const AttnArgs& a, hipStream_t st,
                               bool* supported) {
  if (head_dim == kD) {
    *supported = true;
    switch (group) {
      case 1: return launch_g<1>(a, st);
      case 2: return launch_g<2>(a, st);
      case 4: return launch_g<4>(a, st);
      case 8: return launch_g<8>(a, st);
      default: break;
    }
  }
  // Other shapes run the row kernel (same results, VALU arithmetic).
  return launch_attn_rows(kBF16, head_dim, group, a, st, supported);
}

}  // namespace pkv
