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
// Loads are branch-free: a key past the end of the row's range re-reads the
// last valid key (its weight is zero), and a page id outside the pool is
// replaced by page 0 so no access leaves the cache allocation (the host
// validates page ids; such rows would give undefined values, never a fault).
//
// Multi-row tiles (float32 prefill) loop over their rows; row r sees key j iff
// j <= diag + r ("Causality uses logical positions, not page numbers").

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockKeys = 16;
constexpr int kSegPages = 1024;   // page ids staged in LDS per segment
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

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { *p = dev::f32_to_bf16(x); }
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }

// Reductions over the QPG quads of one softmax group: 4 quads = a 16-lane
// row, 2 quads = half a row.
template <int QPG>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (QPG == 4) {
    x = fmaxf(x, dev::dpp<dev::kRowRor4>(x));
    x = fmaxf(x, dev::dpp<dev::kRowRor8>(x));
  } else {
    x = fmaxf(x, dev::dpp<dev::kRowHalfMirror>(x));
  }
  return x;
}

// Rows with many (head, dim) accumulators and wide register sets (float32, or
// bf16 with 8 heads per group at head_dim 128) need more than 256 VGPRs; they
// run one wave per SIMD instead of spilling.
template <typename T, int D, int G>
constexpr int rows_min_waves() {
  return int(sizeof(T)) * D * G >= 2048 ? 1 : PKV_ROWS_MIN_WAVES;
}

template <typename T, int D, int G, bool kAligned>
__global__ __launch_bounds__(kThreads, (rows_min_waves<T, D, G>())) void attn_rows_kernel(const AttnArgs a) {
  constexpr bool kBF16 = sizeof(T) == 2;
  constexpr int E = Elem<T>::kPer16;   // elements per 16-byte chunk
  constexpr int NCH = D / E;           // chunks per row
  constexpr int KC = NCH / 4;          // score phase: chunks per lane (4 lanes per key)
  constexpr int VL = NCH < 16 ? NCH : 16;  // value phase: lanes per row
  constexpr int VC = NCH / VL;         // value phase: chunks per lane
  constexpr int VT = 64 / VL;          // value phase: rows per load instruction = softmax groups
  constexpr int NU = kBlockKeys / VT;  // value phase: passes per block = keys per group per block
  constexpr int QPG = kBlockKeys / VT; // score phase: quads per softmax group
  static_assert(NCH % 4 == 0 && NCH % VL == 0 && (QPG == 4 || QPG == 2), "unsupported head_dim");
  static_assert(NU % 2 == 0, "value passes come in pairs");

  __shared__ int32_t s_pages[kSegPages];
  // Block weights: bf16 pairs (keys 2w*VT+g, (2w+1)*VT+g) per head, or fp32.
  __shared__ uint32_t s_p[kWaves][NU][VT][G];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];

  const int32_t hkv = a.num_kv_heads;
  const int32_t item_idx = blockIdx.x / hkv;
  const int32_t kvh = blockIdx.x - item_idx * hkv;
  const Item it = a.items[item_idx];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Score phase: quad qk scores key u*VT + g of the block, where g = qk / QPG
  // is its softmax group and u = qk % QPG its pass in the value phase.
  const int qk = lane >> 2, qi = lane & 3;
  const int k_u = qk % QPG, k_g = qk / QPG;
  const int key_in_block = k_u * VT + k_g;
  const int vg = lane / VL, vi = lane % VL;    // value phase: group (= k_g of this lane), chunk column

  const T* kbase = static_cast<const T*>(a.k) + int64_t(kvh) * a.head_stride;
  const T* vbase = static_cast<const T*>(a.v) + int64_t(kvh) * a.head_stride;
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t hq = a.num_qo_heads;
  const int32_t psz = a.page_size, pshift = a.page_shift;
  const uint32_t max_pages = uint32_t(a.max_num_pages);
  auto page_of = [&](int32_t j) { return kAligned ? (j >> pshift) : (pshift >= 0 ? (j >> pshift) : (j / psz)); };
  auto slot_of = [&](int32_t j) {
    return kAligned ? (j & (psz - 1)) : (pshift >= 0 ? (j & (psz - 1)) : (j - (j / psz) * psz));
  };

  for (int r = 0; r < it.num_rows; ++r) {
    const int32_t row = it.q_row0 + r;
    const int32_t lo = it.kv_start;
    const int32_t hi = min(it.kv_end, it.diag + r + 1);

    uint4 qreg[G][KC];
    const T* qrow = static_cast<const T*>(a.q) + int64_t(row) * a.q_stride_token +
                    int64_t(kvh * G) * a.q_stride_head;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        qreg[h][c] = *reinterpret_cast<const uint4*>(qrow + int64_t(h) * a.q_stride_head + (qi + 4 * c) * E);

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
        s_pages[i] = uint32_t(pg) < max_pages ? pg : 0;
      }
      __syncthreads();
      const int32_t tlo = max(lo, sp * psz);
      const int32_t thi = min(hi, (sp + np) * psz);

      // Element offset of key j's row; keys at or past thi re-read key thi-1.
      auto row_off = [&](int32_t j) -> int64_t {
        j = min(j, thi - 1);
        return int64_t(s_pages[page_of(j) - sp]) * a.page_stride + int64_t(slot_of(j)) * a.token_stride;
      };
      auto load = [&](int32_t blk, uint4 (&kr)[KC], uint4 (&vr)[NU][VC]) {
        int64_t koff;
        int64_t voff[NU];
        if constexpr (kAligned) {
          // A 16-key block never crosses a page: one page id for the block.
          const int64_t base = int64_t(s_pages[(blk >> pshift) - sp]) * a.page_stride;
          const int32_t last = thi - 1 - blk;
          const int32_t s0 = blk & (psz - 1);
          koff = base + int64_t(s0 + min(key_in_block, last)) * a.token_stride;
#pragma unroll
          for (int u = 0; u < NU; ++u) voff[u] = base + int64_t(s0 + min(u * VT + vg, last)) * a.token_stride;
        } else {
          koff = row_off(blk + key_in_block);
#pragma unroll
          for (int u = 0; u < NU; ++u) voff[u] = row_off(blk + u * VT + vg);
        }
        const T* krow = kbase + koff;
#pragma unroll
        for (int c = 0; c < KC; ++c) kr[c] = *reinterpret_cast<const uint4*>(krow + (qi + 4 * c) * E);
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int c = 0; c < VC; ++c)
            vr[u][c] = *reinterpret_cast<const uint4*>(vbase + voff[u] + (vi + VL * c) * E);
      };

      auto compute = [&](int32_t blk, uint4 (&kr)[KC], uint4 (&vr)[NU][VC]) {
        const bool kok = blk + key_in_block < thi;
        float scale[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float part = 0.f;
#pragma unroll
          for (int c = 0; c < KC; ++c) dot_chunk<T>(qreg[h][c], kr[c], part);
          float s = dev::quad_sum(part) * a.scale_log2;
          s = kok ? s : -INFINITY;
          const float m_new = fmaxf(m[h], group_max<QPG>(s));
          const bool live = m_new != -INFINITY;       // false only while every key so far was skipped
          scale[h] = live ? dev::fast_exp2(m[h] - m_new) : 1.f;
          const float p = live ? dev::fast_exp2(s - m_new) : 0.f;
          l[h] = l[h] * scale[h] + p;
          m[h] = m_new;
          if constexpr (kBF16) {
            // lane qi of the quad stores heads qi, qi+4, ... as the bf16 half
            // (u % 2) of the pair slot of pass pair u / 2.
            if (h % 4 == qi)
              reinterpret_cast<uint16_t*>(&s_p[wave][k_u / 2][k_g][h])[k_u % 2] = dev::f32_to_bf16(p);
          } else {
            if (h % 4 == qi) s_p[wave][k_u][k_g][h] = __float_as_uint(p);
          }
        }
        dev::wave_lds_sync();
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (__any(scale[h] != 1.f)) {
#pragma unroll
            for (int e = 0; e < VC * E; ++e) acc[h][e] *= scale[h];
          }
        }
        if constexpr (kBF16) {
#pragma unroll
          for (int w = 0; w < NU / 2; ++w) {
            uint32_t pp[G];
#pragma unroll
            for (int h = 0; h < G; ++h) pp[h] = s_p[wave][w][vg][h];
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
          for (int u = 0; u < NU; ++u) {
            float pv[G];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = __uint_as_float(s_p[wave][u][vg][h]);
#pragma unroll
            for (int c = 0; c < VC; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float x = __uint_as_float(word(vr[u][c], i));
#pragma unroll
                for (int h = 0; h < G; ++h) acc[h][c * E + i] = fmaf(pv[h], x, acc[h][c * E + i]);
              }
          }
        }
        dev::wave_lds_sync();
      };

      // Two register sets: the loads of block i+1 are in flight while block i
      // computes.  The prefetch is unconditional (past the end it re-reads the
      // last block, which the caches serve) so that every path through the
      // loop has the same loads outstanding and the wait before a block's
      // compute covers only that block's own loads.
      constexpr int32_t kStride = kWaves * kBlockKeys;
      const int32_t blk_max = kAligned ? ((thi - 1) & ~(kBlockKeys - 1)) : thi - 1;
      uint4 ka[KC], kb[KC], va[NU][VC], vb[NU][VC];
      int32_t blk = tlo + wave * kBlockKeys;
      if (blk < thi) {
        load(blk, ka, va);
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

    // Wave state: rescale every group to the wave max, then sum l over quads
    // and acc over value-phase groups.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mw = dev::quads_max(m[h]);
      const float f = m[h] == -INFINITY ? 0.f : dev::fast_exp2(m[h] - mw);
      l[h] = dev::quads_sum(l[h] * f);
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
          for (int e = 0; e < E; ++e) s_acc[wave][h][(vi + VL * c) * E + e] = acc[h][c * E + e];
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
      for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, s_m[w][h]);
      float ll = 0.f, oo = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = s_m[w][h] == -INFINITY ? 0.f : dev::fast_exp2(s_m[w][h] - mm);
        ll += f * s_l[w][h];
        oo += f * s_acc[w][h][d];
      }
      const bool empty = !(ll > 0.f);
      const float out = empty ? 0.f : oo / ll;
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
    __syncthreads();
  }
}

template <typename T, int D, int G>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const int64_t blocks = int64_t(a.num_items) * a.num_kv_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const bool aligned = a.page_shift >= 4;   // a power-of-two page of at least 16 keys
  if (aligned)
    hipLaunchKernelGGL((attn_rows_kernel<T, D, G, true>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_rows_kernel<T, D, G, false>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(int32_t group, const AttnArgs& a, hipStream_t st, bool* ok) {
  *ok = true;
  switch (group) {
    case 1: return launch_t<T, D, 1>(a, st);
    case 2: return launch_t<T, D, 2>(a, st);
    case 4: return launch_t<T, D, 4>(a, st);
    case 8:
      if (sizeof(T) == 2) return launch_t<T, D, 8>(a, st);
      break;
    default: break;
  }
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_rows(int32_t dtype, int32_t head_dim, int32_t group, const AttnArgs& a,
                            hipStream_t st, bool* supported) {
  *supported = false;
  if (dtype == kBF16) {
    if (head_dim == 128) return launch_g<uint16_t, 128>(group, a, st, supported);
    if (head_dim == 64) return launch_g<uint16_t, 64>(group, a, st, supported);
  } else if (dtype == kF32) {
    if (head_dim == 128) return launch_g<float, 128>(group, a, st, supported);
    if (head_dim == 64) return launch_g<float, 64>(group, a, st, supported);
  }
  return hipSuccess;
}

}  // namespace pkv
