// Paged attention, one query row at a time: the decode kernel.
//
// Decode reads a long history for very little arithmetic, so this kernel is
// built around HBM streaming ("Deep Dive - FlashInfer", "Ragged prefill and
// paged decode"): each workgroup takes one work item (a key chunk of one
// request) for one kv head and all G query heads that share it (GQA: query head
// h reads kv head h / G).  Every K and V row is fetched from HBM exactly once
// per kv head and used for all G heads.
//
// Work split inside a workgroup (4 waves of 64 lanes): waves take interleaved
// blocks of 16 keys.
//   Score phase: a quad of 4 lanes owns one key; each lane loads a quarter of
//     the key row with 16-byte loads (4 lanes x 16 B = 64 contiguous bytes per
//     instruction) and forms partial dot products for the G heads (bf16 pairs
//     through v_dot2c_f32_bf16); two DPP quad exchanges finish them.
//   Softmax: block max over the wave's 16 keys by DPP row rotations and two
//     cross-row shuffles, exp2 in the log2 domain (scores are pre-multiplied by
//     sm_scale * log2 e), running max m and per-quad running sum l.
//   Value phase: 16 lanes own one value row (each lane 16 bytes), 4 rows per
//     load instruction; p comes from a per-wave LDS slot; the accumulator is
//     rescaled once per block.
// At the end the 4 waves' states are merged in LDS and written either as the
// final output (dtype of Q, plus base-2 LSE) or as an fp32 partial state for
// the split merge ("Deep Dive - FlashInfer", "A worked split-KV example").
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

template <typename T>
__device__ __forceinline__ void unpack_chunk(const uint4& v, float* out);

template <>
__device__ __forceinline__ void unpack_chunk<uint16_t>(const uint4& v, float* out) {
  out[0] = dev::bf16_lo(v.x);
  out[1] = dev::bf16_hi(v.x);
  out[2] = dev::bf16_lo(v.y);
  out[3] = dev::bf16_hi(v.y);
  out[4] = dev::bf16_lo(v.z);
  out[5] = dev::bf16_hi(v.z);
  out[6] = dev::bf16_lo(v.w);
  out[7] = dev::bf16_hi(v.w);
}

template <>
__device__ __forceinline__ void unpack_chunk<float>(const uint4& v, float* out) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { *p = dev::f32_to_bf16(x); }
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void attn_rows_kernel(const AttnArgs a) {
  constexpr int E = Elem<T>::kPer16;   // elements per 16-byte chunk
  constexpr int NCH = D / E;           // chunks per row
  constexpr int KC = NCH / 4;          // score phase: chunks per lane (4 lanes per key)
  constexpr int VL = NCH < 16 ? NCH : 16;  // value phase: lanes per row
  constexpr int VC = NCH / VL;         // value phase: chunks per lane
  constexpr int VT = 64 / VL;          // value phase: rows per load instruction
  static_assert(NCH % 4 == 0 && NCH % VL == 0, "head_dim must split into 16-byte chunks");

  __shared__ float s_p[kWaves][kBlockKeys][G];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];

  const int32_t hkv = a.num_kv_heads;
  const int32_t item_idx = blockIdx.x / hkv;
  const int32_t kvh = blockIdx.x - item_idx * hkv;
  const Item it = a.items[item_idx];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int qk = lane >> 2, qi = lane & 3;     // score phase: key in block, quarter of the row
  const int vg = lane / VL, vi = lane % VL;    // value phase: row in pass, chunk column

  const T* kbase = static_cast<const T*>(a.k) + int64_t(kvh) * a.head_stride;
  const T* vbase = static_cast<const T*>(a.v) + int64_t(kvh) * a.head_stride;
  const int32_t* pages = a.kv_indices + it.page_base;
  const int32_t hq = a.num_qo_heads;

  for (int r = 0; r < it.num_rows; ++r) {
    const int32_t row = it.q_row0 + r;
    const int32_t kv_end = min(it.kv_end, it.diag + r + 1);
    const int32_t nkeys = kv_end - it.kv_start;

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

    for (int32_t blk = wave * kBlockKeys; blk < nkeys; blk += kWaves * kBlockKeys) {
      // Score phase: one key per quad.
      const int32_t kj = blk + qk;
      uint4 kreg[KC];
      bool kvalid = kj < nkeys;
      if (kvalid) {
        const int64_t off = dev::token_offset(pages, it.kv_start + kj, a.page_size, a.page_shift,
                                              a.max_num_pages, a.page_stride, a.token_stride);
        kvalid = off >= 0;
        if (kvalid) {
          const T* krow = kbase + off;
#pragma unroll
          for (int c = 0; c < KC; ++c) kreg[c] = *reinterpret_cast<const uint4*>(krow + (qi + 4 * c) * E);
        }
      }
      // Value rows of this block, issued before the score math so both are in flight.
      uint4 vreg[kBlockKeys / VT][VC];
      bool vvalid[kBlockKeys / VT];
#pragma unroll
      for (int u = 0; u < kBlockKeys / VT; ++u) {
        const int32_t vj = blk + u * VT + vg;
        vvalid[u] = vj < nkeys;
        int64_t off = -1;
        if (vvalid[u])
          off = dev::token_offset(pages, it.kv_start + vj, a.page_size, a.page_shift, a.max_num_pages,
                                  a.page_stride, a.token_stride);
        vvalid[u] = off >= 0;
#pragma unroll
        for (int c = 0; c < VC; ++c) {
          if (vvalid[u])
            vreg[u][c] = *reinterpret_cast<const uint4*>(vbase + off + (vi + VL * c) * E);
          else
            vreg[u][c] = make_uint4(0, 0, 0, 0);
        }
      }

      float scale[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float part = 0.f;
        if (kvalid) {
#pragma unroll
          for (int c = 0; c < KC; ++c) dot_chunk<T>(qreg[h][c], kreg[c], part);
        }
        float s = dev::quad_sum(part) * a.scale_log2;
        s = kvalid ? s : -INFINITY;
        const float m_new = fmaxf(m[h], dev::quads_max(s));
        const bool live = m_new != -INFINITY;       // false only if every key so far was skipped
        scale[h] = live ? dev::fast_exp2(m[h] - m_new) : 1.f;   // m[h] = -inf gives 0
        const float p = live ? dev::fast_exp2(s - m_new) : 0.f;
        l[h] = l[h] * scale[h] + p;
        m[h] = m_new;
        if (qi == 0) s_p[wave][qk][h] = p;
      }
      dev::wave_lds_sync();

      // Value phase.
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VC * E; ++e) acc[h][e] *= scale[h];
#pragma unroll
      for (int u = 0; u < kBlockKeys / VT; ++u) {
        float pv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pv[h] = s_p[wave][u * VT + vg][h];
#pragma unroll
        for (int c = 0; c < VC; ++c) {
          float vf[E];
          unpack_chunk<T>(vreg[u][c], vf);
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][c * E + e] = fmaf(pv[h], vf[e], acc[h][c * E + e]);
        }
      }
      dev::wave_lds_sync();
    }

    // Wave-level state: l summed over quads, acc summed over value rows.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = dev::quads_sum(l[h]);
#pragma unroll
      for (int e = 0; e < VC * E; ++e) {
        float x = acc[h][e];
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
  hipLaunchKernelGGL((attn_rows_kernel<T, D, G>), dim3(uint32_t(blocks)), dim3(kThreads), 0, st, a);
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
