// Device helpers for the gfx950 kernels: bf16 <-> f32, DPP lane exchanges,
// wave-local synchronisation and page-table address arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
namespace dev {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// a.x*b.x + a.y*b.y + c with bf16 pairs packed in 32-bit words (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// DPP lane exchange within rows of 16 lanes.  CTRL encodings: quad_perm
// 0x00-0xFF, row_ror:N = 0x120 + N.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowMirror = 0x140;      // lane i <-> 15 - i within a row
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i within each half row

// Sum over the 4 lanes of a quad (every lane gets the total).
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  return x;
}

// Max / sum over the 16 quads of a wave for values that are uniform within
// each quad (every lane gets the result).  Needs all 64 lanes active.
__device__ __forceinline__ float quads_max(float x) {
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor8>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float quads_sum(float x) {
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load with the non-temporal hint: for data read once (the KV
// stream of decode), so it does not displace reusable lines in the caches.
// Streaming reads reach markedly higher HBM bandwidth this way on gfx950.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <bool kNT>
__device__ __forceinline__ uint4 load16(const void* p) {
  if constexpr (kNT) {
    const u32x4_t x = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
  } else {
    return *static_cast<const uint4*>(p);
  }
}

// Element offset of token j's row (slot within its page) given the request's
// page list: page kv_indices[page_base + j / P], slot j % P.  Returns -1 for a
// page id outside [0, max_pages).
__device__ __forceinline__ int64_t token_offset(const int32_t* pages, int32_t j, int32_t page_size,
                                                int32_t page_shift, int32_t max_pages, int64_t page_stride,
                                                int64_t token_stride) {
  int32_t pi, slot;
  if (page_shift >= 0) {
    pi = j >> page_shift;
    slot = j & (page_size - 1);
  } else {
    pi = j / page_size;
    slot = j - pi * page_size;
  }
  const int32_t page = pages[pi];
  if (page < 0 || page >= max_pages) return -1;
  return int64_t(page) * page_stride + int64_t(slot) * token_stride;
}

}  // namespace dev
}  // namespace pkv
