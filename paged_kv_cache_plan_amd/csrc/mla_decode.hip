// MLA paged decode ("FlashInfer 中的 KV-Cache 布局", section on the MLA page
// layout): the cache has no head dimension; each token stores one 576-wide
// latent row, ckv (512) followed by kpe (64).  Every query head h scores a
// token as sm_scale * (q_ckv[h] . ckv + q_kpe[h] . kpe) and the output is the
// softmax-weighted sum of the ckv rows.
//
// One workgroup per (work item, head group of 32 heads).  Blocks of 32 latent
// rows are staged in LDS once and shared by the 32 heads; q of the group stays
// in LDS for the whole item.  Thread (h, sub) of the 256 owns head h of the
// group: in the score phase it forms 4 dot products (keys sub + 8i), in the
// value phase it accumulates output dims [64*sub, 64*sub + 64).

#include "device.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kHeadsPerGroup = 32;
constexpr int kBlock = 32;            // latent rows per LDS block
constexpr int kDimCkv = 512;
constexpr int kDimKpe = 64;
constexpr int kDim = kDimCkv + kDimKpe;
constexpr int kRow = kDim + 8;         // padded LDS row (elements) to spread banks
constexpr int kChunks = kDim / 8;      // 16-byte chunks per latent row

__global__ __launch_bounds__(256) void mla_decode_kernel(const MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kHeadsPerGroup * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kBlock * kRow];
  __shared__ float s_p[kHeadsPerGroup][kBlock];

  const int32_t item_idx = blockIdx.x / a.head_groups;
  const int32_t grp = blockIdx.x - item_idx * a.head_groups;
  const Item it = a.items[item_idx];
  const int t = threadIdx.x;
  const int h = t >> 3, sub = t & 7;
  const int32_t b = it.q_row0;
  const int32_t head0 = grp * kHeadsPerGroup;
  const uint16_t* qc = static_cast<const uint16_t*>(a.q_ckv);
  const uint16_t* qp = static_cast<const uint16_t*>(a.q_kpe);
  const uint16_t* ckv = static_cast<const uint16_t*>(a.ckv);
  const uint16_t* kpe = static_cast<const uint16_t*>(a.kpe);
  const int32_t* pages = a.kv_indices + it.page_base;

  for (int c = t; c < kHeadsPerGroup * kChunks; c += 256) {
    const int hh = c / kChunks, part = c - (c / kChunks) * kChunks;
    const int64_t qrow = int64_t(b) * a.num_heads + head0 + hh;
    const uint4 val = part < kDimCkv / 8
                          ? *reinterpret_cast<const uint4*>(qc + qrow * kDimCkv + part * 8)
                          : *reinterpret_cast<const uint4*>(qp + qrow * kDimKpe + (part - kDimCkv / 8) * 8);
    *reinterpret_cast<uint4*>(&s_q[hh * kRow + part * 8]) = val;
  }

  float m = -INFINITY, l = 0.f;
  float acc[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) acc[e] = 0.f;

  for (int32_t blk = it.kv_start; blk < it.kv_end; blk += kBlock) {
    __syncthreads();   // previous block's readers are done with s_k / s_p
    for (int c = t; c < kBlock * kChunks; c += 256) {
      const int r = c / kChunks, part = c - (c / kChunks) * kChunks;
      const int32_t j = blk + r;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (j < it.kv_end) {
        const int64_t off = dev::token_offset(pages, j, a.page_size, a.page_shift, a.max_num_pages,
                                              a.page_stride, a.token_stride);
        if (off >= 0)
          val = part < kDimCkv / 8 ? *reinterpret_cast<const uint4*>(ckv + off + part * 8)
                                   : *reinterpret_cast<const uint4*>(kpe + off + (part - kDimCkv / 8) * 8);
      }
      *reinterpret_cast<uint4*>(&s_k[r * kRow + part * 8]) = val;
    }
    __syncthreads();

    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = 0.f;
    for (int d = 0; d < kDim; d += 8) {
      const uint4 qv = *reinterpret_cast<const uint4*>(&s_q[h * kRow + d]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 kv = *reinterpret_cast<const uint4*>(&s_k[(sub + 8 * i) * kRow + d]);
        s[i] = dev::dot2_bf16(qv.x, kv.x, s[i]);
        s[i] = dev::dot2_bf16(qv.y, kv.y, s[i]);
        s[i] = dev::dot2_bf16(qv.z, kv.z, s[i]);
        s[i] = dev::dot2_bf16(qv.w, kv.w, s[i]);
      }
    }
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = blk + sub + 8 * i < it.kv_end;
      s[i] = valid ? s[i] * a.scale_log2 : -INFINITY;
      bm = fmaxf(bm, s[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 1));
    bm = fmaxf(bm, __shfl_xor(bm, 2));
    bm = fmaxf(bm, __shfl_xor(bm, 4));
    const float m_new = fmaxf(m, bm);
    const float scale = dev::fast_exp2(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = dev::fast_exp2(s[i] - m_new);
      psum += p;
      s_p[h][sub + 8 * i] = p;
    }
    psum += __shfl_xor(psum, 1);
    psum += __shfl_xor(psum, 2);
    psum += __shfl_xor(psum, 4);
    l = l * scale + psum;
    m = m_new;
#pragma unroll
    for (int e = 0; e < 64; ++e) acc[e] *= scale;
    __syncthreads();
    for (int r = 0; r < kBlock; ++r) {
      const float p = s_p[h][r];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(&s_k[r * kRow + sub * 64 + c * 8]);
        acc[c * 8 + 0] = fmaf(p, dev::bf16_lo(v.x), acc[c * 8 + 0]);
        acc[c * 8 + 1] = fmaf(p, dev::bf16_hi(v.x), acc[c * 8 + 1]);
        acc[c * 8 + 2] = fmaf(p, dev::bf16_lo(v.y), acc[c * 8 + 2]);
        acc[c * 8 + 3] = fmaf(p, dev::bf16_hi(v.y), acc[c * 8 + 3]);
        acc[c * 8 + 4] = fmaf(p, dev::bf16_lo(v.z), acc[c * 8 + 4]);
        acc[c * 8 + 5] = fmaf(p, dev::bf16_hi(v.z), acc[c * 8 + 5]);
        acc[c * 8 + 6] = fmaf(p, dev::bf16_lo(v.w), acc[c * 8 + 6]);
        acc[c * 8 + 7] = fmaf(p, dev::bf16_hi(v.w), acc[c * 8 + 7]);
      }
    }
  }

  const int32_t head = head0 + h;
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse2 = empty ? -INFINITY : m + __log2f(l);
  if (it.out_slot < 0) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + (int64_t(b) * a.num_heads + head) * kDimCkv + sub * 64;
#pragma unroll
    for (int e = 0; e < 64; e += 2)
      *reinterpret_cast<uint32_t*>(orow + e) = dev::pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
    if (sub == 0 && a.lse) a.lse[int64_t(b) * a.num_heads + head] = lse2;
  } else {
    const int64_t prow = int64_t(it.out_slot) * a.num_heads + head;
    float* prow_o = a.part_o + prow * kDimCkv + sub * 64;
#pragma unroll
    for (int e = 0; e < 64; ++e) prow_o[e] = acc[e] * inv;
    if (sub == 0) a.part_lse[prow] = lse2;
  }
}

}  // namespace

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st) {
  if (a.num_heads != a.head_groups * kHeadsPerGroup) return hipErrorInvalidValue;
  const int64_t blocks = int64_t(a.num_items) * a.head_groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_decode_kernel, dim3(uint32_t(blocks)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
