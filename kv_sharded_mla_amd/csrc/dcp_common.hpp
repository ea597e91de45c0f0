// Device helpers shared by the DCP MLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcp {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

#define DCP_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// float -> bf16 payload, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Exact LSE merge of `nparts` partials of one 512-wide row, 4 columns per
// thread (threads 0..127 of a row group).  lse values are read in base 2
// (in_base2) or base e; the merged lse is returned in the same base.
// Partials with lse = -inf carry weight 0.  Returns false if every partial is
// empty (then acc = 0).
__device__ __forceinline__ bool merge_row4(const float* __restrict__ o, int64_t o_stride,
                                          const float* __restrict__ lse, int64_t lse_stride,
                                          int nparts, bool in_base2, int col4, f32x4& acc,
                                          float& lse_out) {
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const float to2 = in_base2 ? 1.0f : kLog2e;
  if (nparts <= 8) {
    // every partial's lse and columns are loaded at once, then the maximum
    // is formed and the partials combined (in order r = 0, 1, ...)
    float l[8];
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nparts) {
        l[k] = lse[k * lse_stride];
        v[k] = *reinterpret_cast<const f32x4*>(o + k * o_stride + 4 * col4);
      }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nparts) m = fmaxf(m, l[k]);
    if (m == -INFINITY) {
      lse_out = -INFINITY;
      return false;
    }
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nparts && l[k] != -INFINITY) {
        const float w = exp2f((l[k] - m) * to2);
        tot += w;
        acc += w * v[k];
      }
    const float inv = 1.0f / tot;
    acc *= inv;
    lse_out = m + (in_base2 ? log2f(tot) : logf(tot));
    return true;
  }
  float m = -INFINITY;
  for (int r = 0; r < nparts; ++r) m = fmaxf(m, lse[r * lse_stride]);
  if (m == -INFINITY) {
    lse_out = -INFINITY;
    return false;
  }
  // work in base 2: w_r = 2^(lse2_r - m2).  The partials are loaded 8 at a
  // time before they are combined (in order r = 0, 1, ...), so the loads
  // overlap instead of each waiting for the previous one.
  float tot = 0.f;
  for (int r0 = 0; r0 < nparts; r0 += 8) {
    float l[8];
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (r0 + k < nparts) {
        l[k] = lse[(r0 + k) * lse_stride];
        v[k] = *reinterpret_cast<const f32x4*>(o + (r0 + k) * o_stride + 4 * col4);
      }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (r0 + k < nparts && l[k] != -INFINITY) {
        const float w = exp2f((l[k] - m) * to2);
        tot += w;
        acc += w * v[k];
      }
  }
  float inv = 1.0f / tot;
  acc *= inv;
  lse_out = m + (in_base2 ? log2f(tot) : logf(tot));
  return true;
}

}  // namespace dcp
