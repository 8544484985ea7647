// Matrix-core building blocks shared by the decode and prefill kernels
// (gfx950): operand vector types, the 16x16 MFMA wrappers for bf16 / fp16, the
// split of fp32 probabilities into a high and a low half-precision part, and
// the streaming 16-byte load.  Device code only; included by the .hip files.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load of K/V (each tile is read once per step): the
// non-temporal hint keeps the stream from displacing cached lines.
__device__ __forceinline__ uint4 load_stream(const char* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(p)));
}

template <typename T>
struct Mfma;

template <>
struct Mfma<BF16> {
  // S^T tile (16 tokens x 16 heads) += K (16 tokens x 32 dims) . Q^T (32 dims x 16 heads)
  __device__ static inline f32x4_t qk(uint4 k, uint4 q, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                   __builtin_bit_cast(bf16x8_t, q), c, 0, 0, 0);
  }
  // O tile (16 heads x 16 dims) += P (16 heads x 16 tokens) . V (16 tokens x 16 dims)
  __device__ static inline f32x4_t pv(uint2 p, uint2 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, p),
                                                     __builtin_bit_cast(i16x4_t, v), c, 0, 0, 0);
  }
  // O tile (16 heads x 16 dims) += P (16 heads x 32 tokens) . V (32 tokens x 16 dims)
  __device__ static inline f32x4_t pv8(uint4 p, uint4 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, p),
                                                   __builtin_bit_cast(bf16x8_t, v), c, 0, 0, 0);
  }
  // As split below, for 2 (split2) or 8 weights, two per instruction where
  // the chip has it: the high parts of two weights are their upper halves
  // side by side (one byte permute), the two remainders are rounded to bf16
  // together.
  __device__ static inline void split2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // upper halves of u0, u1
    const f32x2_t r = {p0 - __uint_as_float(u0 & 0xFFFF0000u),
                       p1 - __uint_as_float(u1 & 0xFFFF0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
  }
  __device__ static inline void split8(const float pe[8], uint4& hi, uint4& lo) {
    split2(pe[0], pe[1], hi.x, lo.x);
    split2(pe[2], pe[3], hi.y, lo.y);
    split2(pe[4], pe[5], hi.z, lo.z);
    split2(pe[6], pe[7], hi.w, lo.w);
  }
  // p (>= 0) = hi + lo with hi = p truncated to bf16 (exact remainder) and
  // lo = remainder rounded to bf16.
  __device__ static inline void split(const float pe[4], uint2& hi, uint2& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = __float_as_uint(pe[e]);
      h[e] = u >> 16;
      const float r = pe[e] - __uint_as_float(u & 0xFFFF0000u);
      l[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r));
    }
    hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
  }
};

template <>
struct Mfma<F16> {
  __device__ static inline f32x4_t pv8(uint4 p, uint4 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, p),
                                                  __builtin_bit_cast(f16x8_t, v), c, 0, 0, 0);
  }
  // As split below, for 2 (split2) or 8 weights, rounding two per
  // instruction.
  __device__ static inline void split2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const f16x2_t hh = __builtin_convertvector(f32x2_t{p0, p1}, f16x2_t);
    const f32x2_t r = {p0 - static_cast<float>(hh[0]), p1 - static_cast<float>(hh[1])};
    hi = __builtin_bit_cast(uint32_t, hh);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, f16x2_t));
  }
  __device__ static inline void split8(const float pe[8], uint4& hi, uint4& lo) {
    split2(pe[0], pe[1], hi.x, lo.x);
    split2(pe[2], pe[3], hi.y, lo.y);
    split2(pe[4], pe[5], hi.z, lo.z);
    split2(pe[6], pe[7], hi.w, lo.w);
  }
  __device__ static inline f32x4_t qk(uint4 k, uint4 q, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, k),
                                                  __builtin_bit_cast(f16x8_t, q), c, 0, 0, 0);
  }
  __device__ static inline f32x4_t pv(uint2 p, uint2 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, p),
                                                 __builtin_bit_cast(f16x4_t, v), c, 0, 0, 0);
  }
  __device__ static inline void split(const float pe[4], uint2& hi, uint2& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 hh = static_cast<_Float16>(pe[e]);
      const float r = pe[e] - static_cast<float>(hh);
      h[e] = __builtin_bit_cast(uint16_t, hh);
      l[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r));
    }
    hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
  }
};

}  // namespace pa
