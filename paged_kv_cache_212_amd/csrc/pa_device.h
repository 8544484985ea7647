// Device-side helpers shared by the library's HIP kernels: element types,
// the pool layout and launch-checking plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

constexpr int kBlockSize = 16;  // tokens per KV block

// Element-type tags: `bits` is the stored integer type, kVecElems = elements
// per 16-byte chunk (the `x` of the K layout).
struct F32 {
  using bits = uint32_t;
  static constexpr int kBytes = 4;
  static constexpr int kVecElems = 4;
  __device__ static inline float to_float(bits v) { return __uint_as_float(v); }
};
struct F16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kVecElems = 8;
  __device__ static inline float to_float(bits v) {
    return static_cast<float>(__builtin_bit_cast(_Float16, v));
  }
};
struct BF16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kVecElems = 8;
  __device__ static inline float to_float(bits v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
};

// One-byte elements: the 8-bit codes of a quantized cache (value = code *
// the pool's scale).  U8 moves them as bytes; E4M3 (OCP 8-bit float, 4
// exponent bits with bias 7, 3 mantissa bits, no infinity) and I8 (two's
// complement) say how the attention widens them.
struct U8 {
  using bits = uint8_t;
  static constexpr int kBytes = 1;
  static constexpr int kVecElems = 16;
};
struct E4M3 : U8 {};
struct I8 : U8 {};

// Encoders of the quantized cache (r = the fp32 reciprocal of the pool's
// scale): y = x * r in one fp32 rounding, then
//   I8:   round half to even, clamp to [-127, 127], two's complement byte;
//   E4M3: clamp to [-448, 448] (the largest finite code), then the hardware
//         conversion, which rounds to nearest even and keeps the sign.
template <typename Code>
struct Encode;
template <>
struct Encode<I8> {
  __device__ static inline uint32_t pair(float a, float b, float r) {
    const int ca = static_cast<int>(fminf(fmaxf(rintf(a * r), -127.f), 127.f));
    const int cb = static_cast<int>(fminf(fmaxf(rintf(b * r), -127.f), 127.f));
    return (static_cast<uint32_t>(ca) & 0xFFu) | ((static_cast<uint32_t>(cb) & 0xFFu) << 8);
  }
};
template <>
struct Encode<E4M3> {
  __device__ static inline uint32_t pair(float a, float b, float r) {
    const float ya = fminf(fmaxf(a * r, -448.f), 448.f);
    const float yb = fminf(fmaxf(b * r, -448.f), 448.f);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false)) & 0xFFFFu;
  }
};
// Codes of four bf16 values (the 16-bit halves of w, low first): byte i = value i.
template <typename Code>
__device__ inline uint32_t encode4_bf16(uint2 w, float r) {
  const float a = __uint_as_float(w.x << 16), b = __uint_as_float(w.x & 0xFFFF0000u);
  const float c = __uint_as_float(w.y << 16), e = __uint_as_float(w.y & 0xFFFF0000u);
  return Encode<Code>::pair(a, b, r) | (Encode<Code>::pair(c, e, r) << 16);
}

// Element offsets inside one (block, kv-head) tile of D*16 elements.
//   K tile: [D/x][16][x]
//   V tile: [16/x][D][x]  (tokens 0..x-1 as D rows of x tokens, then the
//           next x tokens): one 16-byte load gives x consecutive tokens of a dim.
template <typename T>
__device__ __host__ inline int64_t k_elem(int t, int d) {
  return (static_cast<int64_t>(d / T::kVecElems) * kBlockSize + t) * T::kVecElems +
         d % T::kVecElems;
}
template <typename T>
__device__ __host__ inline int64_t v_elem(int t, int d, int D) {
  return (static_cast<int64_t>(t / T::kVecElems) * D + d) * T::kVecElems + t % T::kVecElems;
}
// First element of the (block, kv-head) tile.
__device__ __host__ inline int64_t tile_base(int64_t block, int head, int num_kv_heads, int D) {
  return (block * num_kv_heads + head) * static_cast<int64_t>(D) * kBlockSize;
}

inline bool code_dtype(pa_dtype dt) { return dt == PA_FP8_E4M3 || dt == PA_INT8; }
inline size_t dtype_bytes(pa_dtype dt) { return dt == PA_F32 ? 4 : code_dtype(dt) ? 1 : 2; }
// floating-point element dtypes (K/V values stored as they are)
inline bool dtype_ok(pa_dtype dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }
// any pool dtype: values or 8-bit codes
inline bool pool_dtype_ok(pa_dtype dt) { return dtype_ok(dt) || code_dtype(dt); }

// Converts the state after a launch into a status.
inline pa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace pa
