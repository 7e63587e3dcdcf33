// Device helpers shared by the HIP kernels of the MoE layer path (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // bf16 stored as its bit pattern
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32, which the __bf16
// conversion compiles to). NaN stays a quiet NaN.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Low and high bf16 of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_hw v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte chunk as 4 or 8 floats.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int V = 4;
  __device__ __forceinline__ static void widen(const u32x4& c, float* out) {
    out[0] = __uint_as_float(c.x); out[1] = __uint_as_float(c.y);
    out[2] = __uint_as_float(c.z); out[3] = __uint_as_float(c.w);
  }
  __device__ __forceinline__ static u32x4 narrow(const float* in) {
    return u32x4{__float_as_uint(in[0]), __float_as_uint(in[1]),
                 __float_as_uint(in[2]), __float_as_uint(in[3])};
  }
};
template <> struct Chunk<bf16_t> {
  static constexpr int V = 8;
  __device__ __forceinline__ static void widen(const u32x4& c, float* out) {
    out[0] = bf16_lo(c.x); out[1] = bf16_hi(c.x); out[2] = bf16_lo(c.y); out[3] = bf16_hi(c.y);
    out[4] = bf16_lo(c.z); out[5] = bf16_hi(c.z); out[6] = bf16_lo(c.w); out[7] = bf16_hi(c.w);
  }
  __device__ __forceinline__ static u32x4 narrow(const float* in) {
    return u32x4{pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                 pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7])};
  }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Non-temporal variants for streams touched once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

}  // namespace moe
