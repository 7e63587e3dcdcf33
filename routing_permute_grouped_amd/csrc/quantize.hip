// MX quantization of the FP8 payload ("Expert Parallelism (EP)", llm-infra-atlas,
// section 6 "DeepSeek-V3 量级的示例数字": the dispatch payload is FP8 e4m3 with
// scales, the combine stays in BF16).
//
// Every 32 consecutive values of a row share one power-of-two scale 2^X, stored as the
// E8M0 byte X + 127: X is the smallest integer with max|v| <= 448 * 2^X (448 is the
// largest OCP E4M3 value), so no value saturates, and -127 for an all-zero block. Each
// value becomes the e4m3 code of v / 2^X rounded to nearest, ties to even. One thread
// per block: the scale comes from frexp of the block's max (exact), the division by 2^X
// is an exact ldexp, and the rounding to e4m3 is done on the float32 bits. The scale
// bytes go row by row ([R, C/32]) or in k-step words ([C/128][R] words of 4 bytes, byte
// j of word (s, r) for block 4*s + j of row r), the layout the fc1 GEMM reads.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

// e4m3 code of a float32 value with |v| <= 448: subnormal codes below 2^-6 (steps of
// 2^-9), otherwise the 3-bit mantissa rounded to nearest even (a carry moves to the next
// exponent, which the code layout absorbs). The sign is kept, -0 included.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {                                   // 2^-6
    code = (uint32_t)rintf(a * 512.0f);                  // 0..8; 8 is 2^-6 itself
  } else {
    int e;
    const float m = frexpf(a, &e);                       // a = m * 2^e, 0.5 <= m < 1
    const uint32_t q = (uint32_t)rintf((2.0f * m - 1.0f) * 8.0f);   // 0..8
    code = ((uint32_t)(e - 1 + 7) << 3) + q;
  }
  return sign | code;
}

template <typename TIn, bool KSTEPS>
__global__ __launch_bounds__(kThreads) void quantize_mx_kernel(const TIn* __restrict__ x,
                                                              int64_t nblocks, int64_t R, int C,
                                                              uint8_t* __restrict__ q,
                                                              uint8_t* __restrict__ scales) {
  constexpr int V = Chunk<TIn>::V;   // values per 16-byte chunk
  constexpr int NC = 32 / V;         // chunks per block
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * kThreads) {
    const TIn* src = x + b * 32;     // rows are C values long and C % 32 == 0
    float v[32];
#pragma unroll
    for (int c = 0; c < NC; ++c) Chunk<TIn>::widen(ld16(src + c * V), v + c * V);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int X = -127;
    if (amax > 0.0f) {
      int e;
      const float m = 2.0f * frexpf(amax, &e);           // amax = m * 2^(e-1), 1 <= m < 2
      X = (m <= 1.75f) ? (e - 1) - 8 : (e - 1) - 7;
      X = max(-127, min(127, X));
    }
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w[i] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[i] |= e4m3_code(ldexpf(v[4 * i + j], -X)) << (8 * j);
    }
    st16(q + b * 32, u32x4{w[0], w[1], w[2], w[3]});
    st16(q + b * 32 + 16, u32x4{w[4], w[5], w[6], w[7]});
    if (KSTEPS) {
      const int nb = C / 32;
      const int64_t r = b / nb;
      const int blk = (int)(b - r * nb);
      scales[((int64_t)(blk >> 2) * R + r) * 4 + (blk & 3)] = (uint8_t)(X + 127);
    } else {
      scales[b] = (uint8_t)(X + 127);
    }
  }
}

// float32 -> bf16 with the rounding of every bf16 store (f32_to_bf16)
__global__ __launch_bounds__(kThreads) void round_bf16_kernel(const float* __restrict__ x,
                                                             uint16_t* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    y[i] = (uint16_t)f32_to_bf16(x[i]);
}

}  // namespace

template <typename TIn>
void launch_quantize_t(const void* x, int64_t R, int C, void* q, void* scales, bool ksteps,
                       hipStream_t s) {
  const int64_t nblocks = R * (C / 32);
  const int grid = (int)std::min<int64_t>(8 * cu_count(), (nblocks + kThreads - 1) / kThreads);
  auto kern = ksteps ? quantize_mx_kernel<TIn, true> : quantize_mx_kernel<TIn, false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, s, static_cast<const TIn*>(x),
                     nblocks, R, C, static_cast<uint8_t*>(q), static_cast<uint8_t*>(scales));
}

hipError_t launch_round_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(8 * cu_count(), (n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(round_bf16_kernel, dim3(grid), dim3(kThreads), 0, s, x, y, n);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(int dt, const void* x, int64_t R, int C, void* q, void* scales,
                              bool ksteps, hipStream_t s) {
  if (dt == kF32)
    launch_quantize_t<float>(x, R, C, q, scales, ksteps, s);
  else
    launch_quantize_t<bf16_t>(x, R, C, q, scales, ksteps, s);
  return hipGetLastError();
}

}  // namespace moe
