// Batched 2-D transpose for the backward GEMMs. The m-grouped dgrad and the k-grouped
// wgrad ("Expert Parallelism (EP)", section 5) read both operands K-contiguous, so the
// weights enter the dgrad transposed (w2 [E,D,F] -> [E,F,D]; w1, w3 [E,F,D] -> the two
// halves of [E,D,2F]) and the activations enter the wgrad transposed ([rows, N] -> [N, rows]).
//
// dst[b][c][col0 + r] = src[b][r][c] for r < rows, zero for rows <= r < roundup(rows, 64);
// columns from roundup(rows, 64) on are not written. A workgroup moves one 64 x 64 tile:
// coalesced 16-byte loads of source rows into LDS, then 16-byte stores of destination rows,
// each gathered from one LDS column (the row pitch is padded by one 4-byte word, so the
// eight lanes that share a column group fall in distinct banks).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int TT = 64;        // tile edge
constexpr int kThreads = 256;

template <typename TE>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const TE* __restrict__ src, int R,
                                                             int C, int rows_src,
                                                             const int32_t* __restrict__ nrows_dev,
                                                             TE* __restrict__ dst, int64_t ld_dst,
                                                             int64_t col0) {
  constexpr int V = 16 / sizeof(TE);        // elements per 16-byte chunk
  constexpr int PITCH = TT + 4 / sizeof(TE);  // LDS row pitch in elements
  __shared__ __attribute__((aligned(16))) TE tile[TT * PITCH];
  int rows = rows_src;
  if (nrows_dev) rows = max(0, min(rows, *nrows_dev));
  const int r0 = blockIdx.y * TT, c0 = blockIdx.x * TT;
  if (r0 >= rows) return;
  const int b = blockIdx.z;
  const TE* s = src + (size_t)b * R * C;
  constexpr int CPR = TT / V;   // chunks per tile row
  for (int q = threadIdx.x; q < TT * CPR; q += kThreads) {
    const int r = q / CPR, cc = (q % CPR) * V;
    TE v[V];
    if (r0 + r < rows) {
      const u32x4 raw = ld16(s + (size_t)(r0 + r) * C + c0 + cc);
      __builtin_memcpy(v, &raw, 16);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = TE(0);
    }
#pragma unroll
    for (int e = 0; e < V; ++e) tile[r * PITCH + cc + e] = v[e];
  }
  __syncthreads();
  TE* d = dst + (size_t)b * C * ld_dst;
  for (int q = threadIdx.x; q < TT * CPR; q += kThreads) {
    const int c = q / CPR, rc = (q % CPR) * V;
    TE v[V];
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = tile[(rc + e) * PITCH + c];
    u32x4 raw;
    __builtin_memcpy(&raw, v, 16);
    st16(d + (size_t)(c0 + c) * ld_dst + col0 + r0 + rc, raw);
  }
}

}  // namespace

hipError_t launch_transpose(int dt, const void* src, int batch, int R, int C, int rows_src,
                            const int32_t* nrows_dev, void* dst, int64_t ld_dst, int64_t col0,
                            hipStream_t s) {
  const dim3 grid(C / TT, R / TT, batch), block(kThreads);
  if (dt == kF32)
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, static_cast<const float*>(src),
                       R, C, rows_src, nrows_dev, static_cast<float*>(dst), ld_dst, col0);
  else
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, block, 0, s,
                       static_cast<const bf16_t*>(src), R, C, rows_src, nrows_dev,
                       static_cast<bf16_t*>(dst), ld_dst, col0);
  return hipGetLastError();
}

}  // namespace moe
