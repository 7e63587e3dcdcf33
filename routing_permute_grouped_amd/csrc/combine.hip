// Combine: unpermute and top-k-weighted reduce back to token order, plus the
// shared experts ("Expert Parallelism (EP)", llm-infra-atlas, section 1:
// combine_postprocess "unpermute-1, reduce back to the original order weighted by
// the top-k weights", output "+ shared expert"; section 5: the unpermute is the
// transpose of the permute).
//
// Each token's k expert rows are gathered by 16-byte chunks and reduced in float32
// in slot order; the shared row is added last and the sum is rounded once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokens = 4;
constexpr int kMaxK = 32;

template <typename TIn>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const TIn* __restrict__ y, const int32_t* __restrict__ dst_row, const float* __restrict__ w,
    const TIn* __restrict__ shared, int T, int D, int k, int64_t m_cap, TIn* __restrict__ out) {
  constexpr int V = Chunk<TIn>::V;
  __shared__ int ds[kTokens * kMaxK];
  __shared__ float ws[kTokens * kMaxK];
  const int t_begin = blockIdx.x * kTokens;
  const int ntok = min(kTokens, T - t_begin);
  for (int i = threadIdx.x; i < ntok * k; i += kThreads) {
    const int d = dst_row[(size_t)t_begin * k + i];
    ds[i] = (d >= 0 && d < m_cap) ? d : -1;
    ws[i] = w[(size_t)t_begin * k + i];
  }
  __syncthreads();
  const int nck = D / V;
  for (int i = threadIdx.x; i < ntok * nck; i += kThreads) {
    const int tl = i / nck, c = i - tl * nck;
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int d = ds[tl * k + j];
      if (d < 0) continue;
      const float wj = ws[tl * k + j];
      float yv[V];
      Chunk<TIn>::widen(ld16(y + (size_t)d * D + (size_t)c * V), yv);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = __builtin_fmaf(wj, yv[v], acc[v]);
    }
    const size_t o = (size_t)(t_begin + tl) * D + (size_t)c * V;
    if (shared) {
      float sv[V];
      Chunk<TIn>::widen(ld16(shared + o), sv);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] += sv[v];
    }
    st16(out + o, Chunk<TIn>::narrow(acc));
  }
}

}  // namespace

hipError_t launch_combine(int dt, const void* y_perm, const int32_t* dst_row, const float* topk_w,
                          const void* shared, int T, int D, int k, int64_t m_cap, void* out,
                          hipStream_t s) {
  const dim3 grid((T + kTokens - 1) / kTokens), block(kThreads);
  if (dt == kF32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, static_cast<const float*>(y_perm),
                       dst_row, topk_w, static_cast<const float*>(shared), T, D, k, m_cap,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, block, 0, s,
                       static_cast<const bf16_t*>(y_perm), dst_row, topk_w,
                       static_cast<const bf16_t*>(shared), T, D, k, m_cap,
                       static_cast<bf16_t*>(out));
  return hipGetLastError();
}

}  // namespace moe
