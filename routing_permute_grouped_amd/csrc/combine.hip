// Combine: unpermute and top-k-weighted reduce back to token order, plus the
// shared experts ("Expert Parallelism (EP)", llm-infra-atlas, section 1:
// combine_postprocess "unpermute-1, reduce back to the original order weighted by
// the top-k weights", output "+ shared expert"; section 5: the unpermute is the
// transpose of the permute).
//
// Each token's k expert rows are gathered by 16-byte chunks and reduced in float32
// in slot order; the shared row is added last and the sum is rounded once. Every
// thread keeps four chunks' row reads in flight per slot.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokens = 4;
constexpr int kMaxK = 32;
constexpr int kU = 4;   // 16-byte chunks per thread whose reads are in flight together

template <typename TIn>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const TIn* __restrict__ y, const int32_t* __restrict__ dst_row, const float* __restrict__ w,
    const TIn* __restrict__ shared, int T, int D, int k, int64_t m_cap, int tpb,
    TIn* __restrict__ out) {
  constexpr int V = Chunk<TIn>::V;
  __shared__ int ds[kTokens * kMaxK];
  __shared__ float ws[kTokens * kMaxK];
  const int t_begin = blockIdx.x * tpb;
  const int ntok = min(tpb, T - t_begin);
  for (int i = threadIdx.x; i < ntok * k; i += kThreads) {
    const int d = dst_row[(size_t)t_begin * k + i];
    ds[i] = (d >= 0 && d < m_cap) ? d : -1;
    ws[i] = w[(size_t)t_begin * k + i];
  }
  __syncthreads();
  const int nck = D / V;
  const int total = ntok * nck;
  // kU chunks per thread: for each slot j their kU row reads are in flight together
  for (int i0 = threadIdx.x; i0 < total; i0 += kThreads * kU) {
    float acc[kU][V];
    int tl[kU], cc[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(i0 + u * kThreads, total - 1);
      tl[u] = i / nck;
      cc[u] = i - tl[u] * nck;
#pragma unroll
      for (int v = 0; v < V; ++v) acc[u][v] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
      u32x4 yv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int d = ds[tl[u] * k + j];
        if (d >= 0) yv[u] = ld16_nt(y + (size_t)d * D + (size_t)cc[u] * V);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int d = ds[tl[u] * k + j];
        if (d < 0) continue;
        const float wj = ws[tl[u] * k + j];
        float f[V];
        Chunk<TIn>::widen(yv[u], f);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[u][v] = __builtin_fmaf(wj, f[v], acc[u][v]);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (i0 + u * kThreads >= total) continue;
      const size_t o = (size_t)(t_begin + tl[u]) * D + (size_t)cc[u] * V;
      if (shared) {
        float sv[V];
        Chunk<TIn>::widen(ld16_nt(shared + o), sv);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[u][v] += sv[v];
      }
      st16(out + o, Chunk<TIn>::narrow(acc[u]));
    }
  }
}

}  // namespace

hipError_t launch_combine(int dt, const void* y_perm, const int32_t* dst_row, const float* topk_w,
                          const void* shared, int T, int D, int k, int64_t m_cap, void* out,
                          hipStream_t s) {
  // tokens per workgroup: up to kTokens, fewer when that leaves the grid too small
  int tpb = kTokens;
  while (tpb > 1 && (T + tpb - 1) / tpb < 8 * cu_count()) tpb >>= 1;
  const dim3 grid((T + tpb - 1) / tpb), block(kThreads);
  if (dt == kF32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, static_cast<const float*>(y_perm),
                       dst_row, topk_w, static_cast<const float*>(shared), T, D, k, m_cap, tpb,
                       static_cast<float*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, block, 0, s,
                       static_cast<const bf16_t*>(y_perm), dst_row, topk_w,
                       static_cast<const bf16_t*>(shared), T, D, k, m_cap, tpb,
                       static_cast<bf16_t*>(out));
  return hipGetLastError();
}

}  // namespace moe
