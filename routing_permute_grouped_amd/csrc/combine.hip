// Combine: unpermute and top-k-weighted reduce back to token order, plus the
// shared experts ("Expert Parallelism (EP)", llm-infra-atlas, section 1 "MoE layer 的 forward 通路", its forward-path figure:
// the combine stage after the expert GEMMs, which restores token order and weights
// each expert row by its top-k probability, and the shared experts added to the
// output; section 5: the unpermute is the transpose of the permute).
//
// Each token's k expert rows are gathered by 16-byte chunks and reduced in float32
// in slot order; the shared row is added last and the sum is rounded once. A thread
// takes one chunk at a time and keeps its reads of up to four slots in flight. Without weights the same
// kernel is the plain unpermute-and-sum, which is also the backward of the permute
// (section 5: the permute's mirror is a scatter_add).
//
// The backward of the combine (section 5: the mirror of unpermute-and-reduce is a
// dispatch) runs over the rows of the permuted buffer: the row holding slot
// s = t*k + j gets dy = topk_w[s] * dout[t], rounded once, and the slot's weight
// gradient <dout[t], y_perm[row]> is reduced by the row's wave in a fixed order; pad
// rows get zeros, so the grouped GEMMs of the backward see exact zeros there.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokens = 4;
constexpr int kMaxK = 32;
constexpr int kU = 1;   // 16-byte chunks per thread (more registers per thread cost more
                        // than they give: at most 64 VGPRs keeps 8 waves per SIMD)
constexpr int kJ = 4;   // slots whose reads of those chunks are in flight together
constexpr int kUB = 4;  // the backward's chunks in flight per lane (each with two reads)

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
    ws[i] = w ? w[(size_t)t_begin * k + i] : 1.0f;   // no weights: the plain unpermute
  }
  __syncthreads();
  const int nck = D / V;
  const int total = ntok * nck;
  // kU chunks per thread, the reads of kJ slots in flight together
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
    for (int j0 = 0; j0 < k; j0 += kJ) {
      u32x4 yv[kJ][kU];
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) {
        const int j = j0 + jj;
        if (j >= k) break;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int d = ds[tl[u] * k + j];
          if (d >= 0) yv[jj][u] = ld16_nt(y + (size_t)d * D + (size_t)cc[u] * V);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) {
        const int j = j0 + jj;
        if (j >= k) break;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int d = ds[tl[u] * k + j];
          if (d < 0) continue;
          const float wj = ws[tl[u] * k + j];
          float f[V];
          Chunk<TIn>::widen(yv[jj][u], f);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[u][v] = __builtin_fmaf(wj, f[v], acc[u][v]);
        }
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

// One wave per row of the permuted buffer, rows [0, min(offsets[E], m_cap)); each lane
// takes 16-byte chunks lane, lane+64, ... in increasing order, kUB of them in flight.
// The dot product is summed per lane in chunk order, then over lanes by an xor
// butterfly (every lane ends with the same value, lane 0 stores it).
template <typename TIn>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(
    const TIn* __restrict__ dout, const TIn* __restrict__ y, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ dst_row,
    const float* __restrict__ w, int T, int D, int E, int k, int64_t m_cap, TIn* __restrict__ dy,
    float* __restrict__ dw) {
  constexpr int V = Chunk<TIn>::V;
  const int lane = threadIdx.x & 63;
  const int64_t mend = max((int64_t)0, min((int64_t)offsets[E], m_cap));
  const int64_t nslots = (int64_t)T * k;
  const int nck = D / V;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < mend;
       r += waves) {
    const int s = src_row[r];
    TIn* drow = dy + r * D;
    if (s < 0 || s >= nslots) {   // pad row
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int c = lane; c < nck; c += 64) st16(drow + (size_t)c * V, z);
      continue;
    }
    const TIn* g = dout + (size_t)(s / k) * D;
    const TIn* yr = y + r * D;
    const float wj = w[s];
    float acc = 0.0f;
    for (int c0 = lane; c0 < nck; c0 += 64 * kUB) {
      u32x4 gv[kUB], yv[kUB];
#pragma unroll
      for (int u = 0; u < kUB; ++u) {
        const int c = c0 + 64 * u;
        if (c < nck) {
          gv[u] = ld16(g + (size_t)c * V);
          yv[u] = ld16_nt(yr + (size_t)c * V);
        }
      }
#pragma unroll
      for (int u = 0; u < kUB; ++u) {
        const int c = c0 + 64 * u;
        if (c >= nck) continue;
        float gf[V], yf[V], o[V];
        Chunk<TIn>::widen(gv[u], gf);
        Chunk<TIn>::widen(yv[u], yf);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          acc = __builtin_fmaf(gf[v], yf[v], acc);
          o[v] = wj * gf[v];
        }
        st16(drow + (size_t)c * V, Chunk<TIn>::narrow(o));
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) dw[s] = acc;
  }
  // slots that no row holds (skipped, or outside the rows in use) have zero gradient
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nslots;
       i += (int64_t)gridDim.x * kThreads) {
    const int d = dst_row[i];
    if (d < 0 || d >= mend) dw[i] = 0.0f;
  }
}

}  // namespace

hipError_t launch_combine_backward(int dt, const void* dout, const void* y_perm,
                                   const int32_t* src_row, const int32_t* offsets,
                                   const int32_t* dst_row, const float* topk_w, int T, int D, int E,
                                   int k, int64_t m_cap, void* dy_perm, float* dtopk_w,
                                   hipStream_t s) {
  const int64_t want = (m_cap + 3) / 4;
  const dim3 grid((unsigned)std::min<int64_t>(want, 16 * cu_count())), block(kThreads);
  if (dt == kF32)
    hipLaunchKernelGGL(combine_bwd_kernel<float>, grid, block, 0, s,
                       static_cast<const float*>(dout), static_cast<const float*>(y_perm), src_row,
                       offsets, dst_row, topk_w, T, D, E, k, m_cap, static_cast<float*>(dy_perm),
                       dtopk_w);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<bf16_t>, grid, block, 0, s,
                       static_cast<const bf16_t*>(dout), static_cast<const bf16_t*>(y_perm),
                       src_row, offsets, dst_row, topk_w, T, D, E, k, m_cap,
                       static_cast<bf16_t*>(dy_perm), dtopk_w);
  return hipGetLastError();
}

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
