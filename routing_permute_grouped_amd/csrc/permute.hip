// Dispatch metadata and permute ("Expert Parallelism (EP)", llm-infra-atlas:
// section 1 "preprocess: tokens_per_expert" and "permute: sort local tokens by
// expert so each local expert's tokens are contiguous"; section 2: the output
// layout must be expert-contiguous with every segment aligned to the GEMM M tile).
//
// Three launches:
//   1. hist_kernel     per 256-token block, slots of each expert (LDS atomics: the
//                      counts do not depend on their order)
//   2. scan_kernel     one workgroup: per-expert exclusive scan over the blocks,
//                      counts, padded offsets, tile -> expert map, error flag
//   3. scatter_kernel  per 16-token block: stable ranks of its slots (ballot match
//                      inside a wave, blocks in order), dst_row/src_row, then each
//                      token row is read once and written to its k rows; extra
//                      blocks zero the pad rows of every segment and mark unused rows
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kMaxK = 32;
constexpr int kCopyTokens = 16;
constexpr int kThreads = 256;
static_assert(kHistTokens % kCopyTokens == 0, "copy blocks nest in histogram blocks");

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx, int T,
                                                        int k, int E, int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ bad) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int nbad;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  if (threadIdx.x == 0) nbad = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kHistTokens * k;
  const int64_t a1 = min(a0 + (int64_t)kHistTokens * k, (int64_t)T * k);
  for (int64_t a = a0 + threadIdx.x; a < a1; a += kThreads) {
    const int e = idx[a];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else if (e != -1)
      atomicAdd(&nbad, 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) hist[(size_t)blockIdx.x * E + e] = cnt[e];
  if (threadIdx.x == 0) bad[blockIdx.x] = nbad;
}

// Exclusive scan over the 1024 threads of the block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wsum[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    int s = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int o = __shfl_up(s, d);
      if (lane >= d) s += o;
    }
    if (lane < 16) wsum[lane] = s;  // inclusive totals of waves 0..lane
  }
  __syncthreads();
  return inc - v + (wid ? wsum[wid - 1] : 0);
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ hist,
                                                    const int32_t* __restrict__ bad, int nbh, int E,
                                                    int m_tile, int64_t m_cap,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ tile_expert,
                                                    int32_t* __restrict__ dev_err) {
  __shared__ int off[kMaxExperts + 1];
  __shared__ int wsum[16];
  __shared__ int anybad;
  const int tid = threadIdx.x;
  if (tid == 0) anybad = 0;
  int padded = 0;
  if (tid < E) {
    int run = 0;
    for (int b = 0; b < nbh; ++b) {
      const int c = hist[(size_t)b * E + tid];
      hist[(size_t)b * E + tid] = run;
      run += c;
    }
    counts[tid] = run;
    padded = (run + m_tile - 1) / m_tile * m_tile;
  }
  const int ex = block_exclusive_scan(padded, wsum);
  if (tid < E) off[tid] = ex;
  if (tid == E - 1) off[E] = ex + padded;
  for (int b = tid; b < nbh; b += 1024)
    if (bad[b]) anybad = 1;
  __syncthreads();
  if (tid == 0) *dev_err = anybad;
  for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];
  const int total = off[E];
  const int64_t ntiles = m_cap / m_tile;
  for (int64_t q = tid; q < ntiles; q += 1024) {
    const int64_t r = q * m_tile;
    int owner = -1;
    if (r < total) {
      int lo = 0, hi = E;  // largest e with off[e] <= r
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid;
      }
      owner = lo;
    }
    tile_expert[q] = owner;
  }
}

template <typename TIn>
__global__ __launch_bounds__(kThreads) void scatter_kernel(
    const TIn* __restrict__ x, const int32_t* __restrict__ idx, int T, int D, int k, int E,
    int64_t m_cap, const int32_t* __restrict__ hist_base, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ dst_row,
    int32_t* __restrict__ src_row, TIn* __restrict__ x_perm) {
  constexpr int V = Chunk<TIn>::V;
  const int nck = D / V;
  const int nbc = (T + kCopyTokens - 1) / kCopyTokens;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;

  if (b >= nbc) {
    if (b < nbc + E) {  // zero the pad rows of segment e and mark them unused
      const int e = b - nbc;
      const int r0 = offsets[e] + counts[e], r1 = offsets[e + 1];
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int64_t i = tid; i < (int64_t)(r1 - r0) * nck; i += kThreads) {
        const int64_t r = r0 + i / nck, c = i % nck;
        st16(x_perm + r * D + c * V, z);
      }
      for (int r = r0 + tid; r < r1; r += kThreads) src_row[r] = -1;
    } else {  // rows past the last segment hold no slot
      for (int64_t r = offsets[E] + tid; r < m_cap; r += kThreads) src_row[r] = -1;
    }
    return;
  }

  __shared__ int base[kMaxExperts];
  __shared__ int dsts[kCopyTokens * kMaxK];
  const int t_begin = b * kCopyTokens;
  const int t_end = min(T, t_begin + kCopyTokens);
  const int hb = t_begin / kHistTokens;
  for (int e = tid; e < E; e += kThreads) base[e] = offsets[e] + hist_base[(size_t)hb * E + e];
  __syncthreads();
  // slots of this histogram block that precede this copy block
  for (int64_t a = (int64_t)hb * kHistTokens * k + tid; a < (int64_t)t_begin * k; a += kThreads) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&base[e], 1);
  }
  __syncthreads();

  const int n = (t_end - t_begin) * k;
  const int64_t a0 = (int64_t)t_begin * k;
  if (tid < kWave) {
    const int lane = tid;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int r0 = 0; r0 < n; r0 += kWave) {
      const int a = r0 + lane;
      const int e = a < n ? idx[a0 + a] : -1;
      const bool valid = a < n && e >= 0 && e < E;
      uint64_t same = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool on = valid && ((e >> bit) & 1);
        const uint64_t bal = __ballot(on);
        same &= ((e >> bit) & 1) ? bal : ~bal;
      }
      int pos = -1;
      if (valid) pos = base[e] + __popcll(same & lt);
      if (pos >= m_cap) pos = -1;  // cannot happen with consistent counts; never write past m_cap
      __builtin_amdgcn_wave_barrier();
      if (valid && (same >> lane) == 1ull) base[e] = base[e] + __popcll(same);
      __builtin_amdgcn_wave_barrier();
      if (a < n) {
        dsts[a] = pos;
        dst_row[a0 + a] = pos;
        if (pos >= 0) src_row[pos] = (int32_t)(a0 + a);
      }
    }
  }
  __syncthreads();

  const int ntok = t_end - t_begin;
  for (int i = tid; i < ntok * nck; i += kThreads) {
    const int tl = i / nck, c = i - tl * nck;
    const u32x4 v = ld16(x + (size_t)(t_begin + tl) * D + (size_t)c * V);
    for (int j = 0; j < k; ++j) {
      const int d = dsts[tl * k + j];
      if (d >= 0) st16(x_perm + (size_t)d * D + (size_t)c * V, v);
    }
  }
}

}  // namespace

size_t permute_workspace_bytes(int T, int k, int E) {
  (void)k;
  const size_t nbh = (size_t)(T + kHistTokens - 1) / kHistTokens;
  return nbh * ((size_t)E + 1) * sizeof(int32_t);
}

hipError_t launch_permute(int dt, const void* x, const int32_t* topk_idx, int T, int D, int E,
                          int k, int m_tile, int64_t m_cap, void* x_perm, int32_t* counts,
                          int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                          int32_t* tile_expert, void* workspace, int32_t* dev_err, hipStream_t s) {
  const int nbh = (T + kHistTokens - 1) / kHistTokens;
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* bad = hist + (size_t)nbh * E;
  hipLaunchKernelGGL(hist_kernel, dim3(nbh), dim3(kThreads), 0, s, topk_idx, T, k, E, hist, bad);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, hist, bad, nbh, E, m_tile, m_cap,
                     counts, offsets, tile_expert, dev_err);
  const int nbc = (T + kCopyTokens - 1) / kCopyTokens;
  const dim3 grid(nbc + E + 1);
  if (dt == kF32)
    hipLaunchKernelGGL(scatter_kernel<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(x), topk_idx, T, D, k, E, m_cap, hist, counts,
                       offsets, dst_row, src_row, static_cast<float*>(x_perm));
  else
    hipLaunchKernelGGL(scatter_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(x), topk_idx, T, D, k, E, m_cap, hist, counts,
                       offsets, dst_row, src_row, static_cast<bf16_t*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
