// Router gating and softmax-then-top-k routing ("Expert Parallelism (EP)",
// llm-infra-atlas, section 1: router.gating logits = x @ W_g^T over [T, E], then
// routing = top-k + score function -> probs and routing map).
//
// One wave handles 8 tokens. For each pass over 8 experts, lane l accumulates the
// 16-byte chunks c = l, l+64, ... of x[t] . wg[e] for the 8x8 (token, expert)
// pairs, in increasing d. The 64 lane partials of all 64 pairs are then combined
// with a recursive-halving exchange whose additions are exactly those of a
// butterfly over lane distances 32, 16, 8, 4, 2, 1 (each pair's partials meet in
// the same tree), ending with pair p's logit in lane p. This fixed float32 order
// is what makes the top-k choice reproducible bit for bit.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kTokPerWave = 8;
constexpr int kExpPerPass = 8;
static_assert(kTokPerWave * kExpPerPass == kWave, "one (token, expert) pair per lane");

// float32: a rounded multiply followed by a rounded add (no contraction).
__device__ __forceinline__ void dot_step(float& acc, float a, float b, float) {
#pragma clang fp contract(off)
  const float p = a * b;
  acc = acc + p;
}
// bf16 inputs: the product of two bf16 values is exact in float32 (unless it
// underflows), so a fused multiply-add rounds exactly like multiply-then-add.
__device__ __forceinline__ void dot_step(float& acc, float a, float b, bf16_t) {
  acc = __builtin_fmaf(a, b, acc);
}

// One recursive-halving step: lanes keep the half of the pairs whose bit log2(M)
// matches their own and add the partner's partial of the same pairs.
template <int M>
__device__ __forceinline__ void halve(float (&v)[kWave], bool upper) {
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const float send = upper ? v[i] : v[i + M];
    const float keep = upper ? v[i + M] : v[i];
    v[i] = keep + __shfl_xor(send, M);
  }
}

// Recursive halving over distances 32..1: lane l ends with pair l's full sum.
__device__ __forceinline__ float reduce_pairs(float (&v)[kWave], int lane) {
  halve<32>(v, lane & 32);
  halve<16>(v, lane & 16);
  halve<8>(v, lane & 8);
  halve<4>(v, lane & 4);
  halve<2>(v, lane & 2);
  halve<1>(v, lane & 1);
  return v[0];
}

template <typename TIn>
__global__ __launch_bounds__(kWave) void route_kernel(const TIn* __restrict__ x,
                                                      const TIn* __restrict__ wg,
                                                      const float* __restrict__ bias, int T, int D,
                                                      int E, int k, int renorm,
                                                      int32_t* __restrict__ topk_idx,
                                                      float* __restrict__ topk_w,
                                                      float* __restrict__ logits_out) {
  constexpr int V = Chunk<TIn>::V;
  __shared__ float lg[kTokPerWave][kWave];
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * kTokPerWave;
  const int nchunk = D / V;

  for (int e0 = 0; e0 < E; e0 += kExpPerPass) {
    float acc[kWave];
#pragma unroll
    for (int p = 0; p < kWave; ++p) acc[p] = 0.0f;
    for (int c = lane; c < nchunk; c += kWave) {
      float xv[kTokPerWave][V];
#pragma unroll
      for (int t = 0; t < kTokPerWave; ++t) {
        const int tok = min(t0 + t, T - 1);
        Chunk<TIn>::widen(ld16(x + (size_t)tok * D + (size_t)c * V), xv[t]);
      }
#pragma unroll
      for (int e = 0; e < kExpPerPass; ++e) {
        const int ee = min(e0 + e, E - 1);
        float wv[V];
        Chunk<TIn>::widen(ld16(wg + (size_t)ee * D + (size_t)c * V), wv);
#pragma unroll
        for (int t = 0; t < kTokPerWave; ++t)
#pragma unroll
          for (int i = 0; i < V; ++i) dot_step(acc[t * kExpPerPass + e], xv[t][i], wv[i], TIn());
      }
    }
    float logit = reduce_pairs(acc, lane);
    const int t = lane / kExpPerPass;
    const int e = e0 + lane % kExpPerPass;
    if (e < E) {
      if (bias) logit = logit + bias[e];
      lg[t][e] = logit;
    }
  }
  __syncthreads();

  for (int t = 0; t < kTokPerWave; ++t) {
    const int tok = t0 + t;
    if (tok >= T) break;
    const bool have = lane < E;
    const float l = have ? lg[t][lane] : -INFINITY;
    if (logits_out && have) logits_out[(size_t)tok * E + lane] = l;
    float mx = l;
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    const float ex = have ? expf(l - mx) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);

    bool avail = have;
    int my_idx = 0;
    float my_w = 0.0f, wtot = 0.0f;
    for (int j = 0; j < k; ++j) {
      float key = avail ? l : -INFINITY;
      int id = avail ? lane : 0x7fffffff;
#pragma unroll
      for (int m = kWave / 2; m >= 1; m >>= 1) {
        const float ok = __shfl_xor(key, m);
        const int oi = __shfl_xor(id, m);
        if (ok > key || (ok == key && oi < id)) {
          key = ok;
          id = oi;
        }
      }
      if (lane == id) avail = false;
      const float wj = __shfl(ex, id) / sum;
      wtot += wj;
      if (lane == j) {
        my_idx = id;
        my_w = wj;
      }
    }
    if (lane < k) {
      topk_idx[(size_t)tok * k + lane] = my_idx;
      topk_w[(size_t)tok * k + lane] = renorm ? my_w / wtot : my_w;
    }
  }
}

}  // namespace

hipError_t launch_route(int dt, const void* x, const void* wg, const float* bias, int T, int D,
                        int E, int k, int renorm, int32_t* topk_idx, float* topk_w, float* logits,
                        hipStream_t s) {
  const dim3 grid((T + kTokPerWave - 1) / kTokPerWave), block(kWave);
  if (dt == kF32)
    hipLaunchKernelGGL(route_kernel<float>, grid, block, 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(wg), bias, T, D, E, k, renorm, topk_idx, topk_w,
                       logits);
  else
    hipLaunchKernelGGL(route_kernel<bf16_t>, grid, block, 0, s, static_cast<const bf16_t*>(x),
                       static_cast<const bf16_t*>(wg), bias, T, D, E, k, renorm, topk_idx, topk_w,
                       logits);
  return hipGetLastError();
}

}  // namespace moe
