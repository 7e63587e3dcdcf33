// Router gating and softmax-then-top-k routing ("Expert Parallelism (EP)",
// llm-infra-atlas, section 1 "MoE layer 的 forward 通路", its forward-path figure: the gate
// scores every token against every expert, then a score function and a top-k pick
// each token's experts and their weights).
//
// A pass covers TW tokens x EC experts: lane l accumulates the 16-byte chunks
// c = l, l+64, ... of x[t] . wg[e] for the TW*EC (token, expert) pairs, in increasing d.
// With at most 8 experts every wave takes its own 2 tokens and does the one pass.
// With more, the 4 waves of a block share 8 tokens (every gate-weight chunk a wave
// reads serves 8 tokens) and take the passes over the experts in turn, so there are
// four times as many waves to hide memory latency; the logits meet in LDS and each
// wave then routes 2 of the tokens. The 64 lane partials of every pair are combined
// over lane distances 32, 16, 8, 4, 2, 1: recursive halving while a lane holds more
// than one pair, then plain butterfly steps. Each pair's partials meet in exactly the
// butterfly's order, so every logit is the same float32 value the fixed order defines,
// and the top-k choice is reproducible bit for bit. In the softmax and top-k each lane
// holds the logits of experts lane, lane + 64, ... (up to 16 of them: 1024 experts);
// each top-k round takes every lane's best available expert, then the wave's.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

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

// C partial sums per lane, next lane distance M: halve while C > 1 (keep the half of
// the pairs whose next index bit matches this lane's bit M, add the partner's partial
// of the same pairs), then add across the remaining distances. Lane l ends with the
// full sum of pair l >> (6 - log2(C0)).
template <int C, int M>
__device__ __forceinline__ float reduce_pairs(float* v, int lane) {
  if constexpr (C > 1) {
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
      const float send = upper ? v[i] : v[i + C / 2];
      const float keep = upper ? v[i + C / 2] : v[i];
      v[i] = keep + __shfl_xor(send, M);
    }
    return reduce_pairs<C / 2, M / 2>(v, lane);
  } else if constexpr (M >= 1) {
    v[0] = v[0] + __shfl_xor(v[0], M);
    return reduce_pairs<1, M / 2>(v, lane);
  } else {
    return v[0];
  }
}

// NE: logits per lane in the softmax and top-k (experts e = lane + 64 i, i < NE).
template <typename TIn, int TW, int EC, bool SHARED, int NE>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void route_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, const float* __restrict__ bias, int T,
    int D, int E, int k, int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_out) {
  constexpr int V = Chunk<TIn>::V;
  constexpr int P = TW * EC;                     // (token, expert) pairs per pass
  constexpr int LOGP = P == 16 ? 4 : (P == 32 ? 5 : 6);
  static_assert(P == 16 || P == 32 || P == 64, "pairs per pass");
  constexpr int NL = SHARED ? 1 : kWavesPerBlock;   // logit tables per block
  __shared__ float lg[NL][TW][NE * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  // SHARED: the block's waves share tokens t0 .. t0+TW-1 and split the passes
  const int t0 = SHARED ? blockIdx.x * TW : (blockIdx.x * kWavesPerBlock + wave) * TW;
  const int tab = SHARED ? 0 : wave;
  const int nchunk = D / V;

  for (int e0 = SHARED ? wave * EC : 0; e0 < E; e0 += SHARED ? kWavesPerBlock * EC : EC) {
    float acc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) acc[p] = 0.0f;
    if constexpr (!SHARED) {
      // few experts: the raw chunks of step c + 64 are loaded while step c is summed
      // (the summation order is unchanged)
      u32x4 xr[2][TW], wr[2][EC];
      auto load = [&](int c, int b) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
          xr[b][t] = ld16(x + (size_t)min(t0 + t, T - 1) * D + (size_t)c * V);
#pragma unroll
        for (int e = 0; e < EC; ++e) wr[b][e] = ld16(wg + (size_t)min(e0 + e, E - 1) * D + (size_t)c * V);
      };
      auto sum = [&](int b) {
        float xv[TW][V];
#pragma unroll
        for (int t = 0; t < TW; ++t) Chunk<TIn>::widen(xr[b][t], xv[t]);
#pragma unroll
        for (int e = 0; e < EC; ++e) {
          float wv[V];
          Chunk<TIn>::widen(wr[b][e], wv);
#pragma unroll
          for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int i = 0; i < V; ++i) dot_step(acc[t * EC + e], xv[t][i], wv[i], TIn());
        }
      };
      if (lane < nchunk) load(lane, 0);
      for (int c = lane; c < nchunk; c += 2 * kWave) {   // buffers 0 / 1 hold c / c + 64
        if (c + kWave < nchunk) load(c + kWave, 1);
        sum(0);
        if (c + kWave >= nchunk) break;
        if (c + 2 * kWave < nchunk) load(c + 2 * kWave, 0);
        sum(1);
      }
    } else {
      for (int c = lane; c < nchunk; c += kWave) {
        float xv[TW][V];
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          const int tok = min(t0 + t, T - 1);
          Chunk<TIn>::widen(ld16(x + (size_t)tok * D + (size_t)c * V), xv[t]);
        }
#pragma unroll
        for (int e = 0; e < EC; ++e) {
          const int ee = min(e0 + e, E - 1);
          float wv[V];
          Chunk<TIn>::widen(ld16(wg + (size_t)ee * D + (size_t)c * V), wv);
#pragma unroll
          for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int i = 0; i < V; ++i) dot_step(acc[t * EC + e], xv[t][i], wv[i], TIn());
        }
      }
    }
    float logit = reduce_pairs<P, kWave / 2>(acc, lane);
    const int p = lane >> (6 - LOGP);
    const int t = p / EC;
    const int e = e0 + p % EC;
    if (e < E && (lane & ((1 << (6 - LOGP)) - 1)) == 0) {
      if (bias) logit = logit + bias[e];
      lg[tab][t][e] = logit;
    }
  }
  __syncthreads();

  for (int t = SHARED ? wave : 0; t < TW; t += SHARED ? kWavesPerBlock : 1) {
    const int tok = t0 + t;
    if (tok >= T) break;
    float l[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + kWave * i;
      l[i] = e < E ? lg[tab][t][e] : -INFINITY;
      if (logits_out && e < E) logits_out[(size_t)tok * E + e] = l[i];
    }
    float mx = l[0];
#pragma unroll
    for (int i = 1; i < NE; ++i) mx = fmaxf(mx, l[i]);
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    float ex[NE];
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      ex[i] = lane + kWave * i < E ? expf(l[i] - mx) : 0.0f;
      sum += ex[i];
    }
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);

    uint32_t avail = 0;   // bit i: expert lane + 64 i is still available
#pragma unroll
    for (int i = 0; i < NE; ++i)
      if (lane + kWave * i < E) avail |= 1u << i;
    int my_idx = 0;
    float my_w = 0.0f, wtot = 0.0f;
    for (int j = 0; j < k; ++j) {
      // this lane's best available expert (in increasing index, so a tie keeps the lower)
      float key = -INFINITY, xv = 0.0f;
      int id = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (((avail >> i) & 1u) && (id == 0x7fffffff || l[i] > key)) {
          key = l[i];
          id = lane + kWave * i;
          xv = ex[i];
        }
      // then the wave's: the larger logit, ties to the lower index
#pragma unroll
      for (int m = kWave / 2; m >= 1; m >>= 1) {
        const float ok = __shfl_xor(key, m);
        const int oi = __shfl_xor(id, m);
        const float ox = __shfl_xor(xv, m);
        if (ok > key || (ok == key && oi < id)) {
          key = ok;
          id = oi;
          xv = ox;
        }
      }
      if (id % kWave == lane) avail &= ~(1u << (id / kWave));
      const float wj = xv / sum;
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

template <typename TIn>
void launch_typed(const TIn* x, const TIn* wg, const float* bias, int T, int D, int E, int k,
                  int renorm, int32_t* topk_idx, float* topk_w, float* logits, hipStream_t s) {
  const dim3 block(kWave * kWavesPerBlock);
  if (E <= 8) {
    constexpr int TW = 2;
    const dim3 grid((T + TW * kWavesPerBlock - 1) / (TW * kWavesPerBlock));
    hipLaunchKernelGGL((route_kernel<TIn, TW, 8, false, 1>), grid, block, 0, s, x, wg, bias, T,
                       D, E, k, renorm, topk_idx, topk_w, logits);
  } else {
    constexpr int TW = 8;
    const dim3 grid((T + TW - 1) / TW);
    if (E <= kWave)
      hipLaunchKernelGGL((route_kernel<TIn, TW, 8, true, 1>), grid, block, 0, s, x, wg, bias, T,
                         D, E, k, renorm, topk_idx, topk_w, logits);
    else if (E <= 4 * kWave)
      hipLaunchKernelGGL((route_kernel<TIn, TW, 8, true, 4>), grid, block, 0, s, x, wg, bias, T,
                         D, E, k, renorm, topk_idx, topk_w, logits);
    else
      hipLaunchKernelGGL((route_kernel<TIn, TW, 8, true, 16>), grid, block, 0, s, x, wg, bias, T,
                         D, E, k, renorm, topk_idx, topk_w, logits);
  }
}

}  // namespace

hipError_t launch_route(int dt, const void* x, const void* wg, const float* bias, int T, int D,
                        int E, int k, int renorm, int32_t* topk_idx, float* topk_w, float* logits,
                        hipStream_t s) {
  if (dt == kF32)
    launch_typed(static_cast<const float*>(x), static_cast<const float*>(wg), bias, T, D, E, k,
                 renorm, topk_idx, topk_w, logits, s);
  else
    launch_typed(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(wg), bias, T, D, E, k,
                 renorm, topk_idx, topk_w, logits, s);
  return hipGetLastError();
}

}  // namespace moe
