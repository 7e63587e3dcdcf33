// Router gating and softmax-then-top-k routing ("Expert Parallelism (EP)",
// llm-infra-atlas, section 1 "MoE layer 的 forward 通路", its forward-path figure: the gate
// scores every token against every expert, then a score function and a top-k pick
// each token's experts and their weights).
//
// A pass covers TW tokens x EC experts: lane l accumulates the 16-byte chunks
// c = l, l+64, ... of x[t] . wg[e] for the TW*EC (token, expert) pairs, in increasing d.
// With at most 8 experts every wave takes its own 2 tokens (1 when there are few) and
// does the one pass.
// With more, the 4 waves of a block share 8 tokens (every gate-weight chunk a wave
// reads serves 8 tokens) and take the passes over the experts in turn, so there are
// four times as many waves to hide memory latency; the logits meet in LDS and each
// wave then routes 2 of the tokens. For few tokens (fewer than 8 per two compute units,
// as in decode batches) blocks of 8 waves share 4 tokens instead, so that the grid
// still spreads over the chip and each wave runs one pass up to 64 experts.
// The 64 lane partials of every pair are combined
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
constexpr int kRawBuffer = 0x00020000;   // descriptor word 3: raw buffer, 32-bit data

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

// Element i of a 16-byte chunk, widened exactly to float32.
template <typename TIn>
__device__ __forceinline__ float elem(const u32x4& c, int i);
template <>
__device__ __forceinline__ float elem<float>(const u32x4& c, int i) {
  return __uint_as_float(c[i]);
}
template <>
__device__ __forceinline__ float elem<bf16_t>(const u32x4& c, int i) {
  return (i & 1) ? bf16_hi(c[i >> 1]) : bf16_lo(c[i >> 1]);
}

// Softmax and top-k of one token from its logits in LDS (lgrow[e], e < E), by one wave:
// lane l holds the logits of experts l, l + 64, ... (NE of them); each top-k round takes
// every lane's best available expert, then the wave's.
template <int NE>
__device__ __forceinline__ void route_token(const float* lgrow, int tok, int E, int k,
                                            int renorm, int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w,
                                            float* __restrict__ logits_out, int lane) {
  float l[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + kWave * i;
    l[i] = e < E ? lgrow[e] : -INFINITY;
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

// NE: logits per lane in the softmax and top-k (experts e = lane + 64 i, i < NE).
// WPB: waves per block.
template <typename TIn, int TW, int EC, bool SHARED, int NE, int WPB = kWavesPerBlock>
__global__ __launch_bounds__(kWave * WPB) void route_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, const float* __restrict__ bias, int T,
    int D, int E, int k, int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_out) {
  constexpr int V = Chunk<TIn>::V;
  constexpr int P = TW * EC;                     // (token, expert) pairs per pass
  constexpr int LOGP = P == 8 ? 3 : (P == 16 ? 4 : (P == 32 ? 5 : 6));
  static_assert(P == 8 || P == 16 || P == 32 || P == 64, "pairs per pass");
  constexpr int NL = SHARED ? 1 : WPB;   // logit tables per block
  __shared__ float lg[NL][TW][NE * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // SHARED: the block's waves share tokens t0 .. t0+TW-1 and split the passes
  const int t0 = SHARED ? blockIdx.x * TW : (blockIdx.x * WPB + wave) * TW;
  const int tab = SHARED ? 0 : wave;
  const int nchunk = D / V;
  // every lane takes the same number of chunks, and byte offsets fit 31 bits
  const bool pipelined = nchunk % kWave == 0 &&
                         (int64_t)max(T, E) * D * (int64_t)sizeof(TIn) < ((int64_t)1 << 31);

  for (int e0 = SHARED ? wave * EC : 0; e0 < E; e0 += SHARED ? WPB * EC : EC) {
    float acc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) acc[p] = 0.0f;
    // Element i of every token chunk and every gate-weight chunk is widened once and
    // feeds the TW x EC products of that element; each pair still adds its 8 (4)
    // products of a chunk in increasing d.
    auto sum = [&](const u32x4 (&xc)[TW], const u32x4 (&wc)[EC]) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float xe[TW], we[EC];
#pragma unroll
        for (int t = 0; t < TW; ++t) xe[t] = elem<TIn>(xc[t], i);
#pragma unroll
        for (int e = 0; e < EC; ++e) we[e] = elem<TIn>(wc[e], i);
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int e = 0; e < EC; ++e) dot_step(acc[t * EC + e], xe[t], we[e], TIn());
      }
    };
    u32x4 xr[2][TW], wr[2][EC];
    if (pipelined) {
      // Buffer loads: one descriptor per tensor, the row's byte offset in a scalar
      // register and the chunk's in one vector register shared by every load. The
      // loop runs over pairs of 64-lane steps, is uniform and holds no branch; the
      // loads of the step ahead are issued one step before their sum (after the last
      // pair they fetch the odd last step, or re-read a valid chunk that is not
      // summed), and the compiler's wait before each sum counts exactly the loads
      // still in flight for the step ahead.
      const __amdgpu_buffer_rsrc_t rx =
          __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, T * D * (int)sizeof(TIn), kRawBuffer);
      const __amdgpu_buffer_rsrc_t rw =
          __builtin_amdgcn_make_buffer_rsrc((void*)wg, (short)0, E * D * (int)sizeof(TIn), kRawBuffer);
      int sx[TW], sw[EC];
#pragma unroll
      for (int t = 0; t < TW; ++t) sx[t] = min(t0 + t, T - 1) * D * (int)sizeof(TIn);
#pragma unroll
      for (int e = 0; e < EC; ++e) sw[e] = min(e0 + e, E - 1) * D * (int)sizeof(TIn);
      auto load = [&](int c, int b) {
        int off = c * 16;
        asm volatile("" : "+v"(off));   // the step-ahead load stays a load of its own
#pragma unroll
        for (int t = 0; t < TW; ++t) xr[b][t] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, sx[t], 0);
#pragma unroll
        for (int e = 0; e < EC; ++e) wr[b][e] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, sw[e], 0);
        __builtin_amdgcn_sched_barrier(0);   // and the scheduler keeps them ahead of the sum
      };
      const int nstep = nchunk / kWave;   // chunks per lane
      load(lane, 0);
      for (int j = 0; j < nstep / 2; ++j) {
        const int c = lane + j * 2 * kWave;
        load(c + kWave, 1);
        sum(xr[0], wr[0]);
        load(min(c + 2 * kWave, nchunk - 1), 0);
        sum(xr[1], wr[1]);
      }
      if (nstep & 1) sum(xr[0], wr[0]);   // the odd last step, loaded by the last pair
    } else {
      for (int c = lane; c < nchunk; c += kWave) {
#pragma unroll
        for (int t = 0; t < TW; ++t) xr[0][t] = ld16(x + (size_t)min(t0 + t, T - 1) * D + (size_t)c * V);
#pragma unroll
        for (int e = 0; e < EC; ++e) wr[0][e] = ld16(wg + (size_t)min(e0 + e, E - 1) * D + (size_t)c * V);
        sum(xr[0], wr[0]);
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

  for (int t = SHARED ? wave : 0; t < TW; t += SHARED ? WPB : 1) {
    const int tok = t0 + t;
    if (tok >= T) break;
    route_token<NE>(&lg[tab][t][0], tok, E, k, renorm, topk_idx, topk_w, logits_out, lane);
  }
}

template <typename TIn>
void launch_typed(const TIn* x, const TIn* wg, const float* bias, int T, int D, int E, int k,
                  int renorm, int32_t* topk_idx, float* topk_w, float* logits, hipStream_t s) {
  const dim3 block(kWave * kWavesPerBlock);
  const bool few = (T + 7) / 8 < cu_count() / 2;   // fewer than 8 tokens per two CUs
  if (E <= 8 && few) {
    // few tokens: one per wave, twice the waves for the same chains of chunk steps
    constexpr int TW = 1;
    const dim3 grid((T + TW * kWavesPerBlock - 1) / (TW * kWavesPerBlock));
    hipLaunchKernelGGL((route_kernel<TIn, TW, 8, false, 1>), grid, block, 0, s, x, wg, bias, T,
                       D, E, k, renorm, topk_idx, topk_w, logits);
  } else if (E <= 8) {
    constexpr int TW = 2;
    const dim3 grid((T + TW * kWavesPerBlock - 1) / (TW * kWavesPerBlock));
    hipLaunchKernelGGL((route_kernel<TIn, TW, 8, false, 1>), grid, block, 0, s, x, wg, bias, T,
                       D, E, k, renorm, topk_idx, topk_w, logits);
  } else if (!few) {
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
  } else {
    // Few tokens (decode batches): 8-token blocks would leave most CUs idle and give each
    // wave a long chain of passes, so blocks of 8 waves share 4 tokens and each wave
    // takes one group of 8 experts per pass (one pass in all up to 64 experts).
    constexpr int TW = 4, WPB = 8;
    const dim3 grid((T + TW - 1) / TW), bigblock(kWave * WPB);
    if (E <= kWave)
      hipLaunchKernelGGL((route_kernel<TIn, TW, 8, true, 1, WPB>), grid, bigblock, 0, s, x, wg,
                         bias, T, D, E, k, renorm, topk_idx, topk_w, logits);
    else if (E <= 4 * kWave)
      hipLaunchKernelGGL((route_kernel<TIn, TW, 8, true, 4, WPB>), grid, bigblock, 0, s, x, wg,
                         bias, T, D, E, k, renorm, topk_idx, topk_w, logits);
    else
      hipLaunchKernelGGL((route_kernel<TIn, TW, 8, true, 16, WPB>), grid, bigblock, 0, s, x, wg,
                         bias, T, D, E, k, renorm, topk_idx, topk_w, logits);
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
