// m-grouped expert GEMMs: fc1 with the fused silu(a)*b activation, then fc2
// ("Expert Parallelism (EP)", llm-infra-atlas, section 1 "routed_experts_compute:
// fc1 -> act -> fc2, grouped GEMM (m-grouped)"; section 2: one kernel over
// same-shape expert GEMMs with different row counts, a tile scheduler across the
// groups, rows laid out expert-contiguous and tile aligned). Weight layout from the
// "Expert Tensor Parallel" design note, section 4.3: w1, w3 [E,F,D], w2 [E,D,F].
//
// bf16 kernel (float32 accumulation on MFMA v_mfma_f32_32x32x16_bf16):
//   * output tile 128 rows x (128 h columns from w1 and w3 | 256 y columns); both
//     operands are K-contiguous, so each tile stages A [128 x 64] and a 256-row
//     weight panel [256 x 64] of bf16 per k-step in LDS, double buffered (96 KiB)
//   * LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with the row
//     so both the global->LDS stores and the MFMA fragment reads are conflict free
//   * weights are the MFMA A operand and activations the B operand, so every lane
//     ends with 4 consecutive output columns of one row (8-byte stores)
//   * fc1 interleaves w1 and w3 rows in the panel so the same wave holds a and b of
//     the same (row, column) and applies silu(a)*b before rounding to bf16
//   * persistent grid (one workgroup per CU); the number of row tiles is read on the
//     device from offsets[E]; tiles are walked in groups of 8 row tiles per column
//     sweep, and the workgroup id is remapped so that each XCD's L2 sees a
//     contiguous run of tiles; the expert of a row tile comes from tile_expert.
// float32 kernel: a plain LDS-tiled VALU GEMM (the tiny float32 layer only).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;        // rows per tile
constexpr int BK = 64;         // k per stage
constexpr int PANEL = 256;     // weight rows per stage
constexpr int NTHR = 256;      // 4 waves: 2 (rows) x 2 (weight rows)
constexpr int GROUP_M = 8;     // row tiles per column sweep
constexpr int XCDS = 8;
constexpr int A_BYTES = BM * BK * 2;
constexpr int B_BYTES = PANEL * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

__device__ __forceinline__ float silu_mul(float a, float b) {
  return a / (1.0f + __expf(-a)) * b;
}

// byte offset of chunk `ch` (16 bytes) of row `r` in a 128-byte-row LDS tile
__device__ __forceinline__ int swz(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

template <bool FC1>
__global__ __launch_bounds__(NTHR, 1) void gg_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_expert, int E, int K, int N, int m_tile, int m_cap,
    const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W3, bf16_t* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;   // 64-row half of the tile
  const int wn = wave >> 1;  // 128-row half of the weight panel

  const int mend = min(offsets[E], m_cap);
  const int n_mt = (mend + BM - 1) / BM;
  const int cols_per_tile = FC1 ? 128 : PANEL;
  const int n_nt = (N + cols_per_tile - 1) / cols_per_tile;
  const int total = n_mt * n_nt;
  const int nk = K / BK;

  int vb = blockIdx.x;
  if (gridDim.x % XCDS == 0) vb = (blockIdx.x % XCDS) * (gridDim.x / XCDS) + blockIdx.x / XCDS;

  // this thread's chunk column and first row of the global->LDS copies
  const int ch = tid & 7;
  const int row0 = tid >> 3;  // rows row0 + 32*j

  for (int w = vb; w < total; w += gridDim.x) {
    const int grp = w / (GROUP_M * n_nt);
    const int first = grp * GROUP_M;
    const int gm = min(GROUP_M, n_mt - first);
    const int within = w - grp * GROUP_M * n_nt;
    const int mt = first + within % gm;
    const int nt = within / gm;
    const int m0 = mt * BM;
    const int e = tile_expert[m0 / m_tile];
    if (e < 0 || e >= E) continue;
    const int n0 = nt * cols_per_tile;

    // global sources of this thread's copies
    const bf16_t* asrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = min(m0 + row0 + 32 * j, mend - 1);
      asrc[j] = A + (size_t)r * K + ch * 8;
    }
    const bf16_t* bsrc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = row0 + 32 * j;  // panel row
      int gr;
      const bf16_t* W;
      if (FC1) {
        W = ((r >> 6) & 1) ? W3 : W1;
        gr = n0 + (r >> 7) * 64 + (r & 63);
      } else {
        W = W1;
        gr = n0 + r;
      }
      gr = min(gr, N - 1);
      bsrc[j] = W + ((size_t)e * N + gr) * K + ch * 8;
    }

    u32x4 ra[4], rb[8];
    auto gload = [&](int kt) {
      const size_t ko = (size_t)kt * BK;
#pragma unroll
      for (int j = 0; j < 4; ++j) ra[j] = ld16(asrc[j] + ko);
#pragma unroll
      for (int j = 0; j < 8; ++j) rb[j] = ld16(bsrc[j] + ko);
    };
    auto lstore = [&](int stage) {
      char* sa = smem + stage * STAGE_BYTES;
      char* sb = sa + A_BYTES;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(sa + swz(row0 + 32 * j, ch)) = ra[j];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<u32x4*>(sb + swz(row0 + 32 * j, ch)) = rb[j];
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const char* sa = smem + cur * STAGE_BYTES;
      const char* sb = sa + A_BYTES;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int chk = ks * 2 + (lane >> 5);
        bf16x8 wf[4], af[2];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int r = wn * 128 + nb * 32 + (lane & 31);
          wf[nb] = *reinterpret_cast<const bf16x8*>(sb + swz(r, chk));
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int r = wm * 64 + mb * 32 + (lane & 31);
          af[mb] = *reinterpret_cast<const bf16x8*>(sa + swz(r, chk));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], af[mb], acc[nb][mb], 0, 0, 0);
      }
      if (kt + 1 < nk) lstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: lane holds column m = lane & 31 of each 32x32 block and rows
    // n = 8*g + 4*(lane >> 5) + i (i = 0..3) for g = 0..3
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = m0 + wm * 64 + mb * 32 + (lane & 31);
      if (m >= mend) continue;
      if (FC1) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * 64 + nb * 32 + g * 8 + (lane >> 5) * 4;
            if (n >= N) continue;
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = silu_mul(acc[nb][mb][g * 4 + i], acc[nb + 2][mb][g * 4 + i]);
            uint2 pk;
            pk.x = pack_bf16x2(hv[0], hv[1]);
            pk.y = pack_bf16x2(hv[2], hv[3]);
            *reinterpret_cast<uint2*>(C + (size_t)m * N + n) = pk;
          }
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * 128 + nb * 32 + g * 8 + (lane >> 5) * 4;
            if (n >= N) continue;
            uint2 pk;
            pk.x = pack_bf16x2(acc[nb][mb][g * 4 + 0], acc[nb][mb][g * 4 + 1]);
            pk.y = pack_bf16x2(acc[nb][mb][g * 4 + 2], acc[nb][mb][g * 4 + 3]);
            *reinterpret_cast<uint2*>(C + (size_t)m * N + n) = pk;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32: 16 rows x 64 columns per workgroup, k-steps of 32 staged in LDS
// ---------------------------------------------------------------------------
constexpr int FM = 16, FN = 64, FK = 32;

template <bool FC1>
__global__ __launch_bounds__(256) void gg_f32_kernel(const float* __restrict__ A,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ tile_expert, int E,
                                                     int K, int N, int m_tile, int m_cap,
                                                     const float* __restrict__ W1,
                                                     const float* __restrict__ W3,
                                                     float* __restrict__ C) {
  __shared__ float As[FM][FK + 1];
  __shared__ float B1[FN][FK + 1];
  __shared__ float B3[FC1 ? FN : 1][FK + 1];
  const int mend = min(offsets[E], m_cap);
  const int m0 = blockIdx.x * FM;
  if (m0 >= mend) return;
  const int e = tile_expert[m0 / m_tile];
  if (e < 0 || e >= E) return;
  const int n0 = blockIdx.y * FN;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  float a1[4] = {0, 0, 0, 0}, a3[4] = {0, 0, 0, 0};
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int i = tid; i < FM * FK; i += 256) {
      const int r = i / FK, c = i % FK;
      const int gm = min(m0 + r, mend - 1);
      As[r][c] = A[(size_t)gm * K + k0 + c];
    }
    for (int i = tid; i < FN * FK; i += 256) {
      const int r = i / FK, c = i % FK;
      const int gn = min(n0 + r, N - 1);
      B1[r][c] = W1[((size_t)e * N + gn) * K + k0 + c];
      if (FC1) B3[r][c] = W3[((size_t)e * N + gn) * K + k0 + c];
    }
    __syncthreads();
    for (int kk = 0; kk < FK; ++kk) {
      const float a = As[tr][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a1[j] = fmaf(a, B1[tc + 16 * j][kk], a1[j]);
        if (FC1) a3[j] = fmaf(a, B3[tc + 16 * j][kk], a3[j]);
      }
    }
    __syncthreads();
  }
  const int m = m0 + tr;
  if (m >= mend) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + tc + 16 * j;
    if (n < N) C[(size_t)m * N + n] = FC1 ? a1[j] / (1.0f + expf(-a1[j])) * a3[j] : a1[j];
  }
}

}  // namespace

hipError_t launch_grouped_swiglu(int dt, int phases, const void* x_perm, const int32_t* offsets,
                                 const int32_t* tile_expert, int E, int D, int F, int m_tile,
                                 int64_t m_cap, const void* w1, const void* w3, const void* w2,
                                 void* h, void* y_perm, hipStream_t s) {
  if (dt == kF32) {
    const dim3 block(256);
    const int mtiles = (int)((m_cap + FM - 1) / FM);
    if (phases & 1)
      hipLaunchKernelGGL(gg_f32_kernel<true>, dim3(mtiles, (F + FN - 1) / FN), block, 0, s,
                         static_cast<const float*>(x_perm), offsets, tile_expert, E, D, F, m_tile,
                         (int)m_cap, static_cast<const float*>(w1), static_cast<const float*>(w3),
                         static_cast<float*>(h));
    if (phases & 2)
      hipLaunchKernelGGL(gg_f32_kernel<false>, dim3(mtiles, (D + FN - 1) / FN), block, 0, s,
                         static_cast<const float*>(h), offsets, tile_expert, E, F, D, m_tile,
                         (int)m_cap, static_cast<const float*>(w2), static_cast<const float*>(w2),
                         static_cast<float*>(y_perm));
    return hipGetLastError();
  }
  const dim3 grid(cu_count()), block(NTHR);
  if (phases & 1)
    hipLaunchKernelGGL(gg_bf16_kernel<true>, grid, block, 0, s, static_cast<const bf16_t*>(x_perm),
                       offsets, tile_expert, E, D, F, m_tile, (int)m_cap,
                       static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w3),
                       static_cast<bf16_t*>(h));
  if (phases & 2)
    hipLaunchKernelGGL(gg_bf16_kernel<false>, grid, block, 0, s, static_cast<const bf16_t*>(h),
                       offsets, tile_expert, E, F, D, m_tile, (int)m_cap,
                       static_cast<const bf16_t*>(w2), static_cast<const bf16_t*>(w2),
                       static_cast<bf16_t*>(y_perm));
  return hipGetLastError();
}

}  // namespace moe
