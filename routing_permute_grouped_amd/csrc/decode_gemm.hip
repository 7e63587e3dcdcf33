// Grouped SwiGLU for decode ("Expert Parallelism (EP)", llm-infra-atlas, section 2:
// decode runs the masked grouped GEMM, each local expert's rows sitting in a fixed slab
// whose valid count is known only on the device). Also taken by contiguous segments in
// a row buffer of at most 128 rows (the shared experts of a decode batch).
//
// At decode sizes an expert holds a few rows (tokens), so the GEMM is a stream of the
// active experts' weights past those rows: its bound is HBM, and what it needs is many
// weight bytes in flight per CU, not LDS tiles of a weight panel. Here:
//   * a workgroup (4 waves) takes one expert and 64 output columns, each wave 16 of
//     them: fc1 reads those 16 rows of w1 and of w3 ([E,F,D]), fc2 16 rows of w2
//     ([E,D,F]); an expert with no valid row is skipped (its weights are not read);
//   * a wave streams its weight rows straight into registers in chunks of 128 k values,
//     PD chunks ahead of the MFMAs (ordinary loads, so the compiler's wait counting stays
//     exact); the lane layout is the MFMA operand's, so no LDS copy of the weights;
//   * the expert's rows (at most 128) come through LDS once per chunk for all 4 waves,
//     double-buffered, by direct buffer->LDS loads whose descriptor ends at the expert's
//     last valid row (rows past it read as zeros and touch no memory); 256-byte rows
//     with the 16-byte unit u of row r at u ^ (r % 16), so the 16 rows a quarter-wave
//     reads fall on distinct banks;
//   * v_mfma_f32_16x16x32_bf16 with the weights as operand A (16 output columns) and the
//     rows as operand B (16 rows per block, up to 8 blocks), float32 accumulation; fc1
//     forms silu(a)*b from the w1 and w3 sums in registers, then rounds h to bf16.
// The loop body has no branch around a load: the weight loads are the only ones the
// compiler sees (its waits for them stay exact), the tail re-reads the last chunk
// instead of branching, and one explicit wait before each barrier covers the row copy.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace moe {
namespace {

constexpr int DW = 4;          // waves per workgroup
constexpr int DCOLS = 16;      // output columns per wave
constexpr int KMIN = 128;      // the shortest chunk (K must be a multiple of it)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_frag(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// silu(a) * b; the sigmoid's reciprocal from the hardware's approximate reciprocal
// (about 1 ulp of float32, below the bf16 rounding of h)
__device__ __forceinline__ float silu_mul(float a, float b) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * b;
}

// The rows of expert e: the masked layout's slab [e*cap, e*cap + min(counts[e], cap))
// (offsets null), or the contiguous layout's segment [offsets[e], offsets[e+1]) of an
// m_cap-row buffer, clamped into [0, min(offsets[E], m_cap)] (offsets that break the
// contract can only shrink the work) and to at most cap rows.
struct DecSegs {
  const int32_t* offsets;
  const int32_t* counts;
  int cap, E, m_cap;
  __device__ void get(int e, int& r0, int& rows) const {
    if (offsets) {
      const int lim = max(0, min(offsets[E], m_cap));
      r0 = max(0, min(offsets[e], lim));
      rows = max(0, min(min(offsets[e + 1], lim) - r0, cap));
    } else {
      r0 = e * cap;
      rows = max(0, min(counts[e], cap));
    }
  }
};

// FC1: out [rows, N] = silu(X w1^T) * (X w3^T) with N = F, K = D; else out = X w2^T with
// N = D, K = F (W3 unused), for expert e's rows [r0, r0 + rows), rows <= 16*NB.
// NB: row blocks of 16 computed (exactly the expert's, so the loop has no branch on the
// count). KS: 32-value slices per chunk (4 or 8). PD: weight chunks in flight per wave.
// N is a multiple of 64, K of 32*KS.
template <bool FC1, int NB, int KS, int PD>
__device__ __forceinline__ void dec_body(char* xs, int xbytes, const bf16_t* __restrict__ X,
                                         int e, int r0, int rows, int K, int N,
                                         const bf16_t* __restrict__ W1,
                                         const bf16_t* __restrict__ W3,
                                         bf16_t* __restrict__ out) {
  constexpr int NW = FC1 ? 2 : 1;
  constexpr int NV = KS * NW;                 // weight loads per wave and chunk
  constexpr int ROWB = KS * 64;               // bytes of a row's chunk
  constexpr int UPR = ROWB / 16;              // 16-byte units per row chunk
  constexpr int RPP = 1024 / ROWB;            // rows per 1 KiB copy piece
  constexpr int NP = NB * 16 / RPP / DW;      // copy pieces per wave and chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * (DW * DCOLS) + wave * DCOLS;
  const int nch = K / (32 * KS);
  const int nmain = nch - nch % PD;

  // this lane's weight row; slice s of a chunk (k = 32*s + 8*g .. +7) is 16 bytes at
  // 64*s + 16*g of the row's 256
  const char* wrow[NW];
  wrow[0] = reinterpret_cast<const char*>(W1 + ((size_t)e * N + n0 + fr) * K) + 16 * g;
  if (FC1) wrow[NW - 1] = reinterpret_cast<const char*>(W3 + ((size_t)e * N + n0 + fr) * K) + 16 * g;
  u32x4 wr[PD][NW][KS];
  auto wload = [&](int slot, int c) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int s = 0; s < KS; ++s) wr[slot][w][s] = ld16(wrow[w] + (size_t)c * ROWB + 64 * s);
  };

  // row copies: piece q = wave + 4*i (i < NP) is LDS rows RPP*q .. of a buffer; lane l
  // fills row r = RPP*q + l/UPR, physical unit l%UPR, i.e. the row's unit
  // (l%UPR) ^ (r%16)
  const i32x4 rs = buffer_rsrc(X + (size_t)r0 * K, (uint32_t)rows * K * 2u);
  uint32_t voff[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = RPP * (wave + 4 * i) + lane / UPR;
    voff[i] = (uint32_t)r * K * 2u + (((lane % UPR) ^ (r & 15)) << 4);
  }
  const uint32_t lds0 = lds_addr(xs);
  auto xcopy = [&](int c, int buf) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      dma16(rs, voff[i], (uint32_t)c * ROWB, lds0 + buf * xbytes + (wave + 4 * i) * 1024);
  };

  f32x4 acc[NW][NB];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[w][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // chunk c from its LDS buffer and weight slot j
  auto compute = [&](int c, int j) {
    const char* xb = xs + (c & 1) * xbytes;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int r = 16 * b + fr;
        const bf16x8 xf = as_frag(
            *reinterpret_cast<const u32x4*>(xb + r * ROWB + (((4 * s + g) ^ (r & 15)) << 4)));
#pragma unroll
        for (int w = 0; w < NW; ++w)
          acc[w][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(wr[j][w][s]), xf,
                                                              acc[w][b], 0, 0, 0);
      }
    }
  };
  // chunk c's rows have landed (only the last NV weight loads may be outstanding) and
  // every wave is done with the buffer the next copy overwrites
  auto sync = [&]() { asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NV) : "memory"); };

  // issue order: the rows of chunk 0, then the first PD weight chunks; from then on each
  // chunk's row copy is followed only by one chunk of weight loads before the wait that
  // needs it. Past the last chunk the copies and loads repeat it rather than branch.
  xcopy(0, 0);
#pragma unroll
  for (int p = 0; p < PD; ++p) wload(p, min(p, nch - 1));
  for (int c0 = 0; c0 < nmain; c0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int c = c0 + j;
      sync();
      compute(c, j);
      xcopy(min(c + 1, nch - 1), (c + 1) & 1);
      wload(j, min(c + PD, nch - 1));
    }
  }
  // the remaining nch % PD chunks sit in slots 0 .. (already loaded); no weight loads
  // follow their row copies, so each waits for every load
#pragma unroll
  for (int j = 0; j < PD - 1; ++j) {
    const int c = nmain + j;
    if (c < nch) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      compute(c, j);
      xcopy(min(c + 1, nch - 1), (c + 1) & 1);
    }
  }

  // lane l holds row (token) 16*b + l%16 and output columns n0 + 4*(l/16) .. +3
  const int col = n0 + 4 * g;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int r = 16 * b + fr;
    if (r < rows) {
      bf16_t* p = out + ((size_t)r0 + r) * N + col;
      const f32x4& a = acc[0][b];
      if (FC1) {
        const f32x4& u = acc[NW - 1][b];
        store4(p, silu_mul(a[0], u[0]), silu_mul(a[1], u[1]), silu_mul(a[2], u[2]),
               silu_mul(a[3], u[3]));
      } else {
        store4(p, a[0], a[1], a[2], a[3]);
      }
    }
  }
}

// One workgroup per (64 output columns, expert); TB: the most row blocks any expert may
// have (cap <= 16*TB). The body is chosen by the expert's own number of row blocks.
template <bool FC1, int TB, int KS, int PD>
__global__ __launch_bounds__(DW * 64) void dec_kernel(const bf16_t* __restrict__ X, DecSegs sg,
                                                      int K, int N,
                                                      const bf16_t* __restrict__ W1,
                                                      const bf16_t* __restrict__ W3,
                                                      bf16_t* __restrict__ out) {
  constexpr int XBYTES = TB * 16 * KS * 64;   // one row buffer
  __shared__ __attribute__((aligned(1024))) char xs[2 * XBYTES];
  const int e = blockIdx.y;
  int r0, rows;
  sg.get(e, r0, rows);
  if (rows == 0) return;   // uniform over the workgroup: the expert's weights stay unread
#define DEC_CASE(n)                                                                         \
  case n:                                                                                   \
    if (TB >= n)                                                                            \
      dec_body<FC1, (TB >= n ? n : 1), KS, PD>(xs, XBYTES, X, e, r0, rows, K, N, W1, W3, out); \
    break;
  switch ((rows + 15) >> 4) {
    DEC_CASE(1)
    DEC_CASE(2)
    DEC_CASE(3)
    DEC_CASE(4)
    DEC_CASE(5)
    DEC_CASE(6)
    DEC_CASE(7)
    default:
      if (TB >= 8) dec_body<FC1, (TB >= 8 ? 8 : 1), KS, PD>(xs, XBYTES, X, e, r0, rows, K, N, W1, W3, out);
      break;
  }
#undef DEC_CASE
}

template <bool FC1, int KS, int PD>
void launch_dec(int tb, const void* X, DecSegs sg, int E, int K, int N, const void* W1,
                const void* W3, void* out, hipStream_t s) {
  const dim3 grid((N + DW * DCOLS - 1) / (DW * DCOLS), E);
  const bf16_t* x = static_cast<const bf16_t*>(X);
  const bf16_t* w1 = static_cast<const bf16_t*>(W1);
  const bf16_t* w3 = static_cast<const bf16_t*>(W3);
  bf16_t* o = static_cast<bf16_t*>(out);
  if (tb <= 2)
    hipLaunchKernelGGL((dec_kernel<FC1, 2, KS, PD>), grid, dim3(DW * 64), 0, s, x, sg, K, N, w1,
                       w3, o);
  else if (tb <= 4)
    hipLaunchKernelGGL((dec_kernel<FC1, 4, KS, PD>), grid, dim3(DW * 64), 0, s, x, sg, K, N, w1,
                       w3, o);
  else
    hipLaunchKernelGGL((dec_kernel<FC1, 8, 4, PD>), grid, dim3(DW * 64), 0, s, x, sg, K, N, w1,
                       w3, o);
}

}  // namespace

int decode_rows_max(int dt, int cap, int64_t m_cap, int E, int D, int F) {
  const int64_t rmax = cap > 0 ? cap : m_cap;
  if (dt != kBF16 || rmax < 1 || rmax > 128 || D % KMIN != 0 || F % KMIN != 0) return 0;
  // a few experts (a dense or shared FFN) give too few workgroups to stream at the HBM
  // rate; the split-K tile kernel serves them better
  if ((int64_t)E * (std::min(D, F) / (DW * DCOLS)) < 2 * cu_count()) return 0;
  if ((cap > 0 ? (int64_t)cap : m_cap) * (D > F ? D : F) * 2 >= ((int64_t)1 << 32)) return 0;
  return (int)rmax;
}

hipError_t launch_decode_swiglu(int phases, const void* x, const int32_t* offsets,
                                const int32_t* counts, int cap, int rmax, int E, int D, int F,
                                const void* w1, const void* w3, const void* w2, void* h, void* y,
                                hipStream_t s) {
  const int tb = (rmax + 15) / 16;
  const DecSegs sg{offsets, counts, offsets ? rmax : cap, E, rmax};
  // fc1 keeps two weight streams in flight per chunk, fc2 one: the same registers.
  // (256-value chunks, 512 contiguous bytes per row and request, measured no faster.)
  if (phases & 1) launch_dec<true, 4, 2>(tb, x, sg, E, D, F, w1, w3, h, s);
  if (phases & 2) launch_dec<false, 4, 4>(tb, h, sg, E, F, D, w2, w2, y, s);
  return hipGetLastError();
}

}  // namespace moe
