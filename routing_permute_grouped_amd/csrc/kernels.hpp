// Internal launchers of the MoE layer kernels. Arguments are validated by the C ABI
// layer (moe_capi.hip) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum DType { kF32 = 0, kBF16 = 1 };

// Tokens per histogram block of the permute (the stable rank of a slot is the
// number of earlier slots of its expert: earlier blocks + earlier in the block).
constexpr int kHistTokens = 256;

// Largest top-k the entry points accept.
constexpr int kMaxTopK = 32;

int cu_count();  // compute units of the current device (cached per device)

hipError_t launch_route(int dt, const void* x, const void* wg, const float* bias, int T, int D,
                        int E, int k, int renorm, int32_t* topk_idx, float* topk_w, float* logits,
                        hipStream_t s);

size_t permute_workspace_bytes(int T, int k, int E);

// The allocation-free permute's static scratch: its size and, for the current device,
// its device address (resolved once per device; later calls return the cached address).
constexpr size_t kPermuteScratchBytes = (size_t)1 << 20;
hipError_t permute_scratch(void** ptr);

hipError_t launch_permute(int dt, const void* x, const int32_t* topk_idx, int T, int D, int E,
                          int k, int m_tile, int64_t m_cap, void* x_perm, int32_t* counts,
                          int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                          int32_t* tile_expert, void* workspace, int32_t* dev_err, hipStream_t s);

// The masked layout: slot (t, j) of expert e to row e*cap + rank (rank < cap, else
// dropped: dst_row -1 and bit 2 of *dev_err); counts[e] = min(#slots, cap); src_row
// [E*cap]; rows past counts are not written.
hipError_t launch_permute_masked(int dt, const void* x, const int32_t* topk_idx, int T, int D,
                                 int E, int k, int cap, void* x_masked, int32_t* counts,
                                 int32_t* dst_row, int32_t* src_row, void* workspace,
                                 int32_t* dev_err, hipStream_t s);

// Workspace that lets the grouped GEMM split its last round of tiles over k.
size_t grouped_workspace_bytes();

// phase bit 1: fc1 (x_perm, w1, w3 -> h, and ab = [a | b] when non-null);
// bit 2: fc2 (h, w2 -> y_perm). Rows: the segments [offsets[e], offsets[e+1]) when
// cap == 0 (the first counts[e] hold tokens, the rest are pad rows; counts may be null),
// else the masked slabs [e*cap, e*cap + min(counts[e], cap)).
hipError_t launch_grouped_swiglu(int dt, int phases, const void* x_perm, const int32_t* offsets,
                                 const int32_t* counts, int cap, const int32_t* tile_expert, int E,
                                 int D, int F, int m_tile, int64_t m_cap, const void* w1,
                                 const void* w3, const void* w2, void* h, void* ab, void* y_perm,
                                 void* workspace, size_t ws_bytes, hipStream_t s);

// fc1 on the FP8 payload: x (e4m3 [m_cap, D], E8M0 scales [m_cap, D/32]) against w1, w3
// (e4m3 [E,F,D], scales [E,F,D/32]) -> h = silu(a)*b in bf16
hipError_t launch_grouped_fc1_mx(const void* xq_perm, const void* xs_perm,
                                 const int32_t* offsets, const int32_t* counts, int E, int D, int F,
                                 int64_t m_cap,
                                 const void* w1q, const void* w1s, const void* w3q,
                                 const void* w3s, void* h, void* workspace, size_t ws_bytes,
                                 hipStream_t s);

// decode path of the grouped SwiGLU (bf16; the masked layout with cap <= 128, or
// contiguous segments in m_cap <= 128 rows; D and F multiples of 128): the active
// experts' weights streamed past their few rows. decode_rows_max returns the most rows
// an expert can have there, 0 when the path does not apply (also when E*min(D,F)/64 gives
// fewer than two workgroups per CU); phases bit 0 fc1, bit 1 fc2.
int decode_rows_max(int dt, int cap, int64_t m_cap, int E, int D, int F);
hipError_t launch_decode_swiglu(int phases, const void* x, const int32_t* offsets,
                                const int32_t* counts, int cap, int rmax, int E, int D, int F,
                                const void* w1, const void* w3, const void* w2, void* h, void* y,
                                hipStream_t s);

// MX quantization of x [R, C] (dt) -> e4m3 codes [R, C] and E8M0 scales, [R, C/32]
// bytes or (ksteps) [C/128][R] words of four bytes
// float32 -> bf16 bit patterns, rounded as every bf16 store of the library
hipError_t launch_round_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s);

hipError_t launch_quantize_mx(int dt, const void* x, int64_t R, int C, void* q, void* scales,
                              bool ksteps, hipStream_t s);

// permute of the FP8 payload: the metadata of launch_permute, then the rows of the codes
// (D bytes) and the scales (rows of D/32 bytes in, [D/128][m_cap] k-step words out)
hipError_t launch_permute_mx(const void* xq, const void* xs, const int32_t* topk_idx, int T, int D,
                             int E, int k, int m_tile, int64_t m_cap, void* xq_perm,
                             void* xs_perm, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                             int32_t* src_row, int32_t* tile_expert, void* workspace,
                             int32_t* dev_err, hipStream_t s);

// dh = dy_perm w2[e] (w2 [E,D,F]), then [da | db] from ab -> dab; dh stored if non-null
hipError_t launch_grouped_dgrad_swiglu(int dt, const void* dy_perm, const int32_t* offsets,
                                       const int32_t* counts, const int32_t* tile_expert, int E,
                                       int D, int F,
                                       int m_tile, int64_t m_cap, const void* w2, const void* ab,
                                       void* dab, void* dh, void* workspace, size_t ws_bytes,
                                       hipStream_t s);

// dx_perm = da w1[e] + db w3[e] with dab = [da | db] [m_cap, 2F], w1, w3 [E,F,D]
hipError_t launch_grouped_dgrad_fc1(int dt, const void* dab, const int32_t* offsets,
                                    const int32_t* counts, const int32_t* tile_expert, int E,
                                    int D, int F, int m_tile,
                                    int64_t m_cap, const void* w1, const void* w3, void* dx_perm,
                                    void* workspace, size_t ws_bytes, hipStream_t s);

// out[e] = P[seg e]^T Q[seg e] (P [rows, N1], Q [rows, N2]), rows < NS of it to out_lo,
// the rest to out_hi (float32)
hipError_t launch_grouped_wgrad(int dt, const void* P, const void* Q, const int32_t* offsets,
                                const int32_t* counts, int E, int N1, int N2, int NS,
                                int64_t m_cap, float* out_lo, float* out_hi, hipStream_t s);

// dy_perm rows [0, min(offsets[E], m_cap)): topk_w[s] * dout[s / k] for the row of slot s,
// zero for pad rows; dtopk_w[s] = <dout[t], y_perm[row of s]>, 0 for slots without a row
hipError_t launch_combine_backward(int dt, const void* dout, const void* y_perm,
                                   const int32_t* src_row, const int32_t* offsets,
                                   const int32_t* dst_row, const float* topk_w, int T, int D, int E,
                                   int k, int64_t m_cap, void* dy_perm, float* dtopk_w,
                                   hipStream_t s);

hipError_t launch_combine(int dt, const void* y_perm, const int32_t* dst_row, const float* topk_w,
                          const void* shared, int T, int D, int k, int64_t m_cap, void* out,
                          hipStream_t s);

}  // namespace moe
