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

int cu_count();  // compute units of the current device (cached per device)

hipError_t launch_route(int dt, const void* x, const void* wg, const float* bias, int T, int D,
                        int E, int k, int renorm, int32_t* topk_idx, float* topk_w, float* logits,
                        hipStream_t s);

size_t permute_workspace_bytes(int T, int k, int E);

hipError_t launch_permute(int dt, const void* x, const int32_t* topk_idx, int T, int D, int E,
                          int k, int m_tile, int64_t m_cap, void* x_perm, int32_t* counts,
                          int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                          int32_t* tile_expert, void* workspace, int32_t* dev_err, hipStream_t s);

// Workspace that lets the grouped GEMM split its last round of tiles over k.
size_t grouped_workspace_bytes();

// phase bit 1: fc1 (x_perm, w1, w3 -> h); bit 2: fc2 (h, w2 -> y_perm)
hipError_t launch_grouped_swiglu(int dt, int phases, const void* x_perm, const int32_t* offsets,
                                 const int32_t* tile_expert, int E, int D, int F, int m_tile,
                                 int64_t m_cap, const void* w1, const void* w3, const void* w2,
                                 void* h, void* y_perm, void* workspace, size_t ws_bytes,
                                 hipStream_t s);

hipError_t launch_combine(int dt, const void* y_perm, const int32_t* dst_row, const float* topk_w,
                          const void* shared, int T, int D, int k, int64_t m_cap, void* out,
                          hipStream_t s);

}  // namespace moe
