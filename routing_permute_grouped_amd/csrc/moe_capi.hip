// C ABI entry points: host-side validation, then the kernel launchers.
// Every check runs before any HIP call, so a rejected call never touches the GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "kernels.hpp"

namespace moe {

int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moe

namespace {

constexpr int kMaxExperts = 1024;
constexpr int kMaxK = moe::kMaxTopK;
constexpr int kMaxDim = 1 << 16;

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dim_ok(int d) { return d >= 64 && d <= kMaxDim && d % 64 == 0; }
bool mtile_ok(int mt) { return mt == 16 || mt == 32 || mt == 64 || mt == 128 || mt == 256; }
bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool tk_ok(int T, int k) { return T >= 1 && (int64_t)T * k <= (1 << 30); }
// masked slabs: a multiple of 16 rows each, E*cap rows addressable with int32
bool cap_ok(int E, int cap) { return cap >= 16 && cap % 16 == 0 && (int64_t)E * cap <= INT32_MAX; }

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace

extern "C" {

int64_t moe_capacity(int T, int k, int E, int m_tile) {
  if (T < 1 || k < 1 || E < 1 || !mtile_ok(m_tile) || !tk_ok(T, k)) return -1;
  const int64_t N = (int64_t)T * k;
  const int64_t ne = E < N ? E : N;
  return (N + ne * (m_tile - 1)) / m_tile * m_tile;
}

size_t moe_grouped_workspace_bytes(void) { return moe::grouped_workspace_bytes(); }

size_t moe_permute_workspace_bytes(int T, int k, int E) {
  if (T < 1 || k < 1 || E < 1 || E > kMaxExperts || !tk_ok(T, k)) return 0;
  return moe::permute_workspace_bytes(T, k, E);
}

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null or misaligned pointer, unknown dtype or flag)";
    case MOE_ESHAPE: return "size outside the supported range";
    case MOE_ECAPACITY: return "m_cap below the worst-case capacity or not a multiple of m_tile";
    case MOE_EWORKSPACE: return "workspace smaller than moe_permute_workspace_bytes";
    case MOE_EHIP: return "HIP runtime error while launching";
    case MOE_EUNSUPPORTED: return "no kernel for this combination of dtype and m_tile";
    case MOE_ESCRATCH:
      return "input too large for the static scratch of moe_permute_noalloc "
             "(ceil(T/256) * (E+1) * 4 bytes must not exceed 1 MiB)";
  }
  return "unknown status";
}

moe_status_t moe_route(moe_dtype_t dt, const void* x, const void* wg, const float* bias, int T,
                       int D, int E, int k, int renorm, int32_t* topk_idx, float* topk_w,
                       float* logits, void* stream) {
  if (!dtype_ok(dt) || !aligned16(x) || !aligned16(wg) || !aligned4(topk_idx) || !aligned4(topk_w))
    return MOE_EINVAL;
  if ((bias && !aligned4(bias)) || (logits && !aligned4(logits))) return MOE_EINVAL;
  if (renorm != 0 && renorm != 1) return MOE_EINVAL;
  if (!tk_ok(T, k) || !dim_ok(D) || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxK)
    return MOE_ESHAPE;
  return hip_status(moe::launch_route(dt, x, wg, bias, T, D, E, k, renorm, topk_idx, topk_w,
                                      logits, static_cast<hipStream_t>(stream)));
}

// Checks shared by moe_permute and moe_permute_noalloc (everything but the workspace).
static moe_status_t permute_args(moe_dtype_t dt, const void* x, const int32_t* topk_idx, int T,
                                 int D, int E, int k, int m_tile, int64_t m_cap,
                                 const void* x_perm, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* dst_row,
                                 const int32_t* src_row, const int32_t* tile_expert,
                                 const int32_t* dev_err) {
  if (!dtype_ok(dt) || !aligned16(x) || !aligned16(x_perm) || !aligned4(topk_idx) ||
      !aligned4(counts) || !aligned4(offsets) || !aligned4(dst_row) || !aligned4(src_row) ||
      !aligned4(tile_expert) || !aligned4(dev_err))
    return MOE_EINVAL;
  if (!tk_ok(T, k) || !dim_ok(D) || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxK ||
      !mtile_ok(m_tile))
    return MOE_ESHAPE;
  const int64_t need = moe_capacity(T, k, E, m_tile);
  if (m_cap < need || m_cap % m_tile != 0 || m_cap > INT32_MAX) return MOE_ECAPACITY;
  return MOE_OK;
}

moe_status_t moe_permute(moe_dtype_t dt, const void* x, const int32_t* topk_idx, int T, int D,
                         int E, int k, int m_tile, int64_t m_cap, void* x_perm, int32_t* counts,
                         int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                         int32_t* tile_expert, void* workspace, size_t ws_bytes, int32_t* dev_err,
                         void* stream) {
  const moe_status_t st = permute_args(dt, x, topk_idx, T, D, E, k, m_tile, m_cap, x_perm,
                                       counts, offsets, dst_row, src_row, tile_expert, dev_err);
  if (st != MOE_OK) return st;
  if (!aligned4(workspace)) return MOE_EINVAL;
  if (ws_bytes < moe::permute_workspace_bytes(T, k, E)) return MOE_EWORKSPACE;
  return hip_status(moe::launch_permute(dt, x, topk_idx, T, D, E, k, m_tile, m_cap, x_perm,
                                        counts, offsets, dst_row, src_row, tile_expert, workspace,
                                        dev_err, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute_noalloc(moe_dtype_t dt, const void* x, const int32_t* topk_idx, int T,
                                 int D, int E, int k, int m_tile, int64_t m_cap, void* x_perm,
                                 int32_t* counts, int32_t* offsets, int32_t* dst_row,
                                 int32_t* src_row, int32_t* tile_expert, int32_t* dev_err,
                                 void* stream) {
  const moe_status_t st = permute_args(dt, x, topk_idx, T, D, E, k, m_tile, m_cap, x_perm,
                                       counts, offsets, dst_row, src_row, tile_expert, dev_err);
  if (st != MOE_OK) return st;
  if (moe::permute_workspace_bytes(T, k, E) > moe::kPermuteScratchBytes) return MOE_ESCRATCH;
  void* scratch = nullptr;   // this device's copy of the library's static array
  if (moe::permute_scratch(&scratch) != hipSuccess) return MOE_EHIP;
  return hip_status(moe::launch_permute(dt, x, topk_idx, T, D, E, k, m_tile, m_cap, x_perm,
                                        counts, offsets, dst_row, src_row, tile_expert, scratch,
                                        dev_err, static_cast<hipStream_t>(stream)));
}

static moe_status_t grouped(int phases, moe_dtype_t dt, const void* x_perm,
                            const int32_t* offsets, const int32_t* counts,
                            const int32_t* tile_expert, int E, int D, int F, int m_tile,
                            int64_t m_cap, const void* w1, const void* w3, const void* w2,
                            void* h, void* ab, void* y_perm, void* workspace, size_t ws_bytes,
                            void* stream) {
  if (!dtype_ok(dt) || !aligned4(offsets) || !aligned4(tile_expert) || !aligned16(h))
    return MOE_EINVAL;
  if (counts && !aligned4(counts)) return MOE_EINVAL;
  if (workspace && !aligned16(workspace)) return MOE_EINVAL;
  if (ab && !aligned16(ab)) return MOE_EINVAL;
  if (!workspace) ws_bytes = 0;
  if ((phases & 1) && (!aligned16(x_perm) || !aligned16(w1) || !aligned16(w3))) return MOE_EINVAL;
  if ((phases & 2) && (!aligned16(w2) || !aligned16(y_perm))) return MOE_EINVAL;
  if (E < 1 || E > kMaxExperts || !dim_ok(D) || !dim_ok(F) || !mtile_ok(m_tile)) return MOE_ESHAPE;
  if ((int64_t)D * F >= ((int64_t)1 << 31)) return MOE_ESHAPE;  // one expert's matrix is int32-indexed
  if (m_cap < 1 || m_cap % m_tile != 0 || m_cap > INT32_MAX) return MOE_ECAPACITY;
  return hip_status(moe::launch_grouped_swiglu(dt, phases, x_perm, offsets, counts, 0,
                                               tile_expert, E, D, F, m_tile, m_cap, w1, w3, w2, h,
                                               ab, y_perm, ws_bytes ? workspace : nullptr,
                                               ws_bytes, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_swiglu(moe_dtype_t dt, const void* x_perm, const int32_t* offsets,
                                const int32_t* counts, const int32_t* tile_expert, int E, int D,
                                int F, int m_tile, int64_t m_cap, const void* w1, const void* w3,
                                const void* w2, void* h, void* y_perm, void* workspace,
                                size_t ws_bytes, void* stream) {
  return grouped(3, dt, x_perm, offsets, counts, tile_expert, E, D, F, m_tile, m_cap, w1, w3, w2,
                 h, nullptr, y_perm, workspace, ws_bytes, stream);
}

moe_status_t moe_grouped_fc1_swiglu(moe_dtype_t dt, const void* x_perm, const int32_t* offsets,
                                    const int32_t* counts, const int32_t* tile_expert, int E,
                                    int D, int F, int m_tile, int64_t m_cap, const void* w1,
                                    const void* w3, void* h, void* ab, void* workspace,
                                    size_t ws_bytes, void* stream) {
  return grouped(1, dt, x_perm, offsets, counts, tile_expert, E, D, F, m_tile, m_cap, w1, w3,
                 nullptr, h, ab, nullptr, workspace, ws_bytes, stream);
}

moe_status_t moe_grouped_fc2(moe_dtype_t dt, const void* h, const int32_t* offsets,
                             const int32_t* counts, const int32_t* tile_expert, int E, int D,
                             int F, int m_tile, int64_t m_cap, const void* w2, void* y_perm,
                             void* workspace, size_t ws_bytes, void* stream) {
  return grouped(2, dt, nullptr, offsets, counts, tile_expert, E, D, F, m_tile, m_cap, nullptr,
                 nullptr, w2, const_cast<void*>(h), nullptr, y_perm, workspace, ws_bytes, stream);
}

moe_status_t moe_permute_masked(moe_dtype_t dt, const void* x, const int32_t* topk_idx, int T,
                                int D, int E, int k, int cap, void* x_masked, int32_t* counts,
                                int32_t* dst_row, int32_t* src_row, void* workspace,
                                size_t ws_bytes, int32_t* dev_err, void* stream) {
  if (!dtype_ok(dt) || !aligned16(x) || !aligned16(x_masked) || !aligned4(topk_idx) ||
      !aligned4(counts) || !aligned4(dst_row) || !aligned4(src_row) || !aligned4(workspace) ||
      !aligned4(dev_err))
    return MOE_EINVAL;
  if (!tk_ok(T, k) || !dim_ok(D) || E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxK)
    return MOE_ESHAPE;
  if (!cap_ok(E, cap)) return MOE_ECAPACITY;
  if (ws_bytes < moe::permute_workspace_bytes(T, k, E)) return MOE_EWORKSPACE;
  return hip_status(moe::launch_permute_masked(dt, x, topk_idx, T, D, E, k, cap, x_masked, counts,
                                               dst_row, src_row, workspace, dev_err,
                                               static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_swiglu_masked(moe_dtype_t dt, const void* x_masked,
                                       const int32_t* counts, int E, int D, int F, int cap,
                                       const void* w1, const void* w3, const void* w2, void* h,
                                       void* y, void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dt) || !aligned4(counts) || !aligned16(x_masked) || !aligned16(w1) ||
      !aligned16(w3) || !aligned16(w2) || !aligned16(h) || !aligned16(y))
    return MOE_EINVAL;
  if (workspace && !aligned16(workspace)) return MOE_EINVAL;
  if (!workspace) ws_bytes = 0;
  if (E < 1 || E > kMaxExperts || !dim_ok(D) || !dim_ok(F)) return MOE_ESHAPE;
  if ((int64_t)D * F >= ((int64_t)1 << 31)) return MOE_ESHAPE;
  if (!cap_ok(E, cap)) return MOE_ECAPACITY;
  return hip_status(moe::launch_grouped_swiglu(dt, 3, x_masked, nullptr, counts, cap, nullptr, E,
                                               D, F, 16, (int64_t)E * cap, w1, w3, w2, h, nullptr,
                                               y, ws_bytes ? workspace : nullptr, ws_bytes,
                                               static_cast<hipStream_t>(stream)));
}

moe_status_t moe_quantize_mxfp8(moe_dtype_t dt, const void* x, int64_t R, int C, void* q,
                                void* scales, moe_mx_layout_t layout, void* stream) {
  if (!dtype_ok(dt) || !aligned16(x) || !aligned16(q) || !scales) return MOE_EINVAL;
  if (layout != MOE_MX_ROWS && layout != MOE_MX_KSTEPS) return MOE_EINVAL;
  if (R < 1 || C < 32 || C % 32 != 0 || C > kMaxDim || R > ((int64_t)1 << 31)) return MOE_ESHAPE;
  if (layout == MOE_MX_KSTEPS && C % 128 != 0) return MOE_ESHAPE;
  return hip_status(moe::launch_quantize_mx(dt, x, R, C, q, scales, layout == MOE_MX_KSTEPS,
                                            static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute_mxfp8(const void* xq, const void* xs, const int32_t* topk_idx, int T,
                               int D, int E, int k, int m_tile, int64_t m_cap, void* xq_perm,
                               void* xs_perm, int32_t* counts, int32_t* offsets,
                               int32_t* dst_row, int32_t* src_row, int32_t* tile_expert,
                               void* workspace, size_t ws_bytes, int32_t* dev_err,
                               void* stream) {
  if (!aligned16(xq) || !aligned4(xs) || !aligned16(xq_perm) || !aligned4(xs_perm) ||
      !aligned4(topk_idx) || !aligned4(counts) || !aligned4(offsets) || !aligned4(dst_row) ||
      !aligned4(src_row) || !aligned4(tile_expert) || !aligned4(workspace) || !aligned4(dev_err))
    return MOE_EINVAL;
  if (!tk_ok(T, k) || !dim_ok(D) || D % 128 != 0 || E < 1 || E > kMaxExperts || k < 1 || k > E ||
      k > kMaxK || !mtile_ok(m_tile))
    return MOE_ESHAPE;
  const int64_t need = moe_capacity(T, k, E, m_tile);
  if (m_cap < need || m_cap % m_tile != 0 || m_cap > INT32_MAX) return MOE_ECAPACITY;
  if (ws_bytes < moe::permute_workspace_bytes(T, k, E)) return MOE_EWORKSPACE;
  return hip_status(moe::launch_permute_mx(xq, xs, topk_idx, T, D, E, k, m_tile, m_cap, xq_perm,
                                           xs_perm, counts, offsets, dst_row, src_row,
                                           tile_expert, workspace, dev_err,
                                           static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_fc1_swiglu_mxfp8(const void* xq_perm, const void* xs_perm,
                                          const int32_t* offsets, const int32_t* counts,
                                          const int32_t* tile_expert, int E, int D, int F,
                                          int m_tile, int64_t m_cap, const void* w1q,
                                          const void* w1s, const void* w3q, const void* w3s,
                                          void* h, void* workspace, size_t ws_bytes,
                                          void* stream) {
  if (!aligned16(xq_perm) || !aligned4(xs_perm) || !aligned4(offsets) || !aligned4(tile_expert) ||
      !aligned16(w1q) || !aligned4(w1s) || !aligned16(w3q) || !aligned4(w3s) || !aligned16(h))
    return MOE_EINVAL;
  if (counts && !aligned4(counts)) return MOE_EINVAL;
  if (workspace && !aligned16(workspace)) return MOE_EINVAL;
  if (!workspace) ws_bytes = 0;
  if (E < 1 || E > kMaxExperts || !dim_ok(D) || D % 128 != 0 || !dim_ok(F) || !mtile_ok(m_tile))
    return MOE_ESHAPE;
  if ((int64_t)D * F >= ((int64_t)1 << 31)) return MOE_ESHAPE;
  if (m_cap < 1 || m_cap % m_tile != 0 || m_cap > INT32_MAX) return MOE_ECAPACITY;
  return hip_status(moe::launch_grouped_fc1_mx(xq_perm, xs_perm, offsets, counts, E, D, F, m_cap,
                                               w1q,
                                               w1s, w3q, w3s, h,
                                               ws_bytes ? workspace : nullptr, ws_bytes,
                                               static_cast<hipStream_t>(stream)));
}

static moe_status_t dgrad_common(moe_dtype_t dt, const void* a, const int32_t* offsets,
                                 const int32_t* counts, const int32_t* tile_expert, int E, int D,
                                 int F, int m_tile, int64_t m_cap, void* workspace) {
  if (!dtype_ok(dt) || !aligned4(offsets) || !aligned4(tile_expert) || !aligned16(a))
    return MOE_EINVAL;
  if (counts && !aligned4(counts)) return MOE_EINVAL;
  if (workspace && !aligned16(workspace)) return MOE_EINVAL;
  if (E < 1 || E > kMaxExperts || !dim_ok(D) || !dim_ok(F) || !mtile_ok(m_tile)) return MOE_ESHAPE;
  if ((int64_t)D * F >= ((int64_t)1 << 31)) return MOE_ESHAPE;
  if (m_cap < 1 || m_cap % m_tile != 0 || m_cap > INT32_MAX) return MOE_ECAPACITY;
  return MOE_OK;
}

moe_status_t moe_grouped_dgrad_swiglu(moe_dtype_t dt, const void* dy_perm, const int32_t* offsets,
                                      const int32_t* counts, const int32_t* tile_expert, int E,
                                      int D, int F, int m_tile, int64_t m_cap, const void* w2,
                                      const void* ab, void* dab, void* dh, void* workspace,
                                      size_t ws_bytes, void* stream) {
  if (!aligned16(w2) || !aligned16(ab) || !aligned16(dab) || (dh && !aligned16(dh)))
    return MOE_EINVAL;
  const moe_status_t st = dgrad_common(dt, dy_perm, offsets, counts, tile_expert, E, D, F, m_tile,
                                       m_cap, workspace);
  if (st != MOE_OK) return st;
  if (!workspace) ws_bytes = 0;
  return hip_status(moe::launch_grouped_dgrad_swiglu(dt, dy_perm, offsets, counts, tile_expert, E,
                                                     D, F,
                                                     m_tile, m_cap, w2, ab, dab, dh,
                                                     ws_bytes ? workspace : nullptr, ws_bytes,
                                                     static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_dgrad_fc1(moe_dtype_t dt, const void* dab, const int32_t* offsets,
                                   const int32_t* counts, const int32_t* tile_expert, int E, int D,
                                   int F, int m_tile, int64_t m_cap, const void* w1,
                                   const void* w3, void* dx_perm, void* workspace,
                                   size_t ws_bytes, void* stream) {
  if (!aligned16(w1) || !aligned16(w3) || !aligned16(dx_perm)) return MOE_EINVAL;
  const moe_status_t st = dgrad_common(dt, dab, offsets, counts, tile_expert, E, D, F, m_tile,
                                       m_cap, workspace);
  if (st != MOE_OK) return st;
  if (!workspace) ws_bytes = 0;
  return hip_status(moe::launch_grouped_dgrad_fc1(dt, dab, offsets, counts, tile_expert, E, D, F,
                                                  m_tile,
                                                  m_cap, w1, w3, dx_perm,
                                                  ws_bytes ? workspace : nullptr, ws_bytes,
                                                  static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_wgrad(moe_dtype_t dt, const void* P, const void* Q,
                               const int32_t* offsets, const int32_t* counts, int E, int N1,
                               int N2, int NS, int m_tile, int64_t m_cap, float* out_lo,
                               float* out_hi, void* stream) {
  if (!dtype_ok(dt) || !aligned16(P) || !aligned16(Q) || !aligned4(offsets)) return MOE_EINVAL;
  if (counts && !aligned4(counts)) return MOE_EINVAL;
  if (NS < 0 || NS > N1) return MOE_ESHAPE;
  if ((NS > 0 && !aligned16(out_lo)) || (NS < N1 && !aligned16(out_hi))) return MOE_EINVAL;
  if (E < 1 || E > kMaxExperts || !dim_ok(N1) || !dim_ok(N2) || !mtile_ok(m_tile))
    return MOE_ESHAPE;
  if (m_cap < 1 || m_cap % m_tile != 0 || m_cap > INT32_MAX) return MOE_ECAPACITY;
  // a segment's rows of one operand are addressed with 32-bit byte offsets
  if ((m_cap + 64) * (int64_t)(N1 > N2 ? N1 : N2) >= ((int64_t)1 << 31)) return MOE_ESHAPE;
  return hip_status(moe::launch_grouped_wgrad(dt, P, Q, offsets, counts, E, N1, N2, NS, m_cap,
                                              out_lo,
                                              out_hi, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_round_bf16(const float* x, uint16_t* y, int64_t n, void* stream) {
  if (n < 0 || n >= ((int64_t)1 << 40)) return MOE_ESHAPE;
  if (n > 0 && (!aligned4(x) || !y || (reinterpret_cast<uintptr_t>(y) & 1u))) return MOE_EINVAL;
  return hip_status(moe::launch_round_bf16(x, y, n, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(moe_dtype_t dt, const void* y_perm, const int32_t* dst_row,
                         const float* topk_w, const void* shared, int T, int D, int k,
                         int64_t m_cap, void* out, void* stream) {
  if (!dtype_ok(dt) || !aligned16(y_perm) || !aligned4(dst_row) || (topk_w && !aligned4(topk_w)) ||
      !aligned16(out) || (shared && !aligned16(shared)))
    return MOE_EINVAL;
  if (!tk_ok(T, k) || !dim_ok(D) || k < 1 || k > kMaxK || m_cap < 1 || m_cap > INT32_MAX)
    return MOE_ESHAPE;
  return hip_status(moe::launch_combine(dt, y_perm, dst_row, topk_w, shared, T, D, k, m_cap, out,
                                        static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine_backward(moe_dtype_t dt, const void* dout, const void* y_perm,
                                  const int32_t* src_row, const int32_t* offsets,
                                  const int32_t* dst_row, const float* topk_w, int T, int D, int E,
                                  int k, int64_t m_cap, void* dy_perm, float* dtopk_w,
                                  void* stream) {
  if (!dtype_ok(dt) || !aligned16(dout) || !aligned16(y_perm) || !aligned4(src_row) ||
      !aligned4(offsets) || !aligned4(dst_row) || !aligned4(topk_w) || !aligned16(dy_perm) ||
      !aligned4(dtopk_w))
    return MOE_EINVAL;
  if (!tk_ok(T, k) || !dim_ok(D) || E < 1 || E > kMaxExperts || k < 1 || k > kMaxK || m_cap < 1 ||
      m_cap > INT32_MAX)
    return MOE_ESHAPE;
  return hip_status(moe::launch_combine_backward(dt, dout, y_perm, src_row, offsets, dst_row,
                                                 topk_w, T, D, E, k, m_cap, dy_perm, dtopk_w,
                                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
