/*
 * moe.h - C ABI of the single-GPU MoE expert-layer path on AMD MI355X (gfx950).
 *
 * The layer (page "Expert Parallelism (EP)", llm-infra-atlas, section 1
 * "MoE layer 的 forward 通路") runs four calls in order:
 *
 *   moe_route           router gating and softmax-then-top-k routing
 *   moe_permute         tokens-per-expert metadata and the expert-contiguous,
 *                       M-tile-aligned permuted activations
 *   moe_grouped_swiglu  m-grouped fc1 (w1, w3) -> silu(a)*b -> fc2 (w2)
 *   moe_combine         unpermute and top-k-weighted reduce back to token order
 *
 * For decode, moe_permute_masked and moe_grouped_swiglu_masked replace the middle
 * two calls with fixed-capacity per-expert slabs (the masked layout). With an FP8
 * payload, moe_quantize_mxfp8, moe_permute_mxfp8 and moe_grouped_fc1_swiglu_mxfp8
 * replace the permute and fc1.
 *
 * and its backward ("Expert Parallelism (EP)", section 5: each forward operator
 * has a mirror; permute <-> unpermute, dispatch <-> combine, an m-grouped fc <->
 * an m-grouped dgrad plus a k-grouped wgrad) as five more:
 *
 *   moe_combine_backward      dispatch of the output gradient to the permuted rows
 *                             and the gradient of the top-k weights
 *   moe_grouped_dgrad_swiglu  dh = dY w2[e], then the SwiGLU backward -> [da | db]
 *   moe_grouped_dgrad_fc1     dX = da w1[e] + db w3[e]
 *   moe_grouped_wgrad         k-grouped dW2 = dY^T h, [dW1 | dW3] = [da | db]^T X
 *   moe_combine (no weights)  unpermute-and-sum: dx from dX (+ the shared experts' dx)
 *
 * The backward GEMMs read the weights and activations in the layouts the forward
 * uses; nothing is transposed in memory.
 *
 * moe_round_bf16 exposes the float32 -> bf16 rounding that every stored bf16 value
 * goes through, so that callers and tests can round the same way.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named as device buffers are HIP device memory, 16-byte aligned.
 *   The caller allocates and owns every buffer (outputs and scratch included).
 *   The library never allocates or frees memory and keeps no state between
 *   calls except a per-device cache of the compute-unit count (and, for
 *   moe_permute_noalloc, of its static scratch array's device address).
 * - `stream` is a hipStream_t (NULL = the legacy default stream). A call only
 *   enqueues kernels on it; it never synchronises. Calls are re-entrant.
 * - Dense arrays are row-major and contiguous. All float buffers of one call
 *   share `dt`; topk_w, logits and bias are always float32; indices int32.
 *   bf16 is stored as its 16-bit pattern.
 * - Arguments are validated on the host before any HIP call, so a bad call
 *   returns an error without touching the GPU. Device data that is wrong
 *   (an expert index outside [-1, E)) never causes an out-of-bounds access:
 *   the slot is skipped and moe_permute reports it through *dev_err.
 * - Sizes: T >= 1; D, F multiples of 64; E in [1, 1024]; k in [1, min(E, 32)];
 *   m_tile in {16,32,64,128,256}.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* null or misaligned pointer, unknown dtype/flag           */
  MOE_ESHAPE = 2,       /* a size outside the ranges above                          */
  MOE_ECAPACITY = 3,    /* m_cap < moe_capacity(...) or m_cap % m_tile != 0         */
  MOE_EWORKSPACE = 4,   /* workspace smaller than moe_permute_workspace_bytes(...)  */
  MOE_EHIP = 5,         /* the HIP runtime reported an error while launching        */
  MOE_EUNSUPPORTED = 6, /* valid request with no kernel for it (no call returns it now) */
  MOE_ESCRATCH = 7      /* input too large for the library's static scratch         */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/*
 * moe_route - router gating and routing ("Expert Parallelism (EP)", section 1
 * "MoE layer 的 forward 通路", forward-path figure: the gate gives every token a
 * logit per expert, then a score function and a top-k give each token its experts
 * and their probabilities).
 *
 *   x [T,D] (dt), wg [E,D] (dt), bias [E] float32 or NULL
 *   -> topk_idx [T,k] int32, topk_w [T,k] float32, logits [T,E] float32 or NULL
 *
 * logits[t,e] = sum_d x[t,d]*wg[e,d] (+ bias[e]) in float32 with a fixed order
 * so that the selection is reproducible bit for bit: elements are taken in
 * 16-byte chunks (4 float32 or 8 bf16 values); chunk c belongs to lane c % 64;
 * each lane accumulates its chunks' products in increasing d, starting from
 * +0 (float32: a rounded multiply then a rounded add; bf16: a fused
 * multiply-add, identical because a bf16*bf16 product is exact in float32
 * unless it underflows below 2^-126); the 64 lane sums are then combined by a
 * butterfly over lane distances 32,16,8,4,2,1; the bias is added last.
 * Score: softmax over all E logits. Selection: the k largest logits, best
 * first, ties to the lower expert index. topk_w[t,j] = softmax probability of
 * topk_idx[t,j] (renorm = 1 divides the k weights by their sum).
 * Errors: MOE_EINVAL, MOE_ESHAPE (E > 1024 or k > E), MOE_EHIP.
 */
moe_status_t moe_route(moe_dtype_t dt, const void* x, const void* wg, const float* bias,
                       int T, int D, int E, int k, int renorm,
                       int32_t* topk_idx, float* topk_w, float* logits, void* stream);

/*
 * moe_permute - dispatch metadata and permute ("Expert Parallelism (EP)",
 * section 1, forward-path figure: the per-expert token counts, then the reordering
 * that groups each local expert's tokens together; section 2: the layout contract, every expert
 * segment aligned to the GEMM M tile; section 5: permute is an index_select).
 *
 *   x [T,D] (dt), topk_idx [T,k] int32 (-1 = slot not handled here)
 *   -> counts [E]        rows of each expert
 *      offsets [E+1]     exclusive prefix sum of ceil(counts/m_tile)*m_tile
 *      dst_row [T,k]     row of slot (t,j) in x_perm, -1 for skipped slots
 *      src_row [m_cap]   t*k+j of the slot held by each row, -1 for pad/unused
 *      tile_expert [m_cap/m_tile]  expert of each m_tile-row tile, -1 past offsets[E]
 *      x_perm [m_cap,D]  x_perm[dst_row[t,j]] = x[t]; pad rows inside a segment
 *                        are zero; rows >= offsets[E] are not written
 *      *dev_err          1 if some topk_idx value lies outside [-1, E), else 0
 * Rows of one expert follow the flat slot order t*k+j (a stable sort).
 * workspace: device scratch of at least moe_permute_workspace_bytes(T,k,E).
 * Errors: MOE_EINVAL, MOE_ESHAPE, MOE_ECAPACITY, MOE_EWORKSPACE, MOE_EHIP.
 */
moe_status_t moe_permute(moe_dtype_t dt, const void* x, const int32_t* topk_idx,
                         int T, int D, int E, int k, int m_tile, int64_t m_cap,
                         void* x_perm, int32_t* counts, int32_t* offsets,
                         int32_t* dst_row, int32_t* src_row, int32_t* tile_expert,
                         void* workspace, size_t ws_bytes, int32_t* dev_err, void* stream);

/*
 * moe_permute_noalloc - moe_permute for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, outputs and errors as moe_permute without the workspace. The
 * histogram table the permute needs lives in a static device array of the library,
 * 1 MiB per device, held from the library's first use on a device until the process
 * ends; the call itself allocates nothing. It serves ceil(T/256) * (E+1) * 4 bytes
 * <= 1 MiB (moe_permute_workspace_bytes(T,k,E) <= 1 MiB; e.g. T <= 65536 with
 * E <= 1023) and returns MOE_ESCRATCH beyond that. The first call on a device looks
 * up the array's address (hipGetSymbolAddress); a failure there returns MOE_EHIP.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one GPU (on
 * different streams without ordering between them) race and must not be issued; calls
 * ordered on a stream are safe. Nothing in the array has to start at zero (each call
 * writes the part it reads first).
 */
moe_status_t moe_permute_noalloc(moe_dtype_t dt, const void* x, const int32_t* topk_idx,
                                 int T, int D, int E, int k, int m_tile, int64_t m_cap,
                                 void* x_perm, int32_t* counts, int32_t* offsets,
                                 int32_t* dst_row, int32_t* src_row, int32_t* tile_expert,
                                 int32_t* dev_err, void* stream);

/*
 * moe_permute_masked - the masked (fixed-capacity) layout for decode ("Expert
 * Parallelism (EP)", section 2: the masked grouped GEMM serves decode; section 6
 * "DeepSeek-V3 量级的示例数字": how many rows each local expert receives is known
 * only at run time).
 *
 *   x [T,D] (dt), topk_idx [T,k] int32 (-1 = slot not handled here), cap
 *   -> x_masked [E*cap,D]  expert e's slab is rows [e*cap, (e+1)*cap); slot (t,j)
 *                          of e goes to row e*cap + its stable rank among e's slots
 *                          (the rank moe_permute gives it); rows past counts[e]
 *                          are not written
 *      counts [E]          valid rows of each slab: min(#slots of e, cap)
 *      dst_row [T,k]       row of slot (t,j), -1 if skipped or dropped
 *      src_row [E*cap]     t*k+j of the slot in each row, -1 for unused rows
 *      *dev_err            bit 0: some topk_idx value outside [-1, E); bit 1: some
 *                          expert had more than cap slots (the slots past cap are
 *                          dropped: no row, and moe_combine skips them)
 * cap a multiple of 16 (E*cap < 2^31). workspace as moe_permute
 * (moe_permute_workspace_bytes). moe_combine takes the same dst_row with
 * m_cap = E*cap.
 * Errors: MOE_EINVAL, MOE_ESHAPE, MOE_ECAPACITY (cap), MOE_EWORKSPACE, MOE_EHIP.
 */
moe_status_t moe_permute_masked(moe_dtype_t dt, const void* x, const int32_t* topk_idx,
                                int T, int D, int E, int k, int cap, void* x_masked,
                                int32_t* counts, int32_t* dst_row, int32_t* src_row,
                                void* workspace, size_t ws_bytes, int32_t* dev_err,
                                void* stream);

/*
 * moe_grouped_swiglu_masked - moe_grouped_swiglu on the masked layout (same page and
 * sections): for every expert e, rows [e*cap, e*cap + min(counts[e], cap)) of
 * x_masked [E*cap,D] give h [E*cap,F] and y [E*cap,D] with the same arithmetic,
 * storage and workspace rules as moe_grouped_swiglu; the other rows of h and y are
 * neither read nor written. counts stays on the device (no host synchronisation).
 * bf16 slabs of at most 128 rows (D and F multiples of 128, at least two workgroups of
 * 64 output columns per CU) run on a decode kernel that streams each active expert's
 * weights past its rows; the workspace is then unused.
 * cap a multiple of 16 (E*cap < 2^31); D*F < 2^31.
 * Errors: MOE_EINVAL, MOE_ESHAPE, MOE_ECAPACITY (cap), MOE_EHIP.
 */
moe_status_t moe_grouped_swiglu_masked(moe_dtype_t dt, const void* x_masked,
                                       const int32_t* counts, int E, int D, int F, int cap,
                                       const void* w1, const void* w3, const void* w2,
                                       void* h, void* y, void* workspace, size_t ws_bytes,
                                       void* stream);

/*
 * moe_grouped_swiglu - the m-grouped expert GEMMs ("Expert Parallelism (EP)",
 * section 1, forward-path figure: the routed experts run fc1, the activation and
 * fc2 as m-grouped GEMMs; section 2: one kernel over same-shape expert GEMMs whose
 * row counts differ, scheduled across groups; weight layout from the
 * "Expert Tensor Parallel" design note, section 4.3: w1, w3 [E,F,D], w2 [E,D,F]).
 *
 *   x_perm [m_cap,D], offsets [E+1], counts [E] or NULL, tile_expert [m_cap/m_tile]
 *   (from moe_permute), w1, w3 [E,F,D], w2 [E,D,F]
 *   -> h [m_cap,F]       h = silu(x_perm w1[e]^T) * (x_perm w3[e]^T), stored in dt
 *      y_perm [m_cap,D]  y = h w2[e]^T, stored in dt
 * for the rows [offsets[e], offsets[e+1]) of every expert e; float32
 * accumulation; rows >= offsets[E] are neither read nor written. Pad rows
 * (zero in x_perm) give exact zeros. offsets[e] for e < E must be multiples of
 * m_tile; offsets[E] may be any value <= m_cap (so a dense FFN over T tokens is
 * the call with E = 1, offsets = {0, T}, tile_expert all 0).
 * counts (the permute's) marks the pad rows: rows [offsets[e] + counts[e],
 * offsets[e+1]) of each segment hold no token. With it the tiled kernels neither
 * read those rows nor run the matrix work of a 32-row block that lies wholly in them,
 * and still write exact zeros to their h and y_perm rows; the decode-sized path
 * below reads them (they hold zeros as moe_permute leaves them). NULL: every row of
 * a segment is computed. counts outside [0, offsets[e+1] - offsets[e]] is clamped.
 * Every m_tile is accepted (the bf16 kernel cuts each segment into 256-row tiles
 * from its bounds and a shorter last tile; m_tile only sets the alignment the
 * segments come with). D*F < 2^31.
 * offsets that break this contract (negative, decreasing, past m_cap) give
 * unspecified values in h and y_perm but no access outside rows [0, m_cap).
 *
 * workspace: optional device scratch (16-byte aligned; NULL or ws_bytes 0 for
 * none), owned by the caller and clobbered by the call. With it the bf16 kernels
 * split the output tiles of their last, partly filled round over k across the
 * otherwise idle compute units: each share's float32 sums go to a 256 KiB slot of
 * the workspace and a second kernel adds the shares in a fixed order and applies
 * the epilogue. moe_grouped_workspace_bytes() gives the size that lets every
 * such round split; a smaller one splits less or not at all. The split changes
 * only the float32 summation order of those tiles; results are deterministic for
 * a given device and ws_bytes. Calls that share a workspace must not overlap.
 * float32 ignores the workspace, and so does a bf16 call whose buffer holds at most
 * 128 rows with enough experts (D and F multiples of 128, E*min(D,F)/64 at least two
 * workgroups per CU): such decode-sized calls stream each active expert's weights
 * past its rows instead of tiling (fc1 without ab, fc2).
 * Errors: MOE_EINVAL, MOE_ESHAPE, MOE_ECAPACITY (m_cap % m_tile), MOE_EHIP.
 */
moe_status_t moe_grouped_swiglu(moe_dtype_t dt, const void* x_perm, const int32_t* offsets,
                                const int32_t* counts, const int32_t* tile_expert, int E, int D,
                                int F, int m_tile, int64_t m_cap, const void* w1, const void* w3,
                                const void* w2, void* h, void* y_perm, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * moe_grouped_fc1_swiglu / moe_grouped_fc2 - the two halves of moe_grouped_swiglu
 * as separate calls (same arguments, same results, same kernels): fc1 writes
 * h = silu(x_perm w1[e]^T) * (x_perm w3[e]^T), fc2 writes y_perm = h w2[e]^T.
 * They exist so a caller can time or overlap the two grouped GEMMs on their own.
 * fc1 also stores the pre-activations for the backward when `ab` is non-NULL:
 * ab [m_cap, 2F] = [x_perm w1[e]^T | x_perm w3[e]^T] rounded to dt (h is formed
 * from the unrounded float32 sums); NULL skips it.
 * Errors: as moe_grouped_swiglu.
 */
moe_status_t moe_grouped_fc1_swiglu(moe_dtype_t dt, const void* x_perm, const int32_t* offsets,
                                    const int32_t* counts, const int32_t* tile_expert, int E,
                                    int D, int F, int m_tile, int64_t m_cap, const void* w1,
                                    const void* w3, void* h, void* ab, void* workspace,
                                    size_t ws_bytes, void* stream);
moe_status_t moe_grouped_fc2(moe_dtype_t dt, const void* h, const int32_t* offsets,
                             const int32_t* counts, const int32_t* tile_expert, int E, int D,
                             int F, int m_tile, int64_t m_cap, const void* w2, void* y_perm,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * FP8 payload ("Expert Parallelism (EP)", section 6 "DeepSeek-V3 量级的示例数字": the
 * dispatch payload is FP8 e4m3 with scales, the combine stays BF16). The token rows travel through the permute and fc1 as OCP E4M3 codes
 * (bias 7, no infinities, largest value 448) with MX block scales: one power-of-two
 * scale 2^X per 32 consecutive values of a row, stored as the byte X + 127 (E8M0). X is
 * the smallest integer with max|v| <= 448 * 2^X over the block (no value saturates),
 * -127 for an all-zero block; each code is v / 2^X rounded to the nearest e4m3 value,
 * ties to even. fc1 multiplies on the scaled-FP8 MFMA with float32 accumulation and
 * writes h in bf16; fc2 and the combine are the bf16 calls above.
 *
 * Scale layouts (moe_mx_layout_t). MOE_MX_ROWS: scales [R, C/32] bytes, row by row (the
 * plain MX layout). MOE_MX_KSTEPS: the GEMM's operand layout, 32-bit words [C/128][R]:
 * word (s, r) holds row r's scales of the four blocks of k step s (values
 * 128*s .. 128*s + 127), block 4*s + j in byte j. One k step of the fc1 GEMM reads one
 * word per row, so 32 consecutive rows are 128 consecutive bytes (the row layout would
 * put every row's byte on its own cache line).
 *
 * moe_quantize_mxfp8: x [R,C] (dt) -> q [R,C] uint8 codes and scales in `layout`
 *   (MOE_MX_ROWS: C a multiple of 32; MOE_MX_KSTEPS: C a multiple of 128; C <= 65536).
 *   Used with MOE_MX_ROWS for the token rows before the permute and, once, with
 *   MOE_MX_KSTEPS for w1 and w3 (R = E*F rows of D values).
 * moe_permute_mxfp8: moe_permute's metadata (same outputs, same rules), the code rows of
 *   xq [T,D] copied to xq_perm [m_cap,D], and the scales xs [T,D/32] (MOE_MX_ROWS)
 *   gathered into xs_perm in MOE_MX_KSTEPS over m_cap rows ([D/128][m_cap] words);
 *   pad rows get zero bytes (code 0 is the value 0). Rows at or past offsets[E] are not
 *   written. D a multiple of 128.
 * moe_grouped_fc1_swiglu_mxfp8: h [m_cap,F] (bf16) = silu(a)*b with a, b the float32
 *   products of the dequantized rows and w1q/w1s, w3q/w3s ([E,F,D] codes; scales in
 *   MOE_MX_KSTEPS over the E*F rows, [D/128][E*F] words), per segment as
 *   moe_grouped_fc1_swiglu (workspace likewise); xs_perm as moe_permute_mxfp8 writes it.
 *   D a multiple of 128; every m_tile, as for moe_grouped_swiglu.
 * Errors: MOE_EINVAL (also an unknown layout), MOE_ESHAPE, MOE_ECAPACITY,
 * MOE_EWORKSPACE, MOE_EHIP.
 */
typedef enum { MOE_MX_ROWS = 0, MOE_MX_KSTEPS = 1 } moe_mx_layout_t;

moe_status_t moe_quantize_mxfp8(moe_dtype_t dt, const void* x, int64_t R, int C, void* q,
                                void* scales, moe_mx_layout_t layout, void* stream);
moe_status_t moe_permute_mxfp8(const void* xq, const void* xs, const int32_t* topk_idx,
                               int T, int D, int E, int k, int m_tile, int64_t m_cap,
                               void* xq_perm, void* xs_perm, int32_t* counts, int32_t* offsets,
                               int32_t* dst_row, int32_t* src_row, int32_t* tile_expert,
                               void* workspace, size_t ws_bytes, int32_t* dev_err,
                               void* stream);
moe_status_t moe_grouped_fc1_swiglu_mxfp8(const void* xq_perm, const void* xs_perm,
                                          const int32_t* offsets, const int32_t* counts,
                                          const int32_t* tile_expert, int E, int D, int F,
                                          int m_tile, int64_t m_cap, const void* w1q,
                                          const void* w1s, const void* w3q, const void* w3s,
                                          void* h, void* workspace,
                                          size_t ws_bytes, void* stream);

/*
 * moe_combine - unpermute and weighted reduce ("Expert Parallelism (EP)",
 * section 1, forward-path figure: the last stage restores token order, weighting
 * each expert row by its top-k probability, and the shared experts are added;
 * section 5:
 * unpermute is a scatter_add, the transpose of the permute).
 *
 *   y_perm [m_cap,D], dst_row [T,k], topk_w [T,k] float32, shared [T,D] or NULL
 *   -> out [T,D]: out[t] = sum_j topk_w[t,j] * y_perm[dst_row[t,j]] (+ shared[t]),
 *      slots in order j, float32 accumulation, one rounding to dt.
 * Slots whose dst_row is outside [0, m_cap) are skipped. topk_w NULL means every
 * weight is 1: the plain unpermute-and-sum, which is the backward of moe_permute
 * (dx[t] = sum_j dX[dst_row[t,j]] (+ shared[t])).
 * Errors: MOE_EINVAL, MOE_ESHAPE, MOE_EHIP.
 */
moe_status_t moe_combine(moe_dtype_t dt, const void* y_perm, const int32_t* dst_row,
                         const float* topk_w, const void* shared, int T, int D, int k,
                         int64_t m_cap, void* out, void* stream);

/*
 * moe_combine_backward - the mirror of moe_combine ("Expert Parallelism (EP)",
 * section 5: the backward of unpermute-and-reduce is a dispatch). Routing is
 * taken as given: the router's own backward is not part of this library.
 *
 *   dout [T,D] (dt), y_perm [m_cap,D] (the forward's), src_row [m_cap],
 *   offsets [E+1], dst_row [T,k] (from moe_permute), topk_w [T,k] float32
 *   -> dy_perm [m_cap,D]: the row of slot s = t*k+j gets topk_w[s]*dout[t],
 *                         rounded once to dt; pad rows (src_row -1) below
 *                         offsets[E] get zeros; rows >= offsets[E] are not written
 *      dtopk_w [T,k] float32: <dout[t], y_perm[dst_row[t,j]]>, summed in float32
 *                         in a fixed order (16-byte chunks c of the row to lane
 *                         c % 64 in increasing c, then an xor butterfly over the
 *                         64 lanes); 0 for slots without a row
 * Errors: MOE_EINVAL, MOE_ESHAPE, MOE_EHIP.
 */
moe_status_t moe_combine_backward(moe_dtype_t dt, const void* dout, const void* y_perm,
                                  const int32_t* src_row, const int32_t* offsets,
                                  const int32_t* dst_row, const float* topk_w, int T, int D,
                                  int E, int k, int64_t m_cap, void* dy_perm, float* dtopk_w,
                                  void* stream);

/*
 * moe_grouped_dgrad_swiglu - the m-grouped dgrad of fc2 fused with the backward
 * of silu(a)*b ("Expert Parallelism (EP)", section 5: an m-grouped fc mirrors
 * into an m-grouped dgrad).
 *
 *   dy_perm [m_cap,D], offsets, counts, tile_expert (as moe_grouped_swiglu),
 *   w2 [E,D,F] (the forward's), ab [m_cap,2F] (from moe_grouped_fc1_swiglu)
 *   -> dh = dy_perm w2[e] per segment row, rounded to dt, then
 *      dab [m_cap,2F] = [dh*b*silu'(a) | dh*silu(a)] rounded to dt, with
 *      silu'(a) = s*(1 + a*(1 - s)), s = 1/(1 + exp(-a));
 *      dh [m_cap,F] also stored when non-NULL.
 * Rows >= offsets[E] are neither read nor written. Sizes, m_tile, workspace and
 * errors as moe_grouped_swiglu (the workspace splits a partly filled last round
 * over k the same way).
 */
moe_status_t moe_grouped_dgrad_swiglu(moe_dtype_t dt, const void* dy_perm, const int32_t* offsets,
                                      const int32_t* counts, const int32_t* tile_expert, int E,
                                      int D, int F, int m_tile, int64_t m_cap, const void* w2,
                                      const void* ab, void* dab, void* dh, void* workspace,
                                      size_t ws_bytes, void* stream);

/*
 * moe_grouped_dgrad_fc1 - the m-grouped dgrad of fc1 (same passage): the input
 * gradient of the routed experts.
 *
 *   dab [m_cap,2F] = [da | db] (from moe_grouped_dgrad_swiglu), offsets, counts,
 *   tile_expert, w1, w3 [E,F,D] (the forward's)
 *   -> dx_perm [m_cap,D] = da w1[e] + db w3[e] per segment row (one float32 sum
 *      over the 2F terms, rounded once to dt).
 * Rows >= offsets[E] are neither read nor written. Sizes, m_tile, workspace and
 * errors as moe_grouped_swiglu.
 */
moe_status_t moe_grouped_dgrad_fc1(moe_dtype_t dt, const void* dab, const int32_t* offsets,
                                   const int32_t* counts, const int32_t* tile_expert, int E, int D,
                                   int F, int m_tile, int64_t m_cap, const void* w1,
                                   const void* w3, void* dx_perm, void* workspace,
                                   size_t ws_bytes, void* stream);

/*
 * moe_grouped_wgrad - k-grouped GEMM for the weight gradients ("Expert
 * Parallelism (EP)", section 5: the backward of an m-grouped fc holds a
 * k-grouped GEMM, whose reduction runs over each expert's rows).
 *
 *   P [m_cap, N1], Q [m_cap, N2] (dt, row-major), offsets [E+1] (segment rows),
 *   counts [E] or NULL (with counts the sum stops at offsets[e] + counts[e], the end
 *   of the token rows: pad rows add nothing)
 *   -> out[e][i][j] = sum_{offsets[e] <= r < offsets[e+1]} P[r][i] * Q[r][j]
 *      in float32, i < N1, j < N2; rows i < NS go to out_lo [E,NS,N2], rows
 *      i >= NS to out_hi [E,N1-NS,N2] (either may be NULL when it gets no rows).
 *      Experts without rows get zeros.
 * Uses: [dW1 | dW3] = [da | db]^T x_perm (P = dab, N1 = 2F, NS = F, Q = x_perm,
 * N2 = D); dW2 = dY^T h (P = dy_perm, N1 = NS = D, Q = h, N2 = F).
 * Segments are clamped to [0, min(offsets[E], m_cap)] and may have any length
 * and start (a dense FFN over T rows is E = 1, offsets = {0, T}); rows outside
 * the segments are not read. The float32 sums of one element run in a fixed
 * order. N1, N2 multiples of 64 (<= 65536); (m_cap + 64) * max(N1, N2) < 2^31.
 * Errors: MOE_EINVAL, MOE_ESHAPE, MOE_ECAPACITY, MOE_EHIP.
 */
moe_status_t moe_grouped_wgrad(moe_dtype_t dt, const void* P, const void* Q,
                               const int32_t* offsets, const int32_t* counts, int E, int N1,
                               int N2, int NS, int m_tile, int64_t m_cap, float* out_lo,
                               float* out_hi, void* stream);

/*
 * moe_round_bf16 - the float32 -> bf16 rounding that every bf16 value the library
 * stores goes through (h, y_perm, the shared output and out of a bf16 layer, and the
 * backward's bf16 gradients): round to nearest, ties to even, over the whole float32
 * range (subnormal results kept, overflow to infinity); a NaN stays a NaN (quiet).
 * The pages fix bf16 as the storage type of the combined output ("Expert Parallelism
 * (EP)", section 6 "DeepSeek-V3 量级的示例数字") but not its rounding; IEEE
 * round-to-nearest-even is the reading taken.
 *
 *   x [n] float32 -> y [n] bf16 bit patterns (device memory, caller-owned; x 4-byte and
 *   y 2-byte aligned). n = 0 does nothing.
 * Errors: MOE_EINVAL (null or misaligned pointer with n > 0), MOE_ESHAPE (n < 0 or
 * n >= 2^40), MOE_EHIP.
 */
moe_status_t moe_round_bf16(const float* x, uint16_t* y, int64_t n, void* stream);

/* Worst-case rows of the permuted buffer: with N = T*k slots,
 * m_tile * floor((N + min(E, N) * (m_tile - 1)) / m_tile). Returns -1 on bad sizes. */
int64_t moe_capacity(int T, int k, int E, int m_tile);

/* Workspace bytes with which the grouped GEMM calls on the current device can
 * split every partly filled last round of tiles over k (256 KiB per compute unit). */
size_t moe_grouped_workspace_bytes(void);

/* Device scratch bytes moe_permute needs for (T, k, E). Returns 0 on bad sizes. */
size_t moe_permute_workspace_bytes(int T, int k, int E);

/* Static text of a status code. */
const char* moe_status_str(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
