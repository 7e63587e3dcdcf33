// m-grouped expert GEMMs: fc1 with the fused silu(a)*b activation, then fc2
// ("Expert Parallelism (EP)", llm-infra-atlas, section 1 "MoE layer 的 forward 通路", its forward-path figure:
// the routed experts run fc1, the activation and fc2 as grouped GEMMs; section 2:
// one kernel over same-shape expert GEMMs with different row counts, a tile scheduler
// across the groups, rows laid out expert-contiguous and tile aligned). Weight layout from the
// "Expert Tensor Parallel" design note, section 4.3: w1, w3 [E,F,D], w2 [E,D,F].
// The backward's GEMMs (section 5: an m-grouped fc mirrors into an m-grouped dgrad and
// a k-grouped wgrad) run on the same tile pipeline.
//
// bf16 kernels (float32 accumulation on v_mfma_f32_32x32x16_bf16):
//   * a tile is up to 256 rows of one expert's segment x a 256-row weight panel
//     (fc1: 128 h columns, taken from w1 and w3 in alternating 32-row blocks; fc2 and
//     the dgrads: 256 output columns). Per 64-wide k step the tile stages A [256 x 64]
//     and the panel [256 x 64] in LDS (64 KiB) with direct buffer->LDS loads, two
//     stages (128 KiB).
//   * eight waves, two per SIMD; on a full tile each wave owns 128 rows x 64 panel rows
//     (8 MFMA blocks, 128 accumulators). A half tile (the last 128 rows of a segment
//     whose length is an odd number of 128-row tiles) is split 64 rows x 64 panel rows
//     per wave, so all four SIMDs stay busy.
//   * an operand whose k is contiguous in memory is staged as 128-byte LDS rows with the
//     16-byte chunk index XOR-swizzled by half the row index; an operand stored [k][n]
//     (w2 read by the dgrad of fc2, w1/w3 by the dgrad of fc1, the activations by the
//     wgrad) is staged as 512-byte k rows and read back with the transposing LDS load.
//     Both layouts are free of bank conflicts for the fragment reads.
//   * weights are the MFMA A operand and activations the B operand: each lane ends
//     with 4 consecutive output columns of one row; for fc1 the w1 and w3 blocks of
//     the same columns land in the same wave, which applies silu(a)*b before rounding
//     to bf16 (8-byte stores). fc2, the dgrad of fc1 (same mode) and the dgrad of fc2
//     pass their rounded tile through the LDS stage of the last k step and store rows
//     in 16-byte chunks.
//   * persistent grid (one workgroup per CU). Each workgroup builds the list of
//     256-row blocks per expert from offsets[] on the device (no host sync), walks
//     each expert's (block, column) tiles with up to GROUP_M blocks per column sweep,
//     and the workgroup id is remapped so each XCD's L2 sees a contiguous run of tiles.
// float32 kernels: plain LDS-tiled VALU GEMMs (the tiny float32 layer only).
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;        // rows per full tile
constexpr int BP = 256;        // weight-panel rows per tile
constexpr int BK = 64;         // k per stage
constexpr int NTHR = 512;      // 8 waves, two per SIMD
constexpr int GROUP_M = 4;     // at most this many 256-row blocks per column sweep
constexpr int XCDS = 8;
constexpr int MAXE = 1024;
constexpr int A_BYTES = BM * BK * 2;
constexpr int B_BYTES = BP * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

// silu(a) * b with the sigmoid's reciprocal from the hardware's approximate reciprocal
// (about 1 ulp of float32, far below the bf16 rounding of h) instead of a correctly
// rounded division, which expands to ten instructions per element.
__device__ __forceinline__ float sigmoid(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}
__device__ __forceinline__ float silu_mul(float a, float b) { return a * sigmoid(a) * b; }

// Byte offset of 16-byte chunk `ch` of row `r` in a 128-byte-row LDS tile. The chunk
// is XOR-swizzled with (r / 2) % 8: the 16 rows that 16 consecutive lanes read at one
// logical chunk then cover all sixteen 16-byte bank groups of a 256-byte bank row
// (conflict free for ds_read_b128, which serves 16 lanes per cycle).
__device__ __forceinline__ int swz(int r, int ch) { return r * 128 + ((ch ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  uint2 pk;
  pk.x = pack_bf16x2(a, b);
  pk.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(p) = pk;
}

// What the m-grouped kernel does with its float32 sums (C = A W^T per segment row):
//   kFc1   the panel interleaves w1 and w3 rows: h = silu(a)*b -> C [m][N]; when `ab` is
//          set, the pre-activations a and b are stored too, as ab [m][2N] = [a | b]
//   kFc2   y -> C [m][N]
//   kDgrad the sums are dh (dY w2[e]); dh is rounded to bf16, then with (a, b) read from
//          ab [m][2N]: da = dh*b*silu'(a), db = dh*silu(a) -> C [m][2N] = [da | db];
//          dh itself -> `dh` [m][N] when set
// (the backward of the activation, "Expert Parallelism (EP)", section 5: the fc of the
// forward mirrors into an m-grouped dgrad).
enum Mode { kFc1 = 0, kFc2 = 1, kDgrad = 2 };

struct Epi {
  bf16_t* C;
  bf16_t* ab;
  bf16_t* dh;
  int N;   // output columns (fc1, dgrad: F; fc2: D)
};

// kDgrad for columns n..n+3 of the row starting at element `row` (m * N): v holds the dh
// sums, pa and pb the packed bf16 a and b of those columns.
__device__ __forceinline__ void dgrad4(const Epi& ep, size_t row, int n, const float* v, uint2 pa,
                                       uint2 pb) {
  const float a[4] = {bf16_lo(pa.x), bf16_hi(pa.x), bf16_lo(pa.y), bf16_hi(pa.y)};
  const float b[4] = {bf16_lo(pb.x), bf16_hi(pb.x), bf16_lo(pb.y), bf16_hi(pb.y)};
  float d[4], da[4], db[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d[i] = bf16_to_f32(f32_to_bf16(v[i]));              // dh as stored
    const float s = sigmoid(a[i]);      // sigmoid; silu = a*s
    db[i] = d[i] * (a[i] * s);
    da[i] = d[i] * b[i] * (s * (1.0f + a[i] * (1.0f - s)));
  }
  bf16_t* p = ep.C + 2 * row + n;
  store4(p, da[0], da[1], da[2], da[3]);
  store4(p + ep.N, db[0], db[1], db[2], db[3]);
  if (ep.dh) store4(ep.dh + row + n, d[0], d[1], d[2], d[3]);
}

// Four consecutive output columns n..n+3 of row m; u holds the w3 sums for kFc1.
template <int MODE>
__device__ __forceinline__ void emit4(const Epi& ep, int m, int n, const float* v, const float* u) {
  const size_t row = (size_t)m * ep.N;
  if (MODE == kFc1) {
    store4(ep.C + row + n, silu_mul(v[0], u[0]), silu_mul(v[1], u[1]), silu_mul(v[2], u[2]),
           silu_mul(v[3], u[3]));
    if (ep.ab) {
      bf16_t* p = ep.ab + 2 * row + n;
      store4(p, v[0], v[1], v[2], v[3]);
      store4(p + ep.N, u[0], u[1], u[2], u[3]);
    }
  } else if (MODE == kFc2) {
    store4(ep.C + row + n, v[0], v[1], v[2], v[3]);
  } else {
    dgrad4(ep, row, n, v, *reinterpret_cast<const uint2*>(ep.ab + 2 * row + n),
           *reinterpret_cast<const uint2*>(ep.ab + 2 * row + ep.N + n));
  }
}

// Exclusive prefix sum over the threads of the block (up to 16 waves).
__device__ __forceinline__ int block_scan_excl(int v, int* wtot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wtot[wid] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wid; ++w) before += wtot[w];
  return before + inc - v;
}

// rows: the tile's rows of its segment (pad rows included); vrows: how many of them, from
// the first, hold tokens (rows past them are pad rows, whose outputs are zero).
struct Tile {
  int e, m0, rows, n0, vrows;
};

// Each operand of a tile is staged per k-step as 256 "rows" (A rows or panel rows,
// the MFMA's M or N index) x 64 k values, in one of two LDS layouts:
//  * K-contiguous (the operand's rows hold k contiguous in memory): 256 LDS rows of
//    128 bytes. Piece j of wave w holds rows 64*j + 8*w .. +7; lane l fills row
//    64*j + lrow with lrow = 8*w + l/8, 16-byte slot l%8, which holds logical chunk
//    (l%8) ^ ((row/2)%8). Rows past the tile or the matrix are clamped to the last one.
//  * MN-major (the operand is stored [k][n], n contiguous, e.g. w2 [E,D,F] read as the
//    dgrad's [F x D] panel, or activations [rows, N] read over their rows in the wgrad):
//    64 LDS rows (one per k) of 512 bytes. Piece j of wave w holds k rows
//    2*(8*j + w) and +1 (l / 32); lane l fills 16-byte slot l%32 of its row with the 8
//    columns of logical slot (l%32) ^ (4*(k%4)). Fragments are read back with the
//    gfx950 transposing LDS load (see frag_mn).
// Both layouts fill 1 KiB per wave and piece, at the same LDS offsets.
struct TileLoads {
  i32x4 rsa, rsb, rsb2;
  uint32_t aoff[4], boff[4];
  uint32_t astep, bstep;   // bytes between k-steps (K-contiguous: 128; MN-major: 64 rows)
  int bsplit;              // k-steps read from rsb; the following ones from rsb2, from its start
  int na;                  // A pieces per wave: 4 for a full tile, 2 for a half K-contiguous one
};

// Byte offset of lane's 16 bytes of piece j in an MN-major operand with row pitch ld.
__device__ __forceinline__ uint32_t mn_off(int j, int ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = 2 * (8 * j + wave) + (lane >> 5);
  return (uint32_t)(r * ld + 8 * ((lane & 31) ^ (4 * (r & 3)))) * 2u;
}

// Loads of an m-grouped tile: A = rows [m0, m0 + rows) of a K-contiguous [m][K] buffer;
// the panel = expert e's weights from panel row n0:
//   P_MN false: W1 [E][N][K] (fc1 interleaves W1 and W3 rows in 32-row blocks);
//   P_MN true:  [E][K][N] read MN-major, the first `ksplit` k from W1 [E][ksplit][N] and
//               the rest from W3 [E][K - ksplit][N] (ksplit = K: W1 only).
// EB: bytes per element (2: bf16; 1: the FP8 payload, whose 64-wide k-steps hold 128
// k values in the same 128-byte LDS rows).
template <bool FC1, bool P_MN, int EB = 2>
__device__ __forceinline__ TileLoads tile_loads(const Tile& t, const bf16_t* __restrict__ A,
                                                const bf16_t* __restrict__ W1,
                                                const bf16_t* __restrict__ W3, int K, int N,
                                                int ksplit) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = 8 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ ((lrow >> 1) & 7);
  TileLoads o;
  o.na = t.rows > BM / 2 ? 4 : 2;
  const char* Ab = reinterpret_cast<const char*>(A);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o.aoff[j] = (uint32_t)(min(64 * j + lrow, t.rows - 1) * K) * EB + lchunk * 16;
  // the descriptor ends at the last row holding a token: pad rows read as zeros
  o.rsa = buffer_rsrc(Ab + (size_t)t.m0 * K * EB, (uint32_t)t.vrows * K * EB);
  o.astep = BK * 2;
  if (P_MN) {
    // columns past N read into the next row (or past the end, zero-filled): such panel
    // rows only feed output columns that are not stored
    o.rsb = buffer_rsrc(W1 + (size_t)t.e * ksplit * N + t.n0, (uint32_t)(ksplit * N - t.n0) * 2u);
    o.rsb2 = ksplit < K ? buffer_rsrc(W3 + (size_t)t.e * (K - ksplit) * N + t.n0,
                                      (uint32_t)((K - ksplit) * N - t.n0) * 2u)
                        : o.rsb;
#pragma unroll
    for (int j = 0; j < 4; ++j) o.boff[j] = mn_off(j, N);
    o.bstep = (uint32_t)BK * N * 2u;
    o.bsplit = ksplit / BK;
  } else {
    // fc1: panel rows alternate 32-row blocks of w1 and w3 over the same 32 columns;
    // row 64*j + lrow is in a w3 block exactly when lrow >= 32, i.e. for waves 4..7
    const char* wsel = reinterpret_cast<const char*>((FC1 && wave >= 4) ? W3 : W1);
    o.rsb = buffer_rsrc(wsel + (size_t)t.e * N * K * EB, (uint32_t)N * K * EB);
    o.rsb2 = o.rsb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pr = 64 * j + lrow;
      const int gr = FC1 ? t.n0 + (pr >> 6) * 32 + (pr & 31) : t.n0 + pr;
      o.boff[j] = (uint32_t)(min(gr, N - 1) * K) * EB + lchunk * 16;
    }
    o.bstep = BK * 2;
    o.bsplit = 1 << 30;
  }
  return o;
}

// Loads of k-step kt into the LDS stage at `la` (this wave's first piece): the A pieces
// (part 0) or the panel pieces (part 1).
// NA > 0 gives the number of A pieces at compile time (it must equal o.na), which keeps
// the issue free of branches.
template <int NA = 0>
__device__ __forceinline__ void issue_loads(const TileLoads& o, uint32_t la, int kt, int part) {
  if (part == 0) {
    const uint32_t ko = (uint32_t)kt * o.astep;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (NA > 0 ? j < NA : j < o.na) dma16(o.rsa, o.aoff[j], ko, la + j * 8192);
  } else {
    const uint32_t lb = la + A_BYTES;
    const bool second = kt >= o.bsplit;
    const i32x4 rs = second ? o.rsb2 : o.rsb;
    const uint32_t ko = (uint32_t)(second ? kt - o.bsplit : kt) * o.bstep;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(rs, o.boff[j], ko, lb + j * 8192);
  }
}

// MFMA fragment of 32 rows (MFMA index nbase .. +31) for k slice ks from an MN-major
// stage: lane l gets index nbase + l%32 and k = 16*ks + 8*(l/32) .. +7, as two
// transposing 8-byte LDS loads. Within each 16-lane group, lane j of the load names row
// k0 + j/4 and the 4 columns starting at 4*(j%4) of the group's 16, and the hardware hands
// lane i column i of that 16 x 4 block, i.e. 4 consecutive k of one column. Row k's
// 8-byte units are XOR-swizzled by 8*(k%4) (matching the loads), so the 16 lanes of a
// group and the two groups of a half-wave hit distinct banks.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 frag_mn(const char* stage, int nbase, int ks) {
  const int lane = threadIdx.x & 63;
  const int q = (lane >> 2) & 3;
  const int k = ks * 16 + (lane >> 5) * 8 + q;
  const int u = (nbase >> 2) + ((lane >> 4) & 1) * 4 + (lane & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const __attribute__((address_space(3))) char* p =
      (const __attribute__((address_space(3))) char*)stage + k * 512 + ((u ^ (8 * q)) << 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 512));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// One tile: rows [m0, m0 + rows) of expert e against the weight panel from n0, k-steps
// [kb, ke).
//
// Eight waves, two per SIMD. Full tile: wave w owns rows 128*(w%2) .. +127 and panel
// rows 64*(w/2) .. +63 (4 x 2 MFMA blocks of 32x32, 128 accumulators). Half tile
// (rows <= 128): rows 64*(w%2) .. +63 and the same panel rows (2 x 2 blocks).
// For fc1 the 64 panel rows of a wave are one w1 block and one w3 block covering the
// same 32 h columns, so silu(a)*b is formed in registers.
//
// Pipeline: two LDS stages filled by direct buffer->LDS loads; step kb uses stage
// `stage0`. Iteration kt waits for its own loads of its stage, meets the other waves
// at a barrier (after which every wave has finished reading the other stage and all
// of this one has landed), then runs the MFMAs of kt with the fragments of the next
// 16-wide k slice loaded while the current slice's MFMAs run. The loads of k-step
// kt+1 into the free stage are issued in two halves (A, then the panel) under the
// first two slices, which keeps the memory system from seeing all of a CU's requests
// in one burst (5-8% faster than issuing them right after the barrier). In the last
// step the free stage instead receives the first step of the next tile (`nxt`, step
// `nkb`), so its load latency hides under this tile's last MFMAs and its epilogue;
// `primed` says that this tile's first step was loaded that way.
//
// GUARD: the tile's rows from `vrows` on hold no token (pad rows, read as zeros): a
// wave runs no MFMA for its 32-row blocks that lie wholly among them.
template <bool HALF, bool A_MN, bool P_MN, bool GUARD = false>
__device__ __forceinline__ void mainloop(char* smem, const TileLoads& ld, int kb, int ke,
                                         int stage0, bool primed, const TileLoads& nxt,
                                         bool has_next, int nkb, f32x16 (&acc)[HALF ? 2 : 4][2],
                                         int vrows = BM) {
  constexpr int WM = HALF ? 2 : 4;   // 32-row blocks of A per wave
  constexpr int WN = 2;              // 32-row panel blocks per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);   // first A row of this wave
  const int prow0 = (wave >> 1) * 64;                 // first panel row of this wave
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;
  const int nmb = GUARD ? max(0, min(WM, (vrows - arow0 + 31) >> 5)) : WM;

#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31;
  if (!primed) {
    issue_loads(ld, lds0 + stage0 * STAGE_BYTES, kb, 0);
    issue_loads(ld, lds0 + stage0 * STAGE_BYTES, kb, 1);
  }
  for (int kt = kb; kt < ke; ++kt) {
    const int cur = (stage0 + kt - kb) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* sa = smem + cur * STAGE_BYTES;
    const char* sb = sa + A_BYTES;
    bf16x8 wf[2][WN], af[2][WM];
    auto frag = [&](int ks, int buf) {
      const int chk = ks * 2 + (lane >> 5);
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
        wf[buf][nb] = P_MN ? frag_mn(sb, prow0 + nb * 32, ks)
                           : *reinterpret_cast<const bf16x8*>(sb + swz(prow0 + nb * 32 + fr, chk));
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
        af[buf][mb] = A_MN ? frag_mn(sa, arow0 + mb * 32, ks)
                           : *reinterpret_cast<const bf16x8*>(sa + swz(arow0 + mb * 32 + fr, chk));
    };
    frag(0, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      // the next stage's loads go out in two halves under the first two k slices
      // rather than in one burst after the barrier
      if (ks < 2) {
        if (kt + 1 < ke) issue_loads(ld, lds0 + (cur ^ 1) * STAGE_BYTES, kt + 1, ks);
        else if (has_next) issue_loads(nxt, lds0 + (cur ^ 1) * STAGE_BYTES, nkb, ks);
      }
      if (ks + 1 < BK / 16) frag(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        if (GUARD && mb >= nmb) continue;
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][nb], af[ks & 1][mb],
                                                                acc[mb][nb], 0, 0, 0);
      }
    }
  }
  // No barrier here: the next tile's first step went into the stage nobody reads in
  // this tile's last step, and its second step's loads are issued only after its
  // first barrier, which every wave reaches after finishing this tile's MFMAs.
}

// Barrier for LDS traffic only: this wave's LDS accesses are complete, then every wave
// meets; outstanding global loads (the next tile's first stage) keep flying.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// kDgrad epilogue through LDS. The lane layout of the accumulators (4 consecutive
// columns of 32 different rows per instruction) would make the ab loads and dab stores
// touch 32 rows x 8 bytes per wave instruction; instead dh (rounded to bf16, as stored)
// goes into the LDS stage the tile's last k-step used (free once every wave has passed
// the barrier below), 128 rows x 256 columns per pass, and is read back by rows, so the
// ab loads and the dab and dh stores are whole 16-byte chunks of consecutive columns.
// LDS rows are 512 bytes; the 8-byte unit u of row r is stored at u ^ (r % 32), so the
// 32 rows a half-wave writes hit 32 distinct bank pairs, and a 16-byte row read lands
// on chunk c ^ ((r % 32) / 2) with its halves swapped when r is odd.
template <bool HALF>
__device__ __forceinline__ void dgrad_epilogue(char* stage, const Tile& t, const Epi& ep,
                                               const f32x16 (&acc)[HALF ? 2 : 4][2]) {
  constexpr int WM = HALF ? 2 : 4;
  constexpr int PASSES = HALF ? 1 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);
  const int prow0 = (wave >> 1) * 64;
  const int fr = lane & 31;
  const int N = ep.N;
  // dh as stored (bf16), packed now: half the registers of the float32 sums
  uint2 pk[WM][2][4];
#pragma unroll
  for (int mb = 0; mb < WM; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[mb][nb];
        pk[mb][nb][g] = uint2{pack_bf16x2(a[4 * g], a[4 * g + 1]),
                              pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
      }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    lds_barrier();   // the stage is free: MFMA reads (or the previous pass) are done
    if (HALF || (wave & 1) == p) {
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        const int rl = (HALF ? arow0 : 0) + mb * 32 + fr;   // row within the pass
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int u = (prow0 + nb * 32 + g * 8 + (lane >> 5) * 4) >> 2;
            *reinterpret_cast<uint2*>(stage + rl * 512 + ((u ^ (rl & 31)) << 3)) = pk[mb][nb][g];
          }
      }
    }
    lds_barrier();
    // 128 rows x 32 chunks of 8 columns; 16 rows per round of the 512 threads
    const int c = threadIdx.x & 31;
    const int n = t.n0 + 8 * c;
#pragma unroll
    for (int it0 = 0; it0 < 8; it0 += 4) {
      uint4 va[4], vb[4];
      bool ok[4];
      size_t row[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = (threadIdx.x >> 5) + 16 * (it0 + i);
        const int r = p * 128 + rl;
        ok[i] = r < t.rows && n < N;
        row[i] = (size_t)(t.m0 + r) * N;
        va[i] = vb[i] = uint4{0u, 0u, 0u, 0u};   // pad rows: dh = 0 and a = b = 0 give zeros
        if (ok[i] && r < t.vrows) {
          va[i] = *reinterpret_cast<const uint4*>(ep.ab + 2 * row[i] + n);
          vb[i] = *reinterpret_cast<const uint4*>(ep.ab + 2 * row[i] + N + n);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!ok[i]) continue;
        const int rl = (threadIdx.x >> 5) + 16 * (it0 + i);
        const int m = rl & 31;
        uint4 d = *reinterpret_cast<const uint4*>(stage + rl * 512 + ((c ^ (m >> 1)) << 4));
        if (m & 1) d = uint4{d.z, d.w, d.x, d.y};
        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
        const uint32_t aw[4] = {va[i].x, va[i].y, va[i].z, va[i].w};
        const uint32_t bw[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
        uint32_t oa[4], ob[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float da2[2], db2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float dh = h ? bf16_hi(dw[q]) : bf16_lo(dw[q]);
            const float av = h ? bf16_hi(aw[q]) : bf16_lo(aw[q]);
            const float bv = h ? bf16_hi(bw[q]) : bf16_lo(bw[q]);
            const float sg = sigmoid(av);   // sigmoid; silu = a*s
            db2[h] = dh * (av * sg);
            da2[h] = dh * bv * (sg * (1.0f + av * (1.0f - sg)));
          }
          oa[q] = pack_bf16x2(da2[0], da2[1]);
          ob[q] = pack_bf16x2(db2[0], db2[1]);
        }
        *reinterpret_cast<uint4*>(ep.C + 2 * row[i] + n) = uint4{oa[0], oa[1], oa[2], oa[3]};
        *reinterpret_cast<uint4*>(ep.C + 2 * row[i] + N + n) = uint4{ob[0], ob[1], ob[2], ob[3]};
        if (ep.dh) *reinterpret_cast<uint4*>(ep.dh + row[i] + n) = uint4{d.x, d.y, d.z, d.w};
      }
    }
  }
}

// kFc2 epilogue through LDS, the same passes as the dgrad epilogue: the sums, rounded
// to bf16, go into free LDS of the tile's last k-step, 128 rows x 256 columns per
// pass, and come back by rows, so every store is a whole 16-byte chunk and 32 lanes
// write 512 consecutive bytes of one row. Stored straight from the accumulator layout, a
// wave instruction would touch 32 rows with 16 bytes each. Rows 0-63 of a pass go to
// `lo`, rows 64-127 to `hi` (32 KiB each: the halves of a stage, or the ring's free
// activation and panel slots).
template <bool HALF>
__device__ __forceinline__ void fc2_epilogue(char* lo, char* hi, const Tile& t, const Epi& ep,
                                             const f32x16 (&acc)[HALF ? 2 : 4][2]) {
  auto row = [&](int rl) { return (rl < 64 ? lo : hi) + (rl & 63) * 512; };
  constexpr int WM = HALF ? 2 : 4;
  constexpr int PASSES = HALF ? 1 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);
  const int prow0 = (wave >> 1) * 64;
  const int fr = lane & 31;
  const int N = ep.N;
  uint2 pk[WM][2][4];
#pragma unroll
  for (int mb = 0; mb < WM; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[mb][nb];
        pk[mb][nb][g] = uint2{pack_bf16x2(a[4 * g], a[4 * g + 1]),
                              pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
      }
  const int c = threadIdx.x & 31;
  const int n = t.n0 + 8 * c;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    lds_barrier();   // the stage is free: MFMA reads (or the previous pass) are done
    if (HALF || (wave & 1) == p) {
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        const int rl = (HALF ? arow0 : 0) + mb * 32 + fr;   // row within the pass
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int u = (prow0 + nb * 32 + g * 8 + (lane >> 5) * 4) >> 2;
            *reinterpret_cast<uint2*>(row(rl) + ((u ^ (rl & 31)) << 3)) = pk[mb][nb][g];
          }
      }
    }
    lds_barrier();
    // 128 rows x 32 chunks of 8 columns; 16 rows per round of the 512 threads
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rl = (threadIdx.x >> 5) + 16 * it;
      const int r = p * 128 + rl;
      if (r >= t.rows || n >= N) continue;
      const int m = rl & 31;
      uint4 d = *reinterpret_cast<const uint4*>(row(rl) + ((c ^ (m >> 1)) << 4));
      if (m & 1) d = uint4{d.z, d.w, d.x, d.y};
      *reinterpret_cast<uint4*>(ep.C + (size_t)(t.m0 + r) * N + n) = d;
    }
  }
}

// The end of a tile: the raw float32 sums of a split-K share (`part`, row-major
// [BM][BP]) or the MODE epilogue. Lane l holds column m = l % 32 of every 32x32 block
// and panel rows 8*g + 4*(l / 32) + i (i = 0..3) for g = 0..3.
// ELO, EHI: the free LDS the fc2 epilogue stages through (default: the two halves of the
// stage the last k-step used).
template <int MODE, bool HALF>
__device__ __forceinline__ void finish_tile(char* smem, const Tile& t, const Epi& ep, int kb,
                                            int ke, float* __restrict__ part, int stage0,
                                            const f32x16 (&acc)[HALF ? 2 : 4][2],
                                            char* elo = nullptr, char* ehi = nullptr) {
  constexpr int WM = HALF ? 2 : 4;
  constexpr int WN = 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);
  const int prow0 = (wave >> 1) * 64;
  const int fr = lane & 31;
  if (part) {
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
      const int r = arow0 + mb * 32 + fr;
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int pr = prow0 + nb * 32 + g * 8 + (lane >> 5) * 4;
          const f32x16& a = acc[mb][nb];
          float4 v = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
          *reinterpret_cast<float4*>(part + r * BP + pr) = v;
        }
    }
    return;
  }
  if (MODE == kDgrad) {
    dgrad_epilogue<HALF>(smem + ((stage0 + ke - kb - 1) & 1) * STAGE_BYTES, t, ep, acc);
    return;
  }
  if (MODE == kFc2) {
    char* st = smem + ((stage0 + ke - kb - 1) & 1) * STAGE_BYTES;
    fc2_epilogue<HALF>(elo ? elo : st, ehi ? ehi : st + A_BYTES, t, ep, acc);
    return;
  }
#pragma unroll
  for (int mb = 0; mb < WM; ++mb) {
    const int r = arow0 + mb * 32 + fr;
    if (r >= t.rows) continue;
    const int m = t.m0 + r;
    if (MODE == kFc1) {
      // the wave's two panel blocks are the w1 and w3 rows of the same 32 h columns
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = t.n0 + prow0 / 2 + g * 8 + (lane >> 5) * 4;
        if (n >= ep.N) continue;
        const f32x16& a = acc[mb][0];
        const f32x16& b = acc[mb][1];
        const float v[4] = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
        const float u[4] = {b[4 * g], b[4 * g + 1], b[4 * g + 2], b[4 * g + 3]};
        emit4<MODE>(ep, m, n, v, u);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < WN; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = t.n0 + prow0 + nb * 32 + g * 8 + (lane >> 5) * 4;
          if (n >= ep.N) continue;
          const f32x16& a = acc[mb][nb];
          const float v[4] = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
          emit4<MODE>(ep, m, n, v, v);
        }
      }
    }
  }
}

// One tile of the m-grouped kernel: the main loop, then finish_tile.
template <int MODE, bool HALF, bool P_MN, bool GUARD = false>
__device__ __forceinline__ void run_tile(char* smem, const Tile& t, const TileLoads& ld,
                                         const Epi& ep, int kb, int ke,
                                         float* __restrict__ part, int stage0, bool primed,
                                         const TileLoads& nxt, bool has_next, int nkb) {
  f32x16 acc[HALF ? 2 : 4][2];
  mainloop<HALF, false, P_MN, GUARD>(smem, ld, kb, ke, stage0, primed, nxt, has_next, nkb, acc,
                                     t.vrows);
  finish_tile<MODE, HALF>(smem, t, ep, kb, ke, part, stage0, acc);
}

// ---------------------------------------------------------------------------
// fc1 on the FP8 payload ("Expert Parallelism (EP)", section 6 "DeepSeek-V3 量级的示例
// 数字": the dispatch payload is FP8 e4m3 with scales): activations and w1, w3 in OCP
// e4m3 with one E8M0 scale per 32 values along K, on v_mfma_scale_f32_32x32x64_f8f6f4. A k-step holds 128 k (128-byte LDS
// rows, the bf16 kernel's stage layout); each of its two 64-wide slices is one scaled
// MFMA per block. In that instruction lane l supplies row (or column) l % 32 and 32 of
// the slice's 64 k values as two 16-byte halves, and one scale byte: the first halves
// of lanes l and l + 32 form one 32-value scale block, scaled by lane l's byte, the
// second halves the other, scaled by lane l + 32's (the pairing of k values between the
// two operands follows the same placement, so any consistent order contracts right;
// checked on the device with in-bounds probes before this kernel used them).
// ---------------------------------------------------------------------------
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// The scales in k-step words: word (s, r) at [s * rows + r] holds row r's four E8M0
// bytes for k step s (128 values), so a wave's 32 rows of one step are 128 consecutive
// bytes.
struct MxScales {
  const uint32_t* a;    // [K/128][ra]: the activation rows
  const uint32_t* w1;   // [K/128][E*N]: rows e*N + n
  const uint32_t* w3;
  int64_t ra;
};

// This wave's scale words for k-step kt: its A rows and its two panel blocks (w1 rows,
// then w3 rows, of the same columns).
template <bool HALF>
__device__ __forceinline__ void mx_scale_words(const Tile& t, const MxScales& ms, int E, int N,
                                               int kt, uint32_t (&sa)[HALF ? 2 : 4],
                                               uint32_t (&sw)[2]) {
  constexpr int WM = HALF ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);
  const int prow0 = (wave >> 1) * 64;
  const int fr = lane & 31;
  const uint32_t* a = ms.a + (size_t)kt * ms.ra + t.m0;
#pragma unroll
  for (int mb = 0; mb < WM; ++mb) sa[mb] = a[min(arow0 + mb * 32 + fr, t.rows - 1)];
  const size_t wrow = (size_t)kt * E * N + (size_t)t.e * N + min(t.n0 + prow0 / 2 + fr, N - 1);
  sw[0] = ms.w1[wrow];
  sw[1] = ms.w3[wrow];
}

// The MFMAs of one k step (two 64-wide slices) from the LDS stage at sA / sB, with the
// next stage's loads issued in two halves by `issue(part)`: the A pieces before the
// first MFMA, the panel pieces after the first panel block's MFMAs (a quarter of the
// step; at the start of the second slice they land 2-4% later). Lane half h takes
// 16-byte chunks 4*ks + h and 4*ks + 2 + h of slice ks: the first half of both lanes of
// a row is the slice's first MX block, the second half the other. There is one set of
// fragments (8 registers each; a second set would not fit beside the 128 accumulators),
// and it rolls: the MFMAs go panel block by panel block, and each fragment of the
// second slice is read as soon as the first slice's last MFMA on that register has been
// issued, so every read has several MFMAs to land under. The order is pinned (the
// compiler would otherwise hoist the reads, which needs a second set of registers).
template <bool HALF, typename Issue>
__device__ __forceinline__ void mx_step(const char* sA, const char* sB,
                                        const uint32_t (&sa)[HALF ? 2 : 4],
                                        const uint32_t (&sw)[2],
                                        f32x16 (&acc)[HALF ? 2 : 4][2], Issue issue) {
  constexpr int WM = HALF ? 2 : 4;
  constexpr int WN = 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);
  const int prow0 = (wave >> 1) * 64;
  const int fr = lane & 31;
  const int half = lane >> 5;
  auto frag = [&](const char* base, int r, int ks) {
    const int c0 = 4 * ks + half;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(r, c0));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(r, c0 + 2));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  i32x8 wf[WN], af[WM];
#pragma unroll
  for (int nb = 0; nb < WN; ++nb) wf[nb] = frag(sB, prow0 + nb * 32 + fr, 0);
#pragma unroll
  for (int mb = 0; mb < WM; ++mb) af[mb] = frag(sA, arow0 + mb * 32 + fr, 0);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks == 0) issue(0);
    // lane half h supplies the scale of block 2*ks + h of the step, in byte 0 (the byte
    // the instruction reads with op_sel 0)
    const int sh = 8 * (2 * ks + half);
#pragma unroll
    for (int nb = 0; nb < WN; ++nb) {
#pragma unroll
      for (int mb = 0; mb < WM; ++mb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            wf[nb], af[mb], acc[mb][nb], 0, 0, 0, (int)((sw[nb] >> sh) & 0xFFu), 0,
            (int)((sa[mb] >> sh) & 0xFFu));
        if (ks == 0 && nb == WN - 1) af[mb] = frag(sA, arow0 + mb * 32 + fr, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ks == 0) wf[nb] = frag(sB, prow0 + nb * 32 + fr, 1);
      if (ks == 0 && nb == 0) issue(1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The operands of the FP8 fc1: the load descriptors and per-lane offsets of a tile are
// built from these where they are needed (the next tile's only in the last step), so
// they do not occupy registers through the main loop.
struct MxSrc {
  const bf16_t* A;
  const bf16_t* W1;
  const bf16_t* W3;
  int K, N;
  __device__ TileLoads loads(const Tile& t) const {
    return tile_loads<true, false, 1>(t, A, W1, W3, K, N, K);
  }
};

// The bf16 main loop's pipeline (same stages, barrier, split issue and cross-tile
// prefetch) with FP8 fragments and scaled MFMAs. The steps before the last issue the
// next step of this tile with no branch in the loop body, so the compiler keeps the
// MFMAs between the two halves of the issue; the last step, peeled off, issues the
// first step of the next tile `nt`.
template <bool HALF>
__device__ __forceinline__ void mainloop_mx(char* smem, const TileLoads& ld, int kb, int ke,
                                            int stage0, bool primed, const Tile& nt,
                                            const MxSrc& src, bool has_next, int nkb,
                                            const Tile& t, const MxScales& ms, int E, int N,
                                            f32x16 (&acc)[HALF ? 2 : 4][2]) {
  constexpr int WM = HALF ? 2 : 4;
  constexpr int WN = 2;
  const int wave = threadIdx.x >> 6;
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  if (!primed) {
    issue_loads(ld, lds0 + stage0 * STAGE_BYTES, kb, 0);
    issue_loads(ld, lds0 + stage0 * STAGE_BYTES, kb, 1);
  }
  // the scale words run one step ahead of the MFMAs, like the stage loads
  uint32_t na[WM], nw[WN];
  if (kb >= ke) return;
  mx_scale_words<HALF>(t, ms, E, N, kb, na, nw);
  // step kt: wait for its stage, take its scale words, fetch the next step's
  auto enter = [&](int kt, uint32_t (&sa)[WM], uint32_t (&sw)[WN]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The compiler counts only its own loads (the scale words), not the stage copies
    // issued from inline asm, so it would place its wait for these words before their
    // first MFMA, after the next stage's copies have gone out, and that wait would
    // drain them too. Using the words here, where every load has already landed, puts
    // its wait here instead.
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      sa[i] = na[i];
      asm volatile("" ::"v"(sa[i]));
    }
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      sw[i] = nw[i];
      asm volatile("" ::"v"(sw[i]));
    }
  };
  int kt = kb;
  for (; kt + 1 < ke; ++kt) {
    const int cur = (stage0 + kt - kb) & 1;
    uint32_t sa[WM], sw[WN];
    enter(kt, sa, sw);
    mx_scale_words<HALF>(t, ms, E, N, kt + 1, na, nw);
    const char* sA = smem + cur * STAGE_BYTES;
    const uint32_t lnext = lds0 + (cur ^ 1) * STAGE_BYTES;
    mx_step<HALF>(sA, sA + A_BYTES, sa, sw, acc, [&](int ks) {
      issue_loads<HALF ? 2 : 4>(ld, lnext, kt + 1, ks);
    });
  }
  // the last step: the free stage receives the next tile's first step
  const int cur = (stage0 + kt - kb) & 1;
  uint32_t sa[WM], sw[WN];
  enter(kt, sa, sw);
  const char* sA = smem + cur * STAGE_BYTES;
  const uint32_t lnext = lds0 + (cur ^ 1) * STAGE_BYTES;
  const TileLoads nxt = src.loads(nt);   // nt is this tile when there is no next one
  mx_step<HALF>(sA, sA + A_BYTES, sa, sw, acc, [&](int ks) {
    if (has_next) issue_loads(nxt, lnext, nkb, ks);
  });
}

template <bool HALF>
__device__ __forceinline__ void run_tile_mx(char* smem, const Tile& t, const Epi& ep, int kb,
                                            int ke, float* __restrict__ part, int stage0,
                                            bool primed, const Tile& nt, bool has_next, int nkb,
                                            const MxSrc& src, const MxScales& ms, int E, int N) {
  f32x16 acc[HALF ? 2 : 4][2];
  const TileLoads ld = src.loads(t);
  mainloop_mx<HALF>(smem, ld, kb, ke, stage0, primed, nt, src, has_next, nkb, t, ms, E, N, acc);
  finish_tile<kFc1, HALF>(smem, t, ep, kb, ke, part, stage0, acc);
}

// The rows of each expert: contiguous segments [offsets[e], offsets[e+1]) (cap = 0), of
// which the first counts[e] hold tokens and the rest are zero pad rows (counts may be
// null: then every row is treated as a token row), or the masked layout's slabs, rows
// [e*cap, e*cap + min(counts[e], cap)) (cap > 0).
struct Segs {
  const int32_t* offsets;
  const int32_t* counts;
  int cap;
};

// Per-workgroup schedule tables in LDS: segment bounds and the first 256-row block of
// each expert, built from the offsets or counts on the device.
struct Sched {
  int segoff[MAXE + 1];   // segment starts (clamped to the rows in use)
  int segend[MAXE];       // segment ends
  int segval[MAXE];       // ends of the rows that hold tokens (segoff <= segval <= segend)
  int tstart[MAXE + 1];   // first 256-row block of each expert
  int wtot[16];
};

__device__ void build_sched(Sched& sc, const Segs& sg, int E, int m_cap) {
  const int tid = threadIdx.x;
  if (sg.cap > 0) {
    for (int e = tid; e < E; e += blockDim.x) {
      sc.segoff[e] = e * sg.cap;
      sc.segend[e] = e * sg.cap + max(0, min(sg.counts[e], sg.cap));
      sc.segval[e] = sc.segend[e];
    }
  } else {
    // clamped into [0, min(offsets[E], m_cap)], so offsets that break the contract
    // (negative, decreasing, past m_cap) can only shrink the work, never move it outside;
    // the token rows end inside their segment whatever counts holds
    const int mend = max(0, min(sg.offsets[E], m_cap));
    for (int e = tid; e <= E; e += blockDim.x) sc.segoff[e] = max(0, min(sg.offsets[e], mend));
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
      sc.segend[e] = sc.segoff[e + 1];
      sc.segval[e] = sg.counts ? max(sc.segoff[e], min(sc.segoff[e] + max(sg.counts[e], 0),
                                                       sc.segend[e]))
                               : sc.segend[e];
    }
  }
  __syncthreads();
  const int per = (MAXE + blockDim.x - 1) / blockDim.x;   // experts per thread (<= 4)
  int cnt[4], local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * per + i;
    cnt[i] = (i < per && e < E) ? (max(sc.segend[e] - sc.segoff[e], 0) + BM - 1) / BM : 0;
    local += cnt[i];
  }
  int run = block_scan_excl(local, sc.wtot);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * per + i;
    if (i < per && e < E) sc.tstart[e] = run;
    run += cnt[i];
  }
  if (tid == (int)blockDim.x - 1) sc.tstart[E] = run;
  __syncthreads();
}

// Tiles are numbered expert by expert: expert e owns items [tstart[e], tstart[e+1]) * n_nt,
// nb_e row blocks x n_nt column tiles, walked in groups of up to GROUP_M row blocks per
// column sweep so every weight panel is used by all (or GROUP_M) row blocks of its
// expert back to back.
__device__ Tile decode_item(const Sched& sc, int E, int n_nt, int cols, int w) {
  const int blk = w / n_nt;
  int lo = 0, hi = E;   // largest expert whose first block is <= blk
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sc.tstart[mid] <= blk) lo = mid; else hi = mid;
  }
  const int nb_e = sc.tstart[lo + 1] - sc.tstart[lo];
  const int local = w - sc.tstart[lo] * n_nt;
  const int gsz = min(GROUP_M, nb_e);
  const int grp = local / (gsz * n_nt);
  const int first = grp * gsz;
  const int gm = min(gsz, nb_e - first);
  const int within = local - grp * gsz * n_nt;
  const int mb = sc.tstart[lo] + first + within % gm;
  Tile t;
  t.e = lo;
  t.m0 = sc.segoff[lo] + (mb - sc.tstart[lo]) * BM;
  t.rows = min(BM, sc.segend[lo] - t.m0);
  t.vrows = max(0, min(t.rows, sc.segval[lo] - t.m0));
  t.n0 = (within / gm) * cols;
  return t;
}

// Split-K tail: when the last round of tiles would leave at least half of the G
// workgroups idle, each of its `tail` tiles is cut into S k-ranges (S * tail <= G and
// <= the workspace slots). Share sh of tail tile i is item full + sh*tail + i and writes
// its float32 sums to workspace slot sh*tail + i; gg_tail_reduce adds the shares in
// order sh = 0..S-1. Items [0, full) are whole tiles.
struct Split {
  int full, tail, S, nks;
};

__device__ Split split_plan(int total, int G, int slots, int nk) {
  Split p;
  const int rounds = (total + G - 1) / G;
  p.full = total;
  p.tail = 0;
  p.S = 1;
  p.nks = nk;
  if (total == 0 || rounds == 0) return p;
  const int tail = total - (rounds - 1) * G;
  if (tail > 0 && 2 * tail <= G && slots >= 2 * tail && nk >= 2) {
    int S = min(min(8, G / tail), min(slots / tail, nk));
    const int nks = (nk + S - 1) / S;
    S = (nk + nks - 1) / nks;   // no empty share
    if (S >= 2) {
      p.full = (rounds - 1) * G;
      p.tail = tail;
      p.S = S;
      p.nks = nks;
    }
  }
  return p;
}

// P_MN: the weights are read MN-major (see tile_loads); ksplit as there. MX: fc1 on the
// FP8 payload (A, W1, W3 hold e4m3 bytes, ms their scales).
template <int MODE, bool P_MN, bool MX = false>
__global__ __launch_bounds__(NTHR, 1) void gg_bf16_kernel(
    const bf16_t* __restrict__ A, Segs sg, int E, int K, int N,
    int m_cap, const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W3, int ksplit,
    Epi ep, float* __restrict__ ws, int slots, MxScales ms) {
  constexpr bool FC1 = MODE == kFc1;
  constexpr int EB = MX ? 1 : 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  __shared__ Sched sc;
  build_sched(sc, sg, E, m_cap);

  const int cols = FC1 ? BP / 2 : BP;
  const int n_nt = (N + cols - 1) / cols;
  const int total = sc.tstart[E] * n_nt;
  const int nk = K * EB / (BK * 2);   // 128-byte k-steps
  const Split sp = split_plan(total, gridDim.x, ws ? slots : 0, nk);
  const int items = sp.full + sp.tail * sp.S;
  int vb = blockIdx.x;
  if (gridDim.x % XCDS == 0) vb = (blockIdx.x % XCDS) * (gridDim.x / XCDS) + blockIdx.x / XCDS;

  // work item w: tile, k-range and (for a split-K share) its workspace slot
  struct Work {
    Tile t;
    int kb, ke;
    float* part;
  };
  auto work = [&](int w) {
    Work r;
    int tile = w;
    r.kb = 0;
    r.ke = nk;
    r.part = nullptr;
    if (w >= sp.full) {   // share sh of tail tile i; shares of one k-range are adjacent
      const int j = w - sp.full, sh = j / sp.tail, i = j - sh * sp.tail;
      tile = sp.full + i;
      r.kb = sh * sp.nks;
      r.ke = min(nk, r.kb + sp.nks);
      r.part = ws + (size_t)j * (BM * BP);
    }
    r.t = decode_item(sc, E, n_nt, cols, tile);
    return r;
  };

  if (vb >= items) return;
  Work cur = work(vb);
  if (MX) {
    // FP8 fc1: tile loads are built inside the tile (see MxSrc)
    const MxSrc src{A, W1, W3, K, N};
    int stage0 = 0;
    bool primed = false;
    for (int w = vb; w < items; w += gridDim.x) {
      const bool has_next = w + (int)gridDim.x < items;
      const Work nw = has_next ? work(w + gridDim.x) : cur;
      if (cur.t.rows > BM / 2)
        run_tile_mx<false>(smem, cur.t, ep, cur.kb, cur.ke, cur.part, stage0, primed, nw.t,
                           has_next, nw.kb, src, ms, E, N);
      else
        run_tile_mx<true>(smem, cur.t, ep, cur.kb, cur.ke, cur.part, stage0, primed, nw.t,
                          has_next, nw.kb, src, ms, E, N);
      stage0 = (stage0 + cur.ke - cur.kb) & 1;
      primed = has_next;
      cur = nw;
    }
    return;
  }
  TileLoads ld = tile_loads<FC1, P_MN, EB>(cur.t, A, W1, W3, K, N, ksplit);
  int stage0 = 0;
  bool primed = false;
  for (int w = vb; w < items; w += gridDim.x) {
    const bool has_next = w + (int)gridDim.x < items;
    Work nw = cur;
    TileLoads nl = ld;
    if (has_next) {
      nw = work(w + gridDim.x);
      nl = tile_loads<FC1, P_MN, EB>(nw.t, A, W1, W3, K, N, ksplit);
    }
    // a tile whose token rows end inside it skips the MFMAs of its pad-row blocks
    const bool guard = cur.t.vrows < cur.t.rows;
    if (cur.t.rows > BM / 2) {
      if (guard)
        run_tile<MODE, false, P_MN, true>(smem, cur.t, ld, ep, cur.kb, cur.ke, cur.part, stage0,
                                          primed, nl, has_next, nw.kb);
      else
        run_tile<MODE, false, P_MN>(smem, cur.t, ld, ep, cur.kb, cur.ke, cur.part, stage0,
                                    primed, nl, has_next, nw.kb);
    } else {
      if (guard)
        run_tile<MODE, true, P_MN, true>(smem, cur.t, ld, ep, cur.kb, cur.ke, cur.part, stage0,
                                         primed, nl, has_next, nw.kb);
      else
        run_tile<MODE, true, P_MN>(smem, cur.t, ld, ep, cur.kb, cur.ke, cur.part, stage0,
                                   primed, nl, has_next, nw.kb);
    }
    stage0 = (stage0 + cur.ke - cur.kb) & 1;
    primed = has_next;
    cur = nw;
    ld = nl;
  }
}

// ---------------------------------------------------------------------------
// Ring pipeline for the forward GEMMs (bf16, K-contiguous weights) with at most 64
// experts: two activation slots and three weight-panel slots (160 KiB, all of the LDS),
// so a panel is requested two k-steps before its use and the activations one step
// before. The schedule tables live in registers: lane e holds expert e's segment bounds
// and first 256-row block. Tiles, their order and the split-K plan are those of
// gg_bf16_kernel, so gg_tail_reduce serves both. fc2's epilogue stages its tile in the
// activation and panel slots the tile's last step used (the next tile's first loads
// went to the others).
// ---------------------------------------------------------------------------
constexpr int RING_BYTES = 2 * A_BYTES + 3 * B_BYTES;
constexpr int RING_MAXE = 64;

struct SchedR {
  int off, end, val, ts;   // segment start and end, end of its token rows, first block
};

__device__ __forceinline__ SchedR build_sched_r(const Segs& sg, int E, int m_cap, int& total) {
  const int e = threadIdx.x & 63;
  SchedR s{0, 0, 0, 0};
  if (e < E) {   // the bounds build_sched gives
    if (sg.cap > 0) {
      s.off = e * sg.cap;
      s.end = s.off + max(0, min(sg.counts[e], sg.cap));
      s.val = s.end;
    } else {
      const int mend = max(0, min(sg.offsets[E], m_cap));
      s.off = max(0, min(sg.offsets[e], mend));
      s.end = max(0, min(sg.offsets[e + 1], mend));
      s.val = sg.counts ? max(s.off, min(s.off + max(sg.counts[e], 0), s.end)) : s.end;
    }
  }
  const int nb = (max(s.end - s.off, 0) + BM - 1) / BM;
  int inc = nb;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(inc, d, 64);
    if (e >= d) inc += v;
  }
  s.ts = inc - nb;
  total = __builtin_amdgcn_readlane(inc, 63);
  return s;
}

__device__ __forceinline__ Tile decode_item_r(const SchedR& s, int E, int n_nt, int cols, int w) {
  const int lane = threadIdx.x & 63;
  const int blk = w / n_nt;
  const unsigned long long m = __ballot(lane < E && s.ts <= blk);
  const int lo = 63 - __clzll(m);
  const int ts = __builtin_amdgcn_readlane(s.ts, lo);
  const int off = __builtin_amdgcn_readlane(s.off, lo);
  const int end = __builtin_amdgcn_readlane(s.end, lo);
  const int val = __builtin_amdgcn_readlane(s.val, lo);
  const int nb_e = (max(end - off, 0) + BM - 1) / BM;
  const int local = w - ts * n_nt;
  const int gsz = min(GROUP_M, nb_e);
  const int grp = local / (gsz * n_nt);
  const int first = grp * gsz;
  const int gm = min(gsz, nb_e - first);
  const int within = local - grp * gsz * n_nt;
  Tile t;
  t.e = lo;
  t.m0 = off + (first + within % gm) * BM;
  t.rows = min(BM, end - t.m0);
  t.vrows = max(0, min(t.rows, val - t.m0));
  t.n0 = (within / gm) * cols;
  return t;
}

// Slots of a tile's first k-step: activations a (of 2), panel b (of 3). Consecutive
// k-steps (also across tiles) take consecutive slots.
struct RingPos {
  int a, b;
};

// One tile's main loop on the ring. `aprimed`: the tile's first activation step was
// issued by the previous tile; `bpre`: how many of its first panel steps were. During
// step s the activations of step s+1 and the panel of step s+2 are issued (crossing into
// the next tile: its first activation step and first two panel steps). Each wave's
// panel pieces of step s+2 are the last vector-memory instructions it issues in step s,
// so the wait at the top of step s+1 leaves exactly those 4 in flight. Returns the
// next tile's bpre.
template <bool HALF>
__device__ __forceinline__ int mainloop_ring(char* smem, const TileLoads& ld, int kb, int ke,
                                             RingPos p0, bool aprimed, int bpre,
                                             const TileLoads& nxt, bool has_next, int nkb,
                                             int nn, f32x16 (&acc)[HALF ? 2 : 4][2]) {
  constexpr int WM = HALF ? 2 : 4;
  constexpr int WN = 2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);
  const int prow0 = (wave >> 1) * 64;
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;
  const uint32_t ldsb = lds0 + 2 * A_BYTES - A_BYTES;   // issue_loads adds A_BYTES for the panel

#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int n = ke - kb;
  const int blim = n + (has_next ? min(2, nn) : 0);
  auto issue_b = [&](int j) {
    const int slot = (p0.b + j) % 3;
    if (j < n) issue_loads(ld, ldsb + slot * B_BYTES, kb + j, 1);
    else issue_loads(nxt, ldsb + slot * B_BYTES, nkb + j - n, 1);
  };
  const int fr = lane & 31;
  if (!aprimed) issue_loads(ld, lds0 + p0.a * A_BYTES, kb, 0);
  int bnext = bpre;
  if (bnext < min(2, n)) issue_b(bnext++);
  if (bnext < min(2, n)) issue_b(bnext++);
  int a = p0.a, b = p0.b;
  bool tail4 = false;
  for (int s = 0; s < n; ++s) {
    if (tail4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* sa = smem + a * A_BYTES;
    const char* sb = smem + 2 * A_BYTES + b * B_BYTES;
    const bool dob = bnext <= s + 2 && bnext < blim;
    bf16x8 wf[2][WN], af[2][WM];
    auto frag = [&](int ks, int buf) {
      const int chk = ks * 2 + (lane >> 5);
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
        wf[buf][nb] = *reinterpret_cast<const bf16x8*>(sb + swz(prow0 + nb * 32 + fr, chk));
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
        af[buf][mb] = *reinterpret_cast<const bf16x8*>(sa + swz(arow0 + mb * 32 + fr, chk));
    };
    frag(0, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks == 0) {
        if (s + 1 < n) issue_loads(ld, lds0 + (a ^ 1) * A_BYTES, kb + s + 1, 0);
        else if (has_next) issue_loads(nxt, lds0 + (a ^ 1) * A_BYTES, nkb, 0);
      }
      if (ks == 1 && dob) issue_b(bnext);
      if (ks + 1 < BK / 16) frag(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][nb], af[ks & 1][mb],
                                                                acc[mb][nb], 0, 0, 0);
    }
    tail4 = dob && bnext == s + 2;
    if (dob) ++bnext;
    a ^= 1;
    b = b == 2 ? 0 : b + 1;
  }
  return bnext - n;
}

template <int MODE>
__global__ __launch_bounds__(NTHR, 1) void gg_ring_kernel(
    const bf16_t* __restrict__ A, Segs sg, int E, int K, int N, int m_cap,
    const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W3, Epi ep,
    float* __restrict__ ws, int slots) {
  static_assert(MODE == kFc1 || MODE == kFc2, "the ring serves the forward GEMMs");
  constexpr bool FC1 = MODE == kFc1;
  __shared__ __attribute__((aligned(16))) char smem[RING_BYTES];
  int nblk;
  const SchedR sr = build_sched_r(sg, E, m_cap, nblk);

  const int cols = FC1 ? BP / 2 : BP;
  const int n_nt = (N + cols - 1) / cols;
  const int total = nblk * n_nt;
  const int nk = K / BK;
  const Split sp = split_plan(total, gridDim.x, ws ? slots : 0, nk);
  const int items = sp.full + sp.tail * sp.S;
  int vb = blockIdx.x;
  if (gridDim.x % XCDS == 0) vb = (blockIdx.x % XCDS) * (gridDim.x / XCDS) + blockIdx.x / XCDS;

  struct Work {
    Tile t;
    int kb, ke;
    float* part;
  };
  auto work = [&](int w) {
    Work r;
    int tile = w;
    r.kb = 0;
    r.ke = nk;
    r.part = nullptr;
    if (w >= sp.full) {
      const int j = w - sp.full, sh = j / sp.tail, i = j - sh * sp.tail;
      tile = sp.full + i;
      r.kb = sh * sp.nks;
      r.ke = min(nk, r.kb + sp.nks);
      r.part = ws + (size_t)j * (BM * BP);
    }
    r.t = decode_item_r(sr, E, n_nt, cols, tile);
    return r;
  };

  if (vb >= items) return;
  Work cur = work(vb);
  TileLoads ld = tile_loads<FC1, false, 2>(cur.t, A, W1, W3, K, N, K);
  RingPos p{0, 0};
  bool aprimed = false;
  int bpre = 0;
  for (int w = vb; w < items; w += gridDim.x) {
    const bool has_next = w + (int)gridDim.x < items;
    Work nw = cur;
    TileLoads nl = ld;
    if (has_next) {
      nw = work(w + gridDim.x);
      nl = tile_loads<FC1, false, 2>(nw.t, A, W1, W3, K, N, K);
    }
    const int nn = has_next ? nw.ke - nw.kb : 0;
    // free after the tile's last step: its activation slot and its panel slot (the next
    // tile's first loads went to the others)
    const int nlast = cur.ke - cur.kb - 1;
    char* elo = smem + ((p.a + nlast) & 1) * A_BYTES;
    char* ehi = smem + 2 * A_BYTES + ((p.b + nlast) % 3) * B_BYTES;
    int nbp;
    if (cur.t.rows > BM / 2) {
      f32x16 acc[4][2];
      nbp = mainloop_ring<false>(smem, ld, cur.kb, cur.ke, p, aprimed, bpre, nl, has_next, nw.kb,
                                 nn, acc);
      finish_tile<MODE, false>(smem, cur.t, ep, cur.kb, cur.ke, cur.part, 0, acc, elo, ehi);
    } else {
      f32x16 acc[2][2];
      nbp = mainloop_ring<true>(smem, ld, cur.kb, cur.ke, p, aprimed, bpre, nl, has_next, nw.kb,
                                nn, acc);
      finish_tile<MODE, true>(smem, cur.t, ep, cur.kb, cur.ke, cur.part, 0, acc, elo, ehi);
    }
    const int n = cur.ke - cur.kb;
    p.a ^= n & 1;
    p.b = (p.b + n) % 3;
    aprimed = has_next;
    bpre = nbp;
    cur = nw;
    ld = nl;
  }
}

// Sums the split-K shares of the tail tiles in split order and applies the MODE
// epilogue, rounding once to bf16. G must be the grid size the GEMM ran with.
template <int MODE>
__global__ __launch_bounds__(256) void gg_tail_reduce(Segs sg, int E, int K, int m_cap, int G,
                                                      int slots, const float* __restrict__ ws,
                                                      Epi ep) {
  constexpr bool FC1 = MODE == kFc1;
  __shared__ Sched sc;
  build_sched(sc, sg, E, m_cap);
  const int N = ep.N;
  const int cols = FC1 ? BP / 2 : BP;
  const int n_nt = (N + cols - 1) / cols;
  const Split sp = split_plan(sc.tstart[E] * n_nt, G, slots, K / BK);
  if (sp.tail == 0) return;
  constexpr int Q = (FC1 ? BP / 2 : BP) / 4;   // 4-column groups per row
  const int64_t units = (int64_t)sp.tail * BM * Q;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(u / (BM * Q));
    const int rem = (int)(u - (int64_t)i * BM * Q);
    const int r = rem / Q, q = rem - r * Q;
    const Tile t = decode_item(sc, E, n_nt, cols, sp.full + i);
    if (r >= t.rows) continue;
    const float* base = ws + (size_t)i * (BM * BP) + r * BP;
    const size_t stride = (size_t)sp.tail * (BM * BP);   // next share of the same tile
    const int fl = 4 * q;                                // output column inside the tile
    // fc1: column fl's w1 panel row; its w3 row is 32 later
    const int pa = FC1 ? (fl >> 5) * 64 + (fl & 31) : fl;
    float a[4] = {0, 0, 0, 0}, b[4] = {0, 0, 0, 0};
    for (int sh = 0; sh < sp.S; ++sh) {
      const float4 va = *reinterpret_cast<const float4*>(base + sh * stride + pa);
      a[0] += va.x; a[1] += va.y; a[2] += va.z; a[3] += va.w;
      if (FC1) {
        const float4 vb = *reinterpret_cast<const float4*>(base + sh * stride + pa + 32);
        b[0] += vb.x; b[1] += vb.y; b[2] += vb.z; b[3] += vb.w;
      }
    }
    const int n = t.n0 + fl;
    if (n >= N) continue;
    if (MODE == kDgrad && r >= t.vrows) {   // pad row: zeros, its [a | b] is never read
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
      dgrad4(ep, (size_t)(t.m0 + r) * N, n, z, uint2{0u, 0u}, uint2{0u, 0u});
    } else {
      emit4<MODE>(ep, t.m0 + r, n, a, b);
    }
  }
}

// ---------------------------------------------------------------------------
// k-grouped weight gradient ("Expert Parallelism (EP)", section 5: the backward of an
// m-grouped fc is an m-grouped dgrad plus a k-grouped wgrad). For every expert e with
// segment rows [s_e, s_e+1) (offsets, clamped to the rows in use):
//   out[e][i][j] = sum over r in the segment of P[r][i] * Q[r][j]     (i < N1, j < N2)
// with P [rows][N1] and Q [rows][N2] the activations as the forward and the dgrad leave
// them (row-major): both operands are read MN-major, a k-step being 64 segment rows. Rows
// i < NS of the result go to out_lo [E][NS][N2], the others to out_hi [E][N1-NS][N2]
// (float32), so [dW1 | dW3] from [da | db] lands in two separate arrays. Experts without
// rows get zeros. Tiles are 256 columns of P x 256 columns of Q with the m-grouped
// kernel's pipeline; every expert has the same tile grid, walked in groups of up to
// GROUP_M P blocks per Q sweep. The buffer descriptors of a tile end at its segment's
// last row, so the rows of the last, partial k-step past the segment read as zeros.
// ---------------------------------------------------------------------------
struct WSched {
  int seg[MAXE + 1];   // segment bounds
  int sval[MAXE];      // ends of the rows that hold tokens (the sums run over those only)
  int elist[MAXE];     // experts with token rows, in order
  int nne;
  int wtot[16];
};

__device__ void build_wsched(WSched& sc, const int32_t* __restrict__ offsets,
                             const int32_t* __restrict__ counts, int E, int m_cap) {
  const int tid = threadIdx.x;
  const int mend = max(0, min(offsets[E], m_cap));
  for (int e = tid; e <= E; e += blockDim.x) sc.seg[e] = max(0, min(offsets[e], mend));
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x)
    sc.sval[e] = counts ? max(sc.seg[e], min(sc.seg[e] + max(counts[e], 0), sc.seg[e + 1]))
                        : sc.seg[e + 1];
  __syncthreads();
  const int per = (MAXE + blockDim.x - 1) / blockDim.x;   // experts per thread (<= 4)
  bool has[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * per + i;
    has[i] = i < per && e < E && sc.sval[e] > sc.seg[e];
    local += has[i];
  }
  int run = block_scan_excl(local, sc.wtot);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (has[i]) sc.elist[run++] = tid * per + i;
  if (tid == (int)blockDim.x - 1) sc.nne = run;
  __syncthreads();
}

struct WTile {
  Tile t;       // e, first P column (m0), P columns (rows), first Q column (n0)
  int kseg0;    // first row of the segment
  int klen;     // rows of the segment
  int nk;       // k-steps
};

__device__ __forceinline__ WTile wg_decode(const WSched& sc, int N1, int N2, int w) {
  const int n_t1 = (N1 + BM - 1) / BM, n_t2 = (N2 + BP - 1) / BP;
  const int per = n_t1 * n_t2;
  const int ei = w / per;
  const int local = w - ei * per;
  const int gsz = min(GROUP_M, n_t1);
  const int grp = local / (gsz * n_t2);
  const int first = grp * gsz;
  const int gm = min(gsz, n_t1 - first);
  const int within = local - grp * gsz * n_t2;
  WTile r;
  r.t.e = sc.elist[ei];
  r.t.m0 = (first + within % gm) * BM;
  r.t.rows = min(BM, N1 - r.t.m0);
  r.t.vrows = r.t.rows;
  r.t.n0 = (within / gm) * BP;
  r.kseg0 = sc.seg[r.t.e];
  r.klen = sc.sval[r.t.e] - r.kseg0;
  r.nk = (r.klen + BK - 1) / BK;
  return r;
}

// Both operands MN-major (mn_off); each descriptor starts at the segment's first row and
// the tile's first column and ends at the segment's last row.
__device__ __forceinline__ TileLoads wg_loads(const WTile& w, const bf16_t* __restrict__ P,
                                              const bf16_t* __restrict__ Q, int N1, int N2) {
  TileLoads o;
  o.na = 4;
  o.rsa = buffer_rsrc(P + (size_t)w.kseg0 * N1 + w.t.m0, (uint32_t)(w.klen * N1 - w.t.m0) * 2u);
  o.rsb = buffer_rsrc(Q + (size_t)w.kseg0 * N2 + w.t.n0, (uint32_t)(w.klen * N2 - w.t.n0) * 2u);
  o.rsb2 = o.rsb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o.aoff[j] = mn_off(j, N1);
    o.boff[j] = mn_off(j, N2);
  }
  o.astep = (uint32_t)BK * N1 * 2u;
  o.bstep = (uint32_t)BK * N2 * 2u;
  o.bsplit = 1 << 30;
  return o;
}

// One wgrad tile. The float32 result (256 x 256, 256 KiB) leaves through the LDS stage
// the tile's last k-step used, 64 rows (64 KiB) per pass: the owning waves write their
// accumulators (16-byte unit u of row r stored at u ^ (r % 16): the 16 rows a quarter-wave
// writes hit distinct banks), then every wave stores whole 1 KiB rows to the output.
template <bool HALF>
__device__ __forceinline__ void wg_tile(char* smem, const WTile& w, const TileLoads& ld, int N1,
                                        int N2, int NS, float* __restrict__ out_lo,
                                        float* __restrict__ out_hi, int stage0, bool primed,
                                        const TileLoads& nxt, bool has_next) {
  constexpr int WM = HALF ? 2 : 4;
  constexpr int WN = 2;
  constexpr int PASSES = HALF ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);
  const int prow0 = (wave >> 1) * 64;
  const int fr = lane & 31;
  f32x16 acc[WM][WN];
  mainloop<HALF, true, true>(smem, ld, 0, w.nk, stage0, primed, nxt, has_next, 0, acc);
  char* stage = smem + ((stage0 + w.nk - 1) & 1) * STAGE_BYTES;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    lds_barrier();
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
      const int r = arow0 + mb * 32 + fr;
      // rows [64p, 64p + 64): a block of 32 rows lies in one pass
      if ((arow0 + mb * 32) / 64 != p) continue;
      const int rl = r - 64 * p;
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int u = (prow0 + nb * 32 + g * 8 + (lane >> 5) * 4) >> 2;
          const f32x16& a = acc[mb][nb];
          *reinterpret_cast<float4*>(stage + rl * 1024 + ((u ^ (rl & 15)) << 4)) =
              float4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
        }
    }
    lds_barrier();
    const int j = w.t.n0 + 4 * lane;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rl = wave + 8 * it;
      const int r = 64 * p + rl;
      if (r >= w.t.rows || j >= N2) continue;
      const int i = w.t.m0 + r;
      float* orow = i < NS ? out_lo + ((size_t)w.t.e * NS + i) * N2
                           : out_hi + ((size_t)w.t.e * (N1 - NS) + (i - NS)) * N2;
      *reinterpret_cast<float4*>(orow + j) =
          *reinterpret_cast<const float4*>(stage + rl * 1024 + ((lane ^ (rl & 15)) << 4));
    }
  }
}

__global__ __launch_bounds__(NTHR, 1) void wg_bf16_kernel(
    const bf16_t* __restrict__ P, const bf16_t* __restrict__ Q,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts, int E, int N1,
    int N2, int NS, int m_cap, float* __restrict__ out_lo, float* __restrict__ out_hi) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  __shared__ WSched sc;
  build_wsched(sc, offsets, counts, E, m_cap);
  int vb = blockIdx.x;
  if (gridDim.x % XCDS == 0) vb = (blockIdx.x % XCDS) * (gridDim.x / XCDS) + blockIdx.x / XCDS;

  // experts without rows: zero gradient
  const int q2 = N2 / 4;
  const int64_t per_e = (int64_t)N1 * q2;
  for (int e = 0; e < E; ++e) {
    if (sc.sval[e] > sc.seg[e]) continue;
    for (int64_t u = (int64_t)vb * NTHR + threadIdx.x; u < per_e; u += (int64_t)gridDim.x * NTHR) {
      const int i = (int)(u / q2), j = (int)(u - (int64_t)i * q2) * 4;
      float* orow = i < NS ? out_lo + ((size_t)e * NS + i) * N2
                           : out_hi + ((size_t)e * (N1 - NS) + (i - NS)) * N2;
      *reinterpret_cast<float4*>(orow + j) = float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  const int items = sc.nne * ((N1 + BM - 1) / BM) * ((N2 + BP - 1) / BP);
  if (vb >= items) return;
  WTile cur = wg_decode(sc, N1, N2, vb);
  TileLoads ld_ = wg_loads(cur, P, Q, N1, N2);
  int stage0 = 0;
  bool primed = false;
  for (int w = vb; w < items; w += gridDim.x) {
    const bool has_next = w + (int)gridDim.x < items;
    WTile nw = cur;
    TileLoads nl = ld_;
    if (has_next) {
      nw = wg_decode(sc, N1, N2, w + gridDim.x);
      nl = wg_loads(nw, P, Q, N1, N2);
    }
    if (cur.t.rows > BM / 2)
      wg_tile<false>(smem, cur, ld_, N1, N2, NS, out_lo, out_hi, stage0, primed, nl, has_next);
    else
      wg_tile<true>(smem, cur, ld_, N1, N2, NS, out_lo, out_hi, stage0, primed, nl, has_next);
    stage0 = (stage0 + cur.nk) & 1;
    primed = has_next;
    cur = nw;
    ld_ = nl;
  }
}

// ---------------------------------------------------------------------------
// float32: 16 rows x 64 columns per workgroup, k-steps of 32 staged in LDS (the tiny
// float32 layer only); the same modes as the bf16 kernel, without rounding.
// ---------------------------------------------------------------------------
constexpr int FM = 16, FN = 64, FK = 32;

struct Epi32 {
  float* C;
  float* ab;
  float* dh;
  int N;
};

template <int MODE, bool P_MN>
__global__ __launch_bounds__(256) void gg_f32_kernel(const float* __restrict__ A, Segs sg,
                                                     const int32_t* __restrict__ tile_expert, int E,
                                                     int K, int m_tile, int m_cap,
                                                     const float* __restrict__ W1,
                                                     const float* __restrict__ W3, int ksplit,
                                                     Epi32 ep) {
  constexpr bool FC1 = MODE == kFc1;
  const int N = ep.N;
  __shared__ float As[FM][FK + 1];
  __shared__ float B1[FN][FK + 1];
  __shared__ float B3[FC1 ? FN : 1][FK + 1];
  const int m0 = blockIdx.x * FM;
  int e, mend, vend;   // vend: end of the rows holding tokens (later rows read as zeros)
  if (sg.cap > 0) {   // masked slabs (cap a multiple of FM: a block never straddles two)
    e = m0 / sg.cap;
    if (e >= E) return;
    mend = e * sg.cap + max(0, min(sg.counts[e], sg.cap));
    vend = mend;
  } else {
    mend = min(sg.offsets[E], m_cap);
    if (m0 >= mend) return;
    e = tile_expert[m0 / m_tile];
    vend = mend;
    if (sg.counts && e >= 0 && e < E) vend = min(mend, sg.offsets[e] + max(sg.counts[e], 0));
  }
  if (m0 >= mend || e < 0 || e >= E) return;
  const int n0 = blockIdx.y * FN;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  float a1[4] = {0, 0, 0, 0}, a3[4] = {0, 0, 0, 0};
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int i = tid; i < FM * FK; i += 256) {
      const int r = i / FK, c = i % FK;
      const int gm = min(m0 + r, mend - 1);
      As[r][c] = m0 + r < vend ? A[(size_t)gm * K + k0 + c] : 0.0f;
    }
    if (P_MN) {   // W1 [E][ksplit][N] then W3 [E][K - ksplit][N], read along N
      for (int i = tid; i < FN * FK; i += 256) {
        const int c = i / FN, r = i % FN, k = k0 + c;
        const int gn = min(n0 + r, N - 1);
        B1[r][c] = k < ksplit ? W1[((size_t)e * ksplit + k) * N + gn]
                              : W3[((size_t)e * (K - ksplit) + (k - ksplit)) * N + gn];
      }
    } else {
      for (int i = tid; i < FN * FK; i += 256) {
        const int r = i / FK, c = i % FK;
        const int gn = min(n0 + r, N - 1);
        B1[r][c] = W1[((size_t)e * N + gn) * K + k0 + c];
        if (FC1) B3[r][c] = W3[((size_t)e * N + gn) * K + k0 + c];
      }
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
    if (n >= N) continue;
    const size_t row = (size_t)m * N;
    if (MODE == kFc1) {
      ep.C[row + n] = a1[j] / (1.0f + expf(-a1[j])) * a3[j];
      if (ep.ab) {
        ep.ab[2 * row + n] = a1[j];
        ep.ab[2 * row + N + n] = a3[j];
      }
    } else if (MODE == kFc2) {
      ep.C[row + n] = a1[j];
    } else {
      const float d = a1[j];
      const float a = ep.ab[2 * row + n], b = ep.ab[2 * row + N + n];
      const float s = 1.0f / (1.0f + expf(-a));
      ep.C[2 * row + n] = d * b * (s * (1.0f + a * (1.0f - s)));
      ep.C[2 * row + N + n] = d * (a * s);
      if (ep.dh) ep.dh[row + n] = d;
    }
  }
}

// float32 k-grouped weight gradient: a 64 x 64 block of out[e] per workgroup, k-steps of
// 16 segment rows staged in LDS; rows past the segment's end are masked.
constexpr int WT = 64, WK = 16;

__global__ __launch_bounds__(256) void wg_f32_kernel(const float* __restrict__ P,
                                                     const float* __restrict__ Q,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ counts, int E,
                                                     int N1, int N2, int NS, int m_cap,
                                                     float* __restrict__ out_lo,
                                                     float* __restrict__ out_hi) {
  __shared__ float Ps[WT][WK + 1];
  __shared__ float Qs[WT][WK + 1];
  const int e = blockIdx.y;
  const int nt2 = (N2 + WT - 1) / WT;
  const int i0 = (blockIdx.x / nt2) * WT, j0 = (blockIdx.x % nt2) * WT;
  const int mend = max(0, min(offsets[E], m_cap));
  const int s0 = max(0, min(offsets[e], mend));
  int s1 = max(s0, min(offsets[e + 1], mend));
  if (counts) s1 = min(s1, s0 + max(counts[e], 0));   // token rows only
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  float acc[4][4] = {};
  for (int k0 = s0; k0 < s1; k0 += WK) {
    for (int x = tid; x < WT * WK; x += 256) {
      const int c = x / WT, r = x % WT, k = k0 + c;
      Ps[r][c] = (i0 + r < N1 && k < s1) ? P[(size_t)k * N1 + i0 + r] : 0.0f;
      Qs[r][c] = (j0 + r < N2 && k < s1) ? Q[(size_t)k * N2 + j0 + r] : 0.0f;
    }
    __syncthreads();
    for (int c = 0; c < WK; ++c)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = fmaf(Ps[ti + 16 * a][c], Qs[tj + 16 * b][c], acc[a][b]);
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ti + 16 * a;
    if (i >= N1) continue;
    float* orow = i < NS ? out_lo + ((size_t)e * NS + i) * N2
                         : out_hi + ((size_t)e * (N1 - NS) + (i - NS)) * N2;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + tj + 16 * b;
      if (j < N2) orow[j] = acc[a][b];
    }
  }
}

}  // namespace

size_t grouped_workspace_bytes() { return (size_t)cu_count() * BM * BP * sizeof(float); }

// One m-grouped GEMM per segment with the MODE epilogue: C = A W^T, W [E][N][K]
// (p_mn false), or C = A W with W [E][K][N] split at ksplit between W1 and W3 (p_mn
// true). K: reduction width, ep.N: output columns.
static hipError_t launch_mgrouped(int dt, int mode, bool p_mn, const void* A, Segs sg,
                                  const int32_t* tile_expert, int E, int K,
                                  int m_tile, int64_t m_cap, const void* W1, const void* W3,
                                  int ksplit, void* C, void* ab, void* dh, int N, void* workspace,
                                  size_t ws_bytes, hipStream_t s) {
  if (dt == kF32) {
    const dim3 block(256);
    const dim3 grid((unsigned)((m_cap + FM - 1) / FM), (N + FN - 1) / FN);
    const Epi32 ep{static_cast<float*>(C), static_cast<float*>(ab), static_cast<float*>(dh), N};
    const float* a = static_cast<const float*>(A);
    const float* w1 = static_cast<const float*>(W1);
    const float* w3 = static_cast<const float*>(W3);
    const int mc = (int)m_cap;
    if (mode == kFc1)
      hipLaunchKernelGGL((gg_f32_kernel<kFc1, false>), grid, block, 0, s, a, sg, tile_expert,
                         E, K, m_tile, mc, w1, w3, K, ep);
    else if (mode == kFc2 && !p_mn)
      hipLaunchKernelGGL((gg_f32_kernel<kFc2, false>), grid, block, 0, s, a, sg, tile_expert,
                         E, K, m_tile, mc, w1, w1, K, ep);
    else if (mode == kFc2)
      hipLaunchKernelGGL((gg_f32_kernel<kFc2, true>), grid, block, 0, s, a, sg, tile_expert,
                         E, K, m_tile, mc, w1, w3, ksplit, ep);
    else
      hipLaunchKernelGGL((gg_f32_kernel<kDgrad, true>), grid, block, 0, s, a, sg,
                         tile_expert, E, K, m_tile, mc, w1, w1, ksplit, ep);
    return hipGetLastError();
  }
  const int G = cu_count();
  const dim3 grid(G), block(NTHR);
  float* ws = static_cast<float*>(workspace);
  const int slots = ws ? (int)std::min<size_t>(ws_bytes / (BM * BP * sizeof(float)), 1 << 20) : 0;
  const dim3 rgrid(4 * G), rblock(256);
  const Epi ep{static_cast<bf16_t*>(C), static_cast<bf16_t*>(ab), static_cast<bf16_t*>(dh), N};
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* w1 = static_cast<const bf16_t*>(W1);
  const bf16_t* w3 = static_cast<const bf16_t*>(W3);
  const int mc = (int)m_cap;
  // the ring while an expert's row blocks fit about one column sweep (then every weight
  // panel comes from HBM once and the deeper lookahead pays); with more, later sweeps
  // find their panels in the caches and the ring only costs
  const bool ring = E <= RING_MAXE && m_cap <= (int64_t)(GROUP_M + 1) * BM * E;
  if (mode == kFc1) {
    if (ring)
      hipLaunchKernelGGL(gg_ring_kernel<kFc1>, grid, block, 0, s, a, sg, E, K, N, mc, w1, w3,
                         ep, ws, slots);
    else
      hipLaunchKernelGGL((gg_bf16_kernel<kFc1, false>), grid, block, 0, s, a, sg, E, K, N, mc,
                         w1, w3, K, ep, ws, slots, MxScales{});
    if (slots)
      hipLaunchKernelGGL(gg_tail_reduce<kFc1>, rgrid, rblock, 0, s, sg, E, K, mc, G, slots,
                         ws, ep);
  } else if (mode == kFc2) {
    if (p_mn)
      hipLaunchKernelGGL((gg_bf16_kernel<kFc2, true>), grid, block, 0, s, a, sg, E, K, N, mc,
                         w1, w3, ksplit, ep, ws, slots, MxScales{});
    else if (ring)
      hipLaunchKernelGGL(gg_ring_kernel<kFc2>, grid, block, 0, s, a, sg, E, K, N, mc, w1, w1,
                         ep, ws, slots);
    else
      hipLaunchKernelGGL((gg_bf16_kernel<kFc2, false>), grid, block, 0, s, a, sg, E, K, N,
                         mc, w1, w1, K, ep, ws, slots, MxScales{});
    if (slots)
      hipLaunchKernelGGL(gg_tail_reduce<kFc2>, rgrid, rblock, 0, s, sg, E, K, mc, G, slots,
                         ws, ep);
  } else {
    hipLaunchKernelGGL((gg_bf16_kernel<kDgrad, true>), grid, block, 0, s, a, sg, E, K, N, mc,
                       w1, w1, K, ep, ws, slots, MxScales{});
    if (slots)
      hipLaunchKernelGGL(gg_tail_reduce<kDgrad>, rgrid, rblock, 0, s, sg, E, K, mc, G, slots,
                         ws, ep);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_swiglu(int dt, int phases, const void* x_perm, const int32_t* offsets,
                                 const int32_t* counts, int cap, const int32_t* tile_expert, int E,
                                 int D, int F, int m_tile, int64_t m_cap, const void* w1,
                                 const void* w3, const void* w2, void* h, void* ab, void* y_perm,
                                 void* workspace, size_t ws_bytes, hipStream_t s) {
  const Segs sg{offsets, counts, cap};
  // decode-sized batches (at most 128 rows per expert) stream the weights instead
  const int rmax = ab ? 0 : decode_rows_max(dt, cap, m_cap, E, D, F);
  if (rmax > 0)
    return launch_decode_swiglu(phases, x_perm, cap > 0 ? nullptr : offsets, counts, cap, rmax,
                                E, D, F, w1, w3, w2, h, y_perm, s);
  if (phases & 1) {
    const hipError_t e = launch_mgrouped(dt, kFc1, false, x_perm, sg, tile_expert, E, D, m_tile,
                                         m_cap, w1, w3, D, h, ab, nullptr, F, workspace, ws_bytes,
                                         s);
    if (e != hipSuccess) return e;
  }
  if (phases & 2)
    return launch_mgrouped(dt, kFc2, false, h, sg, tile_expert, E, F, m_tile, m_cap, w2, w2, F,
                           y_perm, nullptr, nullptr, D, workspace, ws_bytes, s);
  return hipSuccess;
}

hipError_t launch_grouped_fc1_mx(const void* xq_perm, const void* xs_perm,
                                 const int32_t* offsets, const int32_t* counts, int E, int D, int F,
                                 int64_t m_cap,
                                 const void* w1q, const void* w1s, const void* w3q,
                                 const void* w3s, void* h, void* workspace, size_t ws_bytes,
                                 hipStream_t s) {
  const int G = cu_count();
  float* ws = static_cast<float*>(workspace);
  const int slots = ws ? (int)std::min<size_t>(ws_bytes / (BM * BP * sizeof(float)), 1 << 20) : 0;
  const Segs sg{offsets, counts, 0};
  const Epi ep{static_cast<bf16_t*>(h), nullptr, nullptr, F};
  const MxScales ms{static_cast<const uint32_t*>(xs_perm), static_cast<const uint32_t*>(w1s),
                    static_cast<const uint32_t*>(w3s), m_cap};
  hipLaunchKernelGGL((gg_bf16_kernel<kFc1, false, true>), dim3(G), dim3(NTHR), 0, s,
                     static_cast<const bf16_t*>(xq_perm), sg, E, D, F, (int)m_cap,
                     static_cast<const bf16_t*>(w1q), static_cast<const bf16_t*>(w3q), D, ep, ws,
                     slots, ms);
  // the reduction counts k-steps as K / 64 bf16 values: the FP8 kernel's 128-byte steps
  // are D / 128
  if (slots)
    hipLaunchKernelGGL(gg_tail_reduce<kFc1>, dim3(4 * G), dim3(256), 0, s, sg, E, D / 2,
                       (int)m_cap, G, slots, ws, ep);
  return hipGetLastError();
}

hipError_t launch_grouped_dgrad_swiglu(int dt, const void* dy_perm, const int32_t* offsets,
                                       const int32_t* counts, const int32_t* tile_expert, int E,
                                       int D, int F,
                                       int m_tile, int64_t m_cap, const void* w2, const void* ab,
                                       void* dab, void* dh, void* workspace, size_t ws_bytes,
                                       hipStream_t s) {
  // dh = dY w2[e]: w2 [E][D][F] is the [K = D][N = F] operand, read MN-major
  return launch_mgrouped(dt, kDgrad, true, dy_perm, Segs{offsets, counts, 0}, tile_expert, E, D,
                         m_tile, m_cap, w2,
                         w2, D, dab, const_cast<void*>(ab), dh, F, workspace, ws_bytes, s);
}

hipError_t launch_grouped_dgrad_fc1(int dt, const void* dab, const int32_t* offsets,
                                    const int32_t* counts, const int32_t* tile_expert, int E,
                                    int D, int F, int m_tile,
                                    int64_t m_cap, const void* w1, const void* w3, void* dx_perm,
                                    void* workspace, size_t ws_bytes, hipStream_t s) {
  // dX = [da | db] [w1[e] ; w3[e]]: K = 2F, k < F from w1 [E][F][D], the rest from w3
  return launch_mgrouped(dt, kFc2, true, dab, Segs{offsets, counts, 0}, tile_expert, E, 2 * F,
                         m_tile, m_cap, w1,
                         w3, F, dx_perm, nullptr, nullptr, D, workspace, ws_bytes, s);
}

hipError_t launch_grouped_wgrad(int dt, const void* P, const void* Q, const int32_t* offsets,
                                const int32_t* counts, int E, int N1, int N2, int NS,
                                int64_t m_cap, float* out_lo, float* out_hi, hipStream_t s) {
  if (dt == kF32) {
    const dim3 grid(((N1 + WT - 1) / WT) * ((N2 + WT - 1) / WT), E), block(256);
    hipLaunchKernelGGL(wg_f32_kernel, grid, block, 0, s, static_cast<const float*>(P),
                       static_cast<const float*>(Q), offsets, counts, E, N1, N2, NS, (int)m_cap,
                       out_lo, out_hi);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(wg_bf16_kernel, dim3(cu_count()), dim3(NTHR), 0, s,
                     static_cast<const bf16_t*>(P), static_cast<const bf16_t*>(Q), offsets, counts,
                     E, N1, N2, NS, (int)m_cap, out_lo, out_hi);
  return hipGetLastError();
}

}  // namespace moe
