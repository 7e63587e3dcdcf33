// m-grouped expert GEMMs: fc1 with the fused silu(a)*b activation, then fc2
// ("Expert Parallelism (EP)", llm-infra-atlas, section 1 "routed_experts_compute:
// fc1 -> act -> fc2, grouped GEMM (m-grouped)"; section 2: one kernel over
// same-shape expert GEMMs with different row counts, a tile scheduler across the
// groups, rows laid out expert-contiguous and tile aligned). Weight layout from the
// "Expert Tensor Parallel" design note, section 4.3: w1, w3 [E,F,D], w2 [E,D,F].
//
// bf16 kernel (float32 accumulation on v_mfma_f32_32x32x16_bf16):
//   * a tile is up to 256 rows of one expert's segment x a 256-row weight panel
//     (fc1: 128 h columns, taken from w1 and w3 in alternating 32-row blocks; fc2:
//     256 y columns). Both operands are K-contiguous; per 64-wide k step the tile
//     stages A [256 x 64] and the panel [256 x 64] in LDS (64 KiB), double
//     buffered through registers (128 KiB).
//   * four waves; on a full tile each wave owns 128 rows x 128 panel rows (16
//     MFMA blocks, 256 accumulators in AGPRs). A half tile (the last 128 rows of a
//     segment whose length is an odd number of 128-row tiles) is split 128 rows x
//     64 panel rows per wave, so all four SIMDs stay busy.
//   * LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with half the
//     row index, so the MFMA fragment reads are conflict free.
//   * weights are the MFMA A operand and activations the B operand: each lane ends
//     with 4 consecutive output columns of one row (8-byte stores); for fc1 the w1
//     and w3 blocks of the same columns land in the same wave, which applies
//     silu(a)*b before rounding to bf16.
//   * persistent grid (one workgroup per CU). Each workgroup builds the list of
//     256-row blocks per expert from offsets[] on the device (no host sync), walks
//     each expert's (block, column) tiles with up to 16 blocks per column sweep, and
//     the workgroup id is remapped so each XCD's L2 sees a contiguous run of tiles.
// float32 kernel: a plain LDS-tiled VALU GEMM (the tiny float32 layer only).
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

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

__device__ __forceinline__ float silu_mul(float a, float b) {
  return a / (1.0f + __expf(-a)) * b;
}

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

struct Tile {
  int e, m0, rows, n0;
};

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Raw buffer descriptor over [base, base + bytes): the hardware zero-fills any lane
// whose offset falls outside the range.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;   // raw (untyped) buffer, 32-bit data format
  return r;
}

// 16 bytes per lane from a buffer straight into LDS: lane l reads base + voff_l + soff
// and the 64 lanes of the wave fill 1 KiB at LDS address `lds` (wave-uniform), lane l
// at lds + 16*l. Buffer addressing takes a 32-bit offset per lane and the k-step in a
// scalar offset, which issues faster than 64-bit flat addresses. Issued as inline
// assembly so the compiler adds no waits of its own for it; the pipeline below waits
// with an explicit s_waitcnt vmcnt(0) and a barrier before any wave reads the stage
// the loads fill.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// Load addresses of one tile at k-step 0, per lane: buffer descriptors for its A rows
// and for expert e's weight matrix, and the byte offsets of the rows this lane fills.
// Piece j of wave w holds rows 64*j + 8*w .. +7; lane l fills row 64*j + lrow with
// lrow = 8*w + l/8, 16-byte slot l%8, which holds logical chunk (l%8) ^ ((row/2)%8).
// Rows past the tile or the matrix are clamped to the last one.
struct TileLoads {
  i32x4 rsa, rsb;
  uint32_t aoff[4], boff[4];
  int na;   // A pieces per wave: 4 for a full tile, 2 for a half tile
};

template <bool FC1>
__device__ __forceinline__ TileLoads tile_loads(const Tile& t, const bf16_t* __restrict__ A,
                                                const bf16_t* __restrict__ W1,
                                                const bf16_t* __restrict__ W3, int K, int N) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = 8 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ ((lrow >> 1) & 7);
  TileLoads o;
  o.na = t.rows > BM / 2 ? 4 : 2;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o.aoff[j] = (uint32_t)(min(64 * j + lrow, t.rows - 1) * K + lchunk * 8) * 2u;
  o.rsa = buffer_rsrc(A + (size_t)t.m0 * K, (uint32_t)t.rows * K * 2u);
  // fc1: panel rows alternate 32-row blocks of w1 and w3 over the same 32 columns;
  // row 64*j + lrow is in a w3 block exactly when lrow >= 32, i.e. for waves 4..7
  const bf16_t* wsel = (FC1 && wave >= 4) ? W3 : W1;
  o.rsb = buffer_rsrc(wsel + (size_t)t.e * N * K, (uint32_t)N * K * 2u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pr = 64 * j + lrow;
    const int gr = FC1 ? t.n0 + (pr >> 6) * 32 + (pr & 31) : t.n0 + pr;
    o.boff[j] = (uint32_t)(min(gr, N - 1) * K + lchunk * 8) * 2u;
  }
  return o;
}

// Loads of k-step kt into the LDS stage at `la` (this wave's first piece): the A pieces
// (part 0) or the panel pieces (part 1).
__device__ __forceinline__ void issue_loads(const TileLoads& o, uint32_t la, int kt, int part) {
  const uint32_t ko = (uint32_t)kt * BK * 2u;
  if (part == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < o.na) dma16(o.rsa, o.aoff[j], ko, la + j * 8192);
  } else {
    const uint32_t lb = la + A_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(o.rsb, o.boff[j], ko, lb + j * 8192);
  }
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
template <bool FC1, bool HALF>
__device__ __forceinline__ void run_tile(char* smem, const Tile& t, const TileLoads& ld,
                                         bf16_t* __restrict__ C, int N, int kb, int ke,
                                         float* __restrict__ part, int stage0, bool primed,
                                         const TileLoads& nxt, bool has_next, int nkb) {
  constexpr int WM = HALF ? 2 : 4;   // 32-row blocks of A per wave
  constexpr int WN = 2;              // 32-row panel blocks per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int arow0 = (wave & 1) * (HALF ? 64 : 128);   // first A row of this wave
  const int prow0 = (wave >> 1) * 64;                 // first panel row of this wave
  const uint32_t lds0 = lds_addr(smem) + wave * 1024;

  f32x16 acc[WM][WN];
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
        wf[buf][nb] = *reinterpret_cast<const bf16x8*>(sb + swz(prow0 + nb * 32 + fr, chk));
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
        af[buf][mb] = *reinterpret_cast<const bf16x8*>(sa + swz(arow0 + mb * 32 + fr, chk));
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
      for (int mb = 0; mb < WM; ++mb)
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][nb], af[ks & 1][mb],
                                                                acc[mb][nb], 0, 0, 0);
    }
  }
  // No barrier here: the next tile's first step went into the stage nobody reads in
  // this tile's last step, and its second step's loads are issued only after its
  // first barrier, which every wave reaches after finishing this tile's MFMAs.

  // Lane holds column m = lane & 31 of every 32x32 block and panel rows
  // 8*g + 4*(lane >> 5) + i (i = 0..3) for g = 0..3.
  if (part) {   // split-K share: raw float32 sums, row-major [BM][BP]
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
#pragma unroll
  for (int mb = 0; mb < WM; ++mb) {
    const int r = arow0 + mb * 32 + fr;
    if (r >= t.rows) continue;
    bf16_t* crow = C + (size_t)(t.m0 + r) * N;
    if (FC1) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = t.n0 + prow0 / 2 + g * 8 + (lane >> 5) * 4;
        if (n >= N) continue;
        const f32x16& a = acc[mb][0];
        const f32x16& b = acc[mb][1];
        store4(crow + n, silu_mul(a[4 * g], b[4 * g]), silu_mul(a[4 * g + 1], b[4 * g + 1]),
               silu_mul(a[4 * g + 2], b[4 * g + 2]), silu_mul(a[4 * g + 3], b[4 * g + 3]));
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < WN; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = t.n0 + prow0 + nb * 32 + g * 8 + (lane >> 5) * 4;
          if (n >= N) continue;
          const f32x16& a = acc[mb][nb];
          store4(crow + n, a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
      }
    }
  }
}

// Per-workgroup schedule tables in LDS: segment starts and the first 256-row block
// of each expert, built from offsets[] on the device.
struct Sched {
  int segoff[MAXE + 1];   // segment starts (clamped to the rows in use)
  int tstart[MAXE + 1];   // first 256-row block of each expert
  int wtot[16];
};

__device__ void build_sched(Sched& sc, const int32_t* __restrict__ offsets, int E, int m_cap) {
  const int tid = threadIdx.x;
  // clamped into [0, min(offsets[E], m_cap)], so offsets that break the contract
  // (negative, decreasing, past m_cap) can only shrink the work, never move it outside
  const int mend = max(0, min(offsets[E], m_cap));
  for (int e = tid; e <= E; e += blockDim.x) sc.segoff[e] = max(0, min(offsets[e], mend));
  __syncthreads();
  const int per = (MAXE + blockDim.x - 1) / blockDim.x;   // experts per thread (<= 4)
  int cnt[4], local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * per + i;
    cnt[i] = (i < per && e < E) ? (max(sc.segoff[e + 1] - sc.segoff[e], 0) + BM - 1) / BM : 0;
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
  t.rows = min(BM, sc.segoff[lo + 1] - t.m0);
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

template <bool FC1>
__global__ __launch_bounds__(NTHR, 1) void gg_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E, int K, int N,
    int m_cap, const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W3,
    bf16_t* __restrict__ C, float* __restrict__ ws, int slots) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  __shared__ Sched sc;
  build_sched(sc, offsets, E, m_cap);

  const int cols = FC1 ? BP / 2 : BP;
  const int n_nt = (N + cols - 1) / cols;
  const int total = sc.tstart[E] * n_nt;
  const int nk = K / BK;
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
  TileLoads ld = tile_loads<FC1>(cur.t, A, W1, W3, K, N);
  int stage0 = 0;
  bool primed = false;
  for (int w = vb; w < items; w += gridDim.x) {
    const bool has_next = w + (int)gridDim.x < items;
    Work nw = cur;
    TileLoads nl = ld;
    if (has_next) {
      nw = work(w + gridDim.x);
      nl = tile_loads<FC1>(nw.t, A, W1, W3, K, N);
    }
    if (cur.t.rows > BM / 2)
      run_tile<FC1, false>(smem, cur.t, ld, C, N, cur.kb, cur.ke, cur.part, stage0, primed, nl,
                           has_next, nw.kb);
    else
      run_tile<FC1, true>(smem, cur.t, ld, C, N, cur.kb, cur.ke, cur.part, stage0, primed, nl,
                          has_next, nw.kb);
    stage0 = (stage0 + cur.ke - cur.kb) & 1;
    primed = has_next;
    cur = nw;
    ld = nl;
  }
}

// Sums the split-K shares of the tail tiles in split order and applies the epilogue
// (fc1: silu(a)*b; fc2: the sum), rounding once to bf16. G must be the grid size the
// GEMM ran with.
template <bool FC1>
__global__ __launch_bounds__(256) void gg_tail_reduce(const int32_t* __restrict__ offsets, int E,
                                                      int K, int N, int m_cap, int G, int slots,
                                                      const float* __restrict__ ws,
                                                      bf16_t* __restrict__ C) {
  __shared__ Sched sc;
  build_sched(sc, offsets, E, m_cap);
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
    if (FC1) {
      const int fl = 4 * q;                              // h column inside the tile
      const int pa = (fl >> 5) * 64 + (fl & 31);         // its w1 panel row; w3 is 32 later
      float4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      for (int sh = 0; sh < sp.S; ++sh) {
        const float4 va = *reinterpret_cast<const float4*>(base + sh * stride + pa);
        const float4 vb = *reinterpret_cast<const float4*>(base + sh * stride + pa + 32);
        a.x += va.x; a.y += va.y; a.z += va.z; a.w += va.w;
        b.x += vb.x; b.y += vb.y; b.z += vb.z; b.w += vb.w;
      }
      const int n = t.n0 + fl;
      if (n < N)
        store4(C + (size_t)(t.m0 + r) * N + n, silu_mul(a.x, b.x), silu_mul(a.y, b.y),
               silu_mul(a.z, b.z), silu_mul(a.w, b.w));
    } else {
      const int nl = 4 * q;
      float4 a = {0, 0, 0, 0};
      for (int sh = 0; sh < sp.S; ++sh) {
        const float4 v = *reinterpret_cast<const float4*>(base + sh * stride + nl);
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      }
      const int n = t.n0 + nl;
      if (n < N) store4(C + (size_t)(t.m0 + r) * N + n, a.x, a.y, a.z, a.w);
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

size_t grouped_workspace_bytes() { return (size_t)cu_count() * BM * BP * sizeof(float); }

hipError_t launch_grouped_swiglu(int dt, int phases, const void* x_perm, const int32_t* offsets,
                                 const int32_t* tile_expert, int E, int D, int F, int m_tile,
                                 int64_t m_cap, const void* w1, const void* w3, const void* w2,
                                 void* h, void* y_perm, void* workspace, size_t ws_bytes,
                                 hipStream_t s) {
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
  const int G = cu_count();
  const dim3 grid(G), block(NTHR);
  float* ws = static_cast<float*>(workspace);
  const int slots = ws ? (int)std::min<size_t>(ws_bytes / (BM * BP * sizeof(float)), 1 << 20) : 0;
  const dim3 rgrid(4 * G), rblock(256);
  if (phases & 1) {
    hipLaunchKernelGGL(gg_bf16_kernel<true>, grid, block, 0, s, static_cast<const bf16_t*>(x_perm),
                       offsets, E, D, F, (int)m_cap, static_cast<const bf16_t*>(w1),
                       static_cast<const bf16_t*>(w3), static_cast<bf16_t*>(h), ws, slots);
    if (slots)
      hipLaunchKernelGGL(gg_tail_reduce<true>, rgrid, rblock, 0, s, offsets, E, D, F, (int)m_cap,
                         G, slots, ws, static_cast<bf16_t*>(h));
  }
  if (phases & 2) {
    hipLaunchKernelGGL(gg_bf16_kernel<false>, grid, block, 0, s, static_cast<const bf16_t*>(h),
                       offsets, E, F, D, (int)m_cap, static_cast<const bf16_t*>(w2),
                       static_cast<const bf16_t*>(w2), static_cast<bf16_t*>(y_perm), ws, slots);
    if (slots)
      hipLaunchKernelGGL(gg_tail_reduce<false>, rgrid, rblock, 0, s, offsets, E, F, D, (int)m_cap,
                         G, slots, ws, static_cast<bf16_t*>(y_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
