// Dispatch metadata and permute ("Expert Parallelism (EP)", llm-infra-atlas:
// section 1 "MoE layer 的 forward 通路", its forward-path figure: the per-expert token counts,
// then the reordering that groups each local expert's tokens together; section 2:
// the output layout must be expert-contiguous with every segment aligned to the GEMM
// M tile).
//
// Two launches while the histogram table is small (hist_kernel, then place_kernel, which
// ranks and copies in one pass; up to 2^24 table reads in all, every benchmark workload),
// else three:
//   1. hist_kernel   per 256-token block, the slots of each expert (LDS atomics:
//                    counts do not depend on their order) and the bad-index count.
//   2. rank_kernel   one workgroup per histogram block reads the small histogram
//                    table and derives the counts, padded offsets and its block's
//                    starting rank per expert (the earlier blocks), so no
//                    single-workgroup scan is needed; it ranks its slots stably
//                    (per-wave counts prefix-summed over the waves, then a ballot
//                    match inside each wave) and writes dst_row / src_row. The last
//                    workgroup writes counts, offsets, tile_expert, the unused rows
//                    and the error flag.
//   3. copy_kernel   streams the rows: each token row is read once (16-byte chunks of
//                    four tokens in flight per thread) and written to its k rows; the
//                    pad rows of every segment are zeroed by the same grid, a row per
//                    wave.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Scratch of the allocation-free permute (moe_permute_noalloc): the histogram table of
// one call, held by every device the library runs on until the process ends. Host code
// never passes `scratch` itself to a kernel (on the host it names a stand-in, not device
// memory): it uses the address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) int32_t scratch[kPermuteScratchBytes / sizeof(int32_t)];

hipError_t permute_scratch(void** ptr) {
  static std::mutex mu;
  static void* cache[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cache[dev] = p;
  }
  *ptr = cache[dev];
  return hipSuccess;
}

namespace {

constexpr int kMaxExperts = 1024;
constexpr int kThreads = 256;
constexpr int kBatch = 8;    // index loads per thread in flight while counting
constexpr int kCopyTokens = 4;   // tokens whose row chunks a copy thread reads together

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx, int T,
                                                        int k, int E, int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ bad) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int nbad;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  if (threadIdx.x == 0) nbad = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kHistTokens * k;
  const int64_t a1 = min(a0 + (int64_t)kHistTokens * k, (int64_t)T * k);
  // kBatch loads per thread go out before their atomics: one memory round trip per batch
  for (int64_t g = a0 + threadIdx.x; g < a1; g += (int64_t)kThreads * kBatch) {
    int ev[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t a = g + (int64_t)i * kThreads;
      ev[i] = a < a1 ? idx[a] : -1;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int e = ev[i];
      if (e >= 0 && e < E)
        atomicAdd(&cnt[e], 1);
      else if (e != -1)
        atomicAdd(&nbad, 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) hist[(size_t)blockIdx.x * E + e] = cnt[e];
  if (threadIdx.x == 0) bad[blockIdx.x] = nbad;
}

// In-place inclusive prefix of the histogram table over its blocks: hist[h][e] becomes
// expert e's slots in histogram blocks 0..h, so block hb's starting rank is row hb-1
// and the totals are the last row. A workgroup takes 64 experts, a lane each, and its
// four waves contiguous quarters of the blocks: each wave sums its quarter, the sums are
// prefix-summed over the waves, and each wave rewrites its quarter. Integer sums: the
// result does not depend on their order.
__global__ __launch_bounds__(kThreads) void hist_scan_kernel(int32_t* __restrict__ hist, int nbh,
                                                             int E) {
  constexpr int kWaves = kThreads / kWave;
  __shared__ int wsum[kWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int e = blockIdx.x * kWave + lane;
  const int per = (nbh + kWaves - 1) / kWaves;
  const int h0 = min(nbh, wv * per), h1 = min(nbh, h0 + per);
  int run = 0;
  if (e < E) {
    for (int h = h0; h < h1; h += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = h + j < h1 ? hist[(int64_t)(h + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) run += v[j];
    }
  }
  wsum[wv][lane] = run;
  __syncthreads();
  run = 0;
  for (int w = 0; w < wv; ++w) run += wsum[w][lane];
  if (e < E) {
    for (int h = h0; h < h1; h += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = h + j < h1 ? hist[(int64_t)(h + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        run += v[j];
        if (h + j < h1) hist[(int64_t)(h + j) * E + e] = run;
      }
    }
  }
}

// The rank pass reads the whole table in each workgroup up to this many entries; above
// it the table is prefix-summed first (hist_scan_kernel) and each workgroup reads two rows.
constexpr int kScanAbove = 2048;

// Exclusive prefix sum over the 256 threads of the block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wsum[wid] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wid; ++w) before += wsum[w];
  return before + inc - v;
}

// src_row[r] = -1 over rows [lo, hi) of every expert e < E, bounds(e, lo, hi) giving the
// range. Each wave takes 64 experts at a time: its lanes read their bounds, then the wave
// walks them one by one with the bounds in scalar registers and its lanes over the rows,
// so no step of the walk waits on LDS. WV is the wave's index (uniform).
template <typename Bounds>
__device__ __forceinline__ void clear_rows(int32_t* __restrict__ src_row, int E, int wv, int lane,
                                           Bounds bounds) {
  constexpr int kWaves = kThreads / kWave;
  for (int e0 = wv * kWave; e0 < E; e0 += kWaves * kWave) {
    int lo = 0, hi = 0;
    if (e0 + lane < E) bounds(e0 + lane, lo, hi);
    const int ne = min(kWave, E - e0);
    for (int j = 0; j < ne; ++j) {
      const int l = __builtin_amdgcn_readlane(lo, j), h = __builtin_amdgcn_readlane(hi, j);
      for (int r = l + lane; r < h; r += kWave) src_row[r] = -1;
    }
  }
}

// MASKED: the masked layout (fixed slabs of `cap` rows, expert e from row e*cap; m_tile
// unused, m_cap = E*cap): ranks at or past cap are dropped, counts are capped, offsets
// and tile_expert are not written.
//
// Workgroup hb < nbh ranks the slots of histogram block hb (tokens [256 hb, 256 hb + 256)):
// its starting rank per expert is the sum of the table rows before hb. Up to kScanAbove
// entries each workgroup reads the whole nbh x E table; above, SCANNED, the table
// holds inclusive prefixes (hist_scan_kernel), row hb-1 is the start and row nbh-1 the
// totals, so the reads stay linear in the token count. Its four waves take contiguous quarters of the block's slots: each
// counts its quarter per expert, the counts are prefix-summed over the waves, and each
// wave then ranks its quarter 64 slots at a time (ballot match), so ranks follow slot
// order. Workgroup nbh writes counts, offsets, tile_expert, the unused rows and the
// error flag.
template <bool MASKED>
__global__ __launch_bounds__(kThreads) void rank_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int m_tile, int cap, int64_t m_cap,
    int nbh, bool scanned,
    const int32_t* __restrict__ hist, const int32_t* __restrict__ bad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ dev_err,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row) {
  constexpr int kWaves = kThreads / kWave;
  constexpr int kChunks = kHistTokens * kMaxTopK / kWaves / kWave;   // 64-slot chunks per wave
  __shared__ int off[kMaxExperts + 1];   // padded segment starts
  __shared__ int cnt[kMaxExperts];       // rows per expert
  __shared__ int base[kMaxExperts];      // rank of this block's first slot per expert
  __shared__ int wcnt[kWaves][kMaxExperts];   // per wave: its slots, then its next rank
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hb = blockIdx.x;
  const bool token_block = hb < nbh;
  const int t_begin = hb * kHistTokens;
  const int t_end = token_block ? min(T, t_begin + kHistTokens) : t_begin;
  const int n = (t_end - t_begin) * k;   // slots of this block
  const int64_t a0 = (int64_t)t_begin * k;
  const int per_wave = (n + kWaves * kWave - 1) / (kWaves * kWave) * kWave;
  const int w0 = min(n, wv * per_wave), w1 = min(n, w0 + per_wave);   // this wave's slots

  for (int e = tid; e < E; e += kThreads) {
    cnt[e] = scanned ? hist[(int64_t)(nbh - 1) * E + e] : 0;
    base[e] = scanned && token_block && hb > 0 ? hist[(int64_t)(hb - 1) * E + e] : 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
  }
  // this wave's expert indices, fetched once (their load overlaps the table's)
  int own[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int a = w0 + i * kWave + lane;
    own[i] = a < w1 ? idx[a0 + a] : -1;
  }
  __syncthreads();
  // per-expert totals and this block's starting rank (earlier histogram blocks);
  // integer LDS atomics, so the sums do not depend on their order
  for (int i0 = tid; !scanned && i0 < nbh * E; i0 += kThreads * kBatch) {
    int cv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j * kThreads;
      cv[j] = i < nbh * E ? hist[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (cv[j] == 0) continue;
      const int i = i0 + j * kThreads;
      const int h = i / E, e = i - h * E;
      atomicAdd(&cnt[e], cv[j]);
      if (h < hb) atomicAdd(&base[e], cv[j]);
    }
  }
  // this wave's slots per expert
#pragma unroll
  for (int i = 0; i < kChunks; ++i)
    if (own[i] >= 0 && own[i] < E) atomicAdd(&wcnt[wv][own[i]], 1);
  __syncthreads();
  if (MASKED) {
    for (int e = tid; e <= E; e += kThreads) off[e] = e * cap;
  } else {
    int padded[4] = {0, 0, 0, 0};
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) padded[i] = (cnt[e] + m_tile - 1) / m_tile * m_tile;
      local += padded[i];
    }
    int run = block_exclusive_scan(local, wsum);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) off[e] = run;
      run += padded[i];
    }
    if (tid == kThreads - 1) off[E] = run;
  }
  // each wave's starting rank per expert: the block's, plus the earlier waves' slots
  for (int e = tid; e < E; e += kThreads) {
    int run = base[e];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = wcnt[w][e];
      wcnt[w][e] = run;
      run += c;
    }
  }
  __syncthreads();

  if (!token_block && MASKED) {   // capped counts, unused slab rows, error flags
    int over = 0;
    for (int e = tid; e < E; e += kThreads) {
      counts[e] = min(cnt[e], cap);
      over |= cnt[e] > cap;
    }
    clear_rows(src_row, E, wv, lane, [&](int e, int& lo, int& hi) {
      lo = e * cap + min(cnt[e], cap);
      hi = (e + 1) * cap;
    });
    int anybad = 0;
    for (int h = tid; h < nbh; h += kThreads) anybad |= bad[h] != 0;
    anybad = __syncthreads_or(anybad);
    over = __syncthreads_or(over);
    if (tid == 0) *dev_err = anybad | (over << 1);
    return;
  }
  if (!token_block) {   // metadata, unused rows, error flag
    for (int i = tid; i < E; i += kThreads) counts[i] = cnt[i];
    for (int i = tid; i <= E; i += kThreads) offsets[i] = off[i];
    const int total = off[E];
    const int64_t ntiles = m_cap / m_tile;
    for (int64_t q = tid; q < ntiles; q += kThreads) {
      const int64_t r = q * m_tile;
      int owner = -1;
      if (r < total) {
        int lo = 0, hi = E;  // largest e with off[e] <= r
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (off[mid] <= r) lo = mid; else hi = mid;
        }
        owner = lo;
      }
      tile_expert[q] = owner;
    }
    clear_rows(src_row, E, wv, lane, [&](int e, int& lo, int& hi) {   // every segment's pad rows
      lo = off[e] + cnt[e];
      hi = off[e + 1];
    });
    for (int64_t r = total + tid; r < m_cap; r += kThreads) src_row[r] = -1;
    int anybad = 0;
    for (int h = tid; h < nbh; h += kThreads) anybad |= bad[h] != 0;
    anybad = __syncthreads_or(anybad);
    if (tid == 0) *dev_err = anybad;
    return;
  }

  // rank this wave's slots in order, 64 at a time; wcnt[wv][e] is the wave's next rank
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  int* next = wcnt[wv];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int r0 = w0 + i * kWave;
    if (r0 >= w1) break;
    const int a = r0 + lane;
    const int e = own[i];
    const bool valid = a < w1 && e >= 0 && e < E;
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t bal = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? bal : ~bal;
    }
    int pos = -1;
    if (valid) {
      const int rank = next[e] + __popcll(same & lt);
      pos = (MASKED && rank >= cap) ? -1 : off[e] + rank;   // masked: past the slab is dropped
    }
    if (pos >= m_cap) pos = -1;  // cannot happen with consistent counts; never write past m_cap
    __builtin_amdgcn_wave_barrier();
    if (valid && (same >> lane) == 1ull) next[e] = next[e] + __popcll(same);
    __builtin_amdgcn_wave_barrier();
    if (a < w1) {
      dst_row[a0 + a] = pos;
      if (pos >= 0) src_row[pos] = (int32_t)(a0 + a);
    }
  }
}

// Row copy. A work item is a group of kCopyTokens consecutive tokens x a slab of 256
// 16-byte chunks of their rows; workgroups take items in turn. Thread i reads chunk i of
// the slab for every token of the group (kCopyTokens reads in flight) and writes it to
// each of the token's destination rows. Then the pad rows of every segment, [offsets[e] + counts[e],
// offsets[e+1]), are zeroed one row per wave: the rows are numbered across experts by a
// prefix sum in LDS and each wave finds its expert by binary search. dst_row, offsets and
// counts come from rank_kernel; E = 0 skips the pad rows (the masked layout has none).
template <typename TIn>
__global__ __launch_bounds__(kThreads) void copy_kernel(
    const TIn* __restrict__ x, int T, int D, int k, int E, const int32_t* __restrict__ dst_row,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    TIn* __restrict__ x_perm) {
  constexpr int V = Chunk<TIn>::V;
  __shared__ int ds[kCopyTokens * kMaxTopK];
  __shared__ int pstart[kMaxExperts];       // first pad row of each expert
  __shared__ int ppre[kMaxExperts + 1];     // pad rows of the experts before e
  __shared__ int wsum[kThreads / kWave];
  const int nck = D / V;
  const int nslab = (nck + kThreads - 1) / kThreads;   // 256-chunk column slabs of a row
  const int64_t items = (int64_t)((T + kCopyTokens - 1) / kCopyTokens) * nslab;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = (int)(it / nslab);
    const int t0 = g * kCopyTokens;
    const int nt = min(kCopyTokens, T - t0);
    __syncthreads();   // the previous item's destinations are no longer read
    for (int i = threadIdx.x; i < nt * k; i += kThreads) ds[i] = dst_row[(int64_t)t0 * k + i];
    __syncthreads();
    const int c = (int)(it - (int64_t)g * nslab) * kThreads + threadIdx.x;
    if (c < nck) {
      u32x4 v[kCopyTokens];
#pragma unroll
      for (int i = 0; i < kCopyTokens; ++i)
        if (i < nt) v[i] = ld16_nt(x + (int64_t)(t0 + i) * D + (int64_t)c * V);
#pragma unroll
      for (int i = 0; i < kCopyTokens; ++i) {
        if (i >= nt) continue;
        for (int j = 0; j < k; ++j) {
          const int d = ds[i * k + j];
          if (d >= 0) st16(x_perm + (int64_t)d * D + (int64_t)c * V, v[i]);
        }
      }
    }
  }
  if (E == 0) return;
  // pad rows, numbered across experts
  int pads[4] = {0, 0, 0, 0};
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x * 4 + i;
    if (e < E) {
      const int r0 = offsets[e] + counts[e];
      pstart[e] = r0;
      pads[i] = max(0, offsets[e + 1] - r0);
    }
    local += pads[i];
  }
  int run = block_exclusive_scan(local, wsum);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x * 4 + i;
    if (e < E) ppre[e] = run;
    run += pads[i];
  }
  if (threadIdx.x == kThreads - 1) ppre[E] = run;
  __syncthreads();
  const int npad = ppre[E];
  const int lane = threadIdx.x & (kWave - 1);
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int nwaves = gridDim.x * (kThreads / kWave);
  for (int q = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave; q < npad; q += nwaves) {
    int lo = 0, hi = E;   // largest e with ppre[e] <= q
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ppre[mid] <= q) lo = mid; else hi = mid;
    }
    TIn* row = x_perm + (int64_t)(pstart[lo] + (q - ppre[lo])) * D;
    for (int c = lane; c < nck; c += kWave) st16(row + (int64_t)c * V, z);
  }
}

// Rank and copy in one launch (the contiguous layout, when the histogram table is small
// enough for every workgroup to read it, or SCANNED into inclusive prefixes; see
// launch_permute). Workgroup g takes tokens [kCopyTokens g, kCopyTokens g + kCopyTokens):
// it sums the table into the per-expert totals and its histogram block's starting ranks
// (reads them off rows nbh-1 and hb-1 when SCANNED), counts the slots of that block that
// precede its tokens, derives the padded offsets, ranks its own slots in slot order
// (ballot match in wave 0), writes dst_row / src_row, and copies its tokens' rows to
// their destination rows. Every workgroup then takes a share of the pad rows (zeroed,
// src_row -1) and of the rows past offsets[E] (src_row -1); workgroup 0 also writes
// counts, offsets, tile_expert and the error flag.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void place_kernel(
    const TIn* __restrict__ x, const int32_t* __restrict__ idx, int T, int D, int k, int E,
    int m_tile, int64_t m_cap, int nbh, bool scanned, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ bad, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ dev_err,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row, TIn* __restrict__ x_perm) {
  constexpr int V = Chunk<TIn>::V;
  __shared__ int off[kMaxExperts + 1];   // padded segment starts
  __shared__ int cnt[kMaxExperts];       // rows per expert
  __shared__ int base[kMaxExperts];      // next free row per expert for this workgroup
  __shared__ int ds[kCopyTokens * kMaxTopK];
  __shared__ int pstart[kMaxExperts];    // first pad row of each expert
  __shared__ int ppre[kMaxExperts + 1];  // pad rows of the experts before e
  __shared__ int wsum[kThreads / kWave];
  __shared__ int wsum2[kThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int t0 = blockIdx.x * kCopyTokens;
  const int nt = min(kCopyTokens, T - t0);
  const int hb = t0 / kHistTokens;
  const int n = nt * k;                  // this workgroup's slots
  const int64_t a0 = (int64_t)t0 * k;

  for (int e = tid; e < E; e += kThreads) {
    cnt[e] = scanned ? hist[(int64_t)(nbh - 1) * E + e] : 0;
    base[e] = scanned && hb > 0 ? hist[(int64_t)(hb - 1) * E + e] : 0;
  }
  int own[kCopyTokens * kMaxTopK / kWave];
  if (tid < kWave) {
#pragma unroll
    for (int i = 0; i < kCopyTokens * kMaxTopK / kWave; ++i) {
      const int a = i * kWave + tid;
      own[i] = a < n ? idx[a0 + a] : -1;
    }
  }
  __syncthreads();
  // totals and the starting rank of histogram block hb (integer atomics: any order)
  for (int i0 = tid; !scanned && i0 < nbh * E; i0 += kThreads * kBatch) {
    int cv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j * kThreads;
      cv[j] = i < nbh * E ? hist[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (cv[j] == 0) continue;
      const int i = i0 + j * kThreads;
      const int h = i / E, e = i - h * E;
      atomicAdd(&cnt[e], cv[j]);
      if (h < hb) atomicAdd(&base[e], cv[j]);
    }
  }
  // slots of block hb before this workgroup's tokens
  const int64_t p0 = (int64_t)hb * kHistTokens * k;
  for (int64_t g = p0 + tid; g < a0; g += (int64_t)kThreads * kBatch) {
    int ev[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t a = g + (int64_t)i * kThreads;
      ev[i] = a < a0 ? idx[a] : -1;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (ev[i] >= 0 && ev[i] < E) atomicAdd(&base[ev[i]], 1);
  }
  __syncthreads();
  {
    int padded[4] = {0, 0, 0, 0};
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) padded[i] = (cnt[e] + m_tile - 1) / m_tile * m_tile;
      local += padded[i];
    }
    int run = block_exclusive_scan(local, wsum);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) off[e] = run;
      run += padded[i];
    }
    if (tid == kThreads - 1) off[E] = run;
  }
  __syncthreads();

  // rank this workgroup's slots in slot order (wave 0), then its rows' destinations
  if (tid < kWave) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
#pragma unroll
    for (int i = 0; i < kCopyTokens * kMaxTopK / kWave; ++i) {
      const int r0 = i * kWave;
      if (r0 >= n) break;
      const int a = r0 + lane;
      const int e = own[i];
      const bool valid = a < n && e >= 0 && e < E;
      uint64_t same = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const uint64_t bal = __ballot(valid && ((e >> bit) & 1));
        same &= ((e >> bit) & 1) ? bal : ~bal;
      }
      int pos = -1;
      if (valid) pos = off[e] + base[e] + __popcll(same & lt);
      if (pos >= m_cap) pos = -1;  // cannot happen with consistent counts; never write past m_cap
      __builtin_amdgcn_wave_barrier();
      if (valid && (same >> lane) == 1ull) base[e] = base[e] + __popcll(same);
      __builtin_amdgcn_wave_barrier();
      if (a < n) {
        ds[a] = pos;
        dst_row[a0 + a] = pos;
        if (pos >= 0) src_row[pos] = (int32_t)(a0 + a);
      }
    }
  }
  __syncthreads();
  const int nck = D / V;
  for (int c = tid; c < nck; c += kThreads) {
    u32x4 v[kCopyTokens];
#pragma unroll
    for (int i = 0; i < kCopyTokens; ++i)
      if (i < nt) v[i] = ld16_nt(x + (int64_t)(t0 + i) * D + (int64_t)c * V);
#pragma unroll
    for (int i = 0; i < kCopyTokens; ++i) {
      if (i >= nt) continue;
      for (int j = 0; j < k; ++j) {
        const int d = ds[i * k + j];
        if (d >= 0) st16(x_perm + (int64_t)d * D + (int64_t)c * V, v[i]);
      }
    }
  }

  // pad rows (zero rows, src_row -1), numbered across experts; rows past offsets[E]
  {
    int pads[4] = {0, 0, 0, 0};
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) {
        pstart[e] = off[e] + cnt[e];
        pads[i] = off[e + 1] - off[e] - cnt[e];
      }
      local += pads[i];
    }
    int run = block_exclusive_scan(local, wsum2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) ppre[e] = run;
      run += pads[i];
    }
    if (tid == kThreads - 1) ppre[E] = run;
  }
  __syncthreads();
  const int npad = ppre[E];
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int nwaves = gridDim.x * (kThreads / kWave);
  for (int q = blockIdx.x * (kThreads / kWave) + tid / kWave; q < npad; q += nwaves) {
    int lo = 0, hi = E;   // largest e with ppre[e] <= q
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ppre[mid] <= q) lo = mid; else hi = mid;
    }
    const int r = pstart[lo] + (q - ppre[lo]);
    TIn* row = x_perm + (int64_t)r * D;
    for (int c = lane; c < nck; c += kWave) st16(row + (int64_t)c * V, z);
    if (lane == 0) src_row[r] = -1;
  }
  const int64_t total = off[E];
  for (int64_t r = total + (int64_t)blockIdx.x * kThreads + tid; r < m_cap;
       r += (int64_t)gridDim.x * kThreads)
    src_row[r] = -1;
  if (blockIdx.x == 0) {   // metadata and the error flag
    for (int i = tid; i < E; i += kThreads) counts[i] = cnt[i];
    for (int i = tid; i <= E; i += kThreads) offsets[i] = off[i];
    const int64_t ntiles = m_cap / m_tile;
    for (int64_t q = tid; q < ntiles; q += kThreads) {
      const int64_t r = q * m_tile;
      int owner = -1;
      if (r < total) {
        int lo = 0, hi = E;  // largest e with off[e] <= r
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (off[mid] <= r) lo = mid; else hi = mid;
        }
        owner = lo;
      }
      tile_expert[q] = owner;
    }
    int anybad = 0;
    for (int h = tid; h < nbh; h += kThreads) anybad |= bad[h] != 0;
    anybad = __syncthreads_or(anybad);
    if (tid == 0) *dev_err = anybad;
  }
}

// Scales of the FP8 payload into k-step words: out[s * m_cap + row] is word s of the
// [T, D/32]-byte scale row of the token that fills permuted row `row` (its src_row
// assignment / k), 0 for a pad row; rows at or past offsets[E] are not written. Threads
// run along the rows, so the stores are whole lines; the loads are single words of the
// scale rows (T * D/32 bytes, small enough to stay in L2).
__global__ __launch_bounds__(kThreads) void scale_ksteps_kernel(
    const uint32_t* __restrict__ xs, int nsw, int k, int E, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ src_row, int64_t m_cap, uint32_t* __restrict__ out) {
  const int64_t used = max<int64_t>(0, min<int64_t>(offsets[E], m_cap));
  const int64_t n = used * nsw;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n;
       g += (int64_t)gridDim.x * kThreads) {
    const int64_t st = g / used, row = g - st * used;
    const int a = src_row[row];
    out[st * m_cap + row] = a >= 0 ? xs[(int64_t)(a / k) * nsw + st] : 0u;
  }
}

// Masked layout for a batch of at most kHistTokens tokens (decode): one launch in place
// of histogram + rank + copy. Every workgroup ranks all T*k slots itself, exactly as
// rank_kernel ranks one histogram block: each wave counts its contiguous share of the
// slots per expert, the counts are prefix-summed over the waves, and each wave ranks
// its slots 64 at a time with ballots. The destinations stay in LDS for the copy of the
// workgroup's share of the rows (items of kCopyTokens tokens x a 256-chunk slab, as in
// copy_kernel), whose first rows are read before the ranking so that their latency
// hides behind it. One more workgroup, the last, copies nothing and writes the maps,
// the capped counts, the unused slab rows of src_row and the error flags. A few hundred
// slots cost each workgroup less than the two launches they save.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void masked_small_kernel(
    const TIn* __restrict__ x, const int32_t* __restrict__ idx, int T, int D, int k, int E,
    int cap, TIn* __restrict__ x_masked, int32_t* __restrict__ counts,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row,
    int32_t* __restrict__ dev_err) {
  constexpr int V = Chunk<TIn>::V;
  constexpr int kWaves = kThreads / kWave;
  constexpr int kChunks = kHistTokens * kMaxTopK / kWaves / kWave;   // 64-slot chunks per wave
  __shared__ int cnt[kMaxExperts];
  __shared__ int wcnt[kWaves][kMaxExperts];   // per wave: its slots, then its next rank
  __shared__ int ds[kHistTokens * kMaxTopK];  // every slot's destination row (-1: none)
  __shared__ int nbad;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool meta = blockIdx.x == gridDim.x - 1;   // the others copy
  const int ncopy = gridDim.x - 1;
  const int n = T * k;
  const int nck = D / V;
  const int nslab = (nck + kThreads - 1) / kThreads;
  const int items = (T + kCopyTokens - 1) / kCopyTokens * nslab;
  const int per_wave = (n + kWaves * kWave - 1) / (kWaves * kWave) * kWave;
  const int w0 = min(n, wv * per_wave), w1 = min(n, w0 + per_wave);   // this wave's slots

  for (int e = tid; e < E; e += kThreads) {
    cnt[e] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
  }
  if (tid == 0) nbad = 0;
  // the first item's rows, read ahead of the ranking (a copy workgroup has one: ncopy <= items)
  u32x4 v[kCopyTokens];
  if (!meta) {
    const int g = blockIdx.x / nslab;
    const int t0 = g * kCopyTokens;
    const int c = (blockIdx.x - g * nslab) * kThreads + tid;
    if (c < nck) {
#pragma unroll
      for (int i = 0; i < kCopyTokens; ++i)
        if (t0 + i < T) v[i] = ld16_nt(x + (int64_t)(t0 + i) * D + (int64_t)c * V);
    }
  }
  int own[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int a = w0 + i * kWave + lane;
    own[i] = a < w1 ? idx[a] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int e = own[i];
    if (e >= 0 && e < E)
      atomicAdd(&wcnt[wv][e], 1);
    else if (e != -1)
      atomicAdd(&nbad, 1);
  }
  __syncthreads();
  // totals, and each wave's starting rank per expert (the earlier waves' slots)
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = wcnt[w][e];
      wcnt[w][e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();

  // rank this wave's slots in order, 64 at a time; wcnt[wv][e] is the wave's next rank
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  int* next = wcnt[wv];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int r0 = w0 + i * kWave;
    if (r0 >= w1) break;
    const int a = r0 + lane;
    const int e = own[i];
    const bool valid = a < w1 && e >= 0 && e < E;
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t bal = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? bal : ~bal;
    }
    int pos = -1;
    if (valid) {
      const int rank = next[e] + __popcll(same & lt);
      pos = rank >= cap ? -1 : e * cap + rank;   // past the slab: dropped
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (same >> lane) == 1ull) next[e] = next[e] + __popcll(same);
    __builtin_amdgcn_wave_barrier();
    if (a < w1) {
      ds[a] = pos;
      if (meta) {
        dst_row[a] = pos;
        if (pos >= 0) src_row[pos] = a;
      }
    }
  }
  __syncthreads();
  if (meta) {   // capped counts, unused slab rows, error flags
    int over = 0;
    for (int e = tid; e < E; e += kThreads) {
      counts[e] = min(cnt[e], cap);
      over |= cnt[e] > cap;
    }
    clear_rows(src_row, E, wv, lane, [&](int e, int& lo, int& hi) {   // unused slab rows
      lo = e * cap + min(cnt[e], cap);
      hi = (e + 1) * cap;
    });
    over = __syncthreads_or(over);
    if (tid == 0) *dev_err = (nbad != 0) | (over << 1);
    return;
  }

  // the rows: this workgroup's items, the first one already in v
  for (int it = blockIdx.x; it < items; it += ncopy) {
    const int g = it / nslab;
    const int t0 = g * kCopyTokens;
    const int nt = min(kCopyTokens, T - t0);
    const int c = (it - g * nslab) * kThreads + tid;
    if (c >= nck) continue;
    if (it != blockIdx.x) {
#pragma unroll
      for (int i = 0; i < kCopyTokens; ++i)
        if (i < nt) v[i] = ld16_nt(x + (int64_t)(t0 + i) * D + (int64_t)c * V);
    }
#pragma unroll
    for (int i = 0; i < kCopyTokens; ++i) {
      if (i >= nt) continue;
      for (int j = 0; j < k; ++j) {
        const int d = ds[(t0 + i) * k + j];
        if (d >= 0) st16(x_masked + (int64_t)d * D + (int64_t)c * V, v[i]);
      }
    }
  }
}

// Prefix-sums a large histogram table in place for the rank pass (true), or leaves a
// small one for each rank workgroup to read whole (false).
bool scan_hist(int32_t* hist, int nbh, int E, hipStream_t s) {
  if ((int64_t)nbh * E <= kScanAbove) return false;
  hipLaunchKernelGGL(hist_scan_kernel, dim3((E + kWave - 1) / kWave), dim3(kThreads), 0, s, hist,
                     nbh, E);
  return true;
}

hipError_t launch_copy(int dt, const void* x, int T, int D, int k, int E,
                              const int32_t* dst_row, const int32_t* counts,
                              const int32_t* offsets, void* x_perm, hipStream_t s) {
  // a workgroup per work item, at most 8 per CU, and at least one per CU for the pad rows
  const int64_t items = (int64_t)((T + kCopyTokens - 1) / kCopyTokens) *
                        ((D / (dt == kF32 ? 4 : 8) + kThreads - 1) / kThreads);
  const int grid = (int)std::min<int64_t>(8 * cu_count(), std::max<int64_t>(items, cu_count()));
  if (dt == kF32)
    hipLaunchKernelGGL(copy_kernel<float>, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const float*>(x), T, D, k, E, dst_row, counts, offsets,
                       static_cast<float*>(x_perm));
  else
    hipLaunchKernelGGL(copy_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(x), T, D, k, E, dst_row, counts, offsets,
                       static_cast<bf16_t*>(x_perm));
  return hipGetLastError();
}

}  // namespace

size_t permute_workspace_bytes(int T, int k, int E) {
  (void)k;
  const size_t nbh = (size_t)(T + kHistTokens - 1) / kHistTokens;
  return nbh * ((size_t)E + 1) * sizeof(int32_t);
}

hipError_t launch_permute(int dt, const void* x, const int32_t* topk_idx, int T, int D, int E,
                          int k, int m_tile, int64_t m_cap, void* x_perm, int32_t* counts,
                          int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                          int32_t* tile_expert, void* workspace, int32_t* dev_err, hipStream_t s) {
  const int nbh = (T + kHistTokens - 1) / kHistTokens;
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* bad = hist + (size_t)nbh * E;
  hipLaunchKernelGGL(hist_kernel, dim3(nbh), dim3(kThreads), 0, s, topk_idx, T, k, E, hist, bad);
  const int ngroups = (T + kCopyTokens - 1) / kCopyTokens;
  // rank and copy in one launch while every workgroup reading the whole table stays cheap
  // (at most 2^24 table reads in all: e.g. 16384 tokens with 64 experts), or reads two
  // rows of the prefix-summed table
  const bool scanned = scan_hist(hist, nbh, E, s);
  if (scanned || (int64_t)ngroups * nbh * E <= ((int64_t)1 << 24)) {
    if (dt == kF32)
      hipLaunchKernelGGL(place_kernel<float>, dim3(ngroups), dim3(kThreads), 0, s,
                         static_cast<const float*>(x), topk_idx, T, D, k, E, m_tile, m_cap, nbh,
                         scanned, hist, bad, counts, offsets, tile_expert, dev_err, dst_row,
                         src_row,
                         static_cast<float*>(x_perm));
    else
      hipLaunchKernelGGL(place_kernel<bf16_t>, dim3(ngroups), dim3(kThreads), 0, s,
                         static_cast<const bf16_t*>(x), topk_idx, T, D, k, E, m_tile, m_cap, nbh,
                         scanned, hist, bad, counts, offsets, tile_expert, dev_err, dst_row,
                         src_row,
                         static_cast<bf16_t*>(x_perm));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(rank_kernel<false>, dim3(nbh + 1), dim3(kThreads), 0, s, topk_idx, T, k, E,
                     m_tile, 0, m_cap, nbh, scanned, hist, bad, counts, offsets, tile_expert, dev_err,
                     dst_row, src_row);
  return launch_copy(dt, x, T, D, k, E, dst_row, counts, offsets, x_perm, s);
}

hipError_t launch_permute_masked(int dt, const void* x, const int32_t* topk_idx, int T, int D,
                                 int E, int k, int cap, void* x_masked, int32_t* counts,
                                 int32_t* dst_row, int32_t* src_row, void* workspace,
                                 int32_t* dev_err, hipStream_t s) {
  if (T <= kHistTokens) {   // a decode batch: one launch
    const int items = (T + kCopyTokens - 1) / kCopyTokens *
                      ((D / (dt == kF32 ? 4 : 8) + kThreads - 1) / kThreads);
    const int grid = std::min(8 * cu_count(), items) + 1;   // + the metadata workgroup
    if (dt == kF32)
      hipLaunchKernelGGL(masked_small_kernel<float>, dim3(grid), dim3(kThreads), 0, s,
                         static_cast<const float*>(x), topk_idx, T, D, k, E, cap,
                         static_cast<float*>(x_masked), counts, dst_row, src_row, dev_err);
    else
      hipLaunchKernelGGL(masked_small_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s,
                         static_cast<const bf16_t*>(x), topk_idx, T, D, k, E, cap,
                         static_cast<bf16_t*>(x_masked), counts, dst_row, src_row, dev_err);
    return hipGetLastError();
  }
  const int nbh = (T + kHistTokens - 1) / kHistTokens;
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* bad = hist + (size_t)nbh * E;
  hipLaunchKernelGGL(hist_kernel, dim3(nbh), dim3(kThreads), 0, s, topk_idx, T, k, E, hist, bad);
  const bool scanned = scan_hist(hist, nbh, E, s);
  hipLaunchKernelGGL(rank_kernel<true>, dim3(nbh + 1), dim3(kThreads), 0, s, topk_idx, T, k, E, 0,
                     cap, (int64_t)E * cap, nbh, scanned, hist, bad, counts, nullptr, nullptr, dev_err,
                     dst_row, src_row);
  // no pad rows to zero in the masked layout (E = 0 skips that pass)
  return launch_copy(dt, x, T, D, k, 0, dst_row, counts, nullptr, x_masked, s);
}

hipError_t launch_permute_mx(const void* xq, const void* xs, const int32_t* topk_idx, int T, int D,
                             int E, int k, int m_tile, int64_t m_cap, void* xq_perm,
                             void* xs_perm, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                             int32_t* src_row, int32_t* tile_expert, void* workspace,
                             int32_t* dev_err, hipStream_t s) {
  const int nbh = (T + kHistTokens - 1) / kHistTokens;
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* bad = hist + (size_t)nbh * E;
  hipLaunchKernelGGL(hist_kernel, dim3(nbh), dim3(kThreads), 0, s, topk_idx, T, k, E, hist, bad);
  const bool scanned = scan_hist(hist, nbh, E, s);
  hipLaunchKernelGGL(rank_kernel<false>, dim3(nbh + 1), dim3(kThreads), 0, s, topk_idx, T, k, E,
                     m_tile, 0, m_cap, nbh, scanned, hist, bad, counts, offsets, tile_expert, dev_err,
                     dst_row, src_row);
  // the code rows are copied as raw bytes (D bytes = D/2 two-byte units, whole 16-byte
  // chunks as D % 128 == 0); pad rows get zero bytes (code 0 is +0). The scales go into
  // k-step words, zero for pad rows.
  const hipError_t e = launch_copy(kBF16, xq, T, D / 2, k, E, dst_row, counts, offsets, xq_perm, s);
  if (e != hipSuccess) return e;
  const int nsw = D / 128;
  const int grid = (int)std::min<int64_t>(8 * cu_count(),
                                          (m_cap * nsw + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(scale_ksteps_kernel, dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const uint32_t*>(xs), nsw, k, E, offsets, src_row, m_cap,
                     static_cast<uint32_t*>(xs_perm));
  return hipGetLastError();
}

}  // namespace moe
