// Dispatch: per-expert histogram, exclusive scan and a stable scatter of the
// (token, slot) pairs into expert-contiguous rows, plus the GEMM tile list.
//
// Sparse expert activation needs the hidden states dispatched to the chosen
// experts and their outputs combined back (A/F 分离 page, "为什么要拆" and
// the "机制" flowchart).  On one GPU the dispatch is a permutation: rows of
// expert e are its tokens in ascending order (a stable counting sort), so
// the result is unique and bit-comparable.
//
// Up to 1024 tokens, one workgroup of 1024 threads does it all; longer
// batches use one workgroup per block of 1024 tokens (count, then a single
// workgroup scan, then scatter).  Deterministic, no global atomics.  Ranks
// come from per-wave 64-bit membership masks: the rank of token t for
// expert e is (rows of e in earlier blocks) + (members in earlier waves of
// its block) + popcount of the members in t's own wave at lower lanes.
#include "common.h"
#include "kernels.h"

namespace afd {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Exclusive scan of one value per thread over the workgroup; returns the
// exclusive prefix, *total receives the sum.
__device__ int block_exclusive_scan(int v, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wsum[w];
      wsum[w] = run;
      run += c;
    }
    wsum[kWaves] = run;
  }
  __syncthreads();
  const int excl = x - v + wsum[wave];
  *total = wsum[kWaves];
  __syncthreads();
  return excl;
}

// Tile lists.  Group g < E is routed expert g (its rows start at the
// exclusive scan `off` of the counts), group E + s is shared expert s (T rows
// from T*k + s*T).  With a big-tile list, a group of at least big_min rows
// gets full big tiles, plus one partial big tile if the remainder exceeds
// half a big tile; all other rows go to small tiles.  Thread tid < E holds
// expert tid's count `c` and offset `off`; all threads of the workgroup call.
__device__ void build_tiles(int T, int k, int E, int S, const TilePlan &tp, int c, int off,
                            int *wsum, Tile *tiles_s, int32_t *num_s, Tile *tiles_b,
                            int32_t *num_b) {
  const int tid = threadIdx.x;
  const int64_t Tk = static_cast<int64_t>(T) * k;
  const int G = E + S;
  int gc = 0, g0 = 0;
  if (tid < E) {
    gc = c;
    g0 = off;
  } else if (tid < G) {
    gc = T;
    g0 = static_cast<int>(Tk) + (tid - E) * T;
  }
  int nbig = 0, rem = gc;
  if (tid < G && tp.bm_big > 0 && gc >= tp.big_min) {
    nbig = gc / tp.bm_big;
    rem = gc - nbig * tp.bm_big;
    if (rem * 2 > tp.bm_big) {
      ++nbig;
      rem = 0;
    }
  }
  const int nsmall = tid < G ? (rem + tp.bm_small - 1) / tp.bm_small : 0;
  int tot_b = 0, tot_s = 0;
  const int bbase = block_exclusive_scan(nbig, wsum, &tot_b);
  const int sbase = block_exclusive_scan(nsmall, wsum, &tot_s);
  for (int m = 0; m < nbig; ++m) {
    Tile t;
    t.group = tid;
    t.row0 = g0 + m * tp.bm_big;
    t.rows = min(tp.bm_big, gc - m * tp.bm_big);
    t.pad = 0;
    tiles_b[bbase + m] = t;
  }
  const int sfirst = g0 + (gc - rem);
  for (int m = 0; m < nsmall; ++m) {
    Tile t;
    t.group = tid;
    t.row0 = sfirst + m * tp.bm_small;
    t.rows = min(tp.bm_small, rem - m * tp.bm_small);
    t.pad = 0;
    tiles_s[sbase + m] = t;
  }
  if (tid == 0) {
    *num_s = tot_s;
    if (num_b) *num_b = tot_b;
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t *__restrict__ ids, int T, int k, int E, int S, TilePlan tp,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, int32_t *__restrict__ slot_row,
    Tile *__restrict__ tiles_s, int32_t *__restrict__ num_s,
    Tile *__restrict__ tiles_b, int32_t *__restrict__ num_b,
    int32_t *__restrict__ counters, int ncounters) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int run[kMaxExperts];
  __shared__ unsigned long long mask[kWaves][kMaxExperts];
  __shared__ int pre[kWaves][kMaxExperts];
  __shared__ int wsum[kWaves + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t Tk = static_cast<int64_t>(T) * k;

  // 1. histogram (LDS atomics; counts do not depend on their order)
  for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = tid; i < Tk; i += kThreads) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();

  // 2. exclusive scan -> offsets; tile list
  const int c = tid < E ? cnt[tid] : 0;
  int total = 0;
  const int off = block_exclusive_scan(c, wsum, &total);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = off;
    run[tid] = off;
  }
  if (tid == 0) offsets[E] = total;
  build_tiles(T, k, E, S, tp, c, off, wsum, tiles_s, num_s, tiles_b, num_b);
  for (int i = tid; i < ncounters; i += kThreads) counters[i] = 0;
  __syncthreads();

  // 3. stable scatter, 1024 tokens per pass
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < T; base += kThreads) {
    for (int i = tid; i < kWaves * E; i += kThreads) mask[i / E][i % E] = 0ull;
    __syncthreads();
    const int t = base + tid;
    const bool valid = t < T;
    if (valid)
      for (int j = 0; j < k; ++j)
        atomicOr(&mask[wave][ids[static_cast<int64_t>(t) * k + j]], 1ull << lane);
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      int r = run[e];
      for (int w = 0; w < kWaves; ++w) {
        pre[w][e] = r;
        r += __popcll(mask[w][e]);
      }
      run[e] = r;
    }
    __syncthreads();
    if (valid)
      for (int j = 0; j < k; ++j) {
        const int e = ids[static_cast<int64_t>(t) * k + j];
        const int rank = pre[wave][e] + __popcll(mask[wave][e] & below);
        perm[rank] = t;
        slot_row[static_cast<int64_t>(t) * k + j] = rank;
      }
    __syncthreads();
  }
}

// ---- multi-workgroup path for long batches (one token block of 1024 per
// workgroup): count, scan, scatter.  Same result as dispatch_kernel.

// Per-wave membership masks of token block `blk` (tokens blk*1024 + tid).
__device__ void block_masks(const int32_t *__restrict__ ids, int T, int k, int E, int blk,
                            unsigned long long (*mask)[kMaxExperts]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kWaves * E; i += kThreads) mask[i / E][i % E] = 0ull;
  __syncthreads();
  const int t = blk * kThreads + tid;
  if (t < T)
    for (int j = 0; j < k; ++j)
      atomicOr(&mask[wave][ids[static_cast<int64_t>(t) * k + j]], 1ull << lane);
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void dispatch_count_kernel(
    const int32_t *__restrict__ ids, int T, int k, int E, int32_t *__restrict__ block_counts) {
  __shared__ unsigned long long mask[kWaves][kMaxExperts];
  block_masks(ids, T, k, E, blockIdx.x, mask);
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int c = 0;
    for (int w = 0; w < kWaves; ++w) c += __popcll(mask[w][e]);
    block_counts[static_cast<int64_t>(blockIdx.x) * E + e] = c;
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_scan_kernel(
    const int32_t *__restrict__ block_counts, int nblk, int T, int k, int E, int S,
    TilePlan tp, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ block_base, Tile *__restrict__ tiles_s, int32_t *__restrict__ num_s,
    Tile *__restrict__ tiles_b, int32_t *__restrict__ num_b, int32_t *__restrict__ counters,
    int ncounters) {
  __shared__ int wsum[kWaves + 1];
  const int tid = threadIdx.x;
  int c = 0;
  if (tid < E)
    for (int b = 0; b < nblk; ++b) c += block_counts[static_cast<int64_t>(b) * E + tid];
  int total = 0;
  const int off = block_exclusive_scan(c, wsum, &total);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = off;
    int run = off;
    for (int b = 0; b < nblk; ++b) {
      block_base[static_cast<int64_t>(b) * E + tid] = run;
      run += block_counts[static_cast<int64_t>(b) * E + tid];
    }
  }
  if (tid == 0) offsets[E] = total;
  build_tiles(T, k, E, S, tp, c, off, wsum, tiles_s, num_s, tiles_b, num_b);
  for (int i = tid; i < ncounters; i += kThreads) counters[i] = 0;
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    const int32_t *__restrict__ ids, int T, int k, int E,
    const int32_t *__restrict__ block_base, int32_t *__restrict__ perm,
    int32_t *__restrict__ slot_row) {
  __shared__ unsigned long long mask[kWaves][kMaxExperts];
  __shared__ int pre[kWaves][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  block_masks(ids, T, k, E, blockIdx.x, mask);
  for (int e = tid; e < E; e += kThreads) {
    int r = block_base[static_cast<int64_t>(blockIdx.x) * E + e];
    for (int w = 0; w < kWaves; ++w) {
      pre[w][e] = r;
      r += __popcll(mask[w][e]);
    }
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int t = blockIdx.x * kThreads + tid;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = ids[static_cast<int64_t>(t) * k + j];
      const int rank = pre[wave][e] + __popcll(mask[wave][e] & below);
      perm[rank] = t;
      slot_row[static_cast<int64_t>(t) * k + j] = rank;
    }
}

}  // namespace

int dispatch_blocks(int T) { return (T + kThreads - 1) / kThreads; }

hipError_t launch_dispatch(const int32_t *ids, int T, int k, int E, int S,
                           const TilePlan &tp, int32_t *counts, int32_t *offsets,
                           int32_t *perm, int32_t *slot_row, Tile *tiles_s,
                           int32_t *num_s, Tile *tiles_b, int32_t *num_b,
                           int32_t *counters, int ncounters, int32_t *block_scratch,
                           hipStream_t s) {
  const int nblk = dispatch_blocks(T);
  if (nblk == 1) {
    dispatch_kernel<<<1, kThreads, 0, s>>>(ids, T, k, E, S, tp, counts, offsets,
                                           perm, slot_row, tiles_s, num_s, tiles_b,
                                           num_b, counters, ncounters);
    return hipGetLastError();
  }
  int32_t *block_counts = block_scratch;
  int32_t *block_base = block_scratch + static_cast<int64_t>(nblk) * E;
  dispatch_count_kernel<<<nblk, kThreads, 0, s>>>(ids, T, k, E, block_counts);
  dispatch_scan_kernel<<<1, kThreads, 0, s>>>(block_counts, nblk, T, k, E, S, tp, counts,
                                              offsets, block_base, tiles_s, num_s, tiles_b,
                                              num_b, counters, ncounters);
  dispatch_scatter_kernel<<<nblk, kThreads, 0, s>>>(ids, T, k, E, block_base, perm, slot_row);
  return hipGetLastError();
}

}  // namespace afd
