// Dispatch: per-expert histogram, exclusive scan and a stable scatter of the
// (token, slot) pairs into expert-contiguous rows, plus the GEMM tile list.
//
// Sparse expert activation needs the hidden states dispatched to the chosen
// experts and their outputs combined back (A/F 分离 page, "为什么要拆" and
// the "机制" flowchart).  On one GPU the dispatch is a permutation: rows of
// expert e are its tokens in ascending order (a stable counting sort), so
// the result is unique and bit-comparable.
//
// One workgroup of 1024 threads does it all; T*k is at most a few times
// 10^5 here, so a single CU finishes in microseconds, deterministically and
// without global atomics.  Ranks inside a pass of 1024 tokens come from
// per-wave 64-bit membership masks: the rank of token t for expert e is
// (rows of e before this pass) + (members in earlier waves) + popcount of
// the members in t's own wave at lower lanes.
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

__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t *__restrict__ ids, int T, int k, int E, int S, int bm,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, int32_t *__restrict__ slot_row,
    Tile *__restrict__ tiles, int32_t *__restrict__ num_tiles,
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
  const int nt = tid < E ? (c + bm - 1) / bm : 0;
  int routed_tiles = 0;
  const int tbase = block_exclusive_scan(nt, wsum, &routed_tiles);
  for (int m = 0; m < nt; ++m) {
    Tile t;
    t.group = tid;
    t.row0 = off + m * bm;
    t.rows = min(bm, c - m * bm);
    t.pad = 0;
    tiles[tbase + m] = t;
  }
  const int ns = (T + bm - 1) / bm;
  for (int i = tid; i < S * ns; i += kThreads) {
    const int sg = i / ns, m = i % ns;
    Tile t;
    t.group = E + sg;
    t.row0 = static_cast<int>(Tk) + sg * T + m * bm;
    t.rows = min(bm, T - m * bm);
    t.pad = 0;
    tiles[routed_tiles + i] = t;
  }
  if (tid == 0) *num_tiles = routed_tiles + S * ns;
  if (tid < ncounters) counters[tid] = 0;
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

}  // namespace

hipError_t launch_dispatch(const int32_t *ids, int T, int k, int E, int S,
                           int bm, int32_t *counts, int32_t *offsets,
                           int32_t *perm, int32_t *slot_row, Tile *tiles,
                           int32_t *num_tiles, int32_t *counters,
                           int ncounters, hipStream_t s) {
  dispatch_kernel<<<1, kThreads, 0, s>>>(ids, T, k, E, S, bm, counts, offsets,
                                         perm, slot_row, tiles, num_tiles,
                                         counters, ncounters);
  return hipGetLastError();
}

}  // namespace afd
