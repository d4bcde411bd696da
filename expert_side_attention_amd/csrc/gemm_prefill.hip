// Compute-bound grouped expert GEMMs (bf16) for prefill-sized batches, where
// each busy expert holds hundreds to thousands of rows and the work is the
// MFMA throughput (the FFN side saturates compute: LLM 推理提速 page,
// "一个在啃带宽，一个在吃算力"; experts are large matrix products: A/F 分离
// page, "为什么要拆").
//
// Tile: 256 rows x 256 weight rows per workgroup (gate/up: 128 gate + 128 up
// rows, i.e. 128 output columns of z; down: 256 output columns), K in
// 64-element (128-byte) stages, so every load request is a whole cache line.
//
// Operands move with direct-to-LDS loads (global_load_lds, no staging
// registers) into two 64 KB stage buffers: the next stage loads while the
// MFMAs read the current one.  Ordering uses an explicit vmcnt(0) wait plus
// a bare s_barrier per stage (a full workgroup fence would drain every
// outstanding load).  The wait is for zero on purpose: with several stages
// of direct-to-LDS loads in flight, a wait that leaves the newest loads
// outstanding does not guarantee that the older ones have landed in LDS (a
// probe of that scheme read stale data a few times per billion reads).  LDS
// rows are 128 bytes with the 16-byte chunk index XOR-ed by (row / 2) % 8, so
// the 16 rows one MFMA operand read touches per quarter wave hit 16
// different 4-bank groups.
//
// Tile order (workgroup ids go to the 8 XCDs round-robin): the eight-wave
// kernel deals row tiles round-robin to the XCDs and runs all column tiles
// of a row tile on one XCD, close in time, so the XCD's L2 serves the
// activation rows to all of them.  The four-wave kernel deals windows of 4
// consecutive row tiles x up to 8 column tiles (about one workgroup per CU
// of an XCD) instead: in a window each activation stage is read by up to 8
// CUs and each weight stage by up to 4 (consecutive row tiles mostly belong
// to one expert), and the 8 XCDs work on 8 consecutive windows at a time.
//
// Two kernels share this layout.  The expert GEMMs run on four waves (one
// per SIMD), each owning 128 rows x 128 weight rows as 8 x 8 tiles of
// 16x16x32 MFMAs with a hand-fixed instruction order (prefill_gemm4_kernel,
// below).  The router logits of long batches (logits mode: rows of X
// against the router weight, the K range split over workgroups, fp32
// partial sums written straight from the accumulators to one plane per
// split, which the top-k kernel adds) run on eight waves (two per SIMD) in a
// 2 x 4 grid, each owning 128 rows x 64 weight rows = 4 x 2 tiles of
// 32x32x16 MFMAs, the next stage's loads issued one at a time between the
// first K steps' MFMAs (prefill_gemm_kernel).
#include "common.h"
#include <atomic>

#include "kernels.h"

namespace afd {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;    // rows per tile
constexpr int kBW = 256;    // weight rows per tile
constexpr int kStage = 128;  // bytes per row per K stage (64 bf16)
constexpr int kRing = 2;    // LDS double buffer
constexpr int kSlot = (kBM + kBW) * kStage;  // 64 KB

// byte offset of 16-byte chunk `chunk` (0..7) of LDS row `row`: the chunk
// index is XOR-ed with (row / 2) % 8 (see the file comment)
__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * kStage + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Four-wave kernel tile order: windows of kWinR consecutive row tiles x cw
// column tiles (column tiles split into ncg groups of at most kWinC), each
// window on one XCD; ws = kWinR * cw workgroups per window
constexpr int kWinR = 4;
constexpr int kWinC = 32 / kWinR;
struct TileWindows {
  int ncg, cw, ws;
};
__host__ __device__ inline TileWindows tile_windows(int ntn) {
  const int ncg = (ntn + kWinC - 1) / kWinC;
  const int cw = (ntn + ncg - 1) / ncg;
  return {ncg, cw, kWinR * cw};
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// One 16-byte-per-lane direct-to-LDS load: lane i of the wave writes LDS
// bytes [16 i, 16 i + 16) above the wave-uniform `lds_dst`.
__device__ __forceinline__ void dma16(const uint8_t *src, uint8_t *lds_dst) {
  // C-style casts: generic -> global / LDS address-space pointers
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}

// MODE: kDown (C = A B0^T, bf16), kGateUp (C = silu(A B0^T) * (A B1^T),
// bf16), kLogits (router logits: A = X rows, B0 = router weight, no tile
// list; blockIdx.y picks one of gridDim.y equal K ranges and the fp32
// partial sums go to plane blockIdx.y of C, planes c_plane floats apart).
enum { kDown = 0, kGateUp = 1, kLogits = 2 };

template <int MODE>
__global__ __launch_bounds__(512) void prefill_gemm_kernel(const GemmArgs p) {
  constexpr bool SWIGLU = MODE == kGateUp;
  constexpr bool LOGITS = MODE == kLogits;
  extern __shared__ __align__(16) uint8_t lds[];  // kRing x (A 32 KB + B 32 KB)
  __shared__ int rowsrc[kBM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;   // 2 x 4 waves: 128 rows x 64 weight rows each
  const int r32 = lane & 31, g = lane >> 5;
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;  // output columns per tile

  const int nmax = p.N > p.Ns ? p.N : p.Ns;
  const int ntn = (nmax + BNO - 1) / BNO;  // the last column tile may be partial
  const int L = blockIdx.x;
  const int j = L >> 3;
  const int mt = (L & 7) + 8 * (j / ntn);
  const int nt = j % ntn;
  Tile tile;
  if constexpr (LOGITS) {
    if (mt * kBM >= p.T) return;
    tile = Tile{0, mt * kBM, min(kBM, p.T - mt * kBM), 0};
  } else {
    if (mt >= *p.num_tiles) return;
    tile = p.tiles[mt];
  }
  const bool shared = tile.group >= p.E;
  const int N = shared ? p.Ns : p.N;
  const int K = shared ? p.Ks : p.K;
  const int n0 = nt * BNO;
  if (n0 >= N) return;
  const int gi = shared ? tile.group - p.E : tile.group;
  const int rows = tile.rows;

  if (tid < kBM) {
    int src = -1;
    if (tid < rows) {
      const int r = tile.row0 + tid;
      src = p.perm ? (r < p.Tk ? p.perm[r] : (r - p.Tk) % p.T) : r;
    }
    rowsrc[tid] = src;
  }
  __syncthreads();

  const int64_t krow = static_cast<int64_t>(K) * 2;
  // this workgroup's stages [s_begin, s_begin + nst) of the K range
  const int nst_all = static_cast<int>(krow / kStage);
  const int s_begin = static_cast<int>(static_cast<int64_t>(blockIdx.y) * nst_all / gridDim.y);
  const int nst = static_cast<int>(static_cast<int64_t>(blockIdx.y + 1) * nst_all / gridDim.y) - s_begin;
  const int64_t mat = static_cast<int64_t>(N) * krow;
  const uint8_t *B0 = (shared ? p.sb0 : p.b0) + gi * mat;
  const uint8_t *B1 = SWIGLU ? (shared ? p.sb1 : p.b1) + gi * mat : B0;

  // Each wave moves rows [32 wave, 32 wave + 32) of the A stage and of the
  // B stage: four 1 KB direct-to-LDS loads each (8 rows of 128 bytes per
  // load).  Lane i fills LDS row 8 h + i / 8, position i % 8, which holds
  // the row's 16-byte chunk (i % 8) ^ ((row / 2) % 8) (bank swizzle).
  // Rows past the tile's end load a valid row (rows of an MFMA tile are
  // independent; those results are never stored); weight rows past N (a
  // partial last column tile) load row N - 1.
  const int src_first = rowsrc[0];
  const uint8_t *asrc[4];
  const uint8_t *bsrc[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const int row = wave * 32 + hh * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);
    const int src = rowsrc[row] >= 0 ? rowsrc[row] : src_first;
    asrc[hh] = p.A + static_cast<int64_t>(src) * p.a_pitch + ch * 16 +
               static_cast<int64_t>(s_begin) * kStage;
    const int n = n0 + (SWIGLU ? (row & (kBW / 2 - 1)) : row);
    const uint8_t *base = (SWIGLU && row >= kBW / 2) ? B1 : B0;
    bsrc[hh] = base + static_cast<int64_t>(min(n, N - 1)) * krow + ch * 16 +
               static_cast<int64_t>(s_begin) * kStage;
  }
  auto issue = [&](int s) {  // stage s -> ring slot s % kRing
    uint8_t *slot = lds + (s % kRing) * kSlot;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      dma16(asrc[hh] + static_cast<int64_t>(s) * kStage, slot + (wave * 4 + hh) * 1024);
      dma16(bsrc[hh] + static_cast<int64_t>(s) * kStage,
            slot + kBM * kStage + (wave * 4 + hh) * 1024);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x16{};

  // weight rows of this wave: gate/up -> gate block (wc * 32) and the up
  // block at the same columns (128 + wc * 32); down -> wc * 64 + {0, 32}
  const int wrow0 = SWIGLU ? wc * 32 + r32 : wc * 64 + r32;
  const int wrow1 = SWIGLU ? kBW / 2 + wc * 32 + r32 : wc * 64 + 32 + r32;

  // prologue: stage 0 in flight
#pragma unroll
  for (int s = 0; s < kRing - 1; ++s)
    if (s < nst) issue(s);
  for (int s = 0; s < nst; ++s) {
    // double buffer: only stage s is in flight here
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    const bool do_issue = s + 1 < nst;
    const int si = s + 1;
    uint8_t *slot = lds + (si % kRing) * kSlot;
    const uint8_t *la = lds + (s % kRing) * kSlot;
    const uint8_t *lb = la + kBM * kStage;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + g;
      bf16x8 fa[4], fb[2];
      fb[0] = bitcast<bf16x8>(ld16(lb + swz64(wrow0, ch)));
      fb[1] = bitcast<bf16x8>(ld16(lb + swz64(wrow1, ch)));
#pragma unroll
      for (int m = 0; m < 4; ++m)
        fa[m] = bitcast<bf16x8>(ld16(la + swz64(wr * 128 + m * 32 + r32, ch)));
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m], fb[n], acc[m][n], 0, 0, 0);
        if (ks < 2 && do_issue) {
          const int idx = ks * 4 + m;  // 0..7
          const int hh = idx >> 1;
          if ((idx & 1) == 0)
            dma16(asrc[hh] + static_cast<int64_t>(si) * kStage, slot + (wave * 4 + hh) * 1024);
          else
            dma16(bsrc[hh] + static_cast<int64_t>(si) * kStage,
                  slot + kBM * kStage + (wave * 4 + hh) * 1024);
        }
      }
    }
  }
  __syncthreads();  // all waves are done with the ring before the epilogue reuses it

  if constexpr (LOGITS) {
    // fp32 partial logits straight from the accumulators: for each register,
    // the 32 lanes of a half-wave write 32 consecutive experts of one token
    float *plane = reinterpret_cast<float *>(p.C) + static_cast<int64_t>(blockIdx.y) * p.c_plane;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = wr * 128 + m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = n0 + wc * 64 + n * 32 + r32;
          if (row < rows && col < N)
            plane[static_cast<int64_t>(tile.row0 + row) * N + col] = acc[m][n][i];
        }
      }
    return;
  }

  // ---- epilogue: stage the bf16 tile in LDS, then whole 16-byte stores.
  // acc[m][n][i]: row 32 m + 8 (i / 4) + 4 g + (i % 4), column r32 of block n.
  uint16_t *o16 = reinterpret_cast<uint16_t *>(lds);
  constexpr int OPITCH = BNO;  // elements per staged row
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = wr * 128 + m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (SWIGLU) {
        o16[row * OPITCH + wc * 32 + r32] = f32_to_bf16(silu_mul(acc[m][0][i], acc[m][1][i]));
      } else {
#pragma unroll
        for (int n = 0; n < 2; ++n)
          o16[row * OPITCH + wc * 64 + n * 32 + r32] = f32_to_bf16(acc[m][n][i]);
      }
    }
  }
  __syncthreads();
  constexpr int CPR = OPITCH * 2 / 16;  // 16-byte pieces per staged row
  const int vcpr = min(CPR, (N - n0) * 2 / 16);
  for (int c = tid; c < kBM * CPR; c += 512) {
    const int row = c / CPR, col = c % CPR;
    if (row < rows && col < vcpr)
      st16(p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch + n0 * 2 + col * 16,
           ld16(lds + row * OPITCH * 2 + col * 16));
  }
}

// Four-wave kernel (one wave per SIMD) of the expert GEMMs: the tile, stage
// layout, loads and tile order above, each wave owning 128 rows x 128
// weight rows as 8 x 8 tiles of 16x16x32 MFMAs (256 accumulators per lane,
// in the accumulation registers), so a stage reads half the LDS fragments
// per MFMA of the eight-wave layout.  With one wave per SIMD the wave keeps
// its matrix core fed by itself, so the instruction order is fixed by hand
// with scheduling fences; the schedule is described at the main loop.
template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_gemm4_kernel(const GemmArgs p) {
  constexpr bool SWIGLU = MODE == kGateUp;
  extern __shared__ __align__(16) uint8_t lds[];  // kRing x (A 32 KB + B 32 KB)
  __shared__ int rowsrc[kBM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;  // 2 x 2 waves: 128 rows x 128 weight rows each
  const int r16 = lane & 15, q = lane >> 4;
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;  // output columns per tile

  const int nmax = p.N > p.Ns ? p.N : p.Ns;
  const int ntn = (nmax + BNO - 1) / BNO;
  const TileWindows tw = tile_windows(ntn);
  const int L = blockIdx.x;
  const int j = L >> 3;
  const int gw = (j / tw.ws) * 8 + (L & 7);  // window; consecutive windows on consecutive XCDs
  const int u = j % tw.ws;
  const int mt = (gw / tw.ncg) * kWinR + u % kWinR;
  const int nt = (gw % tw.ncg) * tw.cw + u / kWinR;
  if (mt >= *p.num_tiles || nt >= ntn) return;
  const Tile tile = p.tiles[mt];
  const bool shared = tile.group >= p.E;
  const int N = shared ? p.Ns : p.N;
  const int K = shared ? p.Ks : p.K;
  const int n0 = nt * BNO;
  if (n0 >= N) return;
  const int gi = shared ? tile.group - p.E : tile.group;
  const int rows = tile.rows;

  {
    int src = -1;
    if (tid < rows) {
      const int r = tile.row0 + tid;
      src = p.perm ? (r < p.Tk ? p.perm[r] : (r - p.Tk) % p.T) : r;
    }
    rowsrc[tid] = src;  // 256 threads, 256 rows
  }
  __syncthreads();

  const int64_t krow = static_cast<int64_t>(K) * 2;
  const int nst = static_cast<int>(krow / kStage);
  const int64_t mat = static_cast<int64_t>(N) * krow;
  const uint8_t *B0 = (shared ? p.sb0 : p.b0) + gi * mat;
  const uint8_t *B1 = SWIGLU ? (shared ? p.sb1 : p.b1) + gi * mat : B0;

  // wave w moves rows [64 w, 64 w + 64) of the A stage and of the B stage:
  // eight 1 KB direct-to-LDS loads each (layout and swizzle as above); the
  // wave's B rows are 64 consecutive weight rows of one matrix
  const int src_first = rowsrc[0];
  const uint8_t *asrc[8];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) {
    const int row = wave * 64 + hh * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);
    const int src = rowsrc[row] >= 0 ? rowsrc[row] : src_first;
    asrc[hh] = p.A + static_cast<int64_t>(src) * p.a_pitch + ch * 16;
  }
  // LDS B row l holds weight row (output column) n0 + col_of(l), a
  // permutation inside each wave's block chosen so that the MFMA column
  // r16 of block n of a wave is column 4 r16 + n (gate/up: 64 columns per
  // wave, blocks 0-3 gate and 4-7 the up rows of the same columns) or 8 r16
  // + n (down: 128 columns per wave): a lane then holds 4 or 8 consecutive
  // output columns of each of its rows and stores them in one piece
  auto col_of = [](int l) {
    return SWIGLU ? (l & ~63) + ((l & 15) << 2) + ((l >> 4) & 3)
                  : (l & ~127) + ((l & 15) << 3) + ((l >> 4) & 7);
  };
  const uint8_t *bsrc[8];
  {
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      const int row = wave * 64 + hh * 8 + (lane >> 3);
      const int ch = (lane & 7) ^ ((row >> 1) & 7);
      const int n = n0 + col_of(SWIGLU ? (row & (kBW / 2 - 1)) : row);
      const uint8_t *base = (SWIGLU && wave >= 2) ? B1 : B0;
      bsrc[hh] = base + static_cast<int64_t>(min(n, N - 1)) * krow + ch * 16;
    }
  }
  // load jj (0..15) of stage t: jj < 8 -> A rows block jj, else B rows block jj - 8
  auto load = [&](int t, int jj) {
    uint8_t *slot = lds + (t % kRing) * kSlot;
    if (jj < 8)
      dma16(asrc[jj] + static_cast<int64_t>(t) * kStage, slot + (wave * 8 + jj) * 1024);
    else
      dma16(bsrc[jj - 8] + static_cast<int64_t>(t) * kStage,
            slot + kBM * kStage + (wave * 8 + jj - 8) * 1024);
  };
  // the same from pointers that advance one stage per use, up to the last
  // stage (past it the last stage is loaded again, into a buffer nothing
  // reads any more)
  auto load_next = [&](int slot_idx, int jj, int64_t adv) {
    uint8_t *slot = lds + slot_idx * kSlot;
    if (jj < 8) {
      dma16(asrc[jj], slot + (wave * 8 + jj) * 1024);
      asrc[jj] += adv;
    } else {
      dma16(bsrc[jj - 8], slot + kBM * kStage + (wave * 8 + jj - 8) * 1024);
      bsrc[jj - 8] += adv;
    }
  };

  // this wave's weight rows: gate/up -> 64 gate rows (blocks 0-3) and the up
  // rows of the same columns (blocks 4-7); down -> 128 rows
  auto wrow = [&](int n) {
    return SWIGLU ? (n < 4 ? wc * 64 + n * 16 : kBW / 2 + wc * 64 + (n - 4) * 16) + r16
                  : wc * 128 + n * 16 + r16;
  };
  // fragments: one register set per 32-element K step (set kk for step kk)
  bf16x8 fa[2][8], fb[2][8];
  // fragment jj (0..15: A blocks, then B blocks) of K step kk of stage t
  auto read = [&](int t, int kk, int jj) {
    const uint8_t *la = lds + (t % kRing) * kSlot;
    if (jj < 8)
      fa[kk][jj] = bitcast<bf16x8>(ld16(la + swz64(wr * 128 + jj * 16 + r16, kk * 4 + q)));
    else
      fb[kk][jj - 8] =
          bitcast<bf16x8>(ld16(la + kBM * kStage + swz64(wrow(jj - 8), kk * 4 + q)));
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0, 0, 0, 0};

  // Schedule of stage s: K step 0 on set 0 while set 1 is read (step 1 of
  // the same stage, one read per two MFMAs in the first half); then every
  // wave waits for its loads of stage s + 1 and meets the others at the
  // barrier, after which nothing reads stage s from LDS any more; K step 1
  // on set 1 while the sixteen loads of stage s + 2 go into stage s's
  // buffer, one per four MFMAs (the weight rows, which miss the L2 more
  // often, before the activation rows), and set 0 is read from stage s + 1.
  // A load thus has about one stage to arrive.  The loop has no branches: the
  // loads advance their own pointers and, past the last stage, repeat it
  // (about 32 branches per stage around conditional loads had cost ~8%).
  // Measured alternatives were slower:
  // the loads packed into the first quarter or half of step 1, weight and
  // activation loads alternating, or the barrier 16 MFMAs before the end of
  // step 0 (which also made the register allocator move accumulators
  // between register files inside the loop).
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) load(0, jj);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) read(0, 0, jj);
  if (nst > 1) {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) load(1, jj);
  }
  // the pointers now address stage 2 (or the last stage)
  {
    const int64_t first = static_cast<int64_t>(min(2, nst - 1)) * kStage;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      asrc[jj] += first;
      bsrc[jj] += first;
    }
  }

  for (int s = 0; s < nst; ++s) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int m = i >> 3, n = i & 7;
      acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[0][m], fb[0][n], acc[m][n], 0, 0, 0);
      if ((i & 1) == 1 && i < 32) read(s, 1, i >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // past the last stage the loads and reads repeat it (in bounds, unused)
    const int s1 = min(s + 1, nst - 1);
    const int64_t adv = s + 3 < nst ? kStage : 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int m = i >> 3, n = i & 7;
      acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[1][m], fb[1][n], acc[m][n], 0, 0, 0);
      if ((i & 3) == 0) load_next(s & 1, ((i >> 2) + 8) & 15, adv);  // weight rows first
      if ((i & 1) == 1 && i < 32) read(s1, 0, i >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the repeated loads of the last stage may still be landing in LDS, which
  // the next workgroup on this CU will own
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue, straight from the accumulators (no LDS staging):
  // acc[m][n][i] is row wr*128 + 16 m + 4 q + i and column 4 r16 + n
  // (gate/up, n < 4 gate and n + 4 up: 4 consecutive z columns, one 8-byte
  // store) or 8 r16 + n (down: 8 consecutive y columns, one 16-byte store)
  // of the wave's columns (see col_of)
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int col0 = SWIGLU ? n0 + wc * 64 + r16 * 4 : n0 + wc * 128 + r16 * 8;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wr * 128 + m * 16 + 4 * q + i;
      if (row >= rows || col0 >= N) continue;
      uint8_t *dst = p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch + col0 * 2;
      if constexpr (SWIGLU) {
        float z[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) z[n] = silu_mul(acc[m][n][i], acc[m][n + 4][i]);
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
      } else {
        st16(dst, u32x4{pack_bf16x2(acc[m][0][i], acc[m][1][i]), pack_bf16x2(acc[m][2][i], acc[m][3][i]),
                        pack_bf16x2(acc[m][4][i], acc[m][5][i]), pack_bf16x2(acc[m][6][i], acc[m][7][i])});
      }
    }
}

// the dynamic-LDS limit is a per-device attribute of each kernel
template <typename KernelFn>
hipError_t set_lds_limit(KernelFn kern, std::atomic<bool> (&attr_set)[64],
                         size_t kLds = kRing * kSlot) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  return hipSuccess;
}

template <int MODE>
hipError_t set_lds_limit() {
  static std::atomic<bool> attr_set[64];
  return set_lds_limit(prefill_gemm_kernel<MODE>, attr_set);
}

template <int MODE>
hipError_t launch_one(const GemmArgs &a, hipStream_t s) {
  constexpr int BNO = MODE == kGateUp ? kBW / 2 : kBW;
  static std::atomic<bool> attr_set[64];
  hipError_t e = set_lds_limit(prefill_gemm4_kernel<MODE>, attr_set);
  if (e != hipSuccess) return e;
  const int nmax = a.N > a.Ns ? a.N : a.Ns;
  const int ntn = (nmax + BNO - 1) / BNO;
  const TileWindows tw = tile_windows(ntn);
  const int64_t windows = static_cast<int64_t>((a.tiles_ub + kWinR - 1) / kWinR) * tw.ncg;
  const int64_t grid = 8LL * ((windows + 7) / 8) * tw.ws;
  if (grid <= 0) return hipSuccess;
  prefill_gemm4_kernel<MODE><<<static_cast<unsigned>(grid), 256, kRing * kSlot, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(GemmKind kind, const GemmArgs &a, hipStream_t s) {
  return kind == GemmKind::GateUp ? launch_one<kGateUp>(a, s) : launch_one<kDown>(a, s);
}

int logits_splits(int T, int h, int E) {
  const int rtiles = (T + kBM - 1) / kBM, ctiles = (E + kBW - 1) / kBW;
  const int nst = h * 2 / kStage;
  int ks = 256 / (rtiles * ctiles);  // about one workgroup per CU
  if (ks > nst / 7) ks = nst / 7;    // at least 7 stages per split
  if (ks > kMaxLogitSplits) ks = kMaxLogitSplits;
  return ks < 1 ? 1 : ks;
}

hipError_t launch_logits_gemm(const uint16_t *x, const uint16_t *wr, int T, int h, int E,
                              float *partials, int splits, hipStream_t s) {
  hipError_t e = set_lds_limit<kLogits>();
  if (e != hipSuccess) return e;
  GemmArgs a{};
  a.A = reinterpret_cast<const uint8_t *>(x);
  a.a_pitch = static_cast<int64_t>(h) * 2;
  a.perm = nullptr;
  a.T = T;
  a.Tk = T;
  a.b0 = reinterpret_cast<const uint8_t *>(wr);
  a.N = a.Ns = E;
  a.K = a.Ks = h;
  a.E = 1;
  a.C = reinterpret_cast<uint8_t *>(partials);
  a.c_plane = static_cast<int64_t>(T) * E;
  const int rtiles = (T + kBM - 1) / kBM, ctiles = (E + kBW - 1) / kBW;
  const dim3 grid(static_cast<unsigned>(8 * ((rtiles + 7) / 8) * ctiles),
                  static_cast<unsigned>(splits));
  prefill_gemm_kernel<kLogits><<<grid, 512, kRing * kSlot, s>>>(a);
  return hipGetLastError();
}

}  // namespace afd
