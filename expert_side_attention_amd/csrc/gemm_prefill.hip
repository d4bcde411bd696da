// Compute-bound grouped expert GEMMs (bf16) for prefill-sized batches, where
// each busy expert holds hundreds to thousands of rows and the work is the
// MFMA throughput (the FFN side saturates compute: LLM 推理提速 page,
// "一个在啃带宽，一个在吃算力"; experts are large matrix products: A/F 分离
// page, "为什么要拆").
//
// Tile: 256 rows x 256 weight rows per workgroup (gate/up: 128 gate + 128 up
// rows, i.e. 128 output columns of z; down: 256 output columns), K in
// 64-element stages.  Four waves in a 2 x 2 grid each own 128 rows x 128
// weight rows = 4 x 4 tiles of 32x32x16 MFMAs (256 fp32 accumulators per
// lane).  Per stage each wave reads 32 KB of operands from LDS for 64 MFMAs,
// half the LDS bandwidth at full MFMA rate.
//
// Operands go global -> registers -> LDS, double-buffered: during stage s
// the MFMAs read buffer s % 2 while stage s+1 (already in registers) is
// written to the other buffer and stage s+2 is loaded, in four parts
// interleaved with the four MFMA k-steps.  The main loop has no branches.  LDS rows are
// 128 bytes with the 16-byte chunk index XOR-ed by (row / 2) mod 8, so the
// 32 rows an MFMA operand read touches spread over all banks.
//
// Tile order: row tiles are dealt round-robin to the 8 XCDs (workgroup ids
// go to XCDs round-robin) and all column tiles of a row tile run on one XCD,
// close in time: the XCD's L2 serves the activation rows to all of them.
#include "common.h"
#include "kernels.h"

namespace afd {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;   // rows per tile
constexpr int kBW = 256;   // weight rows per tile
constexpr int kRow = 128;  // bytes per LDS row (one K stage)

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRow + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

template <bool SWIGLU>
__global__ __launch_bounds__(256) void prefill_gemm_kernel(const GemmArgs p) {
  extern __shared__ __align__(16) uint8_t lds[];  // 2 x (A 32 KB + B 32 KB)
  __shared__ int rowsrc[kBM];
  uint8_t *ldsA = lds;                       // [2][256][128]
  uint8_t *ldsB = lds + 2 * kBM * kRow;      // [2][256][128]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int r32 = lane & 31, g = lane >> 5;
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;  // output columns per tile

  const int nmax = p.N > p.Ns ? p.N : p.Ns;
  const int ntn = (nmax + BNO - 1) / BNO;  // the last column tile may be partial
  const int L = blockIdx.x;
  const int j = L >> 3;
  const int mt = (L & 7) + 8 * (j / ntn);
  const int nt = j % ntn;
  if (mt >= *p.num_tiles) return;
  const Tile tile = p.tiles[mt];
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
  const int nst = static_cast<int>(krow / kRow);
  const int64_t mat = static_cast<int64_t>(N) * krow;
  const uint8_t *B0 = (shared ? p.sb0 : p.b0) + gi * mat;
  const uint8_t *B1 = SWIGLU ? (shared ? p.sb1 : p.b1) + gi * mat : nullptr;

  // Per-thread load slots: chunk c = tid + 256 i, row c / 8, 16-byte chunk
  // c % 8.  Rows past the tile's end read a valid row instead (the rows of an
  // MFMA tile are independent and those results are never stored), and
  // weight rows past N (partial last column tile) read row N - 1, so the main
  // loop has no branches.
  const int src_first = rowsrc[0];
  const uint8_t *asrc[8];
  const uint8_t *bsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
    const int src = rowsrc[row] >= 0 ? rowsrc[row] : src_first;
    asrc[i] = p.A + static_cast<int64_t>(src) * p.a_pitch + ch * 16;
    const uint8_t *base;
    int n;
    if (SWIGLU) {
      base = row < kBW / 2 ? B0 : B1;
      n = n0 + (row & (kBW / 2 - 1));
    } else {
      base = B0;
      n = n0 + row;
    }
    bsrc[i] = base + static_cast<int64_t>(min(n, N - 1)) * krow + ch * 16;
  }
  u32x4 ra[8], rb[8];
  // slots are moved in 4 parts of 2 (A) + 2 (B) so that LDS stores and
  // global loads interleave with the 4 MFMA k-steps of a stage
  auto gload_part = [&](int part, int s) {
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i) {
      ra[i] = ld16(asrc[i] + static_cast<int64_t>(s) * kRow);
      rb[i] = ld16(bsrc[i] + static_cast<int64_t>(s) * kRow);
    }
  };
  auto lstore_part = [&](int part, int buf) {
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      st16(ldsA + buf * kBM * kRow + swz(row, ch), ra[i]);
      st16(ldsB + buf * kBW * kRow + swz(row, ch), rb[i]);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x16{};

  // weight rows of n-block n for this wave
  int wrow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
    wrow[n] = SWIGLU ? ((n >> 1) * (kBW / 2) + wc * 64 + (n & 1) * 32 + r32)
                     : (wc * 128 + n * 32 + r32);

#pragma unroll
  for (int part = 0; part < 4; ++part) gload_part(part, 0);
#pragma unroll
  for (int part = 0; part < 4; ++part) lstore_part(part, 0);
  if (nst > 1) {
#pragma unroll
    for (int part = 0; part < 4; ++part) gload_part(part, 1);
  }
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    const uint8_t *la = ldsA + buf * kBM * kRow;
    const uint8_t *lb = ldsB + buf * kBW * kRow;
    const bool more = s + 1 < nst, more2 = s + 2 < nst;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + g;
      bf16x8 bfr[4], afr[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) bfr[n] = bitcast<bf16x8>(ld16(lb + swz(wrow[n], ch)));
#pragma unroll
      for (int m = 0; m < 4; ++m)
        afr[m] = bitcast<bf16x8>(ld16(la + swz(wr * 128 + m * 32 + r32, ch)));
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[m], bfr[n], acc[m][n], 0, 0, 0);
      // stage s+1 (loaded during the previous stage) into the other buffer,
      // then reuse the registers for stage s+2
      if (more) {
        lstore_part(ks, buf ^ 1);
        if (more2) gload_part(ks, s + 2);
      }
    }
    __syncthreads();
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
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int col = wc * 64 + jj * 32 + r32;
          o16[row * OPITCH + col] = f32_to_bf16(silu_mul(acc[m][jj][i], acc[m][2 + jj][i]));
        }
      } else {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int col = wc * 128 + n * 32 + r32;
          o16[row * OPITCH + col] = f32_to_bf16(acc[m][n][i]);
        }
      }
    }
  }
  __syncthreads();
  constexpr int CPR = OPITCH * 2 / 16;  // 16-byte pieces per staged row
  const int vcpr = min(CPR, (N - n0) * 2 / 16);
  for (int c = tid; c < kBM * CPR; c += 256) {
    const int row = c / CPR, col = c % CPR;
    if (row < rows && col < vcpr)
      st16(p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch + n0 * 2 + col * 16,
           ld16(lds + row * OPITCH * 2 + col * 16));
  }
}

template <bool SWIGLU>
hipError_t launch_one(const GemmArgs &a, hipStream_t s) {
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;
  constexpr size_t kLds = 2 * (kBM + kBW) * kRow;  // 128 KB
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_gemm_kernel<SWIGLU>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nmax = a.N > a.Ns ? a.N : a.Ns;
  const int ntn = (nmax + BNO - 1) / BNO;
  const int64_t grid = 8LL * ((a.tiles_ub + 7) / 8) * ntn;
  if (grid <= 0) return hipSuccess;
  prefill_gemm_kernel<SWIGLU><<<static_cast<unsigned>(grid), 256, kLds, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(GemmKind kind, const GemmArgs &a, hipStream_t s) {
  return kind == GemmKind::GateUp ? launch_one<true>(a, s) : launch_one<false>(a, s);
}

}  // namespace afd
