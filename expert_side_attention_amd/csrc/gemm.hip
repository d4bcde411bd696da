// Grouped expert GEMMs on MFMA: gate/up with a fused SiLU(gate) * up
// epilogue, and down.  Experts are large, compute-hungry matrix products,
// each run on the rows dispatched to it (A/F 分离 page, "为什么要拆"; the
// FFN side saturates compute, LLM 推理提速 page, "一个在啃带宽，一个在吃算力").
// The SwiGLU form and the shared expert as extra groups are this library's
// reading of "experts".
//
// Work decomposition: the dispatch kernel writes a device-side list of row
// tiles (expert, first row, rows); the grid is an upper bound of that list
// times the column tiles, and surplus workgroups exit at once, so no count
// ever travels to the host.  Workgroup id -> tile: the hardware deals
// workgroups to the 8 XCDs round-robin, so tile rows are dealt round-robin
// too and the column tiles of one row tile land on one XCD (its L2 keeps the
// gathered activation rows).
//
// Inner loop: 128-byte K stages (64 bf16 / 128 fp8 / 32 fp32 per row) of A
// (gathered rows) and B (weight rows) go global -> registers -> LDS (double
// buffered, 16-byte padded rows), then each wave multiplies its column
// slice against all row blocks with 16x16 MFMAs.  FP8 keeps a per-stage
// partial sum and folds it into the accumulator with the product of the
// activation (1x128) and weight (128x128) block scales.
#include "common.h"
#include "kernels.h"

namespace afd {
namespace {

constexpr int kRowB = 144;  // LDS row pitch: 128 data bytes + 16 pad

template <Elem EL>
struct ElemInfo;
template <>
struct ElemInfo<Elem::F32> {
  static constexpr int bytes = 4;
};
template <>
struct ElemInfo<Elem::BF16> {
  static constexpr int bytes = 2;
};
template <>
struct ElemInfo<Elem::FP8> {
  static constexpr int bytes = 1;
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

template <Elem EL, int BM, int BN, bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(const GemmArgs p) {
  constexpr int ES = ElemInfo<EL>::bytes;
  constexpr int NB = SWIGLU ? 2 * BN : BN;  // weight rows per stage
  constexpr int MB = BM / 16;               // 16-row blocks
  constexpr int NW = BN / 64;               // 16-col blocks per wave per matrix
  constexpr int NMAT = SWIGLU ? 2 : 1;
  constexpr int ACH = BM * 8;               // 16-byte chunks of an A stage
  constexpr int BCH = NB * 8;
  constexpr int RA = (ACH + 255) / 256;
  constexpr int RB = BCH / 256;
  constexpr bool kFp8 = EL == Elem::FP8;
  static_assert(BN % 64 == 0 && BM % 16 == 0 && BCH % 256 == 0, "tile shape");
  static_assert(!(kFp8 && SWIGLU) || BN == 128, "fp8 z quantisation needs 128 columns");
  static_assert(!kFp8 || BN <= 128, "one weight scale block per stage");

  __shared__ __align__(16) uint8_t smA[2][BM * kRowB];
  __shared__ __align__(16) uint8_t smB[2][NB * kRowB];
  __shared__ int rowsrc[BM];
  __shared__ float sAs[2][kFp8 ? BM : 1];
  __shared__ float red[kFp8 && SWIGLU ? 4 * BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;

  // ---- workgroup -> (row tile, column tile)
  const int ntn = static_cast<int>(gridDim.x) / (8 * ((p.tiles_ub + 7) / 8));
  const int L = blockIdx.x;
  const int j = L >> 3;
  const int mt = (L & 7) + 8 * (j / ntn);
  const int nt = j % ntn;
  if (mt >= *p.num_tiles) return;
  const Tile tile = p.tiles[mt];
  const bool shared = tile.group >= p.E;
  const int N = shared ? p.Ns : p.N;
  const int K = shared ? p.Ks : p.K;
  const int n0 = nt * BN;
  if (n0 >= N) return;
  const int g = shared ? tile.group - p.E : tile.group;
  const int rows = tile.rows;

  if (tid < BM) {
    int src = -1;
    if (tid < rows) {
      const int r = tile.row0 + tid;
      src = p.perm ? (r < p.Tk ? p.perm[r] : (r - p.Tk) % p.T) : r;
    }
    rowsrc[tid] = src;
  }
  __syncthreads();

  // ---- operand pointers
  const int64_t mat_bytes = static_cast<int64_t>(N) * K * ES;
  const uint8_t *B0 = (shared ? p.sb0 : p.b0) + g * mat_bytes;
  const uint8_t *B1 = SWIGLU ? (shared ? p.sb1 : p.b1) + g * mat_bytes : nullptr;
  const int kblocks = K / 128;  // fp8 scale blocks along K
  const float *Bs0 = nullptr, *Bs1 = nullptr;
  if constexpr (kFp8) {
    const int64_t sblk = static_cast<int64_t>(N / 128) * kblocks;
    Bs0 = (shared ? p.sbs0 : p.bs0) + g * sblk + (n0 / 128) * kblocks;
    if (SWIGLU) Bs1 = (shared ? p.sbs1 : p.bs1) + g * sblk + (n0 / 128) * kblocks;
  }
  const int64_t krow = static_cast<int64_t>(K) * ES;  // weight row bytes
  const int nstages = static_cast<int>(krow / 128);

  u32x4 ra[RA], rb[RB];
  auto load = [&](int s) {
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int c = tid + 256 * i;
      if (c < ACH) {
        const int src = rowsrc[c >> 3];
        if (src >= 0) ra[i] = ld16(p.A + src * p.a_pitch + s * 128 + (c & 7) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int c = tid + 256 * i;
      const int rr = c >> 3;
      const uint8_t *base = (SWIGLU && rr >= BN) ? B1 : B0;
      const int n = n0 + (SWIGLU ? rr % BN : rr);
      rb[i] = ld16(base + n * krow + s * 128 + (c & 7) * 16);
    }
  };
  float as_next = 0.0f;
  auto load_scale = [&](int s) {
    if constexpr (kFp8) {
      if (tid < BM) {
        const int src = rowsrc[tid];
        as_next = src >= 0 ? p.a_scale[static_cast<int64_t>(src) * p.a_scale_pitch + s] : 0.0f;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      const int c = tid + 256 * i;
      if (c < ACH) st16(&smA[buf][(c >> 3) * kRowB + (c & 7) * 16], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int c = tid + 256 * i;
      st16(&smB[buf][(c >> 3) * kRowB + (c & 7) * 16], rb[i]);
    }
    if constexpr (kFp8)
      if (tid < BM) sAs[buf][tid] = as_next;
  };

  f32x4 acc[NMAT][MB][NW];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int w = 0; w < NW; ++w) acc[m][b][w] = f32x4{0, 0, 0, 0};

  const int mb_active = (rows + 15) >> 4;
  const int col_w = wave * (BN / 4);  // this wave's first column in the tile

  load(0);
  load_scale(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) {
      load(s + 1);
      load_scale(s + 1);
    }
    Frag32 fb[NMAT][NW];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint8_t *pb = &smB[buf][(m * BN + col_w + w * 16 + r16) * kRowB + q * 32];
        fb[m][w].lo = ld16(pb);
        fb[m][w].hi = ld16(pb + 16);
      }
    float sb0 = 1.0f, sb1 = 1.0f;
    if constexpr (kFp8) {
      sb0 = Bs0[s];
      if (SWIGLU) sb1 = Bs1[s];
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if (b < mb_active) {
        const uint8_t *pa = &smA[buf][(b * 16 + r16) * kRowB + q * 32];
        Frag32 fa;
        fa.lo = ld16(pa);
        fa.hi = ld16(pa + 16);
        if constexpr (kFp8) {
          float sa[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[i] = sAs[buf][b * 16 + q * 4 + i];
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
              const f32x4 part = mma32<EL>(fa, fb[m][w], f32x4{0, 0, 0, 0});
              const float sbm = m ? sb1 : sb0;
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[m][b][w][i] = fmaf(part[i], sa[i] * sbm, acc[m][b][w][i]);
            }
        } else {
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w) acc[m][b][w] = mma32<EL>(fa, fb[m][w], acc[m][b][w]);
        }
      }
    }
    if (s + 1 < nstages) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  if constexpr (SWIGLU && kFp8) {
    // z = silu(g) * u in fp32, then per-row amax over the tile's 128
    // columns (one quantisation group), scale, E4M3 codes.
    float zv[MB][NW][4];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          zv[b][w][i] = silu_mul(acc[0][b][w][i], acc[1][b][w][i]);
          mx = fmaxf(mx, fabsf(zv[b][w][i]));
        }
        mx = group16_max(mx);
        if (r16 == 0) red[wave * BM + b * 16 + q * 4 + i] = mx;
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < MB; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = b * 16 + q * 4 + i;
        if (row < rows) {
          const float amax = fmaxf(fmaxf(red[row], red[BM + row]),
                                   fmaxf(red[2 * BM + row], red[3 * BM + row]));
          const float sc = e4m3_scale(amax);
          uint8_t *crow = p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch;
#pragma unroll
          for (int w = 0; w < NW; ++w)
            crow[n0 + col_w + w * 16 + r16] = static_cast<uint8_t>(f32_to_e4m3(zv[b][w][i] / sc));
          if (wave == 0 && r16 == 0)
            p.c_scale[static_cast<int64_t>(tile.row0 + row) * p.c_scale_pitch + n0 / 128] = sc;
        }
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = b * 16 + q * 4 + i;
        if (row < rows) {
          uint8_t *crow = p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const int col = n0 + col_w + w * 16 + r16;
            const float v = SWIGLU ? silu_mul(acc[0][b][w][i], acc[NMAT - 1][b][w][i])
                                   : acc[0][b][w][i];
            if constexpr (EL == Elem::F32)
              reinterpret_cast<float *>(crow)[col] = v;
            else
              reinterpret_cast<uint16_t *>(crow)[col] = f32_to_bf16(v);
          }
        }
      }
    }
  }
}

template <Elem EL, int BM, int BN, bool SWIGLU>
hipError_t launch_one(const GemmArgs &a, hipStream_t s) {
  const int nmax = a.N > a.Ns ? a.N : a.Ns;
  const int ntn = (nmax + BN - 1) / BN;
  const int64_t grid = 8LL * ((a.tiles_ub + 7) / 8) * ntn;
  if (grid <= 0) return hipSuccess;
  grouped_gemm_kernel<EL, BM, BN, SWIGLU><<<static_cast<unsigned>(grid), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

GemmPlan gemm_plan(int elem, int T, int k, int E) {
  if (elem == 0) return {{32, 0, 0}, GemmKernel::Tiled};
  // rows per expert on average decide the regime: a few dozen rows per
  // expert -> stream the weights once with a tile that holds all of them;
  // hundreds of rows (bf16) -> experts' 256-row blocks go to the
  // compute-bound kernel and small experts / small remainders (<= 128 rows)
  // to the streaming kernel
  const int64_t avg = (static_cast<int64_t>(T) * k + E - 1) / E;
  if (avg <= 48) return {{64, 0, 0}, GemmKernel::Stream};
  if (avg <= 112 || elem == 2) {
    if (elem == 2 && avg > 112) return {{64, 0, 0}, GemmKernel::Tiled};
    return {{128, 0, 0}, GemmKernel::Stream};
  }
  return {{128, 256, 129}, GemmKernel::Stream};
}

hipError_t launch_gemm(GemmKind kind, int elem, int bm, const GemmArgs &a,
                       hipStream_t s) {
  const bool gu = kind == GemmKind::GateUp;
  if (elem == 0) {
    if (bm != 32) return hipErrorInvalidValue;
    return gu ? launch_one<Elem::F32, 32, 64, true>(a, s)
              : launch_one<Elem::F32, 32, 64, false>(a, s);
  }
  if (bm != 64) return hipErrorInvalidValue;
  if (elem == 1)
    return gu ? launch_one<Elem::BF16, 64, 64, true>(a, s)
              : launch_one<Elem::BF16, 64, 128, false>(a, s);
  return gu ? launch_one<Elem::FP8, 64, 128, true>(a, s)
            : launch_one<Elem::FP8, 64, 128, false>(a, s);
}

}  // namespace afd
