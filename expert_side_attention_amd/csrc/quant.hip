// FP8 E4M3 quantisers.  W8A8 is the precision of the plugin page's
// benchmarks (vLLM AFD plugin page, "效能基準測試"); the A/F 分离 page's
// traffic example also moves FP8 hidden states ("深入推導" / 通信账).
// Scales: one fp32 per row per 128 columns for activations, one per
// 128x128 block for weights; s = fl32(amax / 448), q = E4M3(fl32(x / s)).
#include "common.h"
#include "kernels.h"

namespace afd {
namespace {

// 16 lanes per 128-column group, 8 bf16 (16 bytes) per lane.
__global__ __launch_bounds__(256) void quant_1x128_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
    uint8_t *__restrict__ q, float *__restrict__ sc) {
  const int64_t groups_per_row = cols / 128;
  const int64_t g = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 4;
  if (g >= rows * groups_per_row) return;  // uniform over the 16-lane group
  const int sub = threadIdx.x & 15;
  const int64_t row = g / groups_per_row, cg = g % groups_per_row;
  const int64_t base = row * cols + cg * 128 + sub * 8;
  const u32x4 v = ld16(x + base);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = group16_max(amax);
  const float s = e4m3_scale(amax);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0 |= f32_to_e4m3(f[i] / s) << (8 * i);
    w1 |= f32_to_e4m3(f[4 + i] / s) << (8 * i);
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2 *>(q + base) = u32x2{w0, w1};
  if (sub == 0) sc[row * groups_per_row + cg] = s;
}

// The same quantiser on fp32 input (z of the W8A8 gate/up GEMM): 16 lanes
// per 128-column group, 8 floats (two 16-byte loads) per lane.  Rows have a
// pitch of `pitch` floats (>= cols); codes use pitch `qpitch` bytes, scales
// `spitch` floats.
__global__ __launch_bounds__(256) void quant_1x128_f32_kernel(
    const float *__restrict__ x, int64_t rows, int64_t cols, int64_t pitch,
    uint8_t *__restrict__ q, int64_t qpitch, float *__restrict__ sc, int64_t spitch) {
  const int64_t groups_per_row = cols / 128;
  const int64_t g = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 4;
  if (g >= rows * groups_per_row) return;  // uniform over the 16-lane group
  const int sub = threadIdx.x & 15;
  const int64_t row = g / groups_per_row, cg = g % groups_per_row;
  const float *src = x + row * pitch + cg * 128 + sub * 8;
  const u32x4 v0 = ld16(src), v1 = ld16(src + 4);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = __uint_as_float(v0[i]);
    f[4 + i] = __uint_as_float(v1[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = group16_max(amax);
  const float s = e4m3_scale(amax);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0 |= f32_to_e4m3(f[i] / s) << (8 * i);
    w1 |= f32_to_e4m3(f[4 + i] / s) << (8 * i);
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2 *>(q + row * qpitch + cg * 128 + sub * 8) = u32x2{w0, w1};
  if (sub == 0) sc[row * spitch + cg] = s;
}

// One workgroup per 128x128 block; thread = (row tid/2, 64-column half).
__global__ __launch_bounds__(256) void quant_128x128_kernel(
    const uint16_t *__restrict__ w, int64_t rows, int64_t cols,
    uint8_t *__restrict__ q, float *__restrict__ sc) {
  __shared__ float red[4];
  const int64_t nbc = cols / 128;
  const int64_t br = blockIdx.x / nbc, bc = blockIdx.x % nbc;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t base = (br * 128 + r) * cols + bc * 128 + half * 64;
  u32x4 v[8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    v[c] = ld16(w + base + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[c][i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[c][i] & 0xFFFF0000u)));
    }
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = e4m3_scale(amax);
#pragma unroll
  for (int c = 0; c < 8; c += 2) {
    uint32_t o[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        lo |= f32_to_e4m3(__uint_as_float(v[c + h2][i] << 16) / s) << (16 * i);
        lo |= f32_to_e4m3(__uint_as_float(v[c + h2][i] & 0xFFFF0000u) / s) << (16 * i + 8);
        hi |= f32_to_e4m3(__uint_as_float(v[c + h2][2 + i] << 16) / s) << (16 * i);
        hi |= f32_to_e4m3(__uint_as_float(v[c + h2][2 + i] & 0xFFFF0000u) / s) << (16 * i + 8);
      }
      o[2 * h2] = lo;
      o[2 * h2 + 1] = hi;
    }
    st16(q + base + c * 8, u32x4{o[0], o[1], o[2], o[3]});
  }
  if (threadIdx.x == 0) sc[br * nbc + bc] = s;
}

}  // namespace

hipError_t launch_quant_1x128(const uint16_t *x, int64_t rows, int64_t cols,
                              uint8_t *q, float *sc, hipStream_t s) {
  const int64_t groups = rows * (cols / 128);
  const int64_t blocks = (groups * 16 + 255) / 256;
  quant_1x128_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(x, rows, cols, q, sc);
  return hipGetLastError();
}

hipError_t launch_quant_1x128_f32(const float *x, int64_t rows, int64_t cols, int64_t pitch,
                                  uint8_t *q, int64_t qpitch, float *sc, int64_t spitch,
                                  hipStream_t s) {
  const int64_t groups = rows * (cols / 128);
  const int64_t blocks = (groups * 16 + 255) / 256;
  quant_1x128_f32_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(x, rows, cols, pitch, q,
                                                                        qpitch, sc, spitch);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const uint16_t *w, int64_t rows, int64_t cols,
                                uint8_t *q, float *sc, hipStream_t s) {
  const int64_t blocks = (rows / 128) * (cols / 128);
  quant_128x128_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(w, rows, cols, q, sc);
  return hipGetLastError();
}

}  // namespace afd
