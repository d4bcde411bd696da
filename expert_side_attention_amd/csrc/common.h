// Device-side helpers shared by the kernels of the MoE FFN-service layer
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) |
         (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------- E4M3 (OCP FN)
// Encode a float to an E4M3FN code: saturate |v| to 448, round to nearest
// even on the E4M3 grid, keep the sign bit (also for a zero result).
// Normal range (|v| >= 2^-6): round the fp32 mantissa to 3 bits at bit 20
// and re-bias the exponent (127 -> 7); a mantissa carry moves to the next
// binade, which is the next code.  Below 2^-6 the grid step is 2^-9, so the
// code is rint(|v| * 512) (0..8; 8 is the smallest normal, code 0x08).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = (b >> 20) - (120u << 3);
  }
  return sign | code;
}

// Per-group scale: fl32(amax / 448) with IEEE division; 1 if that is 0.
__device__ __forceinline__ float e4m3_scale(float amax) {
  float s = amax / 448.0f;
  return (amax == 0.0f || s == 0.0f) ? 1.0f : s;
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Max over each group of 16 consecutive lanes (lanes with equal lane / 16).
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

// ---------------------------------------------------------------- MFMA
// 16x16 output tile, fp32 accumulate.  For all three element types a lane
// supplies the A row (lane % 16) / B column (lane % 16) and a lane group
// (lane / 16) supplies a slice of K; A and B use the same slice mapping, so
// any consistent assignment of K indices to (lane group, register) is a
// valid product.  Output: lane holds rows 4*(lane/16)+i, column lane%16.
__device__ __forceinline__ f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_fp8_k32(long a, long b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 32 bytes of operand (one lane's share of a 128-byte K stage) -> MFMAs.
struct Frag32 {
  u32x4 lo, hi;
};

template <typename T>
__device__ __forceinline__ T bitcast(const u32x4 &v) {
  return __builtin_bit_cast(T, v);
}

// acc += A(32B) . B(32B) for the given element type.
// BF16: 16 values -> 2 x (16x16x32); FP8: 32 values -> 4 x (16x16x32 fp8);
// F32: 8 values -> 8 x (16x16x4).
enum class Elem { F32 = 0, BF16 = 1, FP8 = 2 };

template <Elem E>
__device__ __forceinline__ f32x4 mma32(const Frag32 &a, const Frag32 &b, f32x4 c) {
  if constexpr (E == Elem::BF16) {
    c = mfma_bf16_k32(bitcast<bf16x8>(a.lo), bitcast<bf16x8>(b.lo), c);
    c = mfma_bf16_k32(bitcast<bf16x8>(a.hi), bitcast<bf16x8>(b.hi), c);
  } else if constexpr (E == Elem::FP8) {
    typedef long l2 __attribute__((ext_vector_type(2)));
    l2 al = __builtin_bit_cast(l2, a.lo), bl = __builtin_bit_cast(l2, b.lo);
    l2 ah = __builtin_bit_cast(l2, a.hi), bh = __builtin_bit_cast(l2, b.hi);
    c = mfma_fp8_k32(al.x, bl.x, c);
    c = mfma_fp8_k32(al.y, bl.y, c);
    c = mfma_fp8_k32(ah.x, bh.x, c);
    c = mfma_fp8_k32(ah.y, bh.y, c);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = mfma_f32_k4(__uint_as_float(a.lo[i]), __uint_as_float(b.lo[i]), c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = mfma_f32_k4(__uint_as_float(a.hi[i]), __uint_as_float(b.hi[i]), c);
  }
  return c;
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

// acc (16 rows x 16 columns) += A[rows][K] . B[cols][K]^T over nck 128-byte
// K chunks; lane (r16, q) supplies row / column r16 and bytes [32 q, 32 q +
// 32) of each chunk; arow / brow point at the lane's row and column.
template <Elem EL>
__device__ __forceinline__ f32x4 mma_rows(const uint8_t *arow, const uint8_t *brow, int nck,
                                          f32x4 acc) {
  for (int k0 = 0; k0 < nck; k0 += 4) {
    Frag32 fa[4], fb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kc = (k0 + u < nck ? k0 + u : k0) * 128;
      fa[u].lo = ld16(arow + kc);
      fa[u].hi = ld16(arow + kc + 16);
      fb[u].lo = ld16(brow + kc);
      fb[u].hi = ld16(brow + kc + 16);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + u < nck) acc = mma32<EL>(fa[u], fb[u], acc);
  }
  return acc;
}

}  // namespace afd
