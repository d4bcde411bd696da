// Top-k selection keys shared by the router kernels: a 64-bit key whose
// order is (logit descending, expert index ascending), so one unsigned
// maximum picks the next expert with ties going to the lower index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afd {

// Sortable key: larger logit first, then smaller index.  Key 0 = removed.
__device__ __forceinline__ unsigned long long topk_key(float v, int e) {
  v += 0.0f;  // -0 -> +0 so equal logits compare equal
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(e));
}

// The logit a key was made from (-0 comes back as +0).
__device__ __forceinline__ float topk_key_value(unsigned long long key) {
  const uint32_t u = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), o, 64);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), o, 64);
    unsigned long long y = (static_cast<unsigned long long>(hi) << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
}

}  // namespace afd
