// Weighted combine of the expert outputs back into token order (the
// "combine" of expert outputs, A/F 分离 page, "机制"):
//   out[t] = sum_{j<k} w[t,j] * Y[slot_row[t,j]] + sum_s Y[T*k + s*T + t]
// accumulated in fp32 in that fixed order (no atomics), so the result is the
// same bits on every run and for any stream schedule.
#include "common.h"
#include "kernels.h"

namespace afd {
namespace {

// One workgroup per token, one 16-byte chunk of the row per thread.  The
// routed rows are read in groups of eight loads issued back to back (k is a
// runtime value, so a plain loop would wait for each row in turn); the sum
// still runs over j in ascending order.
template <bool F32>
__global__ __launch_bounds__(1024) void combine_kernel(
    const uint8_t *__restrict__ Y, const int32_t *__restrict__ slot_row,
    const float *__restrict__ w, int T, int k, int S, int h,
    uint8_t *__restrict__ out) {
  constexpr int ES = F32 ? 4 : 2;
  constexpr int VPC = 16 / ES;  // values per 16-byte chunk
  constexpr int G = 8;          // routed rows in flight
  const int t = blockIdx.x;
  const int64_t Tk = static_cast<int64_t>(T) * k;
  const int chunks = h / VPC;
  const int64_t ypitch = static_cast<int64_t>(h) * ES;
  const int32_t *rows = slot_row + static_cast<int64_t>(t) * k;
  const float *wt = w + static_cast<int64_t>(t) * k;
  auto add = [&](float (&acc)[VPC], const u32x4 &v, float wj) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (F32) {
        acc[i] = fmaf(wj, __uint_as_float(v[i]), acc[i]);
      } else {
        acc[2 * i] = fmaf(wj, __uint_as_float(v[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj, __uint_as_float(v[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
  };
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    float acc[VPC];
#pragma unroll
    for (int i = 0; i < VPC; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += G) {
      u32x4 v[G];
#pragma unroll
      for (int jj = 0; jj < G; ++jj)
        if (j0 + jj < k) v[jj] = ld16(Y + static_cast<int64_t>(rows[j0 + jj]) * ypitch + c * 16);
#pragma unroll
      for (int jj = 0; jj < G; ++jj)
        if (j0 + jj < k) add(acc, v[jj], wt[j0 + jj]);
    }
    for (int sg = 0; sg < S; ++sg) {
      const int64_t r = Tk + static_cast<int64_t>(sg) * T + t;
      const u32x4 v = ld16(Y + r * ypitch + c * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (F32) {
          acc[i] += __uint_as_float(v[i]);
        } else {
          acc[2 * i] += __uint_as_float(v[i] << 16);
          acc[2 * i + 1] += __uint_as_float(v[i] & 0xFFFF0000u);
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (F32)
        o[i] = __float_as_uint(acc[i]);
      else
        o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    }
    st16(out + static_cast<int64_t>(t) * ypitch + c * 16, o);
  }
}

}  // namespace

hipError_t launch_combine(bool f32, const uint8_t *Y, const int32_t *slot_row,
                          const float *w, int T, int k, int S, int h,
                          void *out, hipStream_t s) {
  uint8_t *o = static_cast<uint8_t *>(out);
  const int chunks = h / (f32 ? 4 : 8);
  int threads = ((chunks + 63) / 64) * 64;
  if (threads > 1024) threads = 1024;
  if (f32)
    combine_kernel<true><<<T, threads, 0, s>>>(Y, slot_row, w, T, k, S, h, o);
  else
    combine_kernel<false><<<T, threads, 0, s>>>(Y, slot_row, w, T, k, S, h, o);
  return hipGetLastError();
}

}  // namespace afd
