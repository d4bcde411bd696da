// Router: logits = X W_r^T (+ b), then top-k with ties to the lower expert
// index, then the softmax restricted to the selected experts and
// renormalised.  One workgroup owns TM tokens and all E experts, so the
// whole routing decision of a token stays on chip.
//
// The pages name routing as one of the two costs of the expert path (vLLM
// AFD plugin page, "Attention-FFN 解耦的原理") and experts as sparsely
// activated, a few out of hundreds per token (LLM 推理提速 page,
// "一个在啃带宽，一个在吃算力"); the softmax, the tie rule and the
// renormalisation are this library's reading of that step.
//
// bf16 path (E <= 256): split-K over the 4 waves, operands straight from
// global memory into MFMA registers, partial logits summed in wave order.
// bf16 path (E <= 512): X rows staged through LDS, each wave owning a set of
// 16-expert column blocks.  fp32 path (small layers): one dot product per
// thread.
#include "common.h"
#include "kernels.h"

namespace afd {
namespace {

constexpr int kRowB = 144;  // LDS pitch of a 128-byte K stage row (+16 pad)

// Sortable key: larger logit first, then smaller index.  Key 0 = removed.
__device__ __forceinline__ unsigned long long topk_key(float v, int e) {
  v += 0.0f;  // -0 -> +0 so equal logits compare equal
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(e));
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

// Top-k over the logits of TM tokens held in LDS (row pitch E), one wave per
// token at a time.  NC = candidates per lane (E <= 64 * NC).
template <int TM, int NC>
__device__ void topk_from_lds(const float *sl, float *selv, int t0, int T,
                              int E, int k, int32_t *ids, float *wout) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  float *mysel = selv + wave * kMaxExperts;
  for (int tt = wave; tt < TM; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float *row = sl + tt * E;
    unsigned long long key[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = lane + 64 * c;
      key[c] = e < E ? topk_key(row[e], e) : 0ull;
    }
    for (int j = 0; j < k; ++j) {
      unsigned long long best = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) best = key[c] > best ? key[c] : best;
      best = wave_max_u64(best);
      const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (lane + 64 * c == e) key[c] = 0;
      if (lane == 0) {
        ids[static_cast<int64_t>(t) * k + j] = e;
        mysel[j] = row[e];
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    // slot 0 holds the largest logit of all E experts
    const float m = mysel[0];
    float part = 0.0f;
    for (int j = lane; j < k; j += 64) part += expf(mysel[j] - m);
    const float den = wave_sum(part);
    for (int j = lane; j < k; j += 64)
      wout[static_cast<int64_t>(t) * k + j] = expf(mysel[j] - m) / den;
    __builtin_amdgcn_wave_barrier();
  }
}

// bf16 router.  TM tokens per workgroup, NBPW 16-expert blocks per wave.
template <int TM, int NBPW>
__global__ __launch_bounds__(256) void router_bf16_kernel(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ Wr,
    const float *__restrict__ bias, int T, int h, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ wout) {
  constexpr int MB = TM / 16;
  constexpr int NC = (NBPW * 4 * 16) / 64;  // candidates per lane
  __shared__ __align__(16) uint8_t smem[(2 * TM * kRowB > TM * NBPW * 64 * 4)
                                            ? 2 * TM * kRowB
                                            : TM * NBPW * 64 * 4];
  __shared__ float selv[4 * kMaxExperts];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.x * TM;
  const int nstages = h / 64;  // 64 bf16 = 128 bytes per stage

  // A (X rows) staging: TM rows x 8 chunks of 16 bytes.
  constexpr int ACH = TM * 8;
  u32x4 ra[(ACH + 255) / 256];
  auto load_a = [&](int s) {
#pragma unroll
    for (int i = 0; i < (ACH + 255) / 256; ++i) {
      const int c = tid + 256 * i;
      if (c < ACH) {
        const int row = c >> 3, col = c & 7;
        const int t = t0 + row;
        ra[i] = (t < T) ? ld16(X + static_cast<int64_t>(t) * h + s * 64 + col * 8)
                        : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < (ACH + 255) / 256; ++i) {
      const int c = tid + 256 * i;
      if (c < ACH) st16(smem + buf * TM * kRowB + (c >> 3) * kRowB + (c & 7) * 16, ra[i]);
    }
  };
  // B (router rows) straight to registers: block nb of this wave, row
  // nb*16 + r16, bytes [32q, 32q + 32) of the stage.
  Frag32 rb[NBPW];
  auto load_b = [&](int s) {
#pragma unroll
    for (int j = 0; j < NBPW; ++j) {
      const int e = (wave + 4 * j) * 16 + r16;
      if (e < E) {
        const uint16_t *p = Wr + static_cast<int64_t>(e) * h + s * 64 + q * 16;
        rb[j].lo = ld16(p);
        rb[j].hi = ld16(p + 8);
      } else {
        rb[j].lo = u32x4{0, 0, 0, 0};
        rb[j].hi = u32x4{0, 0, 0, 0};
      }
    }
  };

  f32x4 acc[MB][NBPW];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < NBPW; ++j) acc[m][j] = f32x4{0, 0, 0, 0};

  load_a(0);
  store_a(0);
  load_b(0);
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    Frag32 cb[NBPW];
#pragma unroll
    for (int j = 0; j < NBPW; ++j) cb[j] = rb[j];
    if (s + 1 < nstages) {
      load_a(s + 1);
      load_b(s + 1);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const uint8_t *pa = smem + buf * TM * kRowB + (m * 16 + r16) * kRowB + q * 32;
      Frag32 fa;
      fa.lo = ld16(pa);
      fa.hi = ld16(pa + 16);
#pragma unroll
      for (int j = 0; j < NBPW; ++j) acc[m][j] = mma32<Elem::BF16>(fa, cb[j], acc[m][j]);
    }
    if (s + 1 < nstages) store_a(buf ^ 1);
    __syncthreads();
  }

  // logits -> LDS [TM][E]
  float *sl = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int j = 0; j < NBPW; ++j) {
    const int e = (wave + 4 * j) * 16 + r16;
    if (e < E) {
      const float b = bias ? bias[e] : 0.0f;
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sl[(m * 16 + q * 4 + i) * E + e] = acc[m][j][i] + b;
    }
  }
  __syncthreads();
  topk_from_lds<TM, NC>(sl, selv, t0, T, E, k, ids, wout);
}

// bf16 router, split-K: the 4 waves of a workgroup take disjoint quarters of
// h and each computes all TM x E partial logits straight from global memory
// (no LDS, no barrier in the K loop; operands prefetched NBUF chunks ahead),
// then the four partial sums are added in wave order through LDS, so the
// result does not depend on timing.  NB = 16-expert column blocks (E <= 16 NB).
template <int TM, int NB, int NBUF>
__global__ __launch_bounds__(256) void router_bf16_splitk_kernel(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ Wr,
    const float *__restrict__ bias, int T, int h, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ wout) {
  constexpr int MB = TM / 16;
  constexpr int NC = (NB * 16 + 63) / 64;
  __shared__ float red[4 * TM * NB * 16];
  __shared__ float selv[4 * kMaxExperts];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.x * TM;
  const int kq = h / 4;            // this wave's K range: [wave * kq, wave * kq + kq)
  const int nchunks = kq / 32;     // 32 K elements per MFMA
  const int kbase = wave * kq + q * 8;

  const uint16_t *arow[MB];
  bool avalid[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int t = t0 + m * 16 + r16;
    avalid[m] = t < T;
    arow[m] = X + static_cast<int64_t>(avalid[m] ? t : 0) * h + kbase;
  }
  const uint16_t *brow[NB];
  bool bvalid[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int e = n * 16 + r16;
    bvalid[n] = e < E;
    brow[n] = Wr + static_cast<int64_t>(bvalid[n] ? e : 0) * h + kbase;
  }

  u32x4 fa[NBUF][MB], fb[NBUF][NB];
  auto load = [&](int buf, int c) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
      fa[buf][m] = avalid[m] ? ld16(arow[m] + c * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int n = 0; n < NB; ++n)
      fb[buf][n] = bvalid[n] ? ld16(brow[n] + c * 32) : u32x4{0, 0, 0, 0};
  };
  f32x4 acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[m][n] = f32x4{0, 0, 0, 0};

#pragma unroll
  for (int b = 0; b < NBUF; ++b)
    if (b < nchunks) load(b, b);
  for (int c0 = 0; c0 < nchunks; c0 += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int c = c0 + b;
      if (c < nchunks) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int n = 0; n < NB; ++n)
            acc[m][n] = mfma_bf16_k32(bitcast<bf16x8>(fa[b][m]), bitcast<bf16x8>(fb[b][n]),
                                      acc[m][n]);
        if (c + NBUF < nchunks) load(b, c + NBUF);
      }
    }
  }

  // partial logits -> LDS, then a fixed-order sum over the 4 waves
  constexpr int EP = NB * 16;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * TM + m * 16 + q * 4 + i) * EP + n * 16 + r16] = acc[m][n][i];
  __syncthreads();
  // sums into registers first, then (after a barrier) compacted to pitch E
  constexpr int PER = (TM * EP + 255) / 256;
  float sum[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + 256 * j;
    sum[j] = 0.0f;
    if (i < TM * E) {
      const int tt = i / E, e = i % E;
      float v = red[tt * EP + e];
      v += red[(TM + tt) * EP + e];
      v += red[(2 * TM + tt) * EP + e];
      v += red[(3 * TM + tt) * EP + e];
      if (bias) v += bias[e];
      sum[j] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + 256 * j;
    if (i < TM * E) red[i] = sum[j];
  }
  __syncthreads();
  topk_from_lds<TM, NC>(red, selv, t0, T, E, k, ids, wout);
}

// fp32 router for small layers: one (token, expert) dot product per thread.
template <int TM>
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float *__restrict__ X, const float *__restrict__ Wr,
    const float *__restrict__ bias, int T, int h, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ wout) {
  __shared__ float sl[TM * kMaxExperts];
  __shared__ float selv[4 * kMaxExperts];
  const int t0 = blockIdx.x * TM;
  for (int p = threadIdx.x; p < TM * E; p += 256) {
    const int tt = p / E, e = p % E, t = t0 + tt;
    float a = 0.0f;
    if (t < T) {
      const float *xr = X + static_cast<int64_t>(t) * h;
      const float *wr = Wr + static_cast<int64_t>(e) * h;
      for (int i = 0; i < h; ++i) a = fmaf(xr[i], wr[i], a);
      if (bias) a += bias[e];
    }
    sl[tt * E + e] = a;
  }
  __syncthreads();
  topk_from_lds<TM, kMaxExperts / 64>(sl, selv, t0, T, E, k, ids, wout);
}

}  // namespace

hipError_t launch_router(bool f32, const void *x, const void *wr,
                         const float *bias, int T, int h, int E, int k,
                         int32_t *ids, float *w, hipStream_t s) {
  if (f32) {
    constexpr int TM = 16;
    router_f32_kernel<TM><<<(T + TM - 1) / TM, 256, 0, s>>>(
        static_cast<const float *>(x), static_cast<const float *>(wr), bias, T,
        h, E, k, ids, w);
    return hipGetLastError();
  }
  const uint16_t *X = static_cast<const uint16_t *>(x);
  const uint16_t *W = static_cast<const uint16_t *>(wr);
  if (E <= 64) {
    if (T <= 4096)
      router_bf16_splitk_kernel<16, 4, 4><<<(T + 15) / 16, 256, 0, s>>>(X, W, bias, T, h, E, k, ids, w);
    else
      router_bf16_splitk_kernel<32, 4, 2><<<(T + 31) / 32, 256, 0, s>>>(X, W, bias, T, h, E, k, ids, w);
  } else if (E <= 256) {
    if (T <= 4096)
      router_bf16_splitk_kernel<16, 16, 2><<<(T + 15) / 16, 256, 0, s>>>(X, W, bias, T, h, E, k, ids, w);
    else
      router_bf16_splitk_kernel<32, 16, 1><<<(T + 31) / 32, 256, 0, s>>>(X, W, bias, T, h, E, k, ids, w);
  } else {
    router_bf16_kernel<32, 8><<<(T + 31) / 32, 256, 0, s>>>(X, W, bias, T, h, E, k, ids, w);
  }
  return hipGetLastError();
}

}  // namespace afd
