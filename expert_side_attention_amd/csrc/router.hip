// Router: logits = X W_r^T (+ b), then top-k with ties to the lower expert
// index, then the softmax restricted to the selected experts and
// renormalised.
//
// The pages name routing as one of the two costs of the expert path (vLLM
// AFD plugin page, "Attention-FFN 解耦的原理") and experts as sparsely
// activated, a few out of hundreds per token (LLM 推理提速 page,
// "一个在啃带宽，一个在吃算力"); the softmax, the tie rule and the
// renormalisation are this library's reading of that step.
//
// bf16 path: router_bf16_kernel up to 4096 tokens (K split in four parts,
// each with its own partial plane, for layers of at most 64 experts), above
// that the logits mode of the compute-bound GEMM (split-K partial planes);
// topk_kernel then adds the planes and selects.  fp32 path (small layers): one dot product per thread, one
// workgroup per 16 tokens, top-k in the same kernel.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace afd {
namespace {

// bf16 batches above this many tokens take the LDS-tiled logits GEMM (at
// 8192 tokens of DeepSeek-V3 width logits plus top-k went from 153 to 90 us,
// 74 us with the top-k's loads hoisted; at 2048 the register-operand kernel
// below is faster, 55 against 76 us)
constexpr int kTiledRouterT = 4096;

// Top-k over the logits of TM tokens (row pitch E, in LDS or global memory),
// one wave per token at a time.  NC = candidates per lane (E <= 64 * NC).
// A logit is the sum of `planes` partial values `plane` floats apart, added
// in plane order, plus bias[e] when bias is not null.  With lout set, the
// logits as ranked are also stored there ([T, E], for inspection).
template <int TM, int NC, int WAVES = 4>
__device__ void topk_rows(const float *sl, float *selv, int t0, int T,
                          int E, int k, int32_t *ids, float *wout, int planes = 1,
                          int64_t plane = 0, const float *bias = nullptr,
                          float *lout = nullptr) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  float *mysel = selv + wave * kMaxExperts;
  for (int tt = wave; tt < TM; tt += WAVES) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float *row = sl + static_cast<int64_t>(tt) * E;
    auto logit = [&](int e) {
      // all plane loads first, then the sum in plane order
      float part[kMaxLogitSplits];
#pragma unroll
      for (int pl = 0; pl < kMaxLogitSplits; ++pl)
        part[pl] = pl < planes ? row[pl * plane + e] : 0.0f;
      float v = part[0];
#pragma unroll
      for (int pl = 1; pl < kMaxLogitSplits; ++pl)
        if (pl < planes) v += part[pl];
      if (bias) v += bias[e];
      return v;
    };
    unsigned long long key[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = lane + 64 * c;
      key[c] = 0ull;
      if (e < E) {
        const float v = logit(e);
        key[c] = topk_key(v, e);
        if (lout) lout[static_cast<int64_t>(t) * E + e] = v;
      }
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
        mysel[j] = topk_key_value(best);
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

// bf16 router logits.  The grid is (expert slices of EN) x (token blocks of
// TM) x (K parts), so even small batches spread over many CUs; with more
// than one K part each part writes its own partial plane and the top-k adds
// the planes in order, then the bias.  Inside a workgroup the
// WAVES waves take disjoint slices of h and compute all TM x EN partial
// logits with operands loaded straight from global memory into MFMA
// registers (no LDS, no barrier in the K loop, NBUF chunks of prefetch); the
// partial sums are added in wave order, so the logits do not depend on
// timing.  The top-k runs in the next kernel: a device-wide hand-over inside
// this one would need an L2 write-back and invalidate per workgroup.
template <int TM, int EN, int NBUF, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void router_bf16_kernel(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ Wr,
    const float *__restrict__ bias, int T, int h, int E, float *__restrict__ logits) {
  constexpr int MB = TM / 16, NB = EN / 16;
  constexpr int THREADS = WAVES * 64;
  __shared__ float red[WAVES * TM * EN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int e0 = blockIdx.x * EN, t0 = blockIdx.y * TM;
  // K part blockIdx.z of gridDim.z: [z hs, z hs + hs), split over the waves;
  // its partial logits go to plane z (T x E floats apart)
  const int hs = h / static_cast<int>(gridDim.z);
  const int kq = hs / WAVES;    // this wave's K range [wave * kq, wave * kq + kq) of the part
  const int nchunks = kq / 32;  // 32 K elements per MFMA
  const int kbase = static_cast<int>(blockIdx.z) * hs + wave * kq + q * 8;
  logits += static_cast<int64_t>(blockIdx.z) * T * E;

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
    const int e = e0 + n * 16 + r16;
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

  // partial logits -> LDS, fixed-order sum over the waves -> global
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * TM + m * 16 + q * 4 + i) * EN + n * 16 + r16] = acc[m][n][i];
  __syncthreads();
  for (int i = tid; i < TM * EN; i += THREADS) {
    const int tt = i / EN, el = i % EN;
    const int t = t0 + tt, e = e0 + el;
    if (t < T && e < E) {
      float v = red[tt * EN + el];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v += red[(w * TM + tt) * EN + el];
      if (bias) v += bias[e];
      logits[static_cast<int64_t>(t) * E + e] = v;
    }
  }
}

// Top-k and weights from the logits (the sum of `planes` partial planes plus
// bias, if given): one wave per token, four per workgroup.
template <int NC>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T,
                                                   int E, int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ wout, int planes,
                                                   const float *__restrict__ bias,
                                                   float *__restrict__ lout) {
  __shared__ float selv[4 * kMaxExperts];
  const int t0 = blockIdx.x * 4;
  topk_rows<4, NC, 4>(logits + static_cast<int64_t>(t0) * E, selv, t0, T, E, k, ids, wout,
                      planes, static_cast<int64_t>(T) * E, bias, lout);
}

// fp32 router for small layers: 16 tokens per workgroup, 16 experts per
// 16x16 fp32 MFMA block; the four waves take quarters of K (loads issued in
// batches) and add their partial logits into LDS in wave order, so the
// logits do not depend on timing; then the top-k from LDS.
template <int TM>
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float *__restrict__ X, const float *__restrict__ Wr,
    const float *__restrict__ bias, int T, int h, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ wout, float *__restrict__ lout) {
  static_assert(TM == 16, "one 16-row MFMA block of tokens");
  __shared__ float sl[TM * kMaxExperts];
  __shared__ float selv[4 * kMaxExperts];
  const int t0 = blockIdx.x * TM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t xrow = static_cast<int64_t>(h) * 4;
  const int nck = static_cast<int>(xrow / 128);  // 128-byte K chunks of a row
  const int c0 = wave * nck / 4, c1 = (wave + 1) * nck / 4;
  const int tr = t0 + r16 < T ? t0 + r16 : T - 1;  // rows past T repeat the last token
  const uint8_t *xa = reinterpret_cast<const uint8_t *>(X) + tr * xrow + q * 32 + c0 * 128;
  constexpr int NB = kMaxExperts / 16;
  f32x4 acc[NB];
#pragma unroll
  for (int eb = 0; eb < NB; ++eb) {
    acc[eb] = f32x4{0, 0, 0, 0};
    if (eb * 16 < E) {
      const int e = eb * 16 + r16 < E ? eb * 16 + r16 : E - 1;
      acc[eb] = mma_rows<Elem::F32>(
          xa, reinterpret_cast<const uint8_t *>(Wr) + e * xrow + q * 32 + c0 * 128, c1 - c0,
          acc[eb]);
    }
  }
  // lane holds tokens 4 q + i, expert eb * 16 + r16; waves add in order
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int eb = 0; eb < NB; ++eb) {
        const int e = eb * 16 + r16;
        if (eb * 16 < E && e < E) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float *d = &sl[(4 * q + i) * E + e];
            *d = w == 0 ? acc[eb][i] : *d + acc[eb][i];
          }
        }
      }
    }
    __syncthreads();
  }
  if (bias) {
    for (int p = threadIdx.x; p < TM * E; p += 256) sl[p] += bias[p % E];
    __syncthreads();
  }
  topk_rows<TM, kMaxExperts / 64>(sl, selv, t0, T, E, k, ids, wout, 1, 0, nullptr, lout);
}

}  // namespace

// K parts of the register router: with at most 64 experts a batch has few
// expert slices, so the K range is split in four over workgroups to spread
// the operand reads over more CUs.  A function of the layer shape only, so
// a token's logits do not depend on the batch it came in.
int router_k_parts(int h, int E) { return E <= 64 && h % (4 * 256) == 0 ? 4 : 1; }

hipError_t launch_router(bool f32, const void *x, const void *wr,
                         const float *bias, int T, int h, int E, int k,
                         float *logits, int32_t *ids, float *w, float *logits_out,
                         hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (f32) {
    constexpr int TM = 16;
    router_f32_kernel<TM><<<(T + TM - 1) / TM, 256, 0, s>>>(
        static_cast<const float *>(x), static_cast<const float *>(wr), bias, T,
        h, E, k, ids, w, logits_out);
    return hipGetLastError();
  }
  const uint16_t *X = static_cast<const uint16_t *>(x);
  const uint16_t *W = static_cast<const uint16_t *>(wr);
  const unsigned blocks = static_cast<unsigned>((T + 3) / 4);
  auto topk = [&](int planes, const float *b) {
    if (E <= 64)
      topk_kernel<1><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, w, planes, b, logits_out);
    else if (E <= 256)
      topk_kernel<4><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, w, planes, b, logits_out);
    else
      topk_kernel<8><<<blocks, 256, 0, s>>>(logits, T, E, k, ids, w, planes, b, logits_out);
    return hipGetLastError();
  };
  if (T > kTiledRouterT) {
    // long batches: LDS-tiled 256 x 256 GEMM with the K range split over
    // workgroups; the top-k adds the partial planes in order, then the bias
    const int splits = logits_splits(T, h, E);
    hipError_t e = launch_logits_gemm(X, W, T, h, E, logits, splits, s);
    if (e != hipSuccess) return e;
    return topk(splits, bias);
  }
  // token blocks of 16 (32 above 1024 tokens), expert slices sized so that
  // a batch launches a few hundred workgroups, K split over 8 waves (4 when
  // h is not a multiple of 256)
  const int parts = router_k_parts(h, E);
  const float *kbias = parts == 1 ? bias : nullptr;
#define AFD_ROUTER(TM, EN, NBUF, WAVES)                                                 \
  router_bf16_kernel<TM, EN, NBUF, WAVES>                                              \
      <<<dim3((E + EN - 1) / EN, (T + TM - 1) / TM, parts), WAVES * 64, 0, s>>>(X, W, kbias, T, h, \
                                                                           E, logits)
  // each wave's K slice must be whole 32-element chunks: 8 waves need
  // h % 256 == 0, 4 waves h % 128 == 0 (always true here)
  const bool k8 = h % 256 == 0;
  if (E > 256) {
    if (k8) AFD_ROUTER(16, 64, 4, 8);
    else AFD_ROUTER(16, 64, 4, 4);
  } else if (T > 1024) {
    if (k8) AFD_ROUTER(32, 64, 4, 8);
    else AFD_ROUTER(32, 64, 4, 4);
  } else if (E <= 64 || T <= 256) {
    if (k8) AFD_ROUTER(16, 16, 8, 8);
    else AFD_ROUTER(16, 16, 8, 4);
  } else {
    if (k8) AFD_ROUTER(16, 32, 6, 8);
    else AFD_ROUTER(16, 32, 6, 4);
  }
#undef AFD_ROUTER
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return parts == 1 ? topk(1, nullptr) : topk(parts, bias);
}

int64_t router_logit_floats(int T, int h, int E) {
  if (T <= kTiledRouterT) return static_cast<int64_t>(router_k_parts(h, E)) * T * E;
  // tiled path, t tokens: splits <= 16, and either splits = 1 or
  // splits x row tiles <= 256 with t <= 256 x row tiles, so the planes hold
  // splits x t <= max(t, min(16 t, 65536)) rows
  const int64_t rows16 = 16LL * T < 65536 ? 16LL * T : 65536;
  return (T > rows16 ? T : rows16) * static_cast<int64_t>(E);
}

}  // namespace afd
