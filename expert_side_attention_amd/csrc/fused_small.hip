// The whole layer in one launch for tiny layers and small batches: router,
// top-k and renormalised weights, dispatch, gate/up with SiLU * up, down,
// shared experts and the weighted combine, in a single cooperative grid with
// one grid-wide barrier.  The sync connectors of the AFD plugin run decode
// as one captured graph (vLLM AFD plugin page, "Connector 與後端支援矩陣");
// for layers whose weights are a few MB the separate launches of the
// multi-kernel forward, not the bytes, set the time, and this path replaces
// them with one.
//
// Phases:
//  1. every workgroup, redundantly: the router logits of all T tokens on
//     MFMAs (x and W_r are small and stay in L2), the top-k of every token
//     (ties to the lower expert index), the renormalised weights, the
//     per-expert counts and offsets and the stable dispatch (rows of an
//     expert in ascending token order), all in LDS.  Workgroup 0 also
//     stores them for inspection.
//  2. work items (group, 64-column slice of I): z = silu(x G^T) * (x U^T) on
//     MFMAs for the group's rows, stored to the z buffer.      -- grid barrier
//  3. each workgroup owns blocks of 16 output columns: y = z D^T of every
//     row for those columns (every element of D read once), kept in LDS,
//     then out[t] = sum_j w[t,j] y[row(t,j)] + shared rows, in a fixed
//     order, so results are bitwise repeatable.
// bf16 layers round z to bf16 before the down product, as the multi-kernel
// path does; y stays fp32 until the output.  Loads are issued in batches of
// four 128-byte K chunks before their MFMAs.
#include <hip/hip_cooperative_groups.h>

#include <atomic>

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace afd {
namespace {

namespace cg = cooperative_groups;

constexpr int kThreads = 256;
constexpr int kSlice = 64;  // z columns per work item
constexpr int kMaxRows = kFusedMaxT * (kFusedMaxK + kMaxShared);
// LDS shared by the logits (phase 1) and the y block (phase 3)
constexpr int kUnion = kFusedMaxT * kMaxExperts > kMaxRows * 16 ? kFusedMaxT * kMaxExperts
                                                                : kMaxRows * 16;

template <Elem EL>
struct ES;
template <>
struct ES<Elem::F32> {
  static constexpr int bytes = 4;
};
template <>
struct ES<Elem::BF16> {
  static constexpr int bytes = 2;
};

template <Elem EL>
__global__ __launch_bounds__(kThreads) void fused_small_kernel(const FusedArgs a) {
  constexpr int ESZ = ES<EL>::bytes;
  constexpr bool BF = EL == Elem::BF16;
  cg::grid_group grid = cg::this_grid();

  __shared__ int32_t s_ids[kFusedMaxT * kFusedMaxK];
  __shared__ float s_w[kFusedMaxT * kFusedMaxK];
  __shared__ int32_t s_slot[kFusedMaxT * kFusedMaxK];
  __shared__ int32_t s_perm[kFusedMaxT * kFusedMaxK];
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_items[kMaxExperts + kMaxShared + 1];
  __shared__ float s_sel[4][kFusedMaxK];
  __shared__ float s_u[kUnion];  // logits [T][E], later the y block [rows][16]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int T = a.T, h = a.h, E = a.E, k = a.k, S = a.S;
  const int Tk = T * k;
  const int G = static_cast<int>(gridDim.x), wg = static_cast<int>(blockIdx.x);
  const int64_t xrow = static_cast<int64_t>(h) * ESZ;
  const int nckh = static_cast<int>(xrow / 128);

  // ---- 1a. router logits of all tokens, 16 experts per MFMA block
  {
    const int tr = r16 < T ? r16 : 0;  // rows past T repeat token 0
    const uint8_t *xa = a.x + tr * xrow + q * 32;
    for (int eb = wave; eb * 16 < E; eb += 4) {
      const int e = eb * 16 + r16 < E ? eb * 16 + r16 : E - 1;
      const f32x4 acc = mma_rows<EL>(xa, a.wr + e * xrow + q * 32, nckh, f32x4{0, 0, 0, 0});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * q + i, ee = eb * 16 + r16;
        if (t < T && ee < E) {
          const float v = acc[i] + (a.bias ? a.bias[ee] : 0.0f);
          s_u[t * E + ee] = v;
          if (wg == 0) a.logits[static_cast<int64_t>(t) * E + ee] = v;
        }
      }
    }
  }
  __syncthreads();

  // ---- 1b. top-k, weights and dispatch of every token
  for (int t = wave; t < T; t += 4) {
    const float *row = s_u + t * E;
    unsigned long long key[kMaxExperts / 64];
#pragma unroll
    for (int c = 0; c < kMaxExperts / 64; ++c) {
      const int e = lane + 64 * c;
      key[c] = e < E ? topk_key(row[e], e) : 0ull;
    }
    for (int j = 0; j < k; ++j) {
      unsigned long long best = 0;
#pragma unroll
      for (int c = 0; c < kMaxExperts / 64; ++c) best = key[c] > best ? key[c] : best;
      best = wave_max_u64(best);
      const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
#pragma unroll
      for (int c = 0; c < kMaxExperts / 64; ++c)
        if (lane + 64 * c == e) key[c] = 0;
      if (lane == 0) {
        s_ids[t * k + j] = e;
        s_sel[wave][j] = topk_key_value(best);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    // slot 0 holds the largest logit of all E experts
    const float m = s_sel[wave][0];
    const float p = lane < k ? expf(s_sel[wave][lane] - m) : 0.0f;
    const float den = wave_sum(p);
    if (lane < k) s_w[t * k + lane] = p / den;
    __builtin_amdgcn_wave_barrier();
  }
  for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < Tk; i += kThreads) atomicAdd(&s_cnt[s_ids[i]], 1);
  __syncthreads();
  if (tid == 0) {
    // offsets of the experts' rows, and the work items: slices of every
    // expert that received rows (in index order), then of the shared experts
    int run = 0, items = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = run;
      run += s_cnt[e];
      s_items[e] = items;
      items += s_cnt[e] > 0 ? a.I / kSlice : 0;
    }
    s_off[E] = run;
    for (int j = 0; j < S; ++j) {
      s_items[E + j] = items;
      items += a.Is / kSlice;
    }
    s_items[E + S] = items;
  }
  __syncthreads();
  // stable scatter: the rank of token t among the tokens of expert e is the
  // number of earlier tokens that chose e
  for (int i = tid; i < Tk; i += kThreads) {
    const int t = i / k, e = s_ids[i];
    int rank = 0;
    for (int u = 0; u < t * k; ++u) rank += s_ids[u] == e;
    const int r = s_off[e] + rank;
    s_slot[i] = r;
    s_perm[r] = t;
  }
  __syncthreads();
  if (wg == 0) {
    for (int i = tid; i < Tk; i += kThreads) {
      a.ids[i] = s_ids[i];
      a.w[i] = s_w[i];
      a.slot_row[i] = s_slot[i];
      a.perm[i] = s_perm[i];
    }
    for (int e = tid; e <= E; e += kThreads) {
      if (e < E) a.counts[e] = s_cnt[e];
      a.offsets[e] = s_off[e];
    }
    if (tid == 0) {
      a.num_tiles[0] = 0;
      a.num_big[0] = 0;
      a.sync_timeouts[0] = 0;
    }
  }

  // ---- 2. (group, slice) items: z of the group's rows for 64 columns,
  // 16 columns per wave
  const int n_items = s_items[E + S];
  const int64_t zrow = static_cast<int64_t>(a.zpitch) * ESZ;
  for (int it = wg; it < n_items; it += G) {
    // the group whose item range holds `it`: s_items[lo] <= it < s_items[hi]
    int lo = 0, hi = E + S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_items[mid] <= it) lo = mid;
      else hi = mid;
    }
    const bool shared = lo >= E;
    const int gi = shared ? lo - E : lo;
    const int sig = it - s_items[lo];
    const int N = shared ? a.Is : a.I;
    const int nrows = shared ? T : s_cnt[lo];
    const int row0 = shared ? Tk + gi * T : s_off[lo];
    const int64_t gmat = static_cast<int64_t>(N) * xrow;
    const uint8_t *Gm = (shared ? a.sgate : a.gate) + gi * gmat;
    const uint8_t *Um = (shared ? a.sup : a.up) + gi * gmat;
    const int col = sig * kSlice + wave * 16 + r16;
    for (int b0 = 0; b0 < nrows; b0 += 16) {
      const int ri = b0 + r16 < nrows ? b0 + r16 : b0;
      const int tok = shared ? ri : s_perm[row0 + ri];
      const uint8_t *xa = a.x + tok * xrow + q * 32;
      const f32x4 ag = mma_rows<EL>(xa, Gm + col * xrow + q * 32, nckh, f32x4{0, 0, 0, 0});
      const f32x4 au = mma_rows<EL>(xa, Um + col * xrow + q * 32, nckh, f32x4{0, 0, 0, 0});
      // z (rows 4 q + i, column col) in the element type
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = b0 + 4 * q + i;
        if (rr < nrows) {
          const float gv = ag[i];
          const float z = gv / (1.0f + expf(-gv)) * au[i];
          uint8_t *dst = a.z + (row0 + rr) * zrow + col * ESZ;
          if constexpr (BF)
            *reinterpret_cast<uint16_t *>(dst) = f32_to_bf16(z);
          else
            *reinterpret_cast<float *>(dst) = z;
        }
      }
    }
  }
  grid.sync();

  // ---- 3. down and combine, 16 output columns per block
  const int ngroups = E + S;
  for (int nb = wg; nb < h / 16; nb += G) {
    const int n = nb * 16 + r16;
    // y of every row for these columns: groups dealt to the waves
    for (int g0 = wave; g0 < ngroups; g0 += 4) {
      const bool shared = g0 >= E;
      const int gi = shared ? g0 - E : g0;
      const int nrows = shared ? T : s_cnt[g0];
      if (nrows == 0) continue;
      const int N = shared ? a.Is : a.I;
      const int row0 = shared ? Tk + gi * T : s_off[g0];
      const uint8_t *Dn = (shared ? a.sdown : a.down) +
                          gi * (static_cast<int64_t>(h) * N * ESZ) +
                          static_cast<int64_t>(n) * N * ESZ + q * 32;
      for (int b0 = 0; b0 < nrows; b0 += 16) {
        const int ri = b0 + r16 < nrows ? b0 + r16 : b0;
        const f32x4 ay = mma_rows<EL>(a.z + (row0 + ri) * zrow + q * 32, Dn,
                                      N * ESZ / 128, f32x4{0, 0, 0, 0});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = b0 + 4 * q + i;
          if (rr < nrows) s_u[(row0 + rr) * 16 + r16] = ay[i];
        }
      }
    }
    __syncthreads();
    // out[t][n]: routed slots in order j = 0..k-1, then the shared experts
    for (int p = tid; p < T * 16; p += kThreads) {
      const int t = p >> 4, c = p & 15;
      float acc = 0.0f;
      for (int j = 0; j < k; ++j)
        acc = fmaf(s_w[t * k + j], s_u[s_slot[t * k + j] * 16 + c], acc);
      for (int j = 0; j < S; ++j) acc += s_u[(Tk + j * T + t) * 16 + c];
      const int64_t o = static_cast<int64_t>(t) * h + nb * 16 + c;
      if constexpr (BF)
        reinterpret_cast<uint16_t *>(a.out)[o] = f32_to_bf16(acc);
      else
        reinterpret_cast<float *>(a.out)[o] = acc;
    }
    __syncthreads();
  }
}

template <Elem EL>
hipError_t launch_fused_t(const FusedArgs &a, hipStream_t s) {
  // co-resident workgroups per device, once per device
  constexpr int kMaxDevices = 64;
  static std::atomic<int> resident[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int g = resident[dev].load(std::memory_order_acquire);
  if (g == 0) {
    int ncu = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(fused_small_kernel<EL>), kThreads, 0);
    if (e != hipSuccess) return e;
    g = ncu * per_cu;
    if (g < 1) return hipErrorLaunchOutOfResources;
    resident[dev].store(g, std::memory_order_release);
  }
  // no more workgroups than the larger phase has items: every extra one only
  // adds to the cost of the grid barrier
  const int ek = a.T * a.k < a.E ? a.T * a.k : a.E;
  int want = (ek * a.I + a.S * a.Is) / kSlice;
  if (want < a.h / 16) want = a.h / 16;
  int grid = g < kFusedMaxGrid ? g : kFusedMaxGrid;
  if (grid > want) grid = want;
  void *args[] = {const_cast<FusedArgs *>(&a)};
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(fused_small_kernel<EL>),
                                 dim3(grid), dim3(kThreads), args, 0, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

bool fused_supported(int device) {
  int coop = 0;
  return hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device) ==
             hipSuccess &&
         coop != 0;
}

hipError_t launch_fused_small(bool f32, const FusedArgs &a, hipStream_t s) {
  return f32 ? launch_fused_t<Elem::F32>(a, s) : launch_fused_t<Elem::BF16>(a, s);
}

}  // namespace afd
