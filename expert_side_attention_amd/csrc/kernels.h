// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afd {

// One GEMM work tile: `rows` (<= BM) consecutive dispatched rows starting at
// `row0`, all belonging to `group` (< E: routed expert, >= E: shared expert
// group - E).  Built on the device by the dispatch kernel.
struct Tile {
  int32_t group;
  int32_t row0;
  int32_t rows;
  int32_t pad;
};

constexpr int kMaxExperts = 512;
// Bytes of the per-device scratch array of the allocation-free forward.
constexpr size_t kStaticScratchBytes = size_t{128} << 20;
// Device address of this device's scratch array (looked up on the first
// call per device; allocates nothing).
hipError_t static_scratch(void **ptr);
constexpr int kMaxLogitSplits = 16;
constexpr int kMaxShared = 8;

// Router GEMM + softmax + top-k + renormalisation.
// f32: x, wr are fp32; else bf16.  bias may be null.  bf16 path scratch:
// logits, router_logit_floats(T, h, E) floats.  logits_out (may be null)
// receives the [T, E] logits as ranked.
int64_t router_logit_floats(int T, int h, int E);
hipError_t launch_router(bool f32, const void *x, const void *wr,
                         const float *bias, int T, int h, int E, int k,
                         float *logits, int32_t *ids, float *w, float *logits_out,
                         hipStream_t s);

// Row-tile lists of a forward: small tiles (bm_small rows) and, if
// bm_big > 0, big tiles (bm_big rows) for groups of at least big_min rows.
struct TilePlan {
  int bm_small;
  int bm_big;
  int big_min;
};

// Histogram, scan and stable scatter of the (token, slot) pairs, and the
// two GEMM tile lists (routed experts, then the S shared groups).  Also
// zeroes `counters[0..ncounters)` (the GEMMs' work counters and, for the
// single launch of both weight-streaming GEMMs, the tile counters).
// block_scratch: 2 * dispatch_blocks(T) * E int32 (used when T > 1024).
int dispatch_blocks(int T);
hipError_t launch_dispatch(const int32_t *ids, int T, int k, int E, int S,
                           const TilePlan &tp, int32_t *counts, int32_t *offsets,
                           int32_t *perm, int32_t *slot_row, Tile *tiles_s,
                           int32_t *num_s, Tile *tiles_b, int32_t *num_b,
                           int32_t *counters, int ncounters, int32_t *block_scratch,
                           hipStream_t s);

hipError_t launch_quant_1x128(const uint16_t *x, int64_t rows, int64_t cols,
                              uint8_t *q, float *sc, hipStream_t s);
// fp32 rows with pitches (elements / bytes / floats) for x, q and scales.
hipError_t launch_quant_1x128_f32(const float *x, int64_t rows, int64_t cols, int64_t pitch,
                                  uint8_t *q, int64_t qpitch, float *sc, int64_t spitch,
                                  hipStream_t s);
hipError_t launch_quant_128x128(const uint16_t *w, int64_t rows,
                                int64_t cols, uint8_t *q, float *sc,
                                hipStream_t s);

enum class GemmKind { GateUp = 0, Down = 1 };

// Grouped GEMM over the tile list.  Element type: 0 f32, 1 bf16, 2 fp8.
struct GemmArgs {
  // A operand: rows of `A` (row pitch a_pitch bytes).  For GateUp the row of
  // a routed dispatched row r is perm[r], of a shared row it is the token;
  // for Down it is r itself.
  const uint8_t *A;
  int64_t a_pitch;
  const int32_t *perm;
  const float *a_scale;  // fp8: [rows of A, a_scale_pitch]
  int a_scale_pitch;
  int Tk, T;             // routed rows, tokens
  // B operand (weights [N, K] per group).  b0 = gate (GateUp) or down;
  // b1 = up (GateUp only).  Shared experts use sb0 / sb1.
  const uint8_t *b0, *b1, *sb0, *sb1;
  const float *bs0, *bs1, *sbs0, *sbs1;  // fp8 block scales
  int N, K, Ns, Ks;      // routed and shared dims
  int E;
  const Tile *tiles;
  const int32_t *num_tiles;
  int32_t *work_counter;  // persistent kernels: next work item (starts at 0)
  int tiles_ub;          // upper bound of the tile count (grid sizing)
  // C: output rows indexed by dispatched row, pitch c_pitch bytes.
  uint8_t *C;
  int64_t c_pitch;
  float *c_scale;        // fp8 GateUp: [R, c_scale_pitch]
  int c_scale_pitch;
  int64_t c_plane;       // router logits GEMM: floats between split-K planes
};

// GEMM plan of a forward: the tile lists and the kernel family that runs
// each (big tiles always go to the compute-bound prefill kernel).
enum class GemmKernel { Tiled = 0, Stream = 1, Prefill = 2 };
struct GemmPlan {
  TilePlan tiles;
  GemmKernel small_kernel;
};
GemmPlan gemm_plan(int elem, int T, int k, int E);

// LDS-tiled kernel (all element types).
hipError_t launch_gemm(GemmKind kind, int elem, int bm, const GemmArgs &a,
                       hipStream_t s);
// Weight-streaming persistent kernel (bf16, fp8; bm 64 or 128).  W8A8
// gate/up writes E4M3 z and 1x128 scales itself when this returns true,
// else fp32 z for the standalone quantiser.
bool stream_gate_up_writes_fp8(int elem, int bm);
hipError_t launch_gemm_stream(GemmKind kind, int elem, int bm, const GemmArgs &a,
                              hipStream_t s);
// Both weight-streaming GEMMs (gate/up, then down) of a bf16 forward with
// 64-row tiles in one persistent launch.  gu and dn use the same tile list;
// sync holds 1 + one int per tile of that list, zeroed before the launch
// (the dispatch kernel does it): sync[0] ends as the number of down items
// that gave up waiting for their tile (0 unless defective), sync[1 + t] is
// tile t's counter.  stream_ffn_supported tells whether a layer's shapes
// allow it.
bool stream_ffn_supported(int elem, int bm, int hidden, int inter, int shared_inter);
hipError_t launch_ffn_stream(const GemmArgs &gu, const GemmArgs &dn, int32_t *sync,
                             hipStream_t s);
// Compute-bound kernel (bf16, bm 256).
hipError_t launch_gemm_prefill(GemmKind kind, const GemmArgs &a, hipStream_t s);
// Router logits of long batches on the compute-bound kernel: partials[p][t][e]
// = sum over the p-th of `splits` equal K ranges of x[t] . wr[e] (fp32);
// logits_splits picks `splits` (at most kMaxLogitSplits) for a shape.
int logits_splits(int T, int h, int E);
hipError_t launch_logits_gemm(const uint16_t *x, const uint16_t *wr, int T, int h, int E,
                              float *partials, int splits, hipStream_t s);

// Single-launch forward of tiny fp32 / bf16 layers (cooperative grid with
// one grid-wide barrier).  Limits: T <= kFusedMaxT, k <= kFusedMaxK; I and
// I_s multiples of 128; z holds T k + S T rows of zpitch elements of the
// layer's type.  ids ... num_big receive the routing and dispatch (as the
// multi-kernel forward's workspace holds them).
constexpr int kFusedMaxT = 16;
constexpr int kFusedMaxK = 16;
constexpr int kFusedMaxGrid = 256;
constexpr int64_t kFusedMaxWeightBytes = int64_t{64} << 20;
struct FusedArgs {
  const uint8_t *x, *wr;
  const float *bias;
  const uint8_t *gate, *up, *down, *sgate, *sup, *sdown;
  int T, h, E, k, I, S, Is, zpitch;
  float *logits;
  int32_t *ids;
  float *w;
  int32_t *counts, *offsets, *perm, *slot_row, *num_tiles, *num_big;
  int32_t *sync_timeouts;  // zeroed (the traced count of the GEMMs' single launch)
  uint8_t *z;
  void *out;
};
bool fused_supported(int device);
hipError_t launch_fused_small(bool f32, const FusedArgs &a, hipStream_t s);

// out[t] = sum_j w[t,j] Y[slot_row[t,j]] + sum_s Y[Tk + s*T + t].
hipError_t launch_combine(bool f32, const uint8_t *Y, const int32_t *slot_row,
                          const float *w, int T, int k, int S, int h,
                          void *out, hipStream_t s);

}  // namespace afd
