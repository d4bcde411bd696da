/*
 * afd_ffn.h -- C ABI of the MoE FFN-service layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The library computes the FFN side of Attention-FFN Disaggregation: the
 * FFN service receives the hidden states of one micro-batch and returns the
 * MoE layer's output for them (vLLM AFD plugin page, "系統架構 / 2. FFN
 * Service").  One call of afd_ffn_forward runs, on the caller's HIP stream:
 *
 *   router GEMM + softmax + top-k (ties to the lower expert index) +
 *     renormalisation over the selected k     ("routing computation", plugin
 *                                              page, "Attention-FFN 解耦的原理")
 *   dispatch: per-expert histogram, exclusive scan, stable scatter of the
 *     (token, slot) pairs into expert-contiguous rows ("dispatch", A/F 分离
 *                                              page, "机制")
 *   [W8A8] per-token-per-128-channel FP8 E4M3 quantisation of the input
 *                                             (W8A8 precision of the plugin
 *                                              page's "效能基準測試")
 *   grouped gate/up GEMM with a fused SiLU(gate) * up epilogue, then the
 *     grouped down GEMM, over the routed experts and the always-on shared
 *     experts                                 (experts are large matrix
 *                                              products, A/F 分离 page,
 *                                              "为什么要拆")
 *     (bf16 batches of the decode regime run both GEMMs as one launch, in
 *     which each down item waits for the gate/up items of its row tile;
 *     the config's split_gemms = 1 asks for one launch per GEMM instead)
 *   deterministic weighted combine back into token order ("combine", A/F
 *                                              分离 page, "机制")
 *
 * Conventions for every entry point:
 *  - All tensors are dense, row-major, and live in device memory of the
 *    current HIP device unless stated otherwise.  Weights use the [out, in]
 *    layout, so every product is X W^T with both operands contiguous in K.
 *  - Entry points validate their arguments before anything is enqueued; on
 *    error nothing is enqueued, a non-zero afd_status is returned and
 *    afd_ffn_last_error() describes it.  There is no silent fallback.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *    and the call returns without waiting.  afd_ffn_forward does not
 *    allocate, does not synchronise and does not read device memory on the
 *    host, so it may be captured into a HIP graph.
 *  - Pointers passed to create() are borrowed: they must stay valid and
 *    unmodified until destroy().  The library never frees them.
 */
#ifndef AFD_FFN_H
#define AFD_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AFD_FFN_ABI_VERSION 3u

typedef struct afd_ffn_handle afd_ffn_handle;
typedef void *afd_stream_t; /* a hipStream_t */

typedef enum {
  AFD_OK = 0,
  AFD_ERR_INVALID_ARG = 1,   /* NULL, aliasing, misalignment, bad size,
                                bad config                                  */
  AFD_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels handle   */
  AFD_ERR_CAPACITY = 3,      /* T > max_tokens given at create()            */
  AFD_ERR_OUT_OF_MEMORY = 4, /* workspace allocation failed in create()     */
  AFD_ERR_HIP = 5            /* a HIP runtime call or launch failed         */
} afd_status;

typedef enum {
  AFD_MODE_F32 = 0,       /* fp32 activations, weights and outputs          */
  AFD_MODE_BF16 = 1,      /* bf16 activations/weights, fp32 accumulation    */
  AFD_MODE_W8A8_E4M3 = 2  /* E4M3 weights (128x128 block scales), E4M3
                             activations (1x128 scales), bf16 in/out,
                             bf16 router                                    */
} afd_mode;

/* Layer configuration (host struct, copied by create()).  One handle holds
 * one layer; the FFN service is told per call which layer and micro-batch
 * ("ubatch") it serves (vLLM AFD plugin page, "系統架構 / 1. Attention
 * Service": data-parallel, ubatch, layer and graph state go to the FFN side),
 * which here means: one handle per layer and per micro-batch stream.
 * Limits: 1 <= top_k <= num_experts <= 512; hidden, inter, shared_inter are
 * multiples of 128 (all modes); 0 <= num_shared <= 8 (shared_inter > 0 when
 * num_shared > 0); 1 <= max_tokens <= 1<<20 with max_tokens * top_k < 2^31. */
typedef struct {
  uint32_t abi_version;   /* must be AFD_FFN_ABI_VERSION                     */
  uint32_t mode;          /* afd_mode                                        */
  int32_t hidden;         /* h                                               */
  int32_t num_experts;    /* E, routed experts                               */
  int32_t top_k;          /* k                                               */
  int32_t inter;          /* I, routed-expert intermediate size              */
  int32_t num_shared;     /* S, always-on shared experts (weight 1)          */
  int32_t shared_inter;   /* I_s                                             */
  int32_t max_tokens;     /* largest T passed to forward(); sizes workspace  */
  int32_t has_router_bias;/* 1: router_b is added to the logits              */
  int32_t single_launch;  /* 1: run forwards of at most 16 tokens of a tiny
                             fp32 / bf16 layer (top_k <= 16, expert weights
                             <= 64 MiB) as one cooperative launch (outside
                             graph capture); 0: the kernel sequence          */
  int32_t split_gemms;    /* 0: a bf16 layer in the decode regime (at most
                             48 routed rows per expert on average, hidden a
                             multiple of 256) runs its gate/up and down
                             weight-streaming GEMMs as one launch, the down
                             work of a row tile starting as soon as that
                             tile's z is complete (same results; best for a
                             GPU the FFN service has to itself); 1: always
                             one launch per GEMM (better when other streams
                             share the GPU, e.g. attention on the same chip) */
} afd_ffn_config;

/* Weight pointers (device, borrowed).  The experts are SwiGLU matrix
 * products (A/F 分离 page, "为什么要拆"), W8A8 is the benchmark precision
 * (vLLM AFD plugin page, "效能基準測試").  Element types by mode:
 *   router_w [E, h]           F32: fp32; BF16 and W8A8: bf16
 *   router_b [E]              fp32, only read when has_router_bias = 1
 *   gate_w, up_w [E, I, h]    F32: fp32; BF16: bf16; W8A8: E4M3 bytes
 *   down_w [E, h, I]          as gate_w
 *   gate_s, up_s [E, I/128, h/128], down_s [E, h/128, I/128]
 *                             fp32 block scales, W8A8 only (else ignored)
 *   sh_* : the same for the S shared experts with I_s in place of I.
 * Weight matrices must be 16-byte aligned, router_b and the scales 4-byte
 * aligned (create() returns AFD_ERR_INVALID_ARG otherwise).               */
typedef struct {
  const void *router_w;
  const float *router_b;
  const void *gate_w, *up_w, *down_w;
  const float *gate_s, *up_s, *down_s;
  const void *sh_gate_w, *sh_up_w, *sh_down_w;
  const float *sh_gate_s, *sh_up_s, *sh_down_s;
} afd_ffn_weights;

/* Optional device buffers that forward_traced() fills with intermediate
 * results of the same call (any field may be NULL).  The routing step (vLLM
 * AFD plugin page, "Attention-FFN 解耦的原理": routing computation) and the
 * dispatch / combine of the expert path (A/F 分离 page, "机制"):
 *   topk_ids [T, k] int32   selected experts, slot order = logit descending,
 *                           index ascending
 *   topk_w   [T, k] fp32    renormalised routing weights
 *   counts   [E] int32      rows per expert
 *   offsets  [E+1] int32    exclusive scan of counts
 *   perm     [T*k] int32    token of each dispatched row (expert-contiguous,
 *                           tokens ascending inside an expert)
 *   slot_row [T, k] int32   dispatched row of each (token, slot)
 *   x_q [T, h] uint8, x_s [T, h/128] fp32   W8A8 only: quantised input
 *   logits   [T, E] fp32    the router logits the top-k ranked (fp32
 *                           accumulation of the products, plus the bias)
 *   z_q [R, Z] uint8, z_s [R, Z/128] fp32   W8A8 only: the E4M3 SwiGLU
 *                           output fed to the down product and its 1x128
 *                           scales, R = T*k + S*T dispatched rows (routed
 *                           rows in expert order, then row T*k + s*T + t for
 *                           shared expert s on token t), Z = max(I, I_s);
 *                           shared rows hold I_s valid columns
 *   num_tiles [2] int32     row tiles of the expert GEMMs: weight-streaming
 *                           tiles, then compute-bound 256-row tiles
 *   sync_timeouts [1] int32 down items of the single launch of both
 *                           weight-streaming GEMMs (config split_gemms = 0)
 *                           that stopped waiting for their row tile's z
 *                           after a bound (about a quarter of a second):
 *                           0 unless the library is defective, in which case
 *                           the call's output is not valid; 0 for other
 *                           launch structures                               */
typedef struct {
  int32_t *topk_ids;
  float *topk_w;
  int32_t *counts;
  int32_t *offsets;
  int32_t *perm;
  int32_t *slot_row;
  uint8_t *x_q;
  float *x_s;
  float *logits;
  uint8_t *z_q;
  float *z_s;
  int32_t *num_tiles;
  int32_t *sync_timeouts;
} afd_ffn_trace;

/* Create a layer handle: validates cfg and w, allocates the per-handle
 * workspace for max_tokens tokens (hipMalloc, on the current device).
 * The configuration is checked up front and misuse is refused at once
 * rather than degraded silently (plugin article "Separar Attention de FFN",
 * "Con qué te vas a tropezar" and "Ejecutarlo en una sola máquina").
 * cfg and w are read during the call only; *out receives the handle (NULL
 * on error), owned by the caller until afd_ffn_destroy().  Errors:
 * AFD_ERR_INVALID_ARG (bad or NULL argument, see the limits above),
 * AFD_ERR_UNSUPPORTED, AFD_ERR_OUT_OF_MEMORY.
 * One handle runs one forward at a time; use one handle per micro-batch
 * stream (handles may share the same weights).                           */
int afd_ffn_create(const afd_ffn_config *cfg, const afd_ffn_weights *w,
                   afd_ffn_handle **out);

/* out[T, h] = MoE-FFN(hidden[T, h]): the FFN service's step on the hidden
 * states it receives, whose result goes back to the attention side (vLLM
 * AFD plugin page, "系統架構 / 2. FFN Service"; capturable into a graph as
 * the sync connectors' decode graphs need: "Connector 與後端支援矩陣").
 * hidden/out: device arrays [T, h], row-major, fp32 in F32 mode, bf16
 * otherwise, 16-byte aligned, owned by the caller; they must not overlap.
 * 0 <= T <= max_tokens (T = 0 is a no-op).  Errors: AFD_ERR_INVALID_ARG
 * (NULL, misaligned, overlapping, T < 0, wrong current device),
 * AFD_ERR_CAPACITY (T > max_tokens), AFD_ERR_HIP (launch failure).
 * Asynchronous on `stream`; the handle's workspace is in use until the
 * enqueued work completes.                                                */
int afd_ffn_forward(afd_ffn_handle *h, const void *hidden, void *out,
                    int64_t T, afd_stream_t stream);

/* forward() plus the intermediates of the same call written to `trace`
 * (see afd_ffn_trace; the routing, dispatch and W8A8 steps named there).
 * Trace buffers are device memory owned by the caller, sized for this T.
 * Errors: those of forward(), and AFD_ERR_INVALID_ARG for a NULL trace or
 * for x_q / x_s / z_q / z_s outside W8A8 mode.                            */
int afd_ffn_forward_traced(afd_ffn_handle *h, const void *hidden, void *out,
                           int64_t T, afd_stream_t stream,
                           const afd_ffn_trace *trace);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward as afd_ffn_forward, same kernels and same results for the same T,
 * without a handle.  Its workspace is a fixed scratch array of
 * AFD_FFN_STATIC_SCRATCH_BYTES that the library holds on each device it
 * runs on, from the first call on that device until the process ends; the
 * call allocates nothing (the first call on a device only looks up the
 * array's address).  cfg and w as for create(), read during the call only;
 * hidden/out as for forward(); 0 <= T <= cfg->max_tokens.  Errors: those of
 * create() and forward(), and AFD_ERR_CAPACITY when the workspace of T
 * tokens exceeds the scratch (e.g. 256 tokens of a 4096-wide, 64-expert,
 * top-8 bf16 layer need 27 MB; 512 tokens of a 7168-wide, 256-expert one
 * 86 MB).  Every call on one device shares that device's array, which keeps
 * the last call's contents: calls that overlap in time on one device (two
 * streams, two threads) race and give wrong results.  Serialise them.      */
#define AFD_FFN_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int afd_ffn_forward_static(const afd_ffn_config *cfg, const afd_ffn_weights *w,
                           const void *hidden, void *out, int64_t T,
                           afd_stream_t stream);

/* Free the workspace and the handle (waits for the device to finish work
 * that uses it).  The counterpart of create(): the FFN service's state for
 * one layer (vLLM AFD plugin page, "系統架構 / 2. FFN Service").  The
 * borrowed weights are not touched.  NULL is ignored.                     */
void afd_ffn_destroy(afd_ffn_handle *h);

/* FP8 E4M3 activation quantiser of the W8A8 layer (vLLM AFD plugin page,
 * "效能基準測試": W8A8): one scale per row per 128 columns.
 * x [rows, cols] bf16 -> q [rows, cols] E4M3 bytes, s [rows, cols/128] fp32,
 * s = fl32(amax/448) (1 if that is 0), q = RNE-saturating E4M3 of
 * fl32(x/s).  Device arrays owned by the caller, row-major, contiguous;
 * x and q 16-byte aligned, s 4-byte.  Errors: NULL or misaligned pointer,
 * rows < 0 or cols not a positive multiple of 128 -> AFD_ERR_INVALID_ARG;
 * rows = 0 is a no-op.                                                    */
int afd_quant_fp8_1x128(const void *x, int64_t rows, int64_t cols,
                        uint8_t *q, float *s, afd_stream_t stream);

/* The same quantiser on fp32 input: the W8A8 layer applies it to the
 * SwiGLU output z between the two expert GEMMs (W8A8 is the precision of
 * the vLLM AFD plugin page's "效能基準測試").  x [rows, cols]
 * fp32 device array, row-major, contiguous; q, s as above; all three owned
 * by the caller; x and q 16-byte aligned, s 4-byte.  Errors: NULL or
 * misaligned pointer, or cols not a positive multiple of 128 ->
 * AFD_ERR_INVALID_ARG; rows = 0 is a no-op.                               */
int afd_quant_fp8_1x128_f32(const float *x, int64_t rows, int64_t cols,
                            uint8_t *q, float *s, afd_stream_t stream);

/* FP8 E4M3 weight quantiser of the W8A8 layer (vLLM AFD plugin page,
 * "效能基準測試"): one scale per 128x128 block, same rounding.
 * w [rows, cols] bf16 -> q [rows, cols], s [rows/128, cols/128], device
 * arrays owned by the caller.  rows % 128 == 0, cols % 128 == 0.  A stack
 * [E, N, K] is rows = E*N.  w and q 16-byte aligned, s 4-byte.  Errors:
 * NULL, misaligned or non-multiple-of-128 -> AFD_ERR_INVALID_ARG.         */
int afd_quant_fp8_128x128(const void *w, int64_t rows, int64_t cols,
                          uint8_t *q, float *s, afd_stream_t stream);

/* Kernel-level timing, for finding where the layer's time goes (LLM 推理提速
 * page, "一个在啃带宽，一个在吃算力": the bound of each side is found by
 * profiling).  With stage_mask != 0, subsequent forwards record HIP events
 * (on the forward's stream) around the launches of the selected stages;
 * afd_ffn_profile_read() waits for them and returns the summed milliseconds
 * and launch counts per stage (host arrays of AFD_STAGE_COUNT owned by the
 * caller), then resets.  Errors: NULL handle or arrays, unknown bits ->
 * AFD_ERR_INVALID_ARG; a failed event -> AFD_ERR_HIP.  The compute-bound
 * launches of the gate/up and down stages (256-row tiles) are also timed
 * on their own under AFD_STAGE_GATE_UP_BIG and AFD_STAGE_DOWN_BIG; a forward
 * that runs as one launch (tiny layers, at most 16 tokens) is timed under
 * AFD_STAGE_SINGLE only, and the single launch of both weight-streaming
 * GEMMs (config split_gemms = 0) under AFD_STAGE_FFN (AFD_STAGE_GATE_UP and
 * AFD_STAGE_DOWN then record nothing).  Stage bits:                                                                    */
#define AFD_STAGE_ROUTER   0
#define AFD_STAGE_DISPATCH 1
#define AFD_STAGE_QUANT    2
#define AFD_STAGE_GATE_UP  3
#define AFD_STAGE_DOWN     4
#define AFD_STAGE_COMBINE  5
#define AFD_STAGE_GATE_UP_BIG 6
#define AFD_STAGE_DOWN_BIG 7
#define AFD_STAGE_SINGLE   8  /* the single-launch forward of tiny layers */
#define AFD_STAGE_FFN      9  /* gate/up + down weight streaming, one launch */
#define AFD_STAGE_COUNT    10
int afd_ffn_profile_enable(afd_ffn_handle *h, uint32_t stage_mask);
int afd_ffn_profile_read(afd_ffn_handle *h, double *ms /*[AFD_STAGE_COUNT]*/,
                         int64_t *launches /*[AFD_STAGE_COUNT]*/);

/* Thread-local description of the last error returned on this thread (the
 * message that comes with a refused call: plugin article "Separar Attention
 * de FFN", "Ejecutarlo en una sola máquina").  Owned by the library, valid
 * until the next call on the same thread; "" if none.                     */
const char *afd_ffn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AFD_FFN_H */
