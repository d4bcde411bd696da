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

#define AFD_FFN_ABI_VERSION 1u

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

/* Layer configuration (host struct, copied by create()).
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
} afd_ffn_config;

/* Weight pointers (device, borrowed).  Element types by mode:
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
 * results of the same call (any field may be NULL):
 *   topk_ids [T, k] int32   selected experts, slot order = logit descending,
 *                           index ascending
 *   topk_w   [T, k] fp32    renormalised routing weights
 *   counts   [E] int32      rows per expert
 *   offsets  [E+1] int32    exclusive scan of counts
 *   perm     [T*k] int32    token of each dispatched row (expert-contiguous,
 *                           tokens ascending inside an expert)
 *   slot_row [T, k] int32   dispatched row of each (token, slot)
 *   x_q [T, h] uint8, x_s [T, h/128] fp32   W8A8 only: quantised input    */
typedef struct {
  int32_t *topk_ids;
  float *topk_w;
  int32_t *counts;
  int32_t *offsets;
  int32_t *perm;
  int32_t *slot_row;
  uint8_t *x_q;
  float *x_s;
} afd_ffn_trace;

/* Create a layer handle: validates cfg and w, allocates the per-handle
 * workspace for max_tokens tokens (hipMalloc, on the current device).
 * One handle runs one forward at a time; use one handle per micro-batch
 * stream (handles may share the same weights).                           */
int afd_ffn_create(const afd_ffn_config *cfg, const afd_ffn_weights *w,
                   afd_ffn_handle **out);

/* out[T, h] = MoE-FFN(hidden[T, h]).  hidden/out: fp32 in F32 mode, bf16
 * otherwise, 16-byte aligned; they must not overlap.  0 <= T <= max_tokens
 * (T = 0 is a no-op).  Asynchronous on `stream`; the handle's workspace is in use until
 * the enqueued work completes.                                            */
int afd_ffn_forward(afd_ffn_handle *h, const void *hidden, void *out,
                    int64_t T, afd_stream_t stream);

/* forward() plus copies of intermediates into `trace` (see afd_ffn_trace). */
int afd_ffn_forward_traced(afd_ffn_handle *h, const void *hidden, void *out,
                           int64_t T, afd_stream_t stream,
                           const afd_ffn_trace *trace);

/* Free the workspace and the handle (waits for the device to finish work
 * that uses it).  NULL is ignored.                                        */
void afd_ffn_destroy(afd_ffn_handle *h);

/* FP8 E4M3 activation quantiser: one scale per row per 128 columns.
 * x [rows, cols] bf16 -> q [rows, cols] E4M3 bytes, s [rows, cols/128] fp32,
 * s = fl32(amax/448) (1 if that is 0), q = RNE-saturating E4M3 of
 * fl32(x/s).  cols % 128 == 0; x and q 16-byte aligned, s 4-byte.       */
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

/* FP8 E4M3 weight quantiser: one scale per 128x128 block, same rounding.
 * w [rows, cols] bf16 -> q [rows, cols], s [rows/128, cols/128].
 * rows % 128 == 0, cols % 128 == 0.  A stack [E, N, K] is rows = E*N.
 * w and q 16-byte aligned, s 4-byte.                                      */
int afd_quant_fp8_128x128(const void *w, int64_t rows, int64_t cols,
                          uint8_t *q, float *s, afd_stream_t stream);

/* Kernel-level timing: with stage_mask != 0, subsequent forwards record HIP
 * events (on the forward's stream) around the launches of the selected
 * stages; afd_ffn_profile_read() waits for them and returns the summed
 * milliseconds and launch counts per stage, then resets.  Stage bits:     */
#define AFD_STAGE_ROUTER   0
#define AFD_STAGE_DISPATCH 1
#define AFD_STAGE_QUANT    2
#define AFD_STAGE_GATE_UP  3
#define AFD_STAGE_DOWN     4
#define AFD_STAGE_COMBINE  5
#define AFD_STAGE_COUNT    6
int afd_ffn_profile_enable(afd_ffn_handle *h, uint32_t stage_mask);
int afd_ffn_profile_read(afd_ffn_handle *h, double *ms /*[AFD_STAGE_COUNT]*/,
                         int64_t *launches /*[AFD_STAGE_COUNT]*/);

/* Thread-local description of the last error returned on this thread.    */
const char *afd_ffn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AFD_FFN_H */
