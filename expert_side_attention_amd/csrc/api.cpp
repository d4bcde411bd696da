// C ABI of the MoE FFN-service layer: validation, workspace, and the
// sequence of kernel launches of one forward (router -> dispatch ->
// [quantise] -> gate/up -> down -> combine) on the caller's stream.
//
// The FFN side of Attention-FFN Disaggregation runs this step on the hidden
// states it receives and returns the result (vLLM AFD plugin page, "系統架構
// / 2. FFN Service"); misuse of the FFN side fails at once rather than
// degrading silently (plugin article, "Ejecutarlo en una sola máquina"),
// which is the error policy here: every argument is checked before anything
// is enqueued.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/afd_ffn.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(AFD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
// The kernels move activations, weights and outputs in 16-byte pieces and
// read biases and scales as floats.
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct StageEvents {
  hipEvent_t start, stop;
};

}  // namespace

struct afd_ffn_handle {
  afd_ffn_config cfg;
  afd_ffn_weights w;
  int device;
  int elem;    // 0 f32, 1 bf16, 2 fp8 (GEMM operand type)
  int zpitch;  // Z row length in elements: max(I, I_s)
  int tiles_cap, big_cap;
  void *ws;
  size_t ws_bytes;
  // counters: the two GEMMs' work counters, then the sync words of the
  // single launch of both weight-streaming GEMMs (items that gave up waiting,
  // then one completion counter per small tile)
  int32_t *ids, *counts, *offsets, *perm, *slot_row, *num_tiles, *num_big, *counters;
  int32_t *dispatch_scratch;
  float *topk_w, *logits;
  afd::Tile *tiles, *tiles_big;
  uint8_t *xq;
  float *xs;
  uint8_t *z;
  float *zs;
  float *z32;  // W8A8 with the streaming kernels: fp32 z before quantisation
  uint8_t *y;
  // single-launch path of tiny layers (asked for; k <= 16, expert weights
  // <= 64 MiB)
  bool fused_ok;
  // profiling
  uint32_t prof_mask;
  std::vector<StageEvents> ev_pool;
  std::vector<int> ev_stage;
  size_t ev_used;
};

namespace {

// Upper bound of the small-tile list: every group adds at most one partial
// tile to R / bm full ones.
int64_t tiles_upper_bound(int64_t T, int k, int E, int S, int bm) {
  const int64_t rows = T * k + S * T;
  const int64_t groups = (T * k < E ? T * k : E) + S;
  return rows / bm + groups;
}
// Upper bound of the big-tile list: every big tile holds more than bm / 2 rows.
int64_t big_tiles_upper_bound(int64_t T, int k, int S, int bm) {
  return (T * k + S * T) * 2 / bm + 1;
}

int validate_config(const afd_ffn_config *c) {
  if (!c) return fail(AFD_ERR_INVALID_ARG, "config is NULL");
  if (c->abi_version != AFD_FFN_ABI_VERSION)
    return fail(AFD_ERR_INVALID_ARG, "abi_version %u, library has %u", c->abi_version,
                AFD_FFN_ABI_VERSION);
  if (c->mode > AFD_MODE_W8A8_E4M3) return fail(AFD_ERR_INVALID_ARG, "unknown mode %u", c->mode);
  if (c->num_experts < 1 || c->num_experts > afd::kMaxExperts)
    return fail(c->num_experts < 1 ? AFD_ERR_INVALID_ARG : AFD_ERR_UNSUPPORTED,
                "num_experts %d outside [1, %d]", c->num_experts, afd::kMaxExperts);
  if (c->top_k < 1 || c->top_k > c->num_experts)
    return fail(AFD_ERR_INVALID_ARG, "top_k %d outside [1, num_experts=%d]", c->top_k,
                c->num_experts);
  if (c->hidden < 128 || c->hidden % 128)
    return fail(AFD_ERR_INVALID_ARG, "hidden %d must be a positive multiple of 128", c->hidden);
  if (c->inter < 128 || c->inter % 128)
    return fail(AFD_ERR_INVALID_ARG, "inter %d must be a positive multiple of 128", c->inter);
  if (c->num_shared < 0 || c->num_shared > afd::kMaxShared)
    return fail(AFD_ERR_INVALID_ARG, "num_shared %d outside [0, %d]", c->num_shared,
                afd::kMaxShared);
  if (c->num_shared > 0 && (c->shared_inter < 128 || c->shared_inter % 128))
    return fail(AFD_ERR_INVALID_ARG, "shared_inter %d must be a positive multiple of 128",
                c->shared_inter);
  if (c->max_tokens < 1 || c->max_tokens > (1 << 20))
    return fail(AFD_ERR_INVALID_ARG, "max_tokens %d outside [1, 2^20]", c->max_tokens);
  if (static_cast<int64_t>(c->max_tokens) * (c->top_k + c->num_shared) >= (1LL << 31))
    return fail(AFD_ERR_INVALID_ARG, "max_tokens * (top_k + num_shared) must be < 2^31");
  // one expert matrix is addressed with 32-bit byte offsets inside kernels
  if (static_cast<int64_t>(c->hidden) * c->inter * 4 >= (1LL << 32) ||
      static_cast<int64_t>(c->hidden) * c->shared_inter * 4 >= (1LL << 32))
    return fail(AFD_ERR_UNSUPPORTED, "an expert matrix must be smaller than 4 GiB in fp32");
  if (c->has_router_bias != 0 && c->has_router_bias != 1)
    return fail(AFD_ERR_INVALID_ARG, "has_router_bias must be 0 or 1");
  if (c->single_launch != 0 && c->single_launch != 1)
    return fail(AFD_ERR_INVALID_ARG, "single_launch must be 0 or 1");
  if (c->split_gemms != 0 && c->split_gemms != 1)
    return fail(AFD_ERR_INVALID_ARG, "split_gemms must be 0 or 1");
  return AFD_OK;
}

int validate_weights(const afd_ffn_config *c, const afd_ffn_weights *w) {
  if (!w) return fail(AFD_ERR_INVALID_ARG, "weights is NULL");
  if (!w->router_w || !w->gate_w || !w->up_w || !w->down_w)
    return fail(AFD_ERR_INVALID_ARG, "router_w, gate_w, up_w and down_w are required");
  if (c->has_router_bias && !w->router_b)
    return fail(AFD_ERR_INVALID_ARG, "has_router_bias = 1 but router_b is NULL");
  const bool fp8 = c->mode == AFD_MODE_W8A8_E4M3;
  if (fp8 && (!w->gate_s || !w->up_s || !w->down_s))
    return fail(AFD_ERR_INVALID_ARG, "W8A8 needs gate_s, up_s and down_s");
  if (c->num_shared > 0) {
    if (!w->sh_gate_w || !w->sh_up_w || !w->sh_down_w)
      return fail(AFD_ERR_INVALID_ARG, "num_shared > 0 needs sh_gate_w, sh_up_w, sh_down_w");
    if (fp8 && (!w->sh_gate_s || !w->sh_up_s || !w->sh_down_s))
      return fail(AFD_ERR_INVALID_ARG, "W8A8 with shared experts needs sh_*_s");
  }
  const void *mats[] = {w->router_w, w->gate_w, w->up_w, w->down_w,
                        w->sh_gate_w, w->sh_up_w, w->sh_down_w};
  for (const void *m : mats)
    if (!aligned(m, 16)) return fail(AFD_ERR_INVALID_ARG, "weight matrices must be 16-byte aligned");
  const void *floats[] = {w->router_b, w->gate_s, w->up_s, w->down_s,
                          w->sh_gate_s, w->sh_up_s, w->sh_down_s};
  for (const void *f : floats)
    if (!aligned(f, 4)) return fail(AFD_ERR_INVALID_ARG, "router_b and scales must be 4-byte aligned");
  return AFD_OK;
}

// Fill the handle fields that follow from the configuration.
void init_handle(afd_ffn_handle *h, const afd_ffn_config *cfg, const afd_ffn_weights *w,
                 int device) {
  h->cfg = *cfg;
  h->w = *w;
  h->device = device;
  h->elem = cfg->mode == AFD_MODE_F32 ? 0 : (cfg->mode == AFD_MODE_BF16 ? 1 : 2);
  const int S = cfg->num_shared;
  h->zpitch = (S > 0 && cfg->shared_inter > cfg->inter) ? cfg->shared_inter : cfg->inter;
  // tiny fp32 / bf16 layers (expert weights of a few MB) run in one launch
  // for batches of at most kFusedMaxT tokens
  const int64_t es = h->elem == 0 ? 4 : 2;
  const int64_t wbytes = (static_cast<int64_t>(cfg->num_experts) * 3 * cfg->inter +
                          static_cast<int64_t>(S) * 3 * cfg->shared_inter) *
                         cfg->hidden * es;
  h->fused_ok = cfg->single_launch == 1 && h->elem != 2 && cfg->top_k <= afd::kFusedMaxK &&
                wbytes <= afd::kFusedMaxWeightBytes;
}

// Workspace of forwards of up to T tokens: sets the capacity of the tile
// lists, points every part at its place above `base` (when not null) and
// returns the total bytes.  Parts start on 256-byte boundaries.  Allocates
// nothing.
size_t layout_workspace(afd_ffn_handle *h, int64_t T, char *base) {
  const afd_ffn_config &c = h->cfg;
  const int64_t k = c.top_k, E = c.num_experts, S = c.num_shared, hd = c.hidden;
  h->tiles_cap = static_cast<int>(tiles_upper_bound(T, c.top_k, c.num_experts, c.num_shared, 16));
  h->big_cap = static_cast<int>(big_tiles_upper_bound(T, c.top_k, c.num_shared, 256));
  const int64_t R = T * k + S * T;  // dispatched + shared rows
  const int zes = h->elem == 0 ? 4 : (h->elem == 1 ? 2 : 1);
  const int yes = h->elem == 0 ? 4 : 2;
  struct Part {
    void **dst;
    size_t bytes;
  };
  Part parts[20];
  int n = 0;
  auto add = [&](void *dst, size_t bytes) { parts[n++] = Part{static_cast<void **>(dst), bytes}; };
  add(&h->ids, sizeof(int32_t) * T * k);
  add(&h->topk_w, sizeof(float) * T * k);
  add(&h->slot_row, sizeof(int32_t) * T * k);
  add(&h->perm, sizeof(int32_t) * T * k);
  add(&h->counts, sizeof(int32_t) * E);
  add(&h->offsets, sizeof(int32_t) * (E + 1));
  add(&h->num_tiles, sizeof(int32_t));
  add(&h->num_big, sizeof(int32_t));
  add(&h->counters, (3 + static_cast<size_t>(h->tiles_cap)) * sizeof(int32_t));
  add(&h->dispatch_scratch, sizeof(int32_t) * 2 * afd::dispatch_blocks(static_cast<int>(T)) * E);
  add(&h->logits, sizeof(float) * static_cast<size_t>(afd::router_logit_floats(
                                      static_cast<int>(T), c.hidden, static_cast<int>(E))));
  add(&h->tiles, sizeof(afd::Tile) * h->tiles_cap);
  add(&h->tiles_big, sizeof(afd::Tile) * h->big_cap);
  add(&h->z, static_cast<size_t>(R) * h->zpitch * zes);
  add(&h->y, static_cast<size_t>(R) * hd * yes);
  if (h->elem == 2) {
    add(&h->xq, static_cast<size_t>(T) * hd);
    add(&h->xs, sizeof(float) * T * (hd / 128));
    add(&h->zs, sizeof(float) * R * (h->zpitch / 128));
    add(&h->z32, sizeof(float) * R * h->zpitch);
  }
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    off = align_up(off, 256);
    if (base) *parts[i].dst = base + off;
    off += align_up(parts[i].bytes, 256);
  }
  return off;
}

// Record a profiling event pair around one stage's launches.  Returns the
// pair's index in the pool (-1: stage not profiled); pairs may nest, so the
// index, not a pointer into the growing pool, identifies the pair.
int prof_begin(afd_ffn_handle *h, int stage, hipStream_t s) {
  if (!(h->prof_mask & (1u << stage))) return -1;
  if (h->ev_used == h->ev_pool.size()) {
    StageEvents e;
    if (hipEventCreate(&e.start) != hipSuccess) return -1;
    if (hipEventCreate(&e.stop) != hipSuccess) {
      hipEventDestroy(e.start);
      return -1;
    }
    h->ev_pool.push_back(e);
    h->ev_stage.push_back(stage);
  }
  const size_t i = h->ev_used++;
  h->ev_stage[i] = stage;
  hipEventRecord(h->ev_pool[i].start, s);
  return static_cast<int>(i);
}
void prof_end(afd_ffn_handle *h, int i, hipStream_t s) {
  if (i >= 0) hipEventRecord(h->ev_pool[static_cast<size_t>(i)].stop, s);
}

}  // namespace

extern "C" {

const char *afd_ffn_last_error(void) { return g_last_error.c_str(); }

int afd_ffn_create(const afd_ffn_config *cfg, const afd_ffn_weights *w,
                   afd_ffn_handle **out) {
  if (!out) return fail(AFD_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  rc = validate_weights(cfg, w);
  if (rc) return rc;

  afd_ffn_handle *h = new afd_ffn_handle();
  int dev = 0;
  hipGetDevice(&dev);
  init_handle(h, cfg, w, dev);
  const size_t total = layout_workspace(h, cfg->max_tokens, nullptr);
  hipError_t e = hipMalloc(&h->ws, total);
  if (e != hipSuccess) {
    delete h;
    (void)hipGetLastError();
    return fail(AFD_ERR_OUT_OF_MEMORY, "workspace of %zu bytes: %s", total, hipGetErrorString(e));
  }
  h->ws_bytes = total;
  layout_workspace(h, cfg->max_tokens, static_cast<char *>(h->ws));
  *out = h;
  return AFD_OK;
}

void afd_ffn_destroy(afd_ffn_handle *h) {
  if (!h) return;
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(h->device);
  hipDeviceSynchronize();
  for (auto &e : h->ev_pool) {
    hipEventDestroy(e.start);
    hipEventDestroy(e.stop);
  }
  hipFree(h->ws);
  hipSetDevice(cur);
  delete h;
}

// One GEMM stage: the small-tile list on its kernel, then (if the plan has
// one) the big-tile list on the compute-bound kernel.
static hipError_t launch_gemms(afd_ffn_handle *h, afd::GemmKind kind, const afd::GemmPlan &plan,
                               afd::GemmArgs a, int64_t T, hipStream_t s) {
  const afd_ffn_config &c = h->cfg;
  a.tiles = h->tiles;
  a.num_tiles = h->num_tiles;
  a.tiles_ub = static_cast<int>(
      tiles_upper_bound(T, c.top_k, c.num_experts, c.num_shared, plan.tiles.bm_small));
  hipError_t e;
  switch (plan.small_kernel) {
    case afd::GemmKernel::Stream:
      e = afd::launch_gemm_stream(kind, h->elem, plan.tiles.bm_small, a, s);
      break;
    default:
      e = afd::launch_gemm(kind, h->elem, plan.tiles.bm_small, a, s);
      break;
  }
  if (e != hipSuccess || plan.tiles.bm_big == 0) return e;
  a.tiles = h->tiles_big;
  a.num_tiles = h->num_big;
  a.tiles_ub = static_cast<int>(big_tiles_upper_bound(T, c.top_k, c.num_shared, plan.tiles.bm_big));
  const int ev = prof_begin(
      h, kind == afd::GemmKind::GateUp ? AFD_STAGE_GATE_UP_BIG : AFD_STAGE_DOWN_BIG, s);
  e = afd::launch_gemm_prefill(kind, a, s);
  prof_end(h, ev, s);
  return e;
}

// logits_out: optional [T, E] fp32 copy of the router logits (trace).
static int forward_impl(afd_ffn_handle *h, const void *hidden, void *out, int64_t T,
                        hipStream_t s, float *logits_out) {
  if (!h) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  const afd_ffn_config &c = h->cfg;
  if (T < 0) return fail(AFD_ERR_INVALID_ARG, "T = %lld < 0", static_cast<long long>(T));
  if (T > c.max_tokens)
    return fail(AFD_ERR_CAPACITY, "T = %lld exceeds max_tokens = %d", static_cast<long long>(T),
                c.max_tokens);
  if (T == 0) return AFD_OK;
  if (!hidden || !out) return fail(AFD_ERR_INVALID_ARG, "hidden and out must not be NULL");
  if (!aligned(hidden, 16) || !aligned(out, 16))
    return fail(AFD_ERR_INVALID_ARG, "hidden and out must be 16-byte aligned");
  const int aes = h->elem == 0 ? 4 : 2;
  const size_t act_bytes = static_cast<size_t>(T) * c.hidden * aes;
  const char *hb = static_cast<const char *>(hidden);
  const char *ob = static_cast<const char *>(out);
  if (hb < ob + act_bytes && ob < hb + act_bytes)
    return fail(AFD_ERR_INVALID_ARG, "hidden and out overlap");
  int cur = -1;
  hipGetDevice(&cur);
  if (cur != h->device)
    return fail(AFD_ERR_INVALID_ARG, "current device %d is not the handle's device %d", cur,
                h->device);

  const int Ti = static_cast<int>(T), k = c.top_k, E = c.num_experts, S = c.num_shared;
  const int hd = c.hidden;
  const int Tk = Ti * k;
  hipError_t e;
  int ev;

  // tiny layers, small batches: the whole layer in one cooperative launch
  // (outside graph capture, where the multi-kernel sequence is recorded)
  if (h->fused_ok && Ti <= afd::kFusedMaxT) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_fail(e, "capture status");
    if (cs == hipStreamCaptureStatusNone && afd::fused_supported(h->device)) {
      afd::FusedArgs fa{};
      fa.x = static_cast<const uint8_t *>(hidden);
      fa.wr = static_cast<const uint8_t *>(h->w.router_w);
      fa.bias = c.has_router_bias ? h->w.router_b : nullptr;
      fa.gate = static_cast<const uint8_t *>(h->w.gate_w);
      fa.up = static_cast<const uint8_t *>(h->w.up_w);
      fa.down = static_cast<const uint8_t *>(h->w.down_w);
      fa.sgate = static_cast<const uint8_t *>(h->w.sh_gate_w);
      fa.sup = static_cast<const uint8_t *>(h->w.sh_up_w);
      fa.sdown = static_cast<const uint8_t *>(h->w.sh_down_w);
      fa.T = Ti;
      fa.h = hd;
      fa.E = E;
      fa.k = k;
      fa.I = c.inter;
      fa.S = S;
      fa.Is = S > 0 ? c.shared_inter : c.inter;
      fa.zpitch = h->zpitch;
      fa.logits = logits_out ? logits_out : h->logits;
      fa.ids = h->ids;
      fa.w = h->topk_w;
      fa.counts = h->counts;
      fa.offsets = h->offsets;
      fa.perm = h->perm;
      fa.slot_row = h->slot_row;
      fa.num_tiles = h->num_tiles;
      fa.num_big = h->num_big;
      fa.sync_timeouts = h->counters + 2;
      fa.z = h->z;
      fa.out = out;
      ev = prof_begin(h, AFD_STAGE_SINGLE, s);
      e = afd::launch_fused_small(h->elem == 0, fa, s);
      prof_end(h, ev, s);
      if (e != hipSuccess) return hip_fail(e, "single-launch forward");
      return AFD_OK;
    }
  }

  ev = prof_begin(h, AFD_STAGE_ROUTER, s);
  e = afd::launch_router(h->elem == 0, hidden, h->w.router_w,
                         c.has_router_bias ? h->w.router_b : nullptr, Ti, hd, E, k, h->logits,
                         h->ids, h->topk_w, logits_out, s);
  prof_end(h, ev, s);
  if (e != hipSuccess) return hip_fail(e, "router launch");

  const afd::GemmPlan plan = afd::gemm_plan(h->elem, Ti, k, E);
  // decode-regime bf16 layers: both weight-streaming GEMMs in one launch
  const bool ffn_one_launch =
      c.split_gemms == 0 && plan.small_kernel == afd::GemmKernel::Stream &&
      plan.tiles.bm_big == 0 &&
      afd::stream_ffn_supported(h->elem, plan.tiles.bm_small, hd, c.inter,
                                S > 0 ? c.shared_inter : c.inter);
  const int small_ub =
      static_cast<int>(tiles_upper_bound(T, k, E, S, plan.tiles.bm_small));
  ev = prof_begin(h, AFD_STAGE_DISPATCH, s);
  e = afd::launch_dispatch(h->ids, Ti, k, E, S, plan.tiles, h->counts, h->offsets, h->perm,
                           h->slot_row, h->tiles, h->num_tiles, h->tiles_big, h->num_big,
                           h->counters, ffn_one_launch ? 3 + small_ub : 3,
                           h->dispatch_scratch, s);
  prof_end(h, ev, s);
  if (e != hipSuccess) return hip_fail(e, "dispatch launch");

  const uint8_t *A = static_cast<const uint8_t *>(hidden);
  int64_t a_pitch = static_cast<int64_t>(hd) * aes;
  if (h->elem == 2) {
    ev = prof_begin(h, AFD_STAGE_QUANT, s);
    e = afd::launch_quant_1x128(static_cast<const uint16_t *>(hidden), T, hd, h->xq, h->xs, s);
    prof_end(h, ev, s);
    if (e != hipSuccess) return hip_fail(e, "quantiser launch");
    A = h->xq;
    a_pitch = hd;
  }

  const int zes = h->elem == 0 ? 4 : (h->elem == 1 ? 2 : 1);
  const int yes = h->elem == 0 ? 4 : 2;
  afd::GemmArgs g{};
  g.A = A;
  g.a_pitch = a_pitch;
  g.perm = h->perm;
  g.a_scale = h->xs;
  g.a_scale_pitch = hd / 128;
  g.Tk = Tk;
  g.T = Ti;
  g.b0 = static_cast<const uint8_t *>(h->w.gate_w);
  g.b1 = static_cast<const uint8_t *>(h->w.up_w);
  g.sb0 = static_cast<const uint8_t *>(h->w.sh_gate_w);
  g.sb1 = static_cast<const uint8_t *>(h->w.sh_up_w);
  g.bs0 = h->w.gate_s;
  g.bs1 = h->w.up_s;
  g.sbs0 = h->w.sh_gate_s;
  g.sbs1 = h->w.sh_up_s;
  g.N = c.inter;
  g.K = hd;
  g.Ns = S > 0 ? c.shared_inter : c.inter;
  g.Ks = hd;
  g.E = E;
  g.work_counter = h->counters;
  g.C = h->z;
  g.c_pitch = static_cast<int64_t>(h->zpitch) * zes;
  g.c_scale = h->zs;
  g.c_scale_pitch = h->zpitch / 128;
  // W8A8 on the streaming kernels with 64-row tiles: gate/up writes fp32 z,
  // then the 1x128 quantiser produces the E4M3 rows and scales the down GEMM
  // reads (with 128-row tiles the gate/up epilogue quantises itself)
  const bool z_fp32 = h->elem == 2 && plan.small_kernel == afd::GemmKernel::Stream &&
                      !afd::stream_gate_up_writes_fp8(h->elem, plan.tiles.bm_small);
  if (z_fp32) {
    g.C = reinterpret_cast<uint8_t *>(h->z32);
    g.c_pitch = static_cast<int64_t>(h->zpitch) * 4;
  }
  if (!ffn_one_launch) {
    ev = prof_begin(h, AFD_STAGE_GATE_UP, s);
    e = launch_gemms(h, afd::GemmKind::GateUp, plan, g, T, s);
    prof_end(h, ev, s);
    if (e != hipSuccess) return hip_fail(e, "gate/up GEMM launch");
  }
  if (z_fp32) {
    ev = prof_begin(h, AFD_STAGE_QUANT, s);
    const int64_t R = static_cast<int64_t>(Tk) + static_cast<int64_t>(S) * Ti;
    // routed rows have I columns; shared rows I_s (quantised in two calls
    // when the widths differ)
    e = afd::launch_quant_1x128_f32(h->z32, Tk, c.inter, h->zpitch, h->z, h->zpitch, h->zs,
                                    h->zpitch / 128, s);
    if (e == hipSuccess && S > 0)
      e = afd::launch_quant_1x128_f32(h->z32 + static_cast<int64_t>(Tk) * h->zpitch, R - Tk,
                                      c.shared_inter, h->zpitch,
                                      h->z + static_cast<int64_t>(Tk) * h->zpitch, h->zpitch,
                                      h->zs + static_cast<int64_t>(Tk) * (h->zpitch / 128),
                                      h->zpitch / 128, s);
    prof_end(h, ev, s);
    if (e != hipSuccess) return hip_fail(e, "z quantiser launch");
  }

  afd::GemmArgs d = g;
  d.A = h->z;
  d.a_pitch = static_cast<int64_t>(h->zpitch) * zes;
  d.perm = nullptr;
  d.a_scale = h->zs;
  d.a_scale_pitch = h->zpitch / 128;
  d.b0 = static_cast<const uint8_t *>(h->w.down_w);
  d.b1 = nullptr;
  d.sb0 = static_cast<const uint8_t *>(h->w.sh_down_w);
  d.sb1 = nullptr;
  d.bs0 = h->w.down_s;
  d.bs1 = nullptr;
  d.sbs0 = h->w.sh_down_s;
  d.sbs1 = nullptr;
  d.N = hd;
  d.K = c.inter;
  d.Ns = hd;
  d.Ks = S > 0 ? c.shared_inter : c.inter;
  d.C = h->y;
  d.c_pitch = static_cast<int64_t>(hd) * yes;
  d.c_scale = nullptr;
  d.work_counter = h->counters + 1;
  if (ffn_one_launch) {
    // one work counter (the gate/up one) for the items of both GEMMs
    g.tiles = d.tiles = h->tiles;
    g.num_tiles = d.num_tiles = h->num_tiles;
    g.tiles_ub = d.tiles_ub = small_ub;
    ev = prof_begin(h, AFD_STAGE_FFN, s);
    e = afd::launch_ffn_stream(g, d, h->counters + 2, s);  // sync words
    prof_end(h, ev, s);
    if (e != hipSuccess) return hip_fail(e, "gate/up + down GEMM launch");
  } else {
    ev = prof_begin(h, AFD_STAGE_DOWN, s);
    e = launch_gemms(h, afd::GemmKind::Down, plan, d, T, s);
    prof_end(h, ev, s);
    if (e != hipSuccess) return hip_fail(e, "down GEMM launch");
  }

  ev = prof_begin(h, AFD_STAGE_COMBINE, s);
  e = afd::launch_combine(h->elem == 0, h->y, h->slot_row, h->topk_w, Ti, k, S, hd, out, s);
  prof_end(h, ev, s);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return AFD_OK;
}

int afd_ffn_forward(afd_ffn_handle *h, const void *hidden, void *out, int64_t T,
                    afd_stream_t stream) {
  return forward_impl(h, hidden, out, T, static_cast<hipStream_t>(stream), nullptr);
}

int afd_ffn_forward_traced(afd_ffn_handle *h, const void *hidden, void *out, int64_t T,
                           afd_stream_t stream, const afd_ffn_trace *tr) {
  if (!tr) return fail(AFD_ERR_INVALID_ARG, "trace is NULL");
  if (h && T > 0 && (tr->x_q || tr->x_s || tr->z_q || tr->z_s) && h->elem != 2)
    return fail(AFD_ERR_INVALID_ARG, "x_q / x_s / z_q / z_s are only produced in W8A8 mode");
  int rc = forward_impl(h, hidden, out, T, static_cast<hipStream_t>(stream), tr->logits);
  if (rc || T == 0) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const afd_ffn_config &c = h->cfg;
  const size_t tk = static_cast<size_t>(T) * c.top_k;
  const size_t R = tk + static_cast<size_t>(c.num_shared) * T;
  struct Cp {
    void *dst;
    const void *src;
    size_t bytes;
  } cps[] = {
      {tr->topk_ids, h->ids, tk * 4},
      {tr->topk_w, h->topk_w, tk * 4},
      {tr->counts, h->counts, static_cast<size_t>(c.num_experts) * 4},
      {tr->offsets, h->offsets, static_cast<size_t>(c.num_experts + 1) * 4},
      {tr->perm, h->perm, tk * 4},
      {tr->slot_row, h->slot_row, tk * 4},
      {tr->x_q, h->xq, static_cast<size_t>(T) * c.hidden},
      {tr->x_s, h->xs, static_cast<size_t>(T) * (c.hidden / 128) * 4},
      {tr->z_q, h->z, R * h->zpitch},
      {tr->z_s, h->zs, R * (h->zpitch / 128) * 4},
      {tr->num_tiles, h->num_tiles, 4},
      {tr->num_tiles ? tr->num_tiles + 1 : nullptr, h->num_big, 4},
      {tr->sync_timeouts, h->counters + 2, 4},
  };
  for (auto &cp : cps) {
    if (!cp.dst) continue;
    hipError_t e = hipMemcpyAsync(cp.dst, cp.src, cp.bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "trace copy");
  }
  return AFD_OK;
}

int afd_ffn_forward_static(const afd_ffn_config *cfg, const afd_ffn_weights *w,
                           const void *hidden, void *out, int64_t T, afd_stream_t stream) {
  static_assert(AFD_FFN_STATIC_SCRATCH_BYTES == afd::kStaticScratchBytes, "scratch size");
  int rc = validate_config(cfg);
  if (rc) return rc;
  rc = validate_weights(cfg, w);
  if (rc) return rc;
  if (T < 0) return fail(AFD_ERR_INVALID_ARG, "T = %lld < 0", static_cast<long long>(T));
  if (T > cfg->max_tokens)
    return fail(AFD_ERR_CAPACITY, "T = %lld exceeds max_tokens = %d", static_cast<long long>(T),
                cfg->max_tokens);
  if (T == 0) return AFD_OK;
  // the handle lives on this stack frame; its workspace is the scratch array
  afd_ffn_handle h{};
  init_handle(&h, cfg, w, -1);
  const size_t need = layout_workspace(&h, T, nullptr);
  if (need > afd::kStaticScratchBytes)
    return fail(AFD_ERR_CAPACITY,
                "T = %lld needs %zu bytes of scratch, the library holds %zu per device",
                static_cast<long long>(T), need, afd::kStaticScratchBytes);
  hipError_t e = hipGetDevice(&h.device);
  if (e != hipSuccess) return hip_fail(e, "current device");
  void *base = nullptr;
  e = afd::static_scratch(&base);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  layout_workspace(&h, T, static_cast<char *>(base));
  return forward_impl(&h, hidden, out, T, static_cast<hipStream_t>(stream), nullptr);
}

int afd_quant_fp8_1x128(const void *x, int64_t rows, int64_t cols, uint8_t *q, float *s,
                        afd_stream_t stream) {
  if (!x || !q || !s) return fail(AFD_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4))
    return fail(AFD_ERR_INVALID_ARG, "x and q must be 16-byte aligned, s 4-byte aligned");
  if (rows < 0 || cols <= 0 || cols % 128)
    return fail(AFD_ERR_INVALID_ARG, "rows >= 0 and cols a positive multiple of 128 required");
  if (rows == 0) return AFD_OK;
  if (rows * (cols / 128) * 16 / 256 >= (1LL << 31))
    return fail(AFD_ERR_UNSUPPORTED, "tensor too large for one launch");
  hipError_t e = afd::launch_quant_1x128(static_cast<const uint16_t *>(x), rows, cols, q, s,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AFD_OK : hip_fail(e, "quantiser launch");
}

int afd_quant_fp8_1x128_f32(const float *x, int64_t rows, int64_t cols, uint8_t *q, float *s,
                            afd_stream_t stream) {
  if (!x || !q || !s) return fail(AFD_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4))
    return fail(AFD_ERR_INVALID_ARG, "x and q must be 16-byte aligned, s 4-byte aligned");
  if (rows < 0 || cols <= 0 || cols % 128)
    return fail(AFD_ERR_INVALID_ARG, "rows >= 0 and cols a positive multiple of 128 required");
  if (rows == 0) return AFD_OK;
  if (rows * (cols / 128) * 16 / 256 >= (1LL << 31))
    return fail(AFD_ERR_UNSUPPORTED, "tensor too large for one launch");
  hipError_t e = afd::launch_quant_1x128_f32(x, rows, cols, cols, q, cols, s, cols / 128,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AFD_OK : hip_fail(e, "quantiser launch");
}

int afd_quant_fp8_128x128(const void *w, int64_t rows, int64_t cols, uint8_t *q, float *s,
                          afd_stream_t stream) {
  if (!w || !q || !s) return fail(AFD_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4))
    return fail(AFD_ERR_INVALID_ARG, "w and q must be 16-byte aligned, s 4-byte aligned");
  if (rows <= 0 || cols <= 0 || rows % 128 || cols % 128)
    return fail(AFD_ERR_INVALID_ARG, "rows and cols must be positive multiples of 128");
  if ((rows / 128) * (cols / 128) >= (1LL << 31))
    return fail(AFD_ERR_UNSUPPORTED, "tensor too large for one launch");
  hipError_t e = afd::launch_quant_128x128(static_cast<const uint16_t *>(w), rows, cols, q, s,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AFD_OK : hip_fail(e, "quantiser launch");
}

int afd_ffn_profile_enable(afd_ffn_handle *h, uint32_t stage_mask) {
  if (!h) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (stage_mask >> AFD_STAGE_COUNT) return fail(AFD_ERR_INVALID_ARG, "unknown stage bits");
  h->prof_mask = stage_mask;
  return AFD_OK;
}

int afd_ffn_profile_read(afd_ffn_handle *h, double *ms, int64_t *launches) {
  if (!h || !ms || !launches) return fail(AFD_ERR_INVALID_ARG, "NULL pointer");
  for (int i = 0; i < AFD_STAGE_COUNT; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  for (size_t i = 0; i < h->ev_used; ++i) {
    hipError_t e = hipEventSynchronize(h->ev_pool[i].stop);
    if (e != hipSuccess) return hip_fail(e, "profile event");
    float t = 0.0f;
    e = hipEventElapsedTime(&t, h->ev_pool[i].start, h->ev_pool[i].stop);
    if (e != hipSuccess) return hip_fail(e, "profile event");
    ms[h->ev_stage[i]] += t;
    launches[h->ev_stage[i]] += 1;
  }
  h->ev_used = 0;
  return AFD_OK;
}

}  // extern "C"
