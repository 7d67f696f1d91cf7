// Host side of the C ABI declared in include/flint_moe.h: argument
// validation, workspace layout and the choice of kernel path.  Everything
// here runs on the CPU; the kernels it enqueues are in the other .hip files.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "flint_kernels.h"
#include "flint_moe.h"

#define FLINT_API extern "C" __attribute__((visibility("default")))

struct flint_moe_ctx {
  flint_moe_config cfg;
  std::string last_error;
};

struct flint_mlp_ctx {
  flint_mlp_config cfg;
  std::string last_error;
};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kHeaderBytes = flint::kHeaderWords * sizeof(uint32_t);
static_assert(kHeaderBytes == FLINT_MOE_WS_HEADER_BYTES, "header size in flint_moe.h");

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Prefill regions inside the "extra" area; fills `p` relative to `base` when given.
size_t prefill_extra_bytes(const flint_moe_config& c, int32_t T, flint::PrefillWs* p,
                           uint8_t* base = nullptr) {
  const size_t t = (size_t)T, E = (size_t)c.n_experts, k = (size_t)c.top_k, I = (size_t)c.inter,
               H = (size_t)c.hidden;
  const size_t nb = (t + flint::kPrefillTile - 1) / flint::kPrefillTile;
  const size_t tiles = (size_t)flint::prefill_tiles_max(T, c.n_experts, c.top_k);
  size_t o = 0;
  const size_t counts = o; o = align_up(o + nb * E * sizeof(int32_t));
  const size_t tl = o;     o = align_up(o + (1 + 3 * tiles) * sizeof(int32_t));
  const size_t pos = o;    o = align_up(o + t * k * sizeof(int32_t));
  const size_t h16 = o;    o = align_up(o + (t * k + t) * I * sizeof(uint16_t));
  const size_t y16 = o;    o = align_up(o + t * k * H * sizeof(uint16_t));
  if (p) {
    p->counts = reinterpret_cast<int32_t*>(base + counts);
    p->tiles = reinterpret_cast<int32_t*>(base + tl);
    p->pos = reinterpret_cast<int32_t*>(base + pos);
    p->h16 = reinterpret_cast<_Float16*>(base + h16);
    p->y16 = reinterpret_cast<_Float16*>(base + y16);
  }
  return o;
}

void compute_layout(const flint_moe_config& c, int32_t T, flint_moe_ws_layout* L) {
  const size_t t = (size_t)T, E = (size_t)c.n_experts, k = (size_t)c.top_k, I = (size_t)c.inter,
               H = (size_t)c.hidden;
  size_t o = 0;
  std::memset(L, 0, sizeof(*L));
  L->header = o;   o = align_up(o + kHeaderBytes);
  L->logits = o;   o = align_up(o + t * E * sizeof(float));
  L->topk_ids = o; o = align_up(o + t * k * sizeof(int32_t));
  L->topk_w = o;   o = align_up(o + t * k * sizeof(float));
  L->route = o;    o = align_up(o + (size_t)flint::route_table_ints((int)E, T, (int)k) * sizeof(int32_t));
  L->normed = o;   o = align_up(o + t * H * sizeof(uint16_t));
  const bool prefill = T > flint::kDecodeMaxT;
  L->h = o;        o = align_up(o + (prefill ? 0 : (t * k + t) * I * sizeof(float)));
  L->items = o;    o = align_up(o + (prefill ? 0 : std::min(E, t * k) * (size_t)flint::item_record_ints(T) *
                                                   sizeof(int32_t)));
  const bool lowlat = T <= flint::kLowLatMaxT;
  L->resid1 = o;   o = align_up(o + (lowlat ? t * H * sizeof(uint16_t) : 0));
  L->norm_part = o; o = align_up(o + (lowlat ? (size_t)(H / 8) * t * sizeof(float) : 0));
  L->extra = o;
  if (prefill) o = L->extra + prefill_extra_bytes(c, T, nullptr);
  L->total_bytes = o;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

flint_status fail(flint_moe_ctx* ctx, flint_status s, const std::string& why) {
  if (ctx) ctx->last_error = why;
  return s;
}

flint_status check_config(const flint_moe_config& c, std::string* why) {
  char buf[256];
  if (c.hidden <= 0 || c.inter <= 0 || c.n_experts <= 0 || c.top_k <= 0 || c.max_tokens <= 0) {
    *why = "hidden, inter, n_experts, top_k and max_tokens must be positive";
    return FLINT_ERR_INVALID_ARG;
  }
  if (c.top_k > c.n_experts) {
    *why = "top_k exceeds n_experts";
    return FLINT_ERR_INVALID_ARG;
  }
  if (c.renormalize != 0 && c.renormalize != 1) {
    *why = "renormalize must be 0 or 1";
    return FLINT_ERR_INVALID_ARG;
  }
  if (!std::isfinite(c.routed_scale)) {
    *why = "routed_scale must be finite";
    return FLINT_ERR_INVALID_ARG;
  }
  if (c.format != FLINT_W_BF16 && c.format != FLINT_W_NVFP4) {
    *why = "unknown weight format";
    return FLINT_ERR_INVALID_ARG;
  }
  if (c.hidden != flint::kHidden || c.inter != flint::kInter || c.n_experts > flint::kMaxExperts ||
      c.top_k > flint::kMaxTopK) {
    std::snprintf(buf, sizeof buf,
                  "no kernels for hidden=%d inter=%d n_experts=%d top_k=%d "
                  "(built for hidden=%d, inter=%d, n_experts<=%d, top_k<=%d)",
                  c.hidden, c.inter, c.n_experts, c.top_k, flint::kHidden, flint::kInter,
                  flint::kMaxExperts, flint::kMaxTopK);
    *why = buf;
    return FLINT_ERR_UNSUPPORTED;
  }
  return FLINT_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Clears n 32-bit words (a kernel rather than a memset, so that a caller may
// capture it in a graph).
__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

FLINT_API flint_status flint_moe_init(const flint_moe_config* cfg, flint_moe_ctx** ctx_out) {
  if (!cfg || !ctx_out) return FLINT_ERR_INVALID_ARG;
  std::string why;
  const flint_status s = check_config(*cfg, &why);
  if (s != FLINT_OK) return s;
  flint_moe_ctx* ctx = new (std::nothrow) flint_moe_ctx;
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  ctx->cfg = *cfg;
  *ctx_out = ctx;
  return FLINT_OK;
}

FLINT_API size_t flint_moe_workspace_bytes(const flint_moe_ctx* ctx, int32_t T) {
  if (!ctx || T <= 0) return 0;
  flint_moe_ws_layout L;
  compute_layout(ctx->cfg, T, &L);
  return L.total_bytes;
}

FLINT_API flint_status flint_moe_workspace_layout(const flint_moe_ctx* ctx, int32_t T,
                                                  flint_moe_ws_layout* layout) {
  if (!ctx || !layout || T <= 0) return FLINT_ERR_INVALID_ARG;
  compute_layout(ctx->cfg, T, layout);
  return FLINT_OK;
}

namespace {

// Pre-norm block arguments: gamma == nullptr runs the bare layer on x.
struct NormArgs {
  const uint16_t* gamma = nullptr;
  float eps = 0.f;
};

// The low-latency decode path's own arguments (flint_moe_lowlat_forward).
struct LowLatArgs {
  const uint16_t* wo = nullptr;
  const uint16_t* attn = nullptr;
  const uint16_t* gamma_next = nullptr;
  uint16_t* n_out = nullptr;
  bool fused = true;
};

flint_status forward_impl(flint_moe_ctx* ctx, const flint_moe_weights* w, const uint16_t* x,
                          int32_t T, uint16_t* out, int32_t* topk_ids, float* topk_w,
                          void* workspace, size_t workspace_bytes, void* stream,
                          flint::Launcher& launch, const NormArgs& norm = NormArgs(),
                          bool zero_header_first = false, const LowLatArgs* ll = nullptr) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  ctx->last_error.clear();
  const flint_moe_config& c = ctx->cfg;
  if (T < 0 || T > c.max_tokens) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "T=%d outside [0, max_tokens=%d]", T, c.max_tokens);
    return fail(ctx, FLINT_ERR_INVALID_ARG, buf);
  }
  if (T == 0) return FLINT_OK;
  if (!w || !x || !out || !workspace)
    return fail(ctx, FLINT_ERR_INVALID_ARG, "weights, x, out and workspace must be non-NULL");
  if (ll) {
    if (T > flint::kLowLatMaxT) {
      char buf[128];
      std::snprintf(buf, sizeof buf, "the low-latency path takes T <= %d (got T=%d)",
                    flint::kLowLatMaxT, T);
      return fail(ctx, FLINT_ERR_UNSUPPORTED, buf);
    }
    if (!ll->wo || !ll->attn)
      return fail(ctx, FLINT_ERR_INVALID_ARG, "wo and attn must be non-NULL");
    if (!aligned(ll->wo, 16) || !aligned(ll->attn, 16) ||
        (ll->gamma_next && !aligned(ll->gamma_next, 16)) || (ll->n_out && !aligned(ll->n_out, 16)))
      return fail(ctx, FLINT_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (!ll->gamma_next != !ll->n_out)
      return fail(ctx, FLINT_ERR_INVALID_ARG, "gamma_next and n_out go together");
    const size_t act = (size_t)T * ctx->cfg.hidden * sizeof(uint16_t);
    const size_t attn_bytes = (size_t)T * flint::kAttnWidth * sizeof(uint16_t);
    if (ranges_overlap(ll->attn, attn_bytes, out, act))
      return fail(ctx, FLINT_ERR_INVALID_ARG, "r_out overlaps attn");
    if (ll->n_out && (ranges_overlap(ll->n_out, act, out, act) || ranges_overlap(ll->n_out, act, x, act)))
      return fail(ctx, FLINT_ERR_INVALID_ARG, "n_out overlaps r or r_out");
  }
  if (norm.gamma && !aligned(norm.gamma, 16))
    return fail(ctx, FLINT_ERR_INVALID_ARG, "gamma must be 16-byte aligned");
  if (norm.gamma && !(std::isfinite(norm.eps) && norm.eps >= 0.f))
    return fail(ctx, FLINT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!w->router_w || !w->routed.w13 || !w->routed.w2 || !w->shared.w13 || !w->shared.w2)
    return fail(ctx, FLINT_ERR_INVALID_ARG, "router and expert weight pointers must be non-NULL");
  const void* p16[] = {w->router_w, w->routed.w13, w->routed.w2, w->shared.w13, w->shared.w2, x, out};
  for (const void* p : p16)
    if (!aligned(p, 16)) return fail(ctx, FLINT_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (c.format == FLINT_W_NVFP4) {
    const flint_expert_bank* banks[2] = {&w->routed, &w->shared};
    for (const flint_expert_bank* b : banks) {
      if (!b->w13_scale || !b->w2_scale || !b->w13_gscale || !b->w2_gscale)
        return fail(ctx, FLINT_ERR_INVALID_ARG, "NVFP4 weights need block and tensor scales");
      if (!aligned(b->w13_scale, 16) || !aligned(b->w2_scale, 16))
        return fail(ctx, FLINT_ERR_INVALID_ARG, "block scales must be 16-byte aligned");
      if (!aligned(b->w13_gscale, 4) || !aligned(b->w2_gscale, 4))
        return fail(ctx, FLINT_ERR_INVALID_ARG, "tensor scales must be 4-byte aligned");
    }
  }
  if (w->router_b && !aligned(w->router_b, 4))
    return fail(ctx, FLINT_ERR_INVALID_ARG, "router_b must be 4-byte aligned");
  if ((topk_ids && !aligned(topk_ids, 4)) || (topk_w && !aligned(topk_w, 4)))
    return fail(ctx, FLINT_ERR_INVALID_ARG, "topk_ids / topk_w must be 4-byte aligned");
  if (!aligned(workspace, kAlign))
    return fail(ctx, FLINT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t act_bytes = (size_t)T * c.hidden * sizeof(uint16_t);
  if (ranges_overlap(x, act_bytes, out, act_bytes))
    return fail(ctx, FLINT_ERR_INVALID_ARG, norm.gamma ? "out overlaps r" : "out overlaps x");

  flint_moe_ws_layout L;
  compute_layout(c, T, &L);
  if (workspace_bytes < L.total_bytes) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "workspace of %zu bytes, %zu needed for T=%d", workspace_bytes,
                  L.total_bytes, T);
    return fail(ctx, FLINT_ERR_WORKSPACE, buf);
  }
  const bool prefill = T > flint::kDecodeMaxT;
  if (prefill && c.format != FLINT_W_BF16)
    return fail(ctx, FLINT_ERR_UNSUPPORTED, "NVFP4 weights are supported for T <= 64 only");

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  flint::LayerArgs a{};
  a.x = x;
  a.out = out;
  if (norm.gamma) {
    a.normed = reinterpret_cast<uint16_t*>(ws + L.normed);
    a.x = a.normed;
    a.resid = x;
    a.norm_w = norm.gamma;
    a.eps = norm.eps;
  }
  a.router_w = w->router_w;
  a.router_b = w->router_b;
  a.routed = {static_cast<const uint8_t*>(w->routed.w13), static_cast<const uint8_t*>(w->routed.w2),
              w->routed.w13_scale, w->routed.w2_scale, w->routed.w13_gscale, w->routed.w2_gscale};
  a.shared = {static_cast<const uint8_t*>(w->shared.w13), static_cast<const uint8_t*>(w->shared.w2),
              w->shared.w13_scale, w->shared.w2_scale, w->shared.w13_gscale, w->shared.w2_gscale};
  a.ids_out = topk_ids;
  a.wts_out = topk_w;
  a.ws.header = reinterpret_cast<uint32_t*>(ws + L.header);
  a.ws.logits = reinterpret_cast<float*>(ws + L.logits);
  a.ws.ids = reinterpret_cast<int32_t*>(ws + L.topk_ids);
  a.ws.wts = reinterpret_cast<float*>(ws + L.topk_w);
  a.ws.route = reinterpret_cast<int32_t*>(ws + L.route);
  a.ws.h = reinterpret_cast<float*>(ws + L.h);
  a.ws.items = reinterpret_cast<int32_t*>(ws + L.items);
  a.ws.extra = ws + L.extra;
  if (prefill) prefill_extra_bytes(c, T, &a.ws.pre, ws + L.extra);
  a.T = T;
  a.E = c.n_experts;
  a.k = c.top_k;
  a.renormalize = c.renormalize;
  a.routed_scale = c.routed_scale;
  a.nvfp4 = c.format == FLINT_W_NVFP4;
  if (ll) {
    // r1 = bf16(r + Wo attn) lands in the workspace and is the block's r from
    // there on; x is the incoming residual stream r.
    a.resid0 = x;
    a.attn = ll->attn;
    a.wo = ll->wo;
    a.ws.resid1 = reinterpret_cast<uint16_t*>(ws + L.resid1);
    a.ws.norm_part = reinterpret_cast<float*>(ws + L.norm_part);
    a.resid = a.ws.resid1;
    a.norm_next_w = ll->gamma_next;
    a.normed_next = ll->n_out;
  }

  (void)hipGetLastError();  // do not report an earlier, unrelated failure
  if (zero_header_first) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(8), dim3(256), 0, static_cast<hipStream_t>(stream),
                       a.ws.header, (int)flint::kHeaderWords);
    const hipError_t ez = hipGetLastError();
    if (ez != hipSuccess) return fail(ctx, FLINT_ERR_HIP, hipGetErrorString(ez));
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t err = ll ? flint::launch_lowlat(a, ll->fused, hs, launch)
                         : prefill ? flint::launch_prefill(a, hs, launch)
                                   : flint::launch_decode(a, hs, launch);
  if (err != hipSuccess) return fail(ctx, FLINT_ERR_HIP, hipGetErrorString(err));
  return FLINT_OK;
}

}  // namespace

FLINT_API flint_status flint_moe_forward(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                         const uint16_t* x, int32_t T, uint16_t* out,
                                         int32_t* topk_ids, float* topk_w, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  flint::Launcher launch;
  return forward_impl(ctx, w, x, T, out, topk_ids, topk_w, workspace, workspace_bytes, stream,
                      launch);
}

FLINT_API flint_status flint_moe_forward_timed(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                               const uint16_t* x, int32_t T, uint16_t* out,
                                               int32_t* topk_ids, float* topk_w, void* workspace,
                                               size_t workspace_bytes, void* stream,
                                               void* const* events, int32_t n_events,
                                               int32_t* n_kernels) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  if (!events || n_events < 16 || !n_kernels)
    return fail(ctx, FLINT_ERR_INVALID_ARG, "events (>= 16) and n_kernels are required");
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(ctx, FLINT_ERR_INVALID_ARG, "NULL event handle");
  flint::Launcher launch;
  launch.events = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  launch.n = n_events;
  const flint_status s = forward_impl(ctx, w, x, T, out, topk_ids, topk_w, workspace,
                                      workspace_bytes, stream, launch);
  *n_kernels = launch.used;
  return s;
}

namespace {

flint_status lowlat_common(flint_moe_ctx* ctx, const flint_moe_weights* w, const uint16_t* wo,
                           const uint16_t* attn, const uint16_t* r, const uint16_t* gamma,
                           const uint16_t* gamma_next, float eps, int32_t T, uint16_t* r_out,
                           uint16_t* n_out, int32_t* topk_ids, float* topk_w, void* workspace,
                           size_t workspace_bytes, int32_t fused, void* stream,
                           flint::Launcher& launch) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  if (!gamma && T != 0) return fail(ctx, FLINT_ERR_INVALID_ARG, "gamma must be non-NULL");
  if (fused != 0 && fused != 1) return fail(ctx, FLINT_ERR_INVALID_ARG, "fused must be 0 or 1");
  NormArgs norm;
  norm.gamma = gamma;
  norm.eps = eps;
  LowLatArgs ll;
  ll.wo = wo;
  ll.attn = attn;
  ll.gamma_next = gamma_next;
  ll.n_out = n_out;
  ll.fused = fused != 0;
  return forward_impl(ctx, w, r, T, r_out, topk_ids, topk_w, workspace, workspace_bytes, stream,
                      launch, norm, false, &ll);
}

}  // namespace

FLINT_API flint_status flint_moe_lowlat_forward(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                                const uint16_t* wo, const uint16_t* attn,
                                                const uint16_t* r, const uint16_t* gamma,
                                                const uint16_t* gamma_next, float eps, int32_t T,
                                                uint16_t* r_out, uint16_t* n_out, int32_t* topk_ids,
                                                float* topk_w, void* workspace,
                                                size_t workspace_bytes, int32_t fused, void* stream) {
  flint::Launcher launch;
  return lowlat_common(ctx, w, wo, attn, r, gamma, gamma_next, eps, T, r_out, n_out, topk_ids,
                       topk_w, workspace, workspace_bytes, fused, stream, launch);
}

FLINT_API flint_status flint_moe_lowlat_forward_timed(
    flint_moe_ctx* ctx, const flint_moe_weights* w, const uint16_t* wo, const uint16_t* attn,
    const uint16_t* r, const uint16_t* gamma, const uint16_t* gamma_next, float eps, int32_t T,
    uint16_t* r_out, uint16_t* n_out, int32_t* topk_ids, float* topk_w, void* workspace,
    size_t workspace_bytes, int32_t fused, void* stream, void* const* events, int32_t n_events,
    int32_t* n_kernels) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  if (!events || n_events < 16 || !n_kernels)
    return fail(ctx, FLINT_ERR_INVALID_ARG, "events (>= 16) and n_kernels are required");
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(ctx, FLINT_ERR_INVALID_ARG, "NULL event handle");
  flint::Launcher launch;
  launch.events = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  launch.n = n_events;
  const flint_status s = lowlat_common(ctx, w, wo, attn, r, gamma, gamma_next, eps, T, r_out, n_out,
                                       topk_ids, topk_w, workspace, workspace_bytes, fused, stream,
                                       launch);
  *n_kernels = launch.used;
  return s;
}

FLINT_API flint_status flint_moe_block_forward(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                               const uint16_t* gamma, float eps, const uint16_t* r,
                                               int32_t T, uint16_t* out, int32_t* topk_ids,
                                               float* topk_w, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  if (!gamma && T != 0) return fail(ctx, FLINT_ERR_INVALID_ARG, "gamma must be non-NULL");
  flint::Launcher launch;
  NormArgs norm;
  norm.gamma = gamma;
  norm.eps = eps;
  return forward_impl(ctx, w, r, T, out, topk_ids, topk_w, workspace, workspace_bytes, stream,
                      launch, norm);
}

FLINT_API flint_status flint_moe_block_forward_timed(
    flint_moe_ctx* ctx, const flint_moe_weights* w, const uint16_t* gamma, float eps,
    const uint16_t* r, int32_t T, uint16_t* out, int32_t* topk_ids, float* topk_w,
    void* workspace, size_t workspace_bytes, void* stream, void* const* events, int32_t n_events,
    int32_t* n_kernels) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  if (!gamma && T != 0) return fail(ctx, FLINT_ERR_INVALID_ARG, "gamma must be non-NULL");
  if (!events || n_events < 16 || !n_kernels)
    return fail(ctx, FLINT_ERR_INVALID_ARG, "events (>= 16) and n_kernels are required");
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(ctx, FLINT_ERR_INVALID_ARG, "NULL event handle");
  flint::Launcher launch;
  launch.events = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  launch.n = n_events;
  NormArgs norm;
  norm.gamma = gamma;
  norm.eps = eps;
  const flint_status s = forward_impl(ctx, w, r, T, out, topk_ids, topk_w, workspace,
                                      workspace_bytes, stream, launch, norm);
  *n_kernels = launch.used;
  return s;
}

// ---------------------------------------------------------------- no-allocation forward

namespace {

// The no-allocation forward's workspace: a file-scope device array, one copy
// per GPU the library runs on, kept until the process ends.  Host code never
// passes `scratch` itself to a kernel (in host code the name is only a
// stand-in); it takes the array's device address on each device once, with
// hipGetSymbolAddress, and uses that address everywhere.
constexpr size_t kScratchBytes = FLINT_MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void* ptr = nullptr;   // scratch's address on the device
  bool zeroed = false;   // a forward has cleared its completion counters
};
std::mutex g_scratch_mu;
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

FLINT_API flint_status flint_moe_forward_noalloc(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                                 const uint16_t* x, int32_t T, uint16_t* out,
                                                 int32_t* topk_ids, float* topk_w, void* stream) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  ctx->last_error.clear();
  if (T < 0 || T > ctx->cfg.max_tokens) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "T=%d outside [0, max_tokens=%d]", T, ctx->cfg.max_tokens);
    return fail(ctx, FLINT_ERR_INVALID_ARG, buf);
  }
  if (T == 0) return FLINT_OK;
  flint_moe_ws_layout L;
  compute_layout(ctx->cfg, T, &L);
  if (T > FLINT_MOE_NOALLOC_MAX_TOKENS || L.total_bytes > kScratchBytes) {
    char buf[192];
    std::snprintf(buf, sizeof buf,
                  "the no-allocation forward takes T <= %d (a %zu-byte device scratch array); "
                  "T=%d needs %zu bytes: use flint_moe_forward with a workspace",
                  FLINT_MOE_NOALLOC_MAX_TOKENS, kScratchBytes, T, L.total_bytes);
    return fail(ctx, FLINT_ERR_UNSUPPORTED, buf);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ctx, FLINT_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ctx, FLINT_ERR_UNSUPPORTED, "device index beyond the library's per-device table");
  void* ws = nullptr;
  bool first = false;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    DeviceScratch& d = g_scratch[dev];
    if (!d.ptr) {
      e = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !d.ptr) {
        d.ptr = nullptr;
        return fail(ctx, FLINT_ERR_HIP, e != hipSuccess ? hipGetErrorString(e)
                                                        : "scratch array has no device address");
      }
    }
    ws = d.ptr;
    first = !d.zeroed;
  }
  // The first forward on a device clears the counters on `stream`, after the
  // arguments have been validated and before its kernels.
  flint::Launcher launch;
  const flint_status s = forward_impl(ctx, w, x, T, out, topk_ids, topk_w, ws, kScratchBytes,
                                      stream, launch, NormArgs(), first);
  if (s == FLINT_OK && first) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch[dev].zeroed = true;
  }
  return s;
}

FLINT_API void flint_moe_destroy(flint_moe_ctx* ctx) { delete ctx; }

FLINT_API const char* flint_moe_status_string(flint_status s) {
  switch (s) {
    case FLINT_OK: return "FLINT_OK";
    case FLINT_ERR_INVALID_ARG: return "FLINT_ERR_INVALID_ARG";
    case FLINT_ERR_UNSUPPORTED: return "FLINT_ERR_UNSUPPORTED";
    case FLINT_ERR_WORKSPACE: return "FLINT_ERR_WORKSPACE";
    case FLINT_ERR_HIP: return "FLINT_ERR_HIP";
  }
  return "FLINT_ERR_UNKNOWN";
}

FLINT_API const char* flint_moe_last_error(const flint_moe_ctx* ctx) {
  return ctx ? ctx->last_error.c_str() : "";
}

// ---------------------------------------------------------------- dense MLP

namespace {

void mlp_layout(const flint_mlp_config& c, int32_t T, flint_mlp_ws_layout* L) {
  const size_t t = (size_t)T, H = (size_t)c.hidden, I = (size_t)c.inter;
  const bool prefill = T > flint::kDecodeMaxT;
  size_t o = 0;
  L->normed = o; o = align_up(o + t * H * sizeof(uint16_t));
  L->h = o;      o = align_up(o + t * I * (prefill ? sizeof(uint16_t) : sizeof(float)));
  L->total_bytes = o;
}

flint_status mlp_fail(flint_mlp_ctx* ctx, flint_status s, const std::string& why) {
  if (ctx) ctx->last_error = why;
  return s;
}

flint_status mlp_forward_impl(flint_mlp_ctx* ctx, const uint16_t* w13, const uint16_t* w2,
                              const uint16_t* gamma, float eps, const uint16_t* x, int32_t T,
                              uint16_t* out, void* workspace, size_t workspace_bytes, void* stream,
                              flint::Launcher& launch) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  ctx->last_error.clear();
  const flint_mlp_config& c = ctx->cfg;
  if (T < 0 || T > c.max_tokens) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "T=%d outside [0, max_tokens=%d]", T, c.max_tokens);
    return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, buf);
  }
  if (T == 0) return FLINT_OK;
  if (!w13 || !w2 || !x || !out || !workspace)
    return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "w13, w2, x, out and workspace must be non-NULL");
  const void* p16[] = {w13, w2, x, out};
  for (const void* p : p16)
    if (!aligned(p, 16)) return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (gamma && !aligned(gamma, 16))
    return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "gamma must be 16-byte aligned");
  if (gamma && !(std::isfinite(eps) && eps >= 0.f))
    return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!aligned(workspace, kAlign))
    return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t act_bytes = (size_t)T * c.hidden * sizeof(uint16_t);
  if (ranges_overlap(x, act_bytes, out, act_bytes))
    return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "out overlaps x");
  flint_mlp_ws_layout L;
  mlp_layout(c, T, &L);
  if (workspace_bytes < L.total_bytes) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "workspace of %zu bytes, %zu needed for T=%d", workspace_bytes,
                  L.total_bytes, T);
    return mlp_fail(ctx, FLINT_ERR_WORKSPACE, buf);
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  flint::DenseArgs a{};
  a.x = x;
  a.out = out;
  a.w13 = w13;
  a.w2 = w2;
  a.T = T;
  a.inter = c.inter;
  const bool prefill = T > flint::kDecodeMaxT;
  if (prefill)
    a.h16 = reinterpret_cast<_Float16*>(ws + L.h);
  else
    a.h = reinterpret_cast<float*>(ws + L.h);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (gamma) {
    uint16_t* normed = reinterpret_cast<uint16_t*>(ws + L.normed);
    flint::launch_rmsnorm(x, gamma, eps, normed, T, s, launch);
    a.x = normed;
    a.resid = x;
  }
  const hipError_t err = prefill ? flint::launch_dense_prefill(a, s, launch)
                                 : flint::launch_dense_decode(a, s, launch);
  if (err != hipSuccess) return mlp_fail(ctx, FLINT_ERR_HIP, hipGetErrorString(err));
  return FLINT_OK;
}

}  // namespace

FLINT_API flint_status flint_mlp_init(const flint_mlp_config* cfg, flint_mlp_ctx** ctx_out) {
  if (!cfg || !ctx_out) return FLINT_ERR_INVALID_ARG;
  if (cfg->hidden <= 0 || cfg->max_tokens <= 0 || cfg->inter <= 0) return FLINT_ERR_INVALID_ARG;
  if (cfg->inter % flint::kDenseChunk != 0 || cfg->inter > flint::kDenseMaxInter)
    return FLINT_ERR_INVALID_ARG;
  if (cfg->hidden != flint::kHidden) return FLINT_ERR_UNSUPPORTED;
  flint_mlp_ctx* ctx = new (std::nothrow) flint_mlp_ctx;
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  ctx->cfg = *cfg;
  *ctx_out = ctx;
  return FLINT_OK;
}

FLINT_API size_t flint_mlp_workspace_bytes(const flint_mlp_ctx* ctx, int32_t T) {
  if (!ctx || T <= 0) return 0;
  flint_mlp_ws_layout L;
  mlp_layout(ctx->cfg, T, &L);
  return L.total_bytes;
}

FLINT_API flint_status flint_mlp_workspace_layout(const flint_mlp_ctx* ctx, int32_t T,
                                                  flint_mlp_ws_layout* layout) {
  if (!ctx || !layout || T <= 0) return FLINT_ERR_INVALID_ARG;
  mlp_layout(ctx->cfg, T, layout);
  return FLINT_OK;
}

FLINT_API flint_status flint_mlp_forward(flint_mlp_ctx* ctx, const uint16_t* w13, const uint16_t* w2,
                                         const uint16_t* gamma, float eps, const uint16_t* x,
                                         int32_t T, uint16_t* out, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  flint::Launcher launch;
  return mlp_forward_impl(ctx, w13, w2, gamma, eps, x, T, out, workspace, workspace_bytes, stream,
                          launch);
}

FLINT_API flint_status flint_mlp_forward_timed(flint_mlp_ctx* ctx, const uint16_t* w13,
                                               const uint16_t* w2, const uint16_t* gamma, float eps,
                                               const uint16_t* x, int32_t T, uint16_t* out,
                                               void* workspace, size_t workspace_bytes,
                                               void* stream, void* const* events, int32_t n_events,
                                               int32_t* n_kernels) {
  if (!ctx) return FLINT_ERR_INVALID_ARG;
  if (!events || n_events < 16 || !n_kernels)
    return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "events (>= 16) and n_kernels are required");
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return mlp_fail(ctx, FLINT_ERR_INVALID_ARG, "NULL event handle");
  flint::Launcher launch;
  launch.events = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  launch.n = n_events;
  const flint_status st = mlp_forward_impl(ctx, w13, w2, gamma, eps, x, T, out, workspace,
                                           workspace_bytes, stream, launch);
  *n_kernels = launch.used;
  return st;
}

FLINT_API void flint_mlp_destroy(flint_mlp_ctx* ctx) { delete ctx; }

FLINT_API const char* flint_mlp_last_error(const flint_mlp_ctx* ctx) {
  return ctx ? ctx->last_error.c_str() : "";
}
