/*
 * flint_moe.h — C ABI of the MI355X (gfx950) Flint MoE feed-forward layer.
 *
 * The layer, as the pages define it:
 *   - hidden size 2048; 256 routed experts chosen by sigmoid top-6 routing,
 *     plus one always-on shared expert ("vLLM Day-0 Support for Recursive's
 *     Flint", section "Flint Model Architecture", bullet "MoE Structure";
 *     "Flint on Arc Pro B70", section "Setup"; "RecursiveSI/flint — vLLM
 *     serving recipe", section "Guide / Overview");
 *   - the router and expert GEMVs read only the selected experts' weights
 *     (Day-0 page, section "Optimization Strategies", bullet "Small-batch MoE
 *     Kernels");
 *   - each expert is SwiGLU with SiLU(g) = g / (1 + exp(-g)) ("Flint on Arc
 *     Pro B70", section "norm.py: Triton kernels that assumed CUDA");
 *   - routed outputs are combined by their routing weights and added to the
 *     shared expert's output (Day-0 page, section "Optimization Strategies",
 *     bullet "Low-Latency Decode Path");
 *   - the NVFP4 checkpoint runs weight-only (W4A16) with bf16 activations
 *     (Day-0 page, section "Flint Model Overview and Capabilities").
 *
 * For token t with bf16 input x_t[H]:
 *   z_e   = sum_k Wr[e,k] x_t[k] + b_e                    (fp32 accumulate)
 *   s_e   = 1 / (1 + exp(-z_e))
 *   S_t   = the top_k experts by s_e, ties to the lower index
 *   w_j   = s_{S_j} / sum_i s_{S_i}   (renormalize = 1)  else s_{S_j};  times routed_scale
 *   h_e   = silu(W13_e[0:I] x_t) * (W13_e[I:2I] x_t)       (fp32 accumulate)
 *   out_t = W2_sh h_sh + sum_j w_j W2_{S_j} h_{S_j}          (fp32, rounded once to bf16, RNE)
 * Intermediate precision: for T <= 64 (the decode kernels) h is kept in fp32
 * and never rounded with bf16 weights; with NVFP4 weights (W4A16: 16-bit
 * activations) it is rounded once to bf16 (RNE) between the two GEMVs.  For T > 64 (the MFMA GEMMs) h and each slot's
 * unweighted W2 h cross between launches as fp16 carrying a 2^-8 bias (the
 * stored value is fp16(v * 2^-8)): 11 significant bits, finite for
 * |h|, |W2 h| < 65504 * 2^8 = 1.68e7, values below 2^-6 kept to an absolute
 * 2^-17; w2 enters those GEMMs as fp16 (exact for 2^-14 <= |w| <= 65504).
 *
 * Conventions for every call:
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - "device" pointers point to memory on the GPU that is current when the
 *     call is made; the library never dereferences them on the host.
 *   - The caller owns every buffer (weights, x, out, routing outputs,
 *     workspace).  The library allocates no device memory.
 *   - flint_moe_forward is asynchronous: it validates its arguments on the
 *     host, enqueues kernels on `stream` and returns.  Argument errors are
 *     reported before anything is enqueued; a failed launch returns
 *     FLINT_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - A context may be used by one stream at a time; a workspace may be used
 *     by one forward at a time.  Forwards that overlap on one workspace race.
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct flint_moe_ctx flint_moe_ctx; /* opaque, host memory */

/* Bytes at the start of every workspace that hold the kernels' completion
 * counters.  They must be zero before a workspace is first used; every
 * completed forward leaves them zero again. */
#define FLINT_MOE_WS_HEADER_BYTES 21504

typedef enum flint_status {
  FLINT_OK = 0,
  FLINT_ERR_INVALID_ARG = 1, /* NULL / misaligned / out-of-range argument */
  FLINT_ERR_UNSUPPORTED = 2, /* shape or format the library has no kernels for */
  FLINT_ERR_WORKSPACE = 3,   /* workspace smaller than flint_moe_workspace_bytes() */
  FLINT_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} flint_status;

typedef enum flint_weight_format {
  FLINT_W_BF16 = 0,  /* bf16 weights */
  FLINT_W_NVFP4 = 1  /* E2M1 elements, E4M3FN scale per 16 K-elements, fp32 scale per tensor */
} flint_weight_format;

/* Host struct, copied by flint_moe_init. */
typedef struct flint_moe_config {
  int32_t hidden;       /* H: must be 2048 */
  int32_t n_experts;    /* E: 1..256 routed experts (256 for Flint) */
  int32_t top_k;        /* k: 1..min(8, E) (6 for Flint) */
  int32_t inter;        /* I: must be 512 (the shared expert has the same shape) */
  int32_t max_tokens;   /* >= 1: largest T a forward may be called with */
  int32_t renormalize;  /* 1: w_j = s_j / sum of the k selected scores; 0: w_j = s_j */
  float routed_scale;   /* multiplies every routed weight (1.0 for Flint); finite */
  int32_t format;       /* flint_weight_format */
} flint_moe_config;

/* One bank of experts, n tensors stacked on the leading axis (n = E for the
 * routed bank, n = 1 for the shared expert).  All device pointers, 16-byte
 * aligned.
 *   BF16 : w13 = bf16 [n][2I][H]   rows [0,I) gate, [I,2I) up; K (= H) contiguous
 *          w2  = bf16 [n][H][I]    K (= I) contiguous
 *          scale / gscale pointers ignored (may be NULL)
 *   NVFP4: w13 = uint8 [n][2I][H/2]  two E2M1 codes per byte, even k in the
 *                                    low nibble, nibble bit 3 = sign
 *          w2  = uint8 [n][H][I/2]
 *          w13_scale = uint8 [n][2I][H/16], w2_scale = uint8 [n][H][I/16] (16-byte aligned too)
 *                      E4M3FN, one per 16 consecutive K elements
 *          w13_gscale, w2_gscale = fp32 [n], one per tensor
 *          element value = e2m1(code) * e4m3(scale) * gscale            */
typedef struct flint_expert_bank {
  const void* w13;
  const void* w2;
  const uint8_t* w13_scale;
  const uint8_t* w2_scale;
  const float* w13_gscale;
  const float* w2_gscale;
} flint_expert_bank;

typedef struct flint_moe_weights {
  const uint16_t* router_w; /* device, bf16 [E][H], row-major; bf16 in every format */
  const float* router_b;    /* device, fp32 [E] added to the logit before the sigmoid, or NULL */
  flint_expert_bank routed; /* n = E */
  flint_expert_bank shared; /* n = 1 */
} flint_moe_weights;

/* Byte offsets of the regions of a workspace sized for T tokens.  Exposed so
 * that tests can read the intermediate results of one forward (a region is
 * valid once the forward that wrote it has completed). */
typedef struct flint_moe_ws_layout {
  size_t total_bytes;
  size_t header;     /* FLINT_MOE_WS_HEADER_BYTES of uint32 completion counters; zero before
                        first use and after every completed forward */
  size_t logits;     /* fp32 [T][E]: z (router GEMV + bias) */
  size_t topk_ids;   /* int32 [T][k]: selected experts in rank order */
  size_t topk_w;     /* fp32 [T][k]: routing weights */
  size_t route;      /* int32 routing table (the token -> expert bucketing):
                          [0]                    |U|, the number of distinct selected experts
                          [1, 1+E)               U, ascending (first |U| entries valid)
                          [1+E, 2+2E)            off: slots of U[a] are slots[off[a], off[a+1]),
                                                 off[|U|] = T*k
                          [2+2E, 2+2E+T*k)       slots s = t*k + j grouped by U, ascending
                                                 within a group */
  size_t h;          /* [T*k + T][I]: h of slot s in row s; h of the shared expert for
                        token t in row T*k + t; fp32 rows with bf16 weights, bf16 rows
                        (I values, packed from the start of the region) with NVFP4 */
  size_t extra;      /* path-private scratch (prefill-sized T only) */
  size_t normed;     /* bf16 [T][H]: the block's normalised input n (flint_moe_block_forward
                        and flint_moe_lowlat_forward; unused by flint_moe_forward) */
  size_t resid1;     /* bf16 [T][H]: r1 = bf16(r + Wo a) (flint_moe_lowlat_forward; sized for
                        T <= 8 only) */
  size_t norm_part;  /* fp32 [256][T]: per down block, per token partial sums of squares of
                        r_out (flint_moe_lowlat_forward with gamma_next; T <= 8 only) */
  size_t items;      /* int32 [min(E, T*k)][2 + T] item records (T <= 64): record a < |U| is
                        {U[a], c = its slot count, its c slots ascending} */
} flint_moe_ws_layout;

/* Validate `cfg` and create a context.  Touches no GPU state.
 * Returns INVALID_ARG for NULL pointers or out-of-range fields, UNSUPPORTED
 * for shapes other than H = 2048, I = 512.  *ctx_out is set only on FLINT_OK. */
flint_status flint_moe_init(const flint_moe_config* cfg, flint_moe_ctx** ctx_out);

/* Bytes of workspace a forward of T tokens needs (0 for T <= 0 or NULL ctx).
 * Its first FLINT_MOE_WS_HEADER_BYTES (the header) must be zero before the
 * workspace is used for the first time; every completed forward leaves them
 * zero again. */
size_t flint_moe_workspace_bytes(const flint_moe_ctx* ctx, int32_t T);

/* Fill `layout` with the region offsets of a workspace for T tokens. */
flint_status flint_moe_workspace_layout(const flint_moe_ctx* ctx, int32_t T,
                                        flint_moe_ws_layout* layout);

/* One layer forward over T tokens.
 *   x         device bf16 [T][H] (16-byte aligned)
 *   out       device bf16 [T][H] (16-byte aligned; must not overlap x)
 *   topk_ids  device int32 [T][k] or NULL: receives the selected experts
 *   topk_w    device fp32  [T][k] or NULL: receives their routing weights
 *   workspace device, >= flint_moe_workspace_bytes(ctx, T) bytes, 256-byte aligned
 *   stream    hipStream_t (passed as void*; NULL = the null stream)
 * T == 0 is a no-op returning FLINT_OK.  T < 0 or T > max_tokens: INVALID_ARG.
 * NULL or misaligned pointers, overlapping x and out, and (NVFP4) a NULL scale
 * or tensor-scale pointer: INVALID_ARG.  workspace_bytes below
 * flint_moe_workspace_bytes(ctx, T): FLINT_ERR_WORKSPACE.  NVFP4 weights with
 * T > 64: FLINT_ERR_UNSUPPORTED (the NVFP4 kernels are the decode-sized ones).
 * NaN/Inf inputs are not checked. */
flint_status flint_moe_forward(flint_moe_ctx* ctx, const flint_moe_weights* w,
                               const uint16_t* x, int32_t T, uint16_t* out,
                               int32_t* topk_ids, float* topk_w,
                               void* workspace, size_t workspace_bytes, void* stream);

/* flint_moe_forward with per-kernel timing, for measurement.  `events` holds
 * n_events hipEvent_t handles (passed as void*, created by the caller with
 * timing enabled).  Kernel i of the chosen path is launched with events
 * 2i and 2i+1 as its start and stop events (hipExtLaunchKernelGGL), so they
 * take the start and end timestamps of that kernel's own execution.
 * *n_kernels receives the number of kernels the path launched (at most 8).
 * Requires n_events >= 16.  Not for use under stream capture.  Same
 * arguments, validation and results as flint_moe_forward otherwise. */
flint_status flint_moe_forward_timed(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                     const uint16_t* x, int32_t T, uint16_t* out,
                                     int32_t* topk_ids, float* topk_w, void* workspace,
                                     size_t workspace_bytes, void* stream,
                                     void* const* events, int32_t n_events, int32_t* n_kernels);

/* The pre-norm block around the layer, with the norm and the residual add
 * fused into the layer's first and last kernels.  Flint is a pre-norm decoder
 * ("vLLM Day-0 Support for Recursive's Flint", section "Flint Model
 * Architecture"): the block input r is normalised by RMSNorm, whose output is
 * bf16 ("Flint on Arc Pro B70", section "norm.py: Triton kernels that assumed
 * CUDA"), the layer runs on it, and its output is added back to r:
 *   n_t   = bf16_rne( r_t[k] / sqrt(mean_k r_t[k]^2 + eps) * gamma[k] )   (fp32)
 *   out_t = bf16_rne( r_t + layer(n_t) )        (the layer's fp32 sum, then + r_t, one rounding)
 *   r         device bf16 [T][H] (16-byte aligned): the residual stream
 *   gamma     device bf16 [H] (16-byte aligned): the RMSNorm gain
 *   eps       finite, >= 0 (Flint: 1e-6)
 *   out       device bf16 [T][H] (16-byte aligned; must not overlap r)
 * n_t is left in the workspace region `normed`; the other arguments, the
 * validation and the errors are those of flint_moe_forward.  The decode path
 * (T <= 64) launches no extra kernel: the router kernel normalises the rows it
 * stages, and the down kernel adds r.  Prefill-sized T adds one norm kernel. */
flint_status flint_moe_block_forward(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                     const uint16_t* gamma, float eps, const uint16_t* r,
                                     int32_t T, uint16_t* out, int32_t* topk_ids, float* topk_w,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* flint_moe_block_forward with the per-kernel timing of flint_moe_forward_timed. */
flint_status flint_moe_block_forward_timed(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                           const uint16_t* gamma, float eps, const uint16_t* r,
                                           int32_t T, uint16_t* out, int32_t* topk_ids,
                                           float* topk_w, void* workspace, size_t workspace_bytes,
                                           void* stream, void* const* events, int32_t n_events,
                                           int32_t* n_kernels);

/* flint_moe_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its kernels, arguments, validation and
 * results are those of flint_moe_forward; the workspace is instead a static
 * device array of FLINT_MOE_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends.  The call allocates nothing.
 *   - T <= FLINT_MOE_NOALLOC_MAX_TOKENS (the decode-sized batches); larger T
 *     returns FLINT_ERR_UNSUPPORTED (use flint_moe_forward).
 *   - The first call on a device zeroes the array's completion counters on
 *     `stream`; every completed forward leaves them zero again.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's intermediate results.  Calls that overlap on one GPU (several
 *     streams or threads at once) race: serialise them. */
#define FLINT_MOE_NOALLOC_SCRATCH_BYTES 2097152
#define FLINT_MOE_NOALLOC_MAX_TOKENS 64
flint_status flint_moe_forward_noalloc(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                       const uint16_t* x, int32_t T, uint16_t* out,
                                       int32_t* topk_ids, float* topk_w, void* stream);

/* The low-latency decode path ("vLLM Day-0 Support for Recursive's Flint",
 * section "Optimization Strategies", bullet "Low-Latency Decode Path": for up
 * to 8 requests the MoE layer's routing and expert combine are fused into the
 * neighbouring GEMV kernels).  Around the pre-norm block it computes, per
 * token, the attention output projection with its residual add before the
 * layer and the next layer's norm after it (Flint: 49 pre-norm layers, GQA
 * with 32 query heads, "Flint Model Architecture"):
 *   r1    = bf16_rne( r + Wo a )                     (fp32 accumulate, one rounding)
 *   n     = bf16_rne( RMSNorm(r1) * gamma )          (as flint_moe_block_forward)
 *   r_out = bf16_rne( r1 + layer(n) )
 *   n_out = bf16_rne( RMSNorm(r_out) * gamma_next )  (only with gamma_next)
 *   wo     device bf16 [H][4096] (row-major: output row o has K = 4096 contiguous)
 *   attn   device bf16 [T][4096]: the attention output (32 heads x 128)
 *   r      device bf16 [T][H]: the residual stream entering the projection's add
 *   gamma  device bf16 [H]: the layer's RMSNorm gain;  eps finite, >= 0 (both norms)
 *   gamma_next device bf16 [H] or NULL: the next layer's input-norm gain
 *   r_out  device bf16 [T][H]: the residual stream leaving the layer (no overlap with r, attn)
 *   n_out  device bf16 [T][H] or NULL (NULL exactly when gamma_next is NULL): the next
 *          layer's normalised input (no overlap with r, r_out)
 *   fused  1: three launches (projection + residual add + norm + router GEMV + routing;
 *          gate/up; down + combine + residual add + next norm);
 *          0: the same arithmetic in five launches (projection; norm + router + routing;
 *          gate/up; down; next norm), for comparison
 * T <= 8 (FLINT_ERR_UNSUPPORTED above); all 16-byte aligned; r1 is left in the
 * workspace region `resid1` and n in `normed`.  The other arguments, the
 * validation and the errors are those of flint_moe_forward. */
flint_status flint_moe_lowlat_forward(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                      const uint16_t* wo, const uint16_t* attn, const uint16_t* r,
                                      const uint16_t* gamma, const uint16_t* gamma_next, float eps,
                                      int32_t T, uint16_t* r_out, uint16_t* n_out,
                                      int32_t* topk_ids, float* topk_w, void* workspace,
                                      size_t workspace_bytes, int32_t fused, void* stream);

/* flint_moe_lowlat_forward with the per-kernel timing of flint_moe_forward_timed. */
flint_status flint_moe_lowlat_forward_timed(flint_moe_ctx* ctx, const flint_moe_weights* w,
                                            const uint16_t* wo, const uint16_t* attn,
                                            const uint16_t* r, const uint16_t* gamma,
                                            const uint16_t* gamma_next, float eps, int32_t T,
                                            uint16_t* r_out, uint16_t* n_out, int32_t* topk_ids,
                                            float* topk_w, void* workspace,
                                            size_t workspace_bytes, int32_t fused, void* stream,
                                            void* const* events, int32_t n_events,
                                            int32_t* n_kernels);

/* Release a context.  NULL is allowed. */
void flint_moe_destroy(flint_moe_ctx* ctx);

/* ------------------------------------------------------------------------
 * Dense MLP of Flint's first two layers, which use a dense MLP in place of the
 * MoE ("vLLM Day-0 Support for Recursive's Flint", section "Flint Model
 * Architecture", bullet "MoE Structure").  Its form is read as the experts'
 * SwiGLU ("Flint on Arc Pro B70", section "norm.py: Triton kernels that
 * assumed CUDA"); its intermediate size I_d is not on the pages and is a
 * parameter here.  For token t with bf16 input x_t[H]:
 *   h_t   = silu(W13[0:I_d] x_t) * (W13[I_d:2 I_d] x_t)    (fp32, never rounded for T <= 64)
 *   out_t = bf16_rne( W2 h_t )                             (fp32 accumulate)
 * and with a norm gain (the pre-norm block, as for flint_moe_block_forward):
 *   out_t = bf16_rne( r_t + W2 h(n_t) ),  n_t = bf16_rne(RMSNorm(r_t) * gamma)
 * T <= 64 runs GEMV kernels; larger T runs MFMA GEMMs that keep h in fp16
 * between the two products, with the 2^-8 bias of the layer's prefill path
 * (finite for |h| < 1.68e7).  Same conventions as the layer above (caller-owned
 * memory, asynchronous on `stream`, host-side validation). */
typedef struct flint_mlp_ctx flint_mlp_ctx; /* opaque, host memory */

typedef struct flint_mlp_config {
  int32_t hidden;      /* H: must be 2048 */
  int32_t inter;       /* I_d: a multiple of 512 in [512, 32768] */
  int32_t max_tokens;  /* >= 1 */
} flint_mlp_config;

typedef struct flint_mlp_ws_layout {
  size_t total_bytes;
  size_t normed;  /* bf16 [T][H]: n (pre-norm block only) */
  size_t h;       /* [T][I_d]: fp32 for T <= 64, fp16 above */
} flint_mlp_ws_layout;

/* INVALID_ARG for NULL or out-of-range fields, UNSUPPORTED for H != 2048. */
flint_status flint_mlp_init(const flint_mlp_config* cfg, flint_mlp_ctx** ctx_out);
size_t flint_mlp_workspace_bytes(const flint_mlp_ctx* ctx, int32_t T);  /* 0 for T <= 0 */
flint_status flint_mlp_workspace_layout(const flint_mlp_ctx* ctx, int32_t T,
                                        flint_mlp_ws_layout* layout);

/* One forward over T tokens.
 *   w13   device bf16 [2 I_d][H] (rows [0, I_d) gate, [I_d, 2 I_d) up), 16-byte aligned
 *   w2    device bf16 [H][I_d], 16-byte aligned
 *   gamma device bf16 [H] or NULL: NULL runs the bare MLP on x; otherwise x is the
 *         residual stream r and the pre-norm block is computed (eps finite, >= 0)
 *   x     device bf16 [T][H];  out device bf16 [T][H] (must not overlap x)
 *   workspace device, >= flint_mlp_workspace_bytes(ctx, T), 256-byte aligned
 * T == 0 is a no-op; T < 0 or T > max_tokens: INVALID_ARG. */
flint_status flint_mlp_forward(flint_mlp_ctx* ctx, const uint16_t* w13, const uint16_t* w2,
                               const uint16_t* gamma, float eps, const uint16_t* x, int32_t T,
                               uint16_t* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* flint_mlp_forward with the per-kernel timing of flint_moe_forward_timed. */
flint_status flint_mlp_forward_timed(flint_mlp_ctx* ctx, const uint16_t* w13, const uint16_t* w2,
                                     const uint16_t* gamma, float eps, const uint16_t* x,
                                     int32_t T, uint16_t* out, void* workspace,
                                     size_t workspace_bytes, void* stream, void* const* events,
                                     int32_t n_events, int32_t* n_kernels);

void flint_mlp_destroy(flint_mlp_ctx* ctx);                   /* NULL-safe */
const char* flint_mlp_last_error(const flint_mlp_ctx* ctx);  /* "" if none */

/* ------------------------------------------------------------------------
 * Measurement probe (not part of the layer).  Reads `bytes` bytes at `src`
 * once, as 16-byte non-temporal vector loads: one-shot blocks of 256 threads,
 * each owning a contiguous 64 KiB chunk and issuing all of its loads before
 * using any (the access the layer's gate/up weight loads make), and XORs the
 * 32-bit words block b read into sink[b % FLINT_MOE_CALIB_SINK_WORDS] with
 * atomic XORs.  With a zeroed sink, the XOR over the whole sink afterwards
 * equals the XOR of every 32-bit word of the buffer.  Used to measure the HBM
 * read rate a plain stream reaches, beside the nominal peak.
 *   src   device, 16-byte aligned;  bytes: a positive multiple of 16
 *   sink  device uint32 [FLINT_MOE_CALIB_SINK_WORDS], updated (XOR) in place
 * Asynchronous on `stream`.  INVALID_ARG for NULL / misaligned / bad sizes,
 * FLINT_ERR_HIP if the launch fails. */
#define FLINT_MOE_CALIB_SINK_WORDS 2048
flint_status flint_moe_calib_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                         void* stream);

/* Static name of a status code. */
const char* flint_moe_status_string(flint_status s);

/* Human-readable reason for the last non-OK status returned with this
 * context ("" if none).  Valid until the next call with the context. */
const char* flint_moe_last_error(const flint_moe_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_MOE_H */
