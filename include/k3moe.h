/*
 * k3moe -- forward pass of the Kimi K3 LatentMoE layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer (Kimi K3 course, lesson 6 "LatentMoE", section "show me the actual equation"):
 *
 *   eq. 11   u = sum_{i in T_k(x)} p_i E_i^routed(W_down x)          in R^l
 *            y = sum_{j=1..N_s} E_j^shared(x) + W_up RMSNorm(u)       in R^d
 *   eq. 13   s = Sigmoid(W_r x);  T = argtopk(s + b);  p_j = s_j / sum_{r in T} s_r
 *
 * Routed and shared experts are SwiGLU GLUs (gate, up, down matrices; lesson 6, "Deriving the
 * headline number"); the bias b steers selection only (eq. 13); the RMSNorm sits between the
 * aggregation and W_up (lesson 6, "What extreme sparsity breaks"). With latent_moe = 0 the layer
 * is the conventional full-width MoE the lesson compares against (no W_down, W_up, RMSNorm;
 * experts at width d; table "What scales with what").
 *
 * Number formats. Every weight matrix is MXFP4: E2M1 codes with one E8M0 scale per 32 values
 * along the reduction axis (the K3 weights are 4-bit MX; "Serving K3, 01 architecture", section
 * on quantisation as a property of the artefact). Activations enter and leave as bf16. The routed
 * GEMM inputs (latent z and GLU hidden h) are rounded to bf16 (K3MOE_ACT_BF16) or encoded MXFP8
 * E4M3 in blocks of 32 along the feature axis (K3MOE_ACT_MXFP8; the K3 activations are MXFP8).
 * The shared-expert hidden and the normalised n are bf16; accumulation is fp32.
 *
 * Canonical MX matrix (the exchange format handed to the packer), for W[N, K] mapping K inputs
 * to N outputs:  codes  uint8 [N][K/2], element 2i in the low nibble;
 *                scales uint8 [N][K/32], E8M0 (value 2^(byte - 127)).
 *
 * Memory and streams. Every pointer argument named *_dev or inside the structs below is a device
 * pointer (HIP global memory) owned by the caller. The library never allocates or frees device
 * memory; it keeps the packed-weight pointer given to k3moe_pack_weights. `stream` is a
 * hipStream_t passed as void* (NULL = the legacy default stream). All device work is enqueued
 * asynchronously on that stream; no call blocks on the device except k3moe_profile_end.
 * A context may be used from one host thread and one stream at a time.
 *
 * Errors. Functions return K3MOE_OK (0) or a negative status. Argument and state checks run
 * before any work is enqueued; on error nothing is enqueued. A failed HIP launch returns
 * K3MOE_EHIP. k3moe_last_error() gives a message for the last failure on a context (or of
 * k3moe_create when called with NULL).
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct k3moe_ctx k3moe_ctx;

enum {
  K3MOE_OK = 0,
  K3MOE_EINVAL = -1,       /* bad argument: null pointer, bad size, bad config */
  K3MOE_ESTATE = -2,       /* call out of order: forward before all weights are packed, ... */
  K3MOE_ETOOBIG = -3,      /* T above max_tokens, or sizes beyond the supported limits */
  K3MOE_EHIP = -4,         /* a HIP runtime call or kernel launch failed */
  K3MOE_EUNSUPPORTED = -5  /* valid request the library does not implement */
};

enum { K3MOE_ACT_BF16 = 0, K3MOE_ACT_MXFP8 = 1 };

typedef struct {
  int32_t d_model;        /* d: model width (multiple of 32) */
  int32_t latent;         /* l: latent width the routed experts work in (multiple of 32); ignored
                             when latent_moe = 0 (experts then work at width d) */
  int32_t hidden;         /* routed expert GLU hidden (multiple of 32) */
  int32_t n_experts;      /* E: routed experts, 1..2048 */
  int32_t top_k;          /* k: experts per token, 1..min(E, 64) */
  int32_t n_shared;       /* N_s: shared experts, 0..4 */
  int32_t shared_hidden;  /* shared expert GLU hidden (multiple of 32) */
  int32_t latent_moe;     /* 1: LatentMoE (eq. 11); 0: conventional full-width MoE */
  int32_t act;            /* K3MOE_ACT_BF16 or K3MOE_ACT_MXFP8 for the routed GEMM inputs z, h */
  int32_t max_tokens;     /* largest T a forward call may pass (sizes the workspace) */
  float rms_eps;          /* epsilon inside the RMSNorm square root */
  int32_t lora_rank;      /* r of the BF16 LoRA deltas on every routed expert matrix: 0 (none) or a
                             multiple of 8 up to 32 */
} k3moe_config;

/* One canonical MXFP4 matrix on the device (layout in the header comment). */
typedef struct {
  const void* codes;
  const void* scales;
} k3moe_mx;

/*
 * BF16 LoRA deltas of one routed expert ("Serving K3, 01 architecture": fine-tuning ships BF16 LoRA
 * deltas over the MXFP4 base weights). Each expert matrix W [N, K] becomes W + B A with A [r, K] and
 * B [N, r], both bf16 row-major device arrays (r = lora_rank; any scaling folded into B):
 *   a_gate, a_up [r, le]; b_gate, b_up [hidden, r]; a_down [r, hidden]; b_down [le, r].
 * The product is applied as B (A v) in fp32 on the activation v the base matrix sees.
 */
typedef struct {
  const void* a_gate;
  const void* b_gate;
  const void* a_up;
  const void* b_up;
  const void* a_down;
  const void* b_down;
} k3moe_lora;

/*
 * Weights handed to k3moe_pack_weights. A call packs the dense part when include_dense != 0 and
 * the routed experts [routed_first, routed_first + routed_count); any number of calls may split
 * the experts. Shapes (le = latent when latent_moe = 1, else d_model):
 *   w_router [E, d]; w_down [l, d] and w_up [d, l] (latent_moe only);
 *   router_bias fp32 [E]; rms_gamma fp32 [l] (latent_moe only);
 *   sh_gate[j], sh_up[j] [shared_hidden, d]; sh_down[j] [d, shared_hidden], j < n_shared;
 *   gate[i], up[i] [hidden, le]; down[i] [le, hidden] for expert routed_first + i.
 * The device memory these point to must stay valid until the packing work on the stream is done.
 */
typedef struct {
  int32_t include_dense;
  k3moe_mx w_router;
  k3moe_mx w_down;
  k3moe_mx w_up;
  const float* router_bias;
  const float* rms_gamma;
  const k3moe_mx* sh_gate;  /* host array of n_shared entries (device pointers inside) */
  const k3moe_mx* sh_up;
  const k3moe_mx* sh_down;
  int32_t routed_first;
  int32_t routed_count;
  const k3moe_mx* gate;     /* host arrays of routed_count entries */
  const k3moe_mx* up;
  const k3moe_mx* down;
  const k3moe_lora* lora;   /* host array of routed_count entries; required when lora_rank > 0 */
} k3moe_weights;

/*
 * Optional copies of intermediate results (device pointers; NULL = not captured), written by
 * k3moe_forward_ex on the stream after the forward. Row order of h, h_f32 and expert_out is the
 * dispatched (expert-contiguous) order; inv maps (t, j) to that row.
 *   scores     fp32 [T, E]      s = Sigmoid(W_r x)
 *   topk_idx   int32 [T, k]     selected experts, descending s + b, ties to the lower id
 *   topk_p     fp32 [T, k]      p, renormalised over the selection from s
 *   counts     int32 [E]        rows per expert
 *   offsets    int32 [E + 1]    exclusive prefix sum of counts
 *   perm       int32 [T * k]    token of each dispatched row; rows ordered (expert, token)
 *   inv        int32 [T, k]     dispatched row of (t, j)
 *   z          [T, l]           W_down x after its quantisation point: bf16, or E4M3 codes (uint8)
 *   z_scales   uint8 [T, l/32]  E8M0 scales of z (MXFP8 only)
 *   z_f32      fp32 [T, l]      W_down x before quantisation
 *   h          [T*k, hidden]    GLU hidden after quantisation: bf16, or E4M3 codes
 *   h_scales   uint8 [T*k, hidden/32]
 *   h_f32      fp32 [T*k, hidden]  GLU hidden before quantisation
 *   expert_out fp32 [T*k, le]   routed expert outputs
 *   u          fp32 [T, le]     p-weighted combine (eq. 11)
 *   n          bf16 [T, l]      RMSNorm(u) (latent_moe only)
 *   hs         bf16 [T, n_shared * shared_hidden]  shared GLU hiddens, expert-major columns
 */
typedef struct {
  float* scores;
  int32_t* topk_idx;
  float* topk_p;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  void* z;
  uint8_t* z_scales;
  float* z_f32;
  void* h;
  uint8_t* h_scales;
  float* h_f32;
  float* expert_out;
  float* u;
  void* n;
  void* hs;
} k3moe_taps;

/* Validate `cfg` and create a context. *out receives the context (NULL on failure). */
int k3moe_create(const k3moe_config* cfg, k3moe_ctx** out);

/* Release a context (host memory and HIP events only; NULL is a no-op). */
void k3moe_destroy(k3moe_ctx* ctx);

/* Message for the last failure on `ctx`, or of k3moe_create if ctx is NULL. Never NULL. */
const char* k3moe_last_error(const k3moe_ctx* ctx);

/* Bytes of the packed weight buffer the caller allocates for k3moe_pack_weights (0 on error).
   The routed experts take exactly their canonical MXFP4 size when every dimension is a multiple
   of 128 (15,722,348,544 bytes at E = 896, l = 3584, hidden = 3072). */
size_t k3moe_weight_bytes(const k3moe_ctx* ctx);

/* Bytes of device workspace a forward call needs at T = max_tokens (0 on error). */
size_t k3moe_workspace_bytes(const k3moe_ctx* ctx);

/*
 * Repack canonical MXFP4 weights into the library's tiled layout inside `packed_dev`
 * (k3moe_weight_bytes bytes, 256-byte aligned). The first call binds `packed_dev` to the
 * context; later calls must pass the same pointer (else K3MOE_EINVAL). Packing is lossless.
 */
int k3moe_pack_weights(k3moe_ctx* ctx, const k3moe_weights* w, void* packed_dev, void* stream);

/*
 * y = layer(x) for T tokens. x_dev: bf16 [T, d] row-major; y_dev: bf16 [T, d] row-major (may
 * not alias x); workspace_dev: k3moe_workspace_bytes bytes, 256-byte aligned, contents
 * overwritten. 0 <= T <= max_tokens; T = 0 enqueues nothing. Requires the dense part and every
 * routed expert packed (else K3MOE_ESTATE).
 */
int k3moe_forward(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, void* workspace_dev,
                  void* stream);

/* k3moe_forward plus copies of the intermediates requested in `taps` (may be NULL). */
int k3moe_forward_ex(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, void* workspace_dev,
                     void* stream, const k3moe_taps* taps);

/*
 * k3moe_forward for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the workspace is the library's static device
 * scratch array (K3MOE_SCRATCH_BYTES per GPU, held until the process ends), so only x and y are
 * passed. T's workspace must fit it (else K3MOE_ETOOBIG; at the K3 shape, decode batches up to 64
 * tokens do); k3moe_scratch_fits tells. Calls on one GPU share that array: calls that overlap on
 * one GPU (two streams, two threads) race. Nothing in the array needs clearing between calls.
 */
#define K3MOE_SCRATCH_BYTES ((size_t)64 << 20)
int k3moe_forward_noalloc(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, void* stream);
/* 1 when a forward of T tokens fits the static scratch, else 0. */
int k3moe_scratch_fits(const k3moe_ctx* ctx, int32_t T);

/*
 * Expert-parallel split of a forward ("Serving K3, 01 architecture": expert parallelism is mandatory
 * at scale and its all-to-all has data-dependent sizes; "Kimi K3: architectural innovations",
 * "Compress the expert interface": the latent z is what crosses the interconnect). With the experts in
 * n_ranks contiguous ranges of E / n_ranks, forward = head, then on each rank the experts of its range
 * on the rows it receives, then tail at the tokens' origin. On one GPU the three calls reproduce
 * k3moe_forward (the same kernels run on the same rows).
 *
 * k3moe_forward_head: router, top-k, dispatch tables, W_down and the shared hiddens for T tokens, then
 *   the send side: send_rows_dev [T k, le] the routed input of every (token, slot) in dispatched order
 *   (expert ascending, token ascending; bf16, or E4M3 codes with send_scales_dev [T k, le / 32] E8M0
 *   for MXFP8 activations, else send_scales_dev may be NULL), send_counts_dev int32 [n_ranks] the rows
 *   for each rank (rank i holds experts [i E / n_ranks, (i + 1) E / n_ranks); its rows are
 *   send_rows[sum of earlier counts ..]) and expert_counts_dev int32 [E] rows per expert (may be NULL).
 *   n_ranks divides E. The workspace keeps the routing state the tail needs: pass the same one to
 *   k3moe_forward_tail and do not use it for another call in between.
 * k3moe_experts_forward: on a context holding one rank's experts (n_experts = E / n_ranks, routed
 *   experts packed; the dense part is not needed), the routed experts on R received rows: rows_dev
 *   [R, le] expert-contiguous (expert_counts_dev int32 [n_experts] rows each, in expert order), with
 *   row_scales_dev [R, le / 32] for MXFP8; out_dev fp32 [R, le] the expert outputs in the same order.
 *   0 <= R <= max_tokens * top_k; workspace_dev of k3moe_workspace_bytes.
 * k3moe_forward_tail: combine (eq. 11) of the expert outputs expert_out_dev fp32 [T k, le] (in the
 *   order of the head's send rows), RMSNorm, W_up and the shared experts' down projections -> y_dev.
 */
int k3moe_forward_head(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* workspace_dev, void* stream,
                       int32_t n_ranks, void* send_rows_dev, uint8_t* send_scales_dev, int32_t* send_counts_dev,
                       int32_t* expert_counts_dev);
int k3moe_experts_forward(k3moe_ctx* ctx, const void* rows_dev, const uint8_t* row_scales_dev, int32_t R,
                          const int32_t* expert_counts_dev, float* out_dev, void* workspace_dev, void* stream);
int k3moe_forward_tail(k3moe_ctx* ctx, const float* expert_out_dev, int32_t T, void* y_dev, void* workspace_dev,
                       void* stream);

/*
 * Measurement aid, not part of the layer: reads `bytes` (a multiple of 16) of device memory once with
 * non-temporal 16-byte loads and xors a checksum of every word into *out_dev (uint32, device). Timing
 * it gives the HBM read rate a plain streaming kernel reaches, the practical ceiling the layer's
 * weight streams are compared with.
 */
int k3moe_stream_read(const void* buf_dev, size_t bytes, uint32_t* out_dev, void* stream);

/*
 * Quantile Balancing: the router bias b of eq. 13 from per-expert router-score quantiles ("Serving
 * K3, 01 architecture", hot-expert paragraph; "Kimi K3: architectural innovations", "A router
 * decision is also a scheduling decision": allocation thresholds follow the observed score
 * distribution). The pages give no formula; reading taken: over a calibration batch of T tokens,
 * b_e = -(the m-th largest of expert e's scores), m = round(T k / E) (halves up, within [1, T]),
 * so that s + b >= 0 for exactly m tokens per expert (ties aside).
 * scores_dev: fp32 [T, E] row-major (e.g. the `scores` tap of a forward over the batch);
 * bias_dev: fp32 [E] out, on the stream. 1 <= T <= 16384 (else K3MOE_ETOOBIG); null pointers give
 * K3MOE_EINVAL. The result can be packed as the router bias (k3moe_weights.router_bias).
 */
int k3moe_quantile_bias(k3moe_ctx* ctx, const float* scores_dev, int32_t T, float* bias_dev, void* stream);

/*
 * Per-stage timing. k3moe_profile_begin makes the next forward calls (at most max_calls) record
 * a HIP event before and after each stage on their stream. k3moe_profile_end waits for those
 * events, writes the summed milliseconds of each stage to ms[0 .. n_stages-1] (n_stages =
 * k3moe_stage_count()) and the number of recorded calls to *calls, and stops recording.
 */
int k3moe_profile_begin(k3moe_ctx* ctx, int32_t max_calls);
int k3moe_profile_end(k3moe_ctx* ctx, float* ms, int32_t n_stages, int32_t* calls);
int32_t k3moe_stage_count(void);
const char* k3moe_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* K3MOE_H */
