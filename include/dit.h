/*
 * dit.h -- C ABI of the MI355X (gfx950) DiT denoise-step library (libdit.so).
 *
 * What it computes.  The SGLang-Diffusion page "Disaggregated Diffusion
 * Pipeline" (section "Quick Start", the role table) defines the denoiser as
 * the DiT forward loop plus the scheduler stepping it drives.  The page
 * "Support New Diffusion Models" fixes its interface: the DiT forward takes
 * the latents (hidden_states), the prompt embeddings (encoder_hidden_states)
 * and the timestep (section "2. Pipeline Config"); the denoising stage is fed
 * latents, timesteps in the reference order and a separate sigma list
 * (section "4. Last-Resort Before-Denoising Stage", the DenoisingStage field
 * table), and the raw latent shape stays with the caller.  One call of
 * dit_denoise_step is one iteration of that loop: the DiT forward over the
 * patchified latents followed by the flow-matching Euler update ("Model
 * Configuration Conventions", section "Sampling And Geometry", flow-prediction
 * denoisers).
 *
 * Conventions (all functions):
 *  - Every pointer argument named as device memory must be a device address
 *    valid on the current HIP device; host arguments are plain host memory.
 *  - Device buffers are owned by the caller.  The library allocates no device
 *    memory (its one device array is the static scratch of
 *    dit_block_forward_static); a model handle keeps non-owning pointers to
 *    the weights and the workspace, which must outlive it.
 *  - Calls that take a stream enqueue their work asynchronously on it
 *    (NULL = the default stream) and return without synchronising; the one
 *    exception is dit_denoise_step_cached on a step that may reuse the cache
 *    (it waits for its probe, see there).
 *  - Arguments are validated before anything is enqueued: a call that returns
 *    an error has not touched any caller buffer.  Launch failures are reported
 *    as DIT_ERR_HIP.  There is no silent fallback: an unsupported shape is an
 *    error ("Support New Diffusion Models", section "Reuse component loaders":
 *    an explicitly selected path fails on errors instead of falling back).
 *  - A handle is not thread-safe; distinct handles are independent, and an
 *    error on one never affects another.
 *  - Matrices are row-major.  Weight matrices are [out_features, in_features].
 *  - Element type "T" below is the configuration's dtype: float (DIT_F32) or
 *    bfloat16 bit patterns (DIT_BF16).  The residual stream, latents,
 *    velocity, modulation vectors and all reductions are float32 in both.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIT_OK = 0,
  DIT_ERR_INVALID_ARG = -1, /* null pointer, misaligned pointer, bad scalar  */
  DIT_ERR_SHAPE = -2,       /* inconsistent sizes, index out of range        */
  DIT_ERR_UNSUPPORTED = -3, /* valid but not implemented (e.g. head_dim 96)  */
  DIT_ERR_WORKSPACE = -4,   /* workspace smaller than dit_workspace_size()   */
  DIT_ERR_HIP = -5          /* HIP runtime or launch failure                 */
} dit_status;

typedef enum { DIT_F32 = 0, DIT_BF16 = 1 } dit_dtype;

/* Model and workload description.  Tokens: S = (lat_f/patch_f) *
 * (lat_h/patch_h) * (lat_w/patch_w), laid out over the patch grid in
 * row-major (f', h', w') order; patch vector width P = in_channels * patch_f *
 * patch_h * patch_w.  Requirements checked by dit_create: every size > 0,
 * hidden == heads * head_dim, head_dim in {32, 64, 128}, lat_* divisible by
 * patch_*, rope_* even with rope_f + rope_h + rope_w == head_dim,
 * freq_dim even, ctx_len_max >= 1, ln_eps > 0, rope_theta > 0. */
typedef struct {
  int32_t num_blocks;   /* B                                                  */
  int32_t hidden;       /* D                                                  */
  int32_t heads;        /* H                                                  */
  int32_t head_dim;     /* d = D / H                                          */
  int32_t mlp_hidden;   /* F                                                  */
  int32_t freq_dim;     /* width of the timestep sinusoid (256)              */
  int32_t in_channels;  /* C                                                  */
  int32_t patch_f, patch_h, patch_w;
  int32_t lat_f, lat_h, lat_w;
  int32_t rope_f, rope_h, rope_w; /* channels per axis in each head         */
  int32_t ctx_len_max;  /* largest context length a call may pass (L)        */
  int32_t text_dim;     /* width of the caller's context tokens; == hidden
                           means no text projection                          */
  float rope_theta;     /* rotary base (10000)                               */
  float ln_eps;         /* LayerNorm epsilon (1e-6)                          */
  int32_t dtype;        /* dit_dtype                                          */
  int32_t guidance;     /* 1: size the workspace for guided steps
                           (dit_denoise_step_cfg, two sequences; needs the
                           token count S a multiple of 8); 0: unguided only  */
  int32_t offload;      /* 1: layerwise weight offload.  The per-block
                           weights (dit_block_weights) are then HOST pointers
                           into page-locked memory (hipHostMalloc or
                           equivalent); each step streams every block into
                           one of two workspace slots on an internal copy
                           stream while the previous block runs ("Support New
                           Diffusion Models - SGLang Documentation", section
                           "5. Distributed and memory integration": layerwise
                           offload over the repeated blocks; section "Verify
                           the Port": compared with the resident baseline).
                           The block's modulation table is copied to the
                           device once, by dit_create.  Fields after it that
                           lie in one allocation in declaration order, each
                           at the first 256-byte boundary after the end of
                           the previous one, are moved in a single transfer;
                           any other placement is valid but copied field by
                           field.  0: all weights resident on the device    */
  int32_t cache;        /* 1: size the workspace for cached steps
                           (dit_denoise_step_cached); 0: none               */
} dit_config;

/* Model-wide parameters (device pointers, element type T).  Shapes:
 *   t1_w [D, freq_dim], t1_b [D], t2_w [D, D], t2_b [D]   timestep MLP
 *   mod_w [6D, D], mod_b [6D]   shared modulation projection; output row
 *       block j (rows j*D .. j*D+D-1) is vector j of (shift_a, scale_a,
 *       gate_a, shift_f, scale_f, gate_f)
 *   txt_w [D, text_dim], txt_b [D]   context projection (NULL when
 *       text_dim == hidden)
 *   pe_w [D, P], pe_b [D]   patch embedding
 *   head_table [2, D]   (shift_o, scale_o) offsets of the final layer
 *   out_w [P, D], out_b [P]   final projection to velocity tokens          */
typedef struct {
  const void *t1_w, *t1_b, *t2_w, *t2_b, *mod_w, *mod_b, *txt_w, *txt_b;
  const void *pe_w, *pe_b, *head_table, *out_w, *out_b;
} dit_global_weights;

/* Per-block parameters (device pointers, element type T).  Shapes:
 *   table [6, D]   block offsets added to the shared modulation vectors
 *   qkv_w [3D, D], qkv_b [3D]   rows 0..D-1 q, D..2D-1 k, 2D..3D-1 v; head h
 *       of each is rows h*d .. h*d+d-1 of that block
 *   o_w [D, D], o_b [D]   self-attention output projection
 *   cq_w [D, D], cq_b [D]   cross-attention query projection
 *   ckv_w [2D, D], ckv_b [2D]   cross-attention key (rows 0..D-1) and value
 *       (rows D..2D-1) projection of the context
 *   co_w [D, D], co_b [D]   cross-attention output projection
 *   w1 [F, D], b1 [F], w2 [D, F], b2 [D]   MLP                              */
typedef struct {
  const void *table, *qkv_w, *qkv_b, *o_w, *o_b, *cq_w, *cq_b, *ckv_w, *ckv_b;
  const void *co_w, *co_b, *w1, *b1, *w2, *b2;
} dit_block_weights;

typedef struct {
  dit_global_weights global;
  const dit_block_weights *blocks; /* HOST array of num_blocks entries; copied
                                      by dit_create.  With offload, the
                                      weights these entries point to are in
                                      page-locked host memory and must stay
                                      there for the handle's lifetime        */
} dit_weights;

typedef struct dit_model dit_model;

/* Bytes of device workspace a model of this configuration needs (host call,
 * no device work).  Writes 0 and returns an error for an invalid config. */
dit_status dit_workspace_size(const dit_config *cfg, size_t *bytes);

/* Validate the configuration and the weight pointers (non-NULL, 16-byte
 * aligned), bind them and the caller's workspace (device, >= the size above,
 * 256-byte aligned) to a new handle, and enqueue on `stream` the
 * precomputation of the rotary cos/sin tables into the workspace.  The handle
 * owns only host memory; release it with dit_destroy.
 * The handle stands for the loaded transformer of page "Support New Diffusion
 * Models - SGLang Documentation": section "Read the Reference First" asks for
 * the latent shape and packing, the rotary style and the conditioning tensors
 * that the model fixes once, and section "Verify the Port" lists a rotary
 * shape or style mismatch among the failure points, which is why the rotary
 * split and base are fields of the configuration and their tables are built
 * here, once, rather than per call. */
dit_status dit_create(const dit_config *cfg, const dit_weights *weights, void *workspace,
                      size_t workspace_bytes, void *stream, dit_model **out);

/* Release a handle (host memory only; no device work).  NULL is accepted. */
dit_status dit_destroy(dit_model *model);

/* One DiT block applied in place to the residual stream, teacher-forcible:
 *   x    device float [S, D], read and overwritten with the block output;
 *   ctx  device T [ctx_len, D], the already projected context tokens;
 *   mod  device float [6, D], the block's six modulation vectors in the order
 *        (shift_a, scale_a, gate_a, shift_f, scale_f, gate_f) (the denoise
 *        step passes shared projection + the block's table; a caller may pass
 *        any values).
 * 0 <= block < num_blocks, 1 <= ctx_len <= ctx_len_max.  Uses the workspace:
 * calls on one handle must not overlap on different streams.
 * The block is the repeated unit of the denoiser's transformer that page
 * "Support New Diffusion Models - SGLang Documentation", section "5.
 * Distributed and memory integration", names as the unit of layerwise offload
 * and of sequence parallelism; page "Disaggregated Diffusion Pipeline",
 * section "Quick Start", places the loop over these blocks in the denoiser
 * role.  Its contents (adaLN-modulated self-attention with rotary, plain
 * LayerNorm and ungated cross-attention to the context, adaLN-modulated GELU
 * MLP, gated residuals) are the plainest reading of that block; the pages
 * print no formula for it. */
dit_status dit_block_forward(dit_model *model, int32_t block, float *x, const void *ctx,
                             int32_t ctx_len, const float *mod, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the block of
 * dit_block_forward without a handle or a workspace.  Arguments as there, with
 * the configuration and this block's weights (device pointers) passed
 * directly; cfg->num_blocks is ignored, and guidance, offload and cache must
 * be 0 (else DIT_ERR_UNSUPPORTED).  The rotary tables and every intermediate
 * buffer (LayerNorm output, q, k, transposed values, attention output, MLP
 * hidden, cross K / V^T) live in a library-owned device array of
 * DIT_STATIC_SCRATCH_BYTES, one per device, held until the process ends; a
 * configuration whose one-block workspace (dit_workspace_size with
 * num_blocks = 1) exceeds it is refused with DIT_ERR_WORKSPACE before any
 * device work.  The call allocates nothing (no hipMalloc or hipFree, no heap
 * memory).  Every call on a device shares that device's array and leaves its
 * last contents there; nothing in it needs to start at zero.  Calls that
 * overlap on one device (concurrent streams or threads) race on the array and
 * must be serialised by the caller. */
#define DIT_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
dit_status dit_block_forward_static(const dit_config *cfg, const dit_block_weights *weights,
                                    float *x, const void *ctx, int32_t ctx_len, const float *mod,
                                    void *stream);

/* One denoising step: velocity V = DiT(X, ctx, t), then X += (sigma_next -
 * sigma) * V.
 *   X      device float [C, F, H, W] latents, read and overwritten;
 *   ctx    device T [ctx_len, text_dim] conditioning tokens;
 *   t      timestep fed to the sinusoid (the schedule uses 1000 * sigma);
 *   sigma, sigma_next   the current and next noise levels;
 *   v_out  device float [C, F, H, W] receiving V, or NULL.
 * 1 <= ctx_len <= ctx_len_max. */
dit_status dit_denoise_step(dit_model *model, float *X, const void *ctx, int32_t ctx_len,
                            float t, float sigma, float sigma_next, float *v_out, void *stream);

/* One denoising step with classifier-free guidance: the network runs on the
 * same latents and timestep once with the positive context ctx and once with
 * the negative context ctx_neg (both device T [ctx_len, text_dim]), as one
 * batch of two sequences that reads every weight once; the guided velocity
 * V = V_neg + guidance_scale * (V_pos - V_neg) then drives the same Euler
 * update, X += (sigma_next - sigma) * V, and goes to v_out when given.
 * ("Support New Diffusion Models - SGLang Documentation", section 1
 * "Sampling Params": guidance_scale; section 2 "Pipeline Config": the positive
 * and negative condition kwargs; section 4: negative_prompt_embeds.  The
 * combination is the conventional one; the pages print no formula.)
 * The handle must have been created with guidance = 1 (else
 * DIT_ERR_WORKSPACE); other arguments as for dit_denoise_step. */
dit_status dit_denoise_step_cfg(dit_model *model, float *X, const void *ctx, const void *ctx_neg,
                                int32_t ctx_len, float t, float sigma, float sigma_next,
                                float guidance_scale, float *v_out, void *stream);

/* Block caching across the steps of one sampling run (page "Disaggregated
 * Diffusion Pipeline", section "GLM-Image distributed mode": the denoisers
 * run with Cache-DiT and the knobs FN, BN, WARMUP, RDT, MC, TAYLORSEER and
 * TS_ORDER, values 2, 1, 4, 0.4, 4, true, 2; the page names the knobs only,
 * and the rules below are the reading of those names).
 *
 * Every step runs the first `fn` blocks.  Their residual P = h_fn - h_0 (the
 * stream after them minus the embedded tokens) is compared with P_ref, the
 * same residual on the last step that ran every block: d = sum|P - P_ref| /
 * sum|P_ref|.  A step reuses the cache when (a) it is not one of the first
 * `warmup` steps, (b) an earlier step ran every block, (c) fewer than
 * `max_consecutive` steps in a row have reused it, and (d) d < rdt.  It then
 * skips the middle blocks [fn, num_blocks - bn) and adds a stand-in for their
 * residual M = h_{num_blocks-bn} - h_fn instead: with TaylorSeer, sum_q T_q
 * k^q / q! over the factors in hand (k = steps since the last full step),
 * where after each full step T_0 = M and T_q = (T_{q-1} - previous
 * T_{q-1}) / (steps between the two full steps), q <= ts_order; without
 * TaylorSeer, the last M.  The last `bn` blocks always run.  Guided steps make
 * one decision for both sequences (d sums over both) and keep one residual
 * cache per sequence. */
typedef struct {
  int32_t fn;              /* first blocks run on every step, >= 1        */
  int32_t bn;              /* last blocks run on every step, >= 0;
                              fn + bn <= num_blocks                        */
  int32_t warmup;          /* steps that always run every block, >= 0     */
  float rdt;               /* threshold on d, >= 0 (+inf allowed)          */
  int32_t max_consecutive; /* cached steps in a row at most, >= 0         */
  int32_t taylorseer;      /* 1: Taylor extrapolation of the residual      */
  int32_t ts_order;        /* 0 .. 2                                       */
} dit_cache_params;

/* The decision state after the last cached-path step. */
typedef struct {
  int32_t step;            /* steps taken since dit_cache_begin            */
  int32_t consecutive;     /* cached steps since the last full one         */
  int32_t last_full;       /* index of the last full step, -1 before any   */
  int32_t factors;         /* Taylor factors in hand (0: nothing cached)   */
  int32_t hit;             /* last step: 1 reused the cache, 0 ran it all  */
  int32_t cached_total;    /* steps that reused the cache                  */
  double diff;             /* last step's d; -1 when the step could not
                              reuse the cache and d was not measured       */
} dit_cache_state;

/* Start a sampling run: validate and keep the knobs, clear the state (host
 * call, no device work).  Needs a handle created with cache = 1 (else
 * DIT_ERR_WORKSPACE); invalid knobs give DIT_ERR_INVALID_ARG, fn + bn >
 * num_blocks DIT_ERR_SHAPE, ts_order > 2 DIT_ERR_UNSUPPORTED. */
dit_status dit_cache_begin(dit_model *model, const dit_cache_params *params);

/* Copy the decision state to *state (host call). */
dit_status dit_cache_state_get(const dit_model *model, dit_cache_state *state);

/* One step of the run begun by dit_cache_begin: dit_denoise_step (ctx_neg
 * NULL) or dit_denoise_step_cfg (ctx_neg given; the handle also needs
 * guidance = 1) with the block cache above.  Arguments as there.  When the
 * step could reuse the cache it waits once for `stream` to reach the probe
 * and reads 2 doubles per probe workgroup back to the host to decide; other
 * steps do not synchronise.  The cached residuals live in their own part of
 * the workspace, which other calls on the handle leave alone.  On an error
 * the run must be begun again. */
dit_status dit_denoise_step_cached(dit_model *model, float *X, const void *ctx,
                                   const void *ctx_neg, int32_t ctx_len, float t, float sigma,
                                   float sigma_next, float guidance_scale, float *v_out,
                                   void *stream);

/* Diagnostics: enqueue on `stream` a copy of Taylor factor q (0 <= q <
 * factors in hand, dit_cache_state.factors) of the current cached run into
 * dst, device float [nb * S * D], nb = 2 for a guided run (positive sequence
 * first) and 1 otherwise; rows follow the token order.  With TaylorSeer the
 * cached stand-in is sum_q T_q k^q / q!; this exposes the T_q the last full
 * step left, so a cached step can be checked against a reference fed the same
 * factors.  DIT_ERR_WORKSPACE without cache = 1, DIT_ERR_SHAPE for q out of
 * range or before the first step of a run. */
dit_status dit_cache_factor_get(const dit_model *model, int32_t q, float *dst, void *stream);

/* Flow Euler update X[i] += (sigma_next - sigma) * v[i] for i < n on device
 * float arrays (layout-agnostic).  n == 0 is a no-op; X and v must be 16-byte
 * aligned, n >= 0.  Page "Model Configuration Conventions", section "Sampling
 * And Geometry", names the flow-prediction denoisers and their flow shift;
 * page "Support New Diffusion Models - SGLang Documentation", section "4.
 * Last-Resort Before-Denoising Stage", passes the sigma list beside the
 * timesteps.  A flow-prediction network outputs a velocity, and the first
 * order step between two noise levels moves the latents by their difference
 * times that velocity. */
dit_status dit_euler_step(float *X, const float *v, int64_t n, float sigma, float sigma_next,
                          void *stream);

/* Host: the shifted linear flow schedule, n_steps + 1 values into the host
 * array sigmas: s_k = 1 - k/n_steps, sigma_k = shift*s_k / (1 + (shift-1)*s_k).
 * ("Support New Diffusion Models", sections "Read the Reference First" and
 * "Verify the Port": timestep and sigma schedule; "Model Configuration
 * Conventions", section "Sampling And Geometry": default flow shift.)
 * Requires n_steps >= 1 and shift > 0. */
dit_status dit_flow_sigmas(int32_t n_steps, double shift, double *sigmas);

/* Component entry points.  They run the same kernels the step uses on
 * caller-provided buffers, so each part of the path can be checked and timed
 * on its own at full size without a model handle. */

/* Multi-head attention softmax(q k^T / sqrt(head_dim)) v, non-causal, no mask
 * (the step's self- and cross-attention kernel); element type from dtype:
 *   q   device T [sq, ldq] (head h at columns h*head_dim .. +head_dim-1);
 *   k   device T [sk, ldk] likewise;
 *   vt  device T [heads*head_dim, ldv]: the values transposed, row
 *       h*head_dim + c holds channel c of head h for keys 0..sk-1;
 *       ldv >= sk rounded up to a multiple of 64 (entries past sk are read
 *       but never used);
 *   o   device T [sq, ldo].
 * heads >= 1, head_dim in {32, 64, 128}, sq, sk >= 1; every ld >= heads *
 * head_dim and a multiple of 8 elements. */
dit_status dit_attention(int32_t dtype, int32_t heads, int32_t head_dim, const void *q,
                         int64_t ldq, const void *k, int64_t ldk, const void *vt, int64_t ldv,
                         void *o, int64_t ldo, int32_t sq, int32_t sk, void *stream);

/* Linear layer on the matrix cores, C[M, N] = A[M, K] * W[N, K]^T + bias[N]
 * (the step's projection kernel), followed by one epilogue:
 *   DIT_EPI_STORE     out T [M, ldo]       = C
 *   DIT_EPI_GELU      out T [M, ldo]       = GELU_tanh(C)
 *   DIT_EPI_RESIDUAL  out float [M, ldo]  += gate[n] * C   (gate NULL: 1)
 *   DIT_EPI_STORE_F32 out float [M, ldo]   = C
 * A device T [M, lda], W device T [N, ldw], bias device T [N] or NULL.
 * M, N, K >= 1; K, lda and ldw multiples of 8; lda, ldw >= K;
 * ldo >= N.  tile selects the workgroup tile (0 automatic, 1: 256x256 with
 * 4 waves, 2: 128x128, 3: 64x64, 4: 256x256 with 8 waves, 5: 256x256 with 8
 * waves on 16x16x32 matrix instructions; fp32 always uses 64x64); other
 * values give DIT_ERR_INVALID_ARG. */
enum { DIT_EPI_STORE = 0, DIT_EPI_GELU = 1, DIT_EPI_RESIDUAL = 2, DIT_EPI_STORE_F32 = 3 };
dit_status dit_gemm(int32_t dtype, int32_t epilogue, const void *A, int64_t lda, const void *W,
                    int64_t ldw, int32_t M, int32_t N, int32_t K, const void *bias, void *out,
                    int64_t ldo, const float *gate, int32_t tile, void *stream);

/* LayerNorm without affine parameters over rows of x (device float [rows, D]),
 * y = LN(x) * (1 + scale) + shift when shift and scale (device float [D]) are
 * both given, plain LN(x) when both are NULL; y is device T [rows, D].
 * D a multiple of 4 and <= 5120, eps > 0. */
dit_status dit_layernorm_modulate(int32_t dtype, int32_t D, float eps, const float *x,
                                  int32_t rows, const float *shift, const float *scale, void *y,
                                  void *stream);

/* Time path: the six modulation vectors of every block (device float
 * [num_blocks, 6, D]), the final layer's (shift_o, scale_o) (device float
 * [2, D]) and temb (device float [D]) at timestep t. */
dit_status dit_time_embedding(dit_model *model, float t, float *block_mod, float *head_mod,
                              float *temb, void *stream);

/* Per-launch timing (diagnostics).  While enabled on a handle, every kernel
 * launch of the handle's calls (blocks, steps, time embedding) carries two
 * HIP events that the runtime records at the kernel's own dispatch and
 * completion on the call's stream (extended launch).  Enabling clears
 * earlier records; disabling keeps them for reading.  dit_profile_read waits
 * for the recorded events of one kind and returns the number of launches and
 * their summed duration in milliseconds.  Kinds are 0 .. dit_profile_kind_count()-1,
 * named by dit_profile_kind_name (static strings, NULL when out of range). */
dit_status dit_profile_enable(dit_model *model, int32_t enable);
dit_status dit_profile_read(dit_model *model, int32_t kind, int64_t *launches, double *total_ms);
int32_t dit_profile_kind_count(void);
const char *dit_profile_kind_name(int32_t kind);

/* Human-readable name of a status code (static string). */
const char *dit_status_string(dit_status status);

#ifdef __cplusplus
}
#endif
#endif /* DIT_H */
