/*
 * wam.h -- C ABI of the MI355X (gfx950) library computing one flow-matching denoising step of
 * DreamZero's chunk-causal joint video+action DiT ("World Action Model").
 *
 * Sources (page titles; sections):
 *   [ARCH]  "DreamZero (WAM) 模型架构": §2.1 encoders, §2.3 Causal WAN DiT (input sequence,
 *           single causal block, output split, causal mask), §2.4 per-embodiment action linears,
 *           §3 flow-matching interpolation, §4 inference (encode once, denoise loop).
 *   [WS1]   "DreamZero 单卡推理" (PhyAI ws1): architecture table (DiT runner keeps the attention
 *           KV; scheduler owns reference KV, CFG branches, DiT calls, the update), request format
 *           (negative prompt, 512 text tokens), continuous requests (frame position, KV reset),
 *           Fixed4 vs dynamic16.
 *   [HYPER] hyper.ai summary of arXiv 2602.15922, 方法: chunked AR generation, mask (noisy chunk
 *           sees clean earlier chunks, never future tokens), KV replaced by real observations.
 *   [N569]  walk-through "World Action Models are Zero-shot Policies": inference with KV cache,
 *           CFG passes, DiT caching by cosine similarity of successive velocities, Flash schedule.
 *
 * Conventions shared by every entry point
 *   - All tensors are caller-owned DEVICE buffers (one GPU), dense and contiguous, 16-byte aligned
 *     (256-byte recommended). Structs are host memory. The library never allocates or frees device
 *     memory and never synchronises: work is enqueued on `stream` (a hipStream_t; NULL = default).
 *   - Matrices (Linear weights, stored [out][in]) and activations/caches use the element type of
 *     wam_config.dtype: WAM_BF16 = bfloat16 bit patterns, WAM_F32 = IEEE float (debug mode).
 *     Vectors (biases, norm gains, modulation tables) and the latents/velocities are always float.
 *   - Arguments are validated on the host before anything is enqueued: a non-zero status means
 *     nothing was launched. WAM_E_HIP reports a launch failure (text in wam_last_error()); a
 *     device fault surfaces at the caller's next synchronisation.
 *   - Calls on different streams need distinct workspaces; the caches they write must not overlap.
 *
 * Time convention: t in [0,1], t = 0 pure noise, t = 1 clean; x_t = t x1 + (1-t) eps; the model
 * predicts the velocity x1 - eps; one Euler step is x += (t_next - t) v.
 */
#ifndef WAM_H_
#define WAM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WAM_OK = 0,
  WAM_E_ARG = -1,         /* null pointer or out-of-range scalar */
  WAM_E_SHAPE = -2,       /* sizes inconsistent or unsupported (e.g. head_dim not 64/128) */
  WAM_E_CAPACITY = -3,    /* KV cache too small for the rows to be written */
  WAM_E_HIP = -4,         /* a HIP launch failed */
  WAM_E_UNSUPPORTED = -5
} wam_status;

typedef enum { WAM_BF16 = 0, WAM_F32 = 1 } wam_dtype;

/* Model and chunk geometry. [ARCH] §5 table: 40 layers, width 5120, 40 heads of 128; §2.3: FFN
 * 5120->13824; 1536-d encoder features; 24-step action horizon. Chunk = frames_per_chunk latent
 * frames of grid_h x grid_w patch tokens (raster order), then action_tokens action tokens. */
typedef struct {
  int dim, heads, head_dim, ffn_dim, layers, freq_dim;
  int patch_dim, action_dim, action_tokens;
  int frames_per_chunk, grid_h, grid_w;
  int ctx_in_dim, ctx_text_len, ctx_img_len;
  int branches;            /* 1, or 2 = CFG batch (branch 0 conditional, branch 1 negative prompt) */
  float rope_theta, eps;   /* 10000, 1e-6 */
  wam_dtype dtype;
  int variant;             /* 0, or WAM_VARIANT_* bits (architectural variants of [ARCH] §2.3) */
  int precision;           /* WAM_PRECISION_NATIVE (0) or WAM_PRECISION_MXFP8 (see below) */
  int ctx_state_len;       /* proprioceptive state rows at the end of the condition sequence (0: none) */
  int state_dim;           /* width of one state vector (multiple of 64) when ctx_state_len > 0 */
} wam_config;

/* Arithmetic of the six block projections (w_qkv, w_o, w_cq, w_co, w_ff1, w_ff2).
 * NATIVE: in dtype. MXFP8 ([N569] real-time optimisations: low-precision projections; bf16 dtype
 *   only, dim and ffn_dim multiples of 128): each projection's input rows are quantised to MXFP8
 *   (see wam_mx_quantize) and multiplied with the layer's packed MXFP8 weights (wam_mx_pack_block)
 *   by the scaled matrix instructions, fp32 accumulation; outputs, epilogues and every other
 *   operation as NATIVE. The condition projections (wam_ctx_build), embeddings and heads stay in
 *   dtype. */
enum { WAM_PRECISION_NATIVE = 0, WAM_PRECISION_MXFP8 = 1, WAM_PRECISION_MXFP4W = 2 };
/* MXFP4W: as MXFP8, but the packed weights are MXFP4 (e2m1 elements, see wam_mx4_quantize); the
 * activations stay MXFP8 and the instructions take one fp8 and one fp4 operand. */

/* Architectural variants drawn on the architecture page next to the adopted readings.
 * FRAME_CAUSAL: inside a chunk a video token sees the video tokens of its own and earlier frames
 *   and an action token the whole chunk (cached chunks and earlier chunks of a pass stay visible).
 * RMS_NORM: the block norms (both modulated norms and the affine norm before cross-attention) and
 *   the output-head norm divide by the root mean square without subtracting the mean.
 * SWIGLU: the feed-forward is (SiLU(y W_g^T + b_g) * (y W_u^T + b_u)) W_2^T + b_2 with w_ff1 [2F][D]
 *   and b_ff1 [2F] holding the gate and up rows interleaved (row 2j gate j, row 2j+1 up j).
 * IMG_XATTN: the image part of the condition sequence gets its own key / value projections
 *   (w_cki, b_cki, g_cki, w_cvi, b_cvi of the block) and its own softmax: the cross-attention output
 *   is attn(q, K_txt, V_txt) + attn(q, K_img, V_img) before W_co (the backbone's image-to-video
 *   layout). Needs ctx_img_len > 0, ctx_text_len a multiple of 8, and ctx_stride of the condition
 *   KV >= ctx_text_len + ctx_img_len rounded up to 32. */
enum { WAM_VARIANT_FRAME_CAUSAL = 1, WAM_VARIANT_RMS_NORM = 2, WAM_VARIANT_SWIGLU = 4, WAM_VARIANT_IMG_XATTN = 8 };

/* One block's parameters ([ARCH] §2.3 single causal block). Matrices [out][in] in dtype;
 * everything else float. mod: [6][D] per-layer offset added to the shared time modulation
 * (shift1, scale1, gate1, shift2, scale2, gate2). */
typedef struct {
  const void *mod;
  const void *w_qkv, *b_qkv;   /* [3D][D], [3D]  rows: q | k | v */
  const void *g_q, *g_k;       /* [D] RMSNorm gains of q and k */
  const void *w_o, *b_o;       /* [D][D], [D] */
  const void *ln3_w, *ln3_b;   /* [D] affine LayerNorm before cross-attention */
  const void *w_cq, *b_cq, *g_cq;
  const void *w_ck, *b_ck, *g_ck;
  const void *w_cv, *b_cv;
  const void *w_co, *b_co;
  const void *w_ff1, *b_ff1;   /* [F][D], [F] (SwiGLU variant: [2F][D], [2F], see below) */
  const void *w_ff2, *b_ff2;   /* [D][F], [D] */
  const void *mx;              /* MXFP8 precision only (else ignored): this layer's packed projections,
                                  wam_mx_block_bytes(cfg) bytes written by wam_mx_pack_block, 256-aligned */
  const void *w_cki, *b_cki, *g_cki;   /* IMG_XATTN only (else ignored): image keys [D][D], [D], RMSNorm gain [D] */
  const void *w_cvi, *b_cvi;           /* IMG_XATTN only: image values [D][D], [D] */
  const void *pk;              /* bf16 NATIVE precision only (else ignored), optional: this layer's six
                                  projections in the fragment-packed layout, wam_pack_block_bytes(cfg) bytes
                                  written by wam_pack_block, 256-byte aligned. When set, the block's products
                                  read it and w_qkv, w_o, w_cq, w_co, w_ff1 and w_ff2 are not read (they may
                                  be NULL); the results equal the unpacked ones. NULL: unpacked matrices. */
} wam_block_weights;

/* Action encoder and decoder of one embodiment ([ARCH] §2.4: each robot body has its own linear from
 * its action space to the width and back, the shared DiT in between, routed by the embodiment id).
 * Shapes as ae_* / ao_* of wam_weights: every embodiment's actions are padded to cfg->action_dim. */
typedef struct {
  const void *ae_w, *ae_b;   /* [D][action_dim], [D] */
  const void *ao_w, *ao_b;   /* [action_dim][D], [action_dim] */
} wam_action_io;

typedef struct {
  const wam_block_weights *blocks;           /* host array [layers] */
  const void *t_w1, *t_b1, *t_w2, *t_b2;     /* time MLP: [D][freq_dim], [D]; [D][D], [D] */
  const void *t_wp, *t_bp;                   /* shared modulation projection [6D][D], [6D] */
  const void *pe_w, *pe_b;                   /* patch embedding [D][patch_dim], [D] */
  const void *ae_w, *ae_b;                   /* action embedding [D][action_dim], [D] */
  const void *head_mod;                      /* [2][D] output-head shift/scale offsets */
  const void *vo_w, *vo_b;                   /* video head [patch_dim][D], [patch_dim] */
  const void *ao_w, *ao_b;                   /* action head [action_dim][D], [action_dim] */
  const void *txt_w, *txt_b;                 /* text features -> width [D][ctx_in_dim], [D] */
  const void *img_w, *img_b;                 /* image features -> width (NULL when ctx_img_len = 0) */
  const wam_action_io *embodiments;          /* optional host array [n_embodiments] (see below) */
  int n_embodiments;
  const void *st_w, *st_b;                   /* state encoder [D][state_dim], [D] (NULL when ctx_state_len = 0) */
} wam_weights;

/* Routing by embodiment id ([ARCH] §2.4): *out = *w with ae_* / ao_* taken from w->embodiments[id].
 * Every call then runs that embodiment's action encoder and decoder (one request, both CFG branches,
 * is one embodiment). Host only, nothing launched; out may alias w. Errors: WAM_E_ARG (id outside
 * [0, n_embodiments), NULL table or matrices). */
wam_status wam_weights_for_embodiment(const wam_weights *w, int id, wam_weights *out);

/* Self-attention KV cache of clean chunks ([WS1] architecture: the DiT runner keeps the KV;
 * [HYPER] 方法: executed chunks are replaced by real observations). Keys after RMSNorm and RoPE.
 *   k: [layers][branches][heads][capacity][head_dim]
 *   v: [layers][branches][heads][head_dim][capacity]   (value rows stored key-contiguous)
 * `length` rows are committed. A forward pass writes its own keys/values into rows
 * [length, length + n_chunks*Lq) as scratch; committed rows are never modified except by
 * wam_kv_append, which fills exactly those rows and then advances `length`.
 * capacity must be a multiple of 64, length a multiple of 8. */
typedef struct {
  void *k, *v;
  int branches, capacity, length;
} wam_kv_cache;

/* Cross-attention keys/values of the condition sequence, built once per request ([ARCH] §4:
 * conditions are encoded once and cached).
 *   k: [layers][branches][heads][ctx_len][head_dim]      (after RMSNorm)
 *   v: [layers][branches][heads][head_dim][ctx_stride]   (ctx_stride multiple of 64, >= ctx_len) */
typedef struct {
  void *k, *v;
  int branches, ctx_len, ctx_stride;
} wam_ctx_kv;

/* Bytes of device workspace needed by any call with up to `n_chunks` chunks in one pass
 * (1 for an incremental step or an append; >1 for a full-sequence pass). */
size_t wam_workspace_bytes(const wam_config *cfg, int n_chunks);

/* Condition build ([ARCH] §2.1: text and image features concatenated into one condition
 * sequence; §4: encoded once). ctx_b = [txt_b W_txt^T + b ; img W_img^T + b ; state W_st^T + b] per
 * branch, then per layer Kc = RMSNorm(ctx Wck^T + b) g_ck and Vc = ctx Wcv^T + b into `out`.
 *   txt:   [branches][ctx_text_len][ctx_in_dim] dtype (branch 1 = negative prompt features)
 *   img:   [ctx_img_len][ctx_in_dim] dtype, shared by the branches (NULL when ctx_img_len = 0)
 *   state: [ctx_state_len][state_dim] dtype, the observed proprioceptive state shared by the
 *          branches (NULL when ctx_state_len = 0). The walk-throughs name a state encoder beside the
 *          text encoder, fused into the DiT; here it is one Linear whose rows join the condition
 *          sequence after the image rows. */
wam_status wam_ctx_build(const wam_config *cfg, const wam_weights *w, const void *txt, const void *img,
                         const void *state, wam_ctx_kv *out, void *ws, size_t ws_bytes, void *stream);

/* New observation: recompute only the state rows of every layer's condition keys / values (the
 * text and image rows built by wam_ctx_build are kept). state as in wam_ctx_build. Errors:
 * WAM_E_ARG / WAM_E_SHAPE (no state rows configured), nothing launched. */
wam_status wam_ctx_set_state(const wam_config *cfg, const wam_weights *w, const void *state, wam_ctx_kv *ctx,
                             void *ws, size_t ws_bytes, void *stream);

/* Shared time modulation for `n` timesteps t[0..n) (host floats, n <= 16): e [n][D] and
 * e6 [n][6][D] (device float). [ARCH] §2.3: sinusoidal time embedding; the modulation's shift and
 * scale come from it. Embedded scalar s = 1000 (1 - t). */
wam_status wam_time_embed(const wam_config *cfg, const wam_weights *w, const float *t, int n, float *e,
                          float *e6, void *ws, size_t ws_bytes, void *stream);

/* One pass of the DiT stack over `n_chunks` chunks for all branches ([WS1]: the DiT runner predicts
 * the video and action outputs and maintains the attention KV).
 *   x_video:  [n_chunks * Lv][patch_dim] float, x_action: [n_chunks * La][action_dim] float
 *             (the same noisy latents feed every branch)
 *   t_video, t_action: HOST arrays [n_chunks] (per-group timesteps; equal values = shared t)
 *   start_frame: frame index of the first frame of chunk 0 within the attention window
 *   v_video: [branches][n_chunks * Lv][patch_dim] float, v_action: [branches][n_chunks*La][action_dim]
 * n_chunks = 1 is the incremental step: the chunk attends to all committed cache rows and to
 * itself. n_chunks > 1 is the full-sequence pass under the chunk-causal mask ([HYPER] 方法): chunk c
 * attends to the committed rows and to chunks 0..c. Writes cache rows [length, length+n*Lq).
 * Requires length + n_chunks*Lq <= capacity (else WAM_E_CAPACITY). */
wam_status wam_dit_stack_fwd(const wam_config *cfg, const wam_weights *w, wam_kv_cache *cache,
                             const wam_ctx_kv *ctx, int n_chunks, const float *x_video, const float *x_action,
                             const float *t_video, const float *t_action, int start_frame, float *v_video,
                             float *v_action, void *ws, size_t ws_bytes, void *stream);

/* Commit one clean chunk ([HYPER] 方法: the executed chunk's predicted frames are replaced in the
 * KV cache by the real observation): a stack pass at t = 1 whose keys/values are written into rows
 * [length, length+Lq) of every layer; then cache->length += Lq (host bookkeeping, done only when
 * everything was enqueued). x_video [Lv][patch_dim], x_action [La][action_dim] float. */
wam_status wam_kv_append(const wam_config *cfg, const wam_weights *w, wam_kv_cache *cache, const wam_ctx_kv *ctx,
                         const float *x_video, const float *x_action, int start_frame, void *ws,
                         size_t ws_bytes, void *stream);

/* One causal DiT block ([ARCH] §2.3: norm -> modulation -> causal self-attention -> residual ->
 * norm -> cross-attention -> residual -> norm -> FFN -> residual) on the residual stream
 *   h:  [branches][n_chunks * Lq][D] float, updated in place
 *   e6: [n_chunks][2][6][D] float (device): shared time modulation per chunk and token group
 *       (0 = video, 1 = action), e.g. from wam_time_embed with t = {t_v0, t_a0, t_v1, ...}; the
 *       block adds its own mod offset
 * `layer` selects the layer's slices of the caches; this block's keys/values (after RMSNorm and
 * RoPE) go to rows [length, length + n_chunks * Lq) of that layer, and the queries attend to the
 * committed rows and to these rows under the chunk-causal rule of wam_dit_stack_fwd.
 * commit != 0 ([WS1] architecture: the DiT runner maintains the attention KV): once everything is
 * enqueued, cache->length += n_chunks * Lq. The length is shared by all layers, so a caller that runs
 * the stack block by block passes commit only with its last block, after every layer has written
 * its rows at the same length (as wam_kv_append does in one call). Errors as wam_dit_stack_fwd
 * (nothing enqueued, length unchanged). */
wam_status wam_dit_block_fwd(const wam_config *cfg, const wam_block_weights *bw, int layer, wam_kv_cache *cache,
                             const wam_ctx_kv *ctx, float *h, const float *e6, int n_chunks, int start_frame,
                             int commit, void *ws, size_t ws_bytes, void *stream);

/* Guidance + Euler + similarity ([N569]: conditional/unconditional passes combined; DiT caching
 * by the cosine similarity of successive velocities).
 *   v_video [branches][n_video], v_action [branches][n_action]: per-branch velocities
 *   guided g = guidance * v_cond + (1 - guidance) * v_uncond (branches = 2) or v (branches = 1)
 *   x_video += dt_video * g_video; x_action += dt_action * g_action
 *   g_video / g_action (optional, may be NULL): the guided velocities; g_video may alias prev_video
 *   prev_video (optional): if given, cos_parts[0..3) = (<g,prev>, |g|^2, |prev|^2) over the video
 *   part, fp32 partial sums in a fixed order for given sizes (deterministic). cos_parts is device
 *   memory.
 * With prev_video, ws must hold 12 * min(512, max(1, ceil((n_video + n_action) / 4096))) bytes
 * (at most 6 KB; wam_workspace_bytes(cfg, 1) always suffices), else WAM_E_ARG. */
wam_status wam_flow_step(float *x_video, float *x_action, const float *v_video, const float *v_action, int branches,
                         float guidance, int n_video, int n_action, float dt_video, float dt_action,
                         float *g_video, float *g_action, const float *prev_video, float *cos_parts, void *ws,
                         size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): wam_flow_step without a workspace. The cosine partials go to a
 * device scratch array owned by the library, 6144 bytes (512 workgroups x 3 floats) on each GPU it
 * runs on, held until the process ends; the call never allocates or frees memory. Every size
 * wam_flow_step accepts fits that scratch (its grid is capped at 512 workgroups); a larger need is
 * rejected with WAM_E_ARG. All calls on one GPU share the scratch, which keeps the last call's
 * partials: calls that overlap on one GPU (different streams, or threads without ordering) race.
 * Nothing in it needs clearing: each call writes every partial it reads. Arguments, results and
 * errors otherwise as wam_flow_step (bit-identical results for the same inputs). */
wam_status wam_flow_step_noalloc(float *x_video, float *x_action, const float *v_video, const float *v_action,
                                 int branches, float guidance, int n_video, int n_action, float dt_video,
                                 float dt_action, float *g_video, float *g_action, const float *prev_video,
                                 float *cos_parts, void *stream);

/* One chunk's denoising loop ([N569] dynamic DiT caching; [WS1] dynamic16 scheduler): n_steps Euler
 * steps over the host times grid[0..n_steps] (both token groups at grid[k]), CFG with `guidance`,
 * with velocity reuse: steps 0 and 1 always run the DiT; at step k >= 2, if the cosine similarity of
 * the two most recent DiT-computed guided video velocities exceeds tau (and fewer than
 * max_consecutive_reuse steps in a row were reused; negative = no limit), the DiT is skipped and
 * the latest computed guided velocities drive the Euler update.
 *   x_video [Lv * P], x_action [La * A] (float, device): updated in place
 *   v_video [branches][Lv][P], v_action [branches][La][A] (float, device): scratch for the DiT output
 *   g_video [Lv * P], g_action [La * A] (float, device): the latest computed guided velocities (out)
 *   cos_parts (float[3], device): scratch for the similarity partial sums
 *   dit_calls (host, may be NULL): DiT passes run; reused (host, n_steps bytes, may be NULL): 1 where
 *   a step reused the velocity
 * The decision needs the similarity on the host: with tau <= 1 the call synchronises `stream` once
 * per DiT pass (12 bytes read back); with tau > 1 reuse is impossible and nothing synchronises.
 * Workspace: wam_workspace_bytes(cfg, 1). The cache is read, not committed (use wam_kv_append). */
wam_status wam_denoise_chunk(const wam_config *cfg, const wam_weights *w, wam_kv_cache *cache, const wam_ctx_kv *ctx,
                             float *x_video, float *x_action, const float *grid, int n_steps, float guidance, float tau,
                             int max_consecutive_reuse, int start_frame, float *v_video, float *v_action,
                             float *g_video, float *g_action, float *cos_parts, void *ws, size_t ws_bytes,
                             void *stream, int *dit_calls, unsigned char *reused);

/* The Euler loop of wam_denoise_chunk with the reuse decisions given instead of taken: step k reuses
 * the latest computed guided velocities iff replay[k] != 0 (host, n_steps bytes; replay[0] and
 * replay[1] must be 0: the first two steps always run the DiT). For decisions another implementation
 * took, e.g. when a similarity lies so close to the threshold that rounding may flip it ([N569] DiT
 * caching: the rule compares a similarity with a predefined threshold).
 *   cosines (host, n_steps floats, may be NULL): the similarity the rule would compare at step k (of
 *   the two most recent DiT-computed guided video velocities), NaN where it compares none (k < 2).
 *   With cosines the call synchronises `stream` once per DiT pass (12 bytes read back); without, never.
 * Other arguments, results and errors as wam_denoise_chunk; WAM_E_ARG for a NULL mask or a set
 * replay[0] / replay[1], nothing enqueued then. */
wam_status wam_denoise_chunk_replay(const wam_config *cfg, const wam_weights *w, wam_kv_cache *cache,
                                    const wam_ctx_kv *ctx, float *x_video, float *x_action, const float *grid,
                                    int n_steps, float guidance, const unsigned char *replay, int start_frame,
                                    float *v_video, float *v_action, float *g_video, float *g_action, float *cos_parts,
                                    void *ws, size_t ws_bytes, void *stream, int *dit_calls, float *cosines);

/* The same loop with the UniPC solver in place of Euler ([WS1] names UniPC as the scheduler's
 * solver; no formula on the pages: the published predictor UniP-p / corrector UniC-p in
 * data-prediction form with B(h) = e^h - 1, for alpha_t = t, sigma_t = 1 - t, lambda_t =
 * log(alpha_t / sigma_t), data prediction m = x + sigma_t g). Arguments as wam_denoise_chunk, plus:
 *   order 1..3: predictor order; steps from t = 0, to t = 1 and the step after one from t = 0 run
 *     at order 1 (lambda is infinite at the ends; the order-1 predictor is the Euler step)
 *   corrector != 0: after each DiT pass, the previous step is corrected with the fresh output
 *     (same order as its predictor); skipped after a reused velocity
 *   state: device scratch of 5 * (Lv * P + La * A) floats (data predictions and the previous
 *     state), owned by the caller, contents irrelevant on entry
 * The grid must increase strictly within [0, 1]. Errors as wam_denoise_chunk, plus WAM_E_ARG for
 * an order outside 1..3, a NULL state or a bad grid. */
wam_status wam_denoise_chunk_unipc(const wam_config *cfg, const wam_weights *w, wam_kv_cache *cache,
                                   const wam_ctx_kv *ctx, float *x_video, float *x_action, const float *grid,
                                   int n_steps, float guidance, float tau, int max_consecutive_reuse, int start_frame,
                                   int order, int corrector, float *v_video, float *v_action, float *g_video,
                                   float *g_action, float *cos_parts, float *state, void *ws, size_t ws_bytes,
                                   void *stream, int *dit_calls, unsigned char *reused);

/* Kernel-level calls, exposed so each kernel can be verified on its own (same kernels as above).
 *
 * Linear layer ([ARCH] §2.3: every projection of the block): C[m][n] = act(sum_k A[m][k] W[n][k] +
 * bias[n]) with A [M][lda], W [N][ldw], C [M][ldc] in `dtype`; bias float [N] or NULL; act 0 = none,
 * 1 = GELU (tanh approximation, the FFN's activation), 2 = SwiGLU pairs (N even: C[m][j] =
 * SiLU(z[m][2j]) * z[m][2j+1] with z = A W^T + bias, so C has N / 2 columns). K must be a multiple of 64;
 * A and W must each stay below 2 GiB (the kernels address them with 32-bit buffer offsets), else
 * WAM_E_SHAPE. M = 0 launches nothing and returns WAM_OK.
 * ws / ws_bytes: optional device scratch (256-byte aligned) for split-K partial products; with
 * NULL, or too little room, the product runs unsplit. A split product sums its fp32 partials in a
 * fixed order, so results are deterministic, but they may differ from the unsplit product in the
 * last bits. The stack and block calls use the split-K region of their own workspace. */
wam_status wam_op_linear(wam_dtype dtype, const void *A, int lda, const void *W, int ldw, const float *bias, void *C,
                         int ldc, int M, int N, int K, int act, void *ws, size_t ws_bytes, void *stream);

/* Finishing row kernel of a split product, on its own ([ARCH] §2.3 single block: the gated residual
 * that closes the self-attention and FFN sub-blocks, then the adaLN of the sub-block that follows;
 * the block runs this kernel after every product it splits over K):
 *   v[m][n] = (sum over s < splits, in order, of part[s][m][n]) + bias[n]
 *   h[m][n] += gate[n] v[m][n], gate = e6[gate_idx] + mod_gate[gate_idx] (gate_idx in 0..5), or
 *              gate = 1 (gate_idx < 0; mod_gate unused)
 *   y[m][n] = bf16(norm(h[m])[n] (1 + e6[scale_idx][n] + mod_norm[scale_idx][n])
 *                  + e6[shift_idx][n] + mod_norm[shift_idx][n])
 * norm: LayerNorm without affine over the row (RMSNorm when rms != 0) with eps, in fp32.
 * part fp32 [splits][M][N]; h fp32 [M][N], updated in place; e6, mod_gate, mod_norm fp32 [6][N]
 * (e6 the time modulation of the rows, mod_* the layer offsets); bias fp32 [N] or NULL; y bf16
 * [M][N]. All device pointers, owned by the caller, 16-byte aligned. 2 <= splits <= 4; N a multiple
 * of 4 up to 8192; else WAM_E_SHAPE / WAM_E_ARG. M = 0 launches nothing. Deterministic. */
wam_status wam_op_split_finish(const float *part, int splits, int M, int N, const float *bias, float *h,
                               const float *e6, const float *mod_gate, int gate_idx, const float *mod_norm,
                               int shift_idx, int scale_idx, int rms, float eps, void *y, void *stream);

/* Modulated norm of fp32 rows, on its own ([ARCH] §2.3: the adaLN before self-attention and FFN;
 * the block's first norm of a pass, and every norm of a product that is not split):
 *   y[m][n] = bf16(norm(x[m])[n] (1 + e6[scale_idx][n] + mod[scale_idx][n]) + e6[shift_idx][n] + mod[shift_idx][n])
 * x fp32 [M][D]; e6, mod fp32 [6][D]; y bf16 [M][D]; norm as in wam_op_split_finish. Device pointers,
 * 16-byte aligned; D a multiple of 4 up to 8192; indices in 0..5; else WAM_E_SHAPE / WAM_E_ARG. */
wam_status wam_op_modulated_norm(const float *x, int M, int D, const float *e6, const float *mod, int shift_idx,
                                 int scale_idx, int rms, float eps, void *y, void *stream);

/* Post-processing of the QKV projection output, on its own ([ARCH] §2.3 single block: q and k are
 * RMS-normalised with learned gains and rotated by the 3-D rotary embedding before attention; the
 * pass's keys and values enter the attention cache). For branch b < br and row r < rows:
 *   q_out[b][h][r][:]          = rot_r(rmsnorm(q[b rows + r]) g_q)[h d .. h d + d)
 *   k_cache[b][h][row0 + r][:] = rot_r(rmsnorm(k[b rows + r]) g_k)[h d .. h d + d)
 *   v_cache[b][h][j][row0 + r] = v[b rows + r][h d + j]
 * where q | k | v are columns [0, D), [D, 2D), [2D, 3D) of qkv (bf16 [br rows][3D], D = H d), rmsnorm
 * is over all D columns with eps in fp32, and rot_r rotates the pairs (2i, 2i+1) of every head by
 * (cos, sin) = rope[r][i] for the video rows of a chunk (r mod Lq < Lv) and leaves the action rows
 * unrotated. g_q, g_k fp32 [D]; rope fp32 [rows][d/2][2]; q_out bf16 [br][H][rows][d]; k_cache bf16
 * [br][H][cap][d]; v_cache bf16 [br][H][d][cap] (keys contiguous). Device pointers owned by the caller,
 * 16-byte aligned. d is 64 or 128; rows, cap, row0 multiples of 8; row0 + rows <= cap; D <= 8192; else
 * WAM_E_SHAPE / WAM_E_ARG. */
wam_status wam_op_qkv_cache(const void *qkv, int br, int rows, int Lq, int Lv, int H, int d, const float *g_q,
                            const float *g_k, float eps, const float *rope, void *q_out, void *k_cache, void *v_cache,
                            int cap, int row0, void *stream);

/* Low-precision projections ([N569] real-time optimisations: quantised projections) in the OCP
 * microscaling format that gfx950's scaled matrix instructions read (MXFP8): fp8 e4m3 codes (bias
 * 7, subnormals, largest finite 448) sharing one e8m0 power-of-two scale per 32 consecutive elements
 * of a row. Quantisation: per block e = max(floor(log2(amax)) - 8, -127), scale byte e + 127, codes
 * = e4m3 of x * 2^-e saturated to +-448, rounded to nearest even (deterministic, bit-exact).
 *   wam_mx_quantize: src [rows][ld] (bf16 or float, dtype) -> codes [rows][ldq] bytes (ldq multiple
 *   of 16), scales [rows][cols / 32] bytes; cols multiple of 32.
 *   wam_op_linear_mx: C[m][n] = act(sum_k dequant(A)[m][k] dequant(W)[n][k] + bias[n]) with A codes
 *   [M][lda] and scales [M][K/32], W codes [N][ldw] and scales [N][K/32], fp32 accumulation, C bf16
 *   [M][ldc] (W MXFP8, or MXFP4 with w_format below); act as wam_op_linear; K multiple of 128, N
 *   multiple of 4, lda / ldw multiples of 16,
 *   codes 16-byte and scales 4-byte aligned. Errors: WAM_E_SHAPE / WAM_E_ARG, nothing launched.
 *   ws: optional scratch for split-K partials (as wam_op_linear). */
wam_status wam_mx_quantize(wam_dtype dtype, const void *src, int ld, int rows, int cols, void *codes, int ldq,
                           void *scales, void *stream);
/* MXFP4 (weights): e2m1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit: 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6), block exponent e = max(floor(log2(amax)) - 2, -127), codes = e2m1 of x * 2^-e
 * saturated to +-6, nearest even; two codes per byte, low nibble first (k even), codes [rows][ldq]
 * bytes with ldq >= cols / 2 a multiple of 16; scales as wam_mx_quantize. */
wam_status wam_mx4_quantize(wam_dtype dtype, const void *src, int ld, int rows, int cols, void *codes, int ldq,
                            void *scales, void *stream);
enum { WAM_MX_E4M3 = 0, WAM_MX_E2M1 = 1 };
/* w_format: WAM_MX_E4M3 (W codes [N][ldw] bytes, ldw >= K) or WAM_MX_E2M1 (packed nibbles, ldw >= K/2). */
wam_status wam_op_linear_mx(const void *A, const void *A_scales, int lda, const void *W, const void *W_scales, int ldw,
                            int w_format, const float *bias, void *C, int ldc, int M, int N, int K, int act, void *ws,
                            size_t ws_bytes, void *stream);

/* Attention ([ARCH] §2.3 causal self-attention and cross-attention; [HYPER] 方法 mask):
 * for branch b, head h, query q < Lq: softmax over keys j < limit(q) of (Q.K_j) / sqrt(head_dim), times V,
 * limit(q) = kv_total, or min(kv_total, kv_base + (q / chunk_q + 1) * chunk_q) when chunk_q > 0.
 *   Q  [br][H][Lq][d], K [br][H][k_rows][d] (k_rows >= kv_total), Vt [br][H][d][v_stride]
 *   (v_stride multiple of 8, >= kv_total), O [br*Lq][H*d]; all in dtype; d = 64 or 128.
 * ws / ws_bytes: optional device scratch (256-byte aligned). When the query blocks of 128 would fill
 * fewer than half of the GPU's CUs and there are at least 8 key tiles of 32, bf16 attention splits
 * each block's keys into up to 8 ranges (flash-decoding style) if the scratch holds their partial
 * outputs (66 x 64 fp32 per 32 queries and range); the ranges are merged in a fixed order, so the
 * result is deterministic, and equals the unsplit result up to rounding. Without scratch (NULL, or
 * too small) nothing is split. The stack and block calls use their own workspace. */
/* Packed projections of one layer for WAM_PRECISION_MXFP8 / MXFP4W. Layout (each region 256-byte
 * aligned, in this order for w_qkv, w_o, w_cq, w_co, w_ff1, w_ff2): codes (e4m3 [N][K], or e2m1
 * [N][K/2] packed for MXFP4W) then e8m0 scales [N][K/32] of the [N][K] matrix. wam_mx_block_bytes: the arena size (0 for a configuration the
 * format cannot serve: dtype not bf16, dim or ffn_dim not multiples of 128). wam_mx_pack_block
 * quantises bw's bf16 matrices into dst (device, 256-byte aligned, dst_bytes >= the arena size); run
 * once per layer after the weights are loaded. Errors: WAM_E_ARG / WAM_E_SHAPE, nothing launched. */
size_t wam_mx_block_bytes(const wam_config *cfg);
wam_status wam_mx_pack_block(const wam_config *cfg, const wam_block_weights *bw, void *dst, size_t dst_bytes,
                             void *stream);

/* Fragment-packed weights (bf16): the same projections ([ARCH] §2.3 single causal block: q/k/v,
 * attention output, cross-attention query and output, the two FFN matrices), stored once in the order
 * the matrix instructions read them, so the products stream each weight fragment from memory in whole
 * 1 KB lines instead of staging it through the compute unit's shared memory. Layout of a packed W
 * [N][K] (N % 32 == 0, K % 64 == 0): N * K bf16 in blocks of 32 rows x 16 k, block (b, c) at element
 * offset (b * K / 16 + c) * 512, 64 lanes x 8 bf16 in it, lane l holding W[32 b + l % 32][16 c + 8 (l / 32)
 * .. + 7]; a band of 32 rows therefore occupies the bytes it would unpacked.
 *   wam_pack_weight: packs W [N][ldw] (device, 16-byte aligned, ldw >= K a multiple of 8) into dst
 *   (device, N * K * 2 bytes, 16-byte aligned); N * K * 2 < 2^31.
 *   wam_op_linear_packed: C = act(A Wp^T + bias) as wam_op_linear (bf16 only; A [M][lda], lda >= K a
 *   multiple of 8; C [M][ldc], ldc a multiple of 4; act 0 / 1 / 2; ws as wam_op_linear) with W given
 *   packed. Where both products take the same split of K (none, or the same number of ranges, as at
 *   the block's projection shapes), the result equals the unpacked product bit for bit: the same
 *   matrix instructions consume the same operands in the same k order.
 *   wam_pack_block_bytes: the packed size of one layer's six projections (w_qkv, w_o, w_cq, w_co,
 *   w_ff1, w_ff2 back to back, in this order), 0 for a configuration that cannot be packed (dtype not
 *   bf16, or a matrix of 2 GiB or more). wam_pack_block packs bw's six matrices into dst (device,
 *   256-byte aligned, dst_bytes >= that size); run once per layer after the weights are loaded, then
 *   set the block's pk to dst.
 * Errors: WAM_E_ARG / WAM_E_SHAPE / WAM_E_UNSUPPORTED, nothing launched. */
wam_status wam_pack_weight(const void *W, int ldw, int N, int K, void *dst, void *stream);
wam_status wam_op_linear_packed(const void *A, int lda, const void *Wp, const float *bias, void *C, int ldc, int M,
                                int N, int K, int act, void *ws, size_t ws_bytes, void *stream);
size_t wam_pack_block_bytes(const wam_config *cfg);
wam_status wam_pack_block(const wam_config *cfg, const wam_block_weights *bw, void *dst, size_t dst_bytes,
                          void *stream);

wam_status wam_op_attention(wam_dtype dtype, const void *Q, const void *K, const void *Vt, void *O, int br, int heads,
                            int head_dim, int Lq, int k_rows, int v_stride, int kv_base, int chunk_q, int kv_total,
                            void *ws, size_t ws_bytes, void *stream);

/* MXFP8 attention ([N569] real-time optimisations, mixed precision: the fp8 QKV projection and an
 * fp8 e4m3 softmax), head_dim 128, same visibility rule as wam_op_attention. Operands are OCP MXFP8:
 * e4m3 codes with one e8m0 scale byte (value 2^(byte - 127)) per 32 consecutive values.
 *   Q  [br][H][Lq][128] codes, Q_scales [br][H][Lq][4]        (blocks along the head dimension)
 *   K  [br][H][k_rows][128] codes, K_scales [br][H][k_rows][4]
 *   Vt [br][H][128][v_stride] codes (key-contiguous), Vt_scales [br][H][v_stride / 32][128]: the
 *      scale of key block kb of value row r is byte kb * 128 + r (blocks along keys)
 *   O  [br * Lq][H * 128] bfloat16.
 * Scores in fp32 from the scaled matrix instruction; softmax with an integer reference (log2 units);
 * each query's probabilities are quantised to MXFP8 in blocks of 32 keys (block rule of
 * wam_mx_quantize) before the product with the values; the normaliser is the sum of the unquantised
 * probabilities. Keys at or past kv_total never reach the output, whatever their codes hold; the scale
 * of the 32-key block that holds key kv_total - 1 must be the one of its valid keys (quantise zero-padded
 * rows). v_stride: a multiple of 64, >= kv_total rounded up to 64. Alignment: codes, Vt_scales and O
 * 16 bytes, Q/K scales 4 bytes. Errors: WAM_E_ARG / WAM_E_SHAPE, nothing launched. */
wam_status wam_op_attention_mx(const void *Q, const void *Q_scales, const void *K, const void *K_scales, const void *Vt,
                               const void *Vt_scales, void *O, int br, int heads, int Lq, int k_rows, int v_stride,
                               int kv_base, int chunk_q, int kv_total, void *stream);

/* Sliding attention window ([WS1] continuous requests: the attention window releases old KV and
 * the frame position restarts; [HYPER] 方法: cached clean chunks are the only past a chunk sees).
 * Drops the oldest `drop_rows` committed rows of every layer and branch (whole chunks: a multiple
 * of the tokens per chunk, at most cache->length) and moves the kept chunks' frame positions back by
 * `frame_shift` frames: the frame-axis rotary pairs of their video keys are rotated by
 * -frame_shift * freq(j) (rotations compose, so a key rotated for frame f becomes the key of frame
 * f - frame_shift); values and action keys only move. The rows are moved in place, on `stream`; on
 * success cache->length -= drop_rows, and the next chunk should be appended / denoised with its start
 * frame lowered by frame_shift (frame_shift = dropped chunks x frames_per_chunk restarts the window's
 * positions at its first kept chunk). drop_rows = 0 does nothing. Errors: WAM_E_ARG (NULL or
 * misaligned pointers), WAM_E_SHAPE (drop_rows not whole chunks or above the length; cache
 * geometry); nothing is enqueued then. */
wam_status wam_kv_evict(const wam_config *cfg, wam_kv_cache *cache, int drop_rows, int frame_shift, void *stream);

/* Host-side: forget every committed row ([WS1] continuous requests: at a window boundary the
 * old KV is released and the frame position restarts). No device work. */
void wam_kv_reset(wam_kv_cache *cache);

/* Text of the last non-OK status returned on this thread (empty string if none). */
const char *wam_last_error(void);

/* Measurement hook for the QKV projection (the largest product of a block): while enabled, every
 * pass that runs block `layer` with full q/k/v records a HIP event pair around that product on its
 * stream, up to `max_samples` pairs (1..4096, else WAM_E_ARG). layer < 0 disables and frees the
 * events. The events are created on the current device, which the timed passes must use. One
 * process-wide timer, not thread-safe. Events are host-side objects: no device memory is
 * allocated. */
wam_status wam_qkv_timer_config(int layer, int max_samples);

/* Durations (ms) of the recorded samples, oldest first: ms[0 .. min(*n, cap)), *n = the number
 * recorded since the last read (which restarts the count). Waits for the recorded events: the one
 * call of this library that blocks the host. ms is a HOST array (may be NULL when cap = 0). */
wam_status wam_qkv_timer_read(float *ms, int cap, int *n);

/* Measurement hook: the matrix-core rate the hardware sustains. Launches `workgroups` x 256 threads
 * (one wave per SIMD), each wave issuing iters x 8 independent bf16 32x32x16 MFMAs (32768 flops
 * each: workgroups x 4 x iters x 8 x 32768 flops in all);
 * out: device floats, workgroups x 256 (written so the products are not optimised away). Time it
 * with events on `stream`. Errors: WAM_E_ARG (NULL out, workgroups outside [1, 65536], iters < 1). */
wam_status wam_mfma_peak_probe(float *out, int workgroups, int iters, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* WAM_H_ */
