/*
 * dg.h -- C ABI of the DiffusionGemma denoise-step library for MI355X (gfx950).
 *
 * The library runs the hot path of a block-diffusion text generator: a causally
 * encoded prompt KV cache, then rounds of denoising over a 256-token canvas.
 * Pages describing the method (secondary summaries of the DiffusionGemma report):
 *   [mlqm]     mlqm.cn/news/993655, sections 一 (multinomial diffusion), 二 (MoE,
 *              causal prompt / bidirectional canvas attention, self-conditioning),
 *              四 (entropy-ordered commit, re-noise, 0.8 -> 0.4 temperature,
 *              adaptive stop), 五 (where the step's time goes)
 *   [chooseai] chooseai.io/news/4338: encoder caches the prompt, decoder attends
 *              bidirectionally; block-autoregressive multi-canvas sampling
 *   [bohu]     bohuyeshan.top, section 一: a developer implements one denoise step;
 *              a finished canvas enters the KV cache before the next one starts
 *
 * Conventions
 *   - Every pointer named d_* is device memory on the current HIP device,
 *     allocated and owned by the caller; h_* pointers are host memory.  The
 *     library borrows them for the duration of the call (asynchronous on the
 *     given stream: buffers must stay valid until the stream reaches the work).
 *   - Handles (dg_model, dg_state) own only host metadata, except that a model
 *     owns derived weight copies in device memory, made once in dg_model_create
 *     and freed by dg_model_destroy: the fused QKV matrices ((Hq + 2 Hkv) hd d
 *     elements per layer), the transposed embedding for the self-conditioning
 *     contraction (V d elements, self-conditioning models), and the expert
 *     weights in MFMA-fragment order (3 E F d elements per layer, or bytes in
 *     FP8), which every expert product of a bf16 model reads -- the weight
 *     streaming for few routed rows and the grouped 128 x 128 products for
 *     many -- whenever ffn_hidden is a multiple of 128 (fp32 models pack for
 *     the streaming products only and keep reading the caller's tensors in
 *     the grouped ones), and (FP8 LM head) the E4M3 codes and scales of the
 *     embedding's rows (V d bytes + 4 V).  A bf16 model so packed, and every
 *     FP8 model, reads the caller's w_gate / w_up / w_down only inside
 *     dg_model_create: the caller may release them afterwards (the
 *     borrowed-weights rule below covers every other tensor).
 *   - The four step calls allocate nothing and never synchronise the device,
 *     except dg_encode_prompt / dg_commit_canvas_to_kv which only enqueue work.
 *   - Errors: a negative status is returned and a thread-local message is set
 *     (dg_last_error).  On an argument or capacity error no work is enqueued and
 *     the state is unchanged.  No exception or abort crosses the ABI.
 *   - Determinism: identical inputs and seeds give bitwise identical outputs
 *     (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dg_status;
#define DG_OK 0
#define DG_ERR_ARG (-1)          /* invalid argument (null pointer, bad size or config) */
#define DG_ERR_CAPACITY (-2)     /* context would exceed max_ctx, or state buffer too small */
#define DG_ERR_HIP (-3)          /* a HIP runtime call failed */
#define DG_ERR_UNSUPPORTED (-4)  /* shape outside what the kernels implement */

#define DG_DTYPE_F32 0
#define DG_DTYPE_BF16 1
#define DG_DTYPE_FP8_E4M3 2   /* expert and LM-head weights only: OCP FP8 E4M3 with one fp32 scale per output channel */

#define DG_STOP_NONE 0    /* run the whole step budget */
#define DG_STOP_MEAN 1    /* stop once the mean canvas entropy < stop_tau */
#define DG_STOP_PAGES 2   /* mean entropy < stop_tau and argmax unchanged from the previous step ([mlqm] 四) */

typedef struct dg_config {
  int32_t n_layers;
  int32_t d_model;      /* 256, 512, 768, 1024, 2048, 3072 or 4096 */
  int32_t n_q_heads;
  int32_t n_kv_heads;   /* divides n_q_heads */
  int32_t head_dim;     /* 64 or 128 */
  int32_t n_experts;    /* 1..128 */
  int32_t ffn_hidden;   /* multiple of 64 */
  int32_t top_k;        /* 1..min(8, n_experts) */
  int32_t vocab;        /* multiple of 64, at most 262144 */
  int32_t canvas_len;   /* 1..256; the pages' canvas is 256 tokens ([mlqm] 一) */
  int32_t dtype;        /* DG_DTYPE_F32 or DG_DTYPE_BF16: weight and matmul operand type */
  int32_t self_cond;    /* 1: add (softmax of the previous step) @ E @ W_sc^T to the embeddings */
  float rope_theta;
  float rms_eps;
  /* Storage of the expert weights: 0 = dtype; DG_DTYPE_FP8_E4M3 (bf16 models
   * with d_model % 512 == 0 and ffn_hidden % 256 == 0): dg_model_create
   * quantises the caller's bf16 experts to OCP FP8 E4M3 (chooseai.io speed
   * paragraph and bohuyeshan.top 一: the model is served in FP8), one fp32
   * scale per output channel, scale = fl32(fl64(max |w_row|) / 448) (1 for a
   * zero row), code = E4M3(fl32(w / scale)) rounded to nearest even and
   * saturating; the expert products then use code * scale.  The model keeps
   * only the packed codes and scales (3 E F d bytes + (2 F + d) E 4 bytes per
   * layer); every batch runs the weight-streaming expert products. */
  int32_t expert_dtype;
  /* Storage of the LM head's weights (the tied embedding E [V, d]): 0 = dtype;
   * DG_DTYPE_FP8_E4M3 (bf16 models): dg_model_create quantises each row of E
   * (one vocabulary id, one output channel of the head) to E4M3 by the rule
   * above, and the LM head computes logit[r][v] = scale[v] * (x_r . codes of
   * row v), fp32 sums of bf16 products, before the temperature and the head
   * statistics.  The embedding lookup and the self-conditioning contraction
   * keep reading the bf16 E.  The model holds V d bytes of codes and V fp32
   * scales in addition.  Full-vocabulary and top-k truncated sampling and
   * the training-side pass (dg_corrupt_forward_loss) all read it. */
  int32_t head_dtype;
} dg_config;

typedef struct dg_sampler_params {
  float t_start;        /* temperature at step 0 (0.8 on the pages) */
  float t_end;          /* temperature at step max_steps-1 (0.4) */
  float entropy_bound;  /* commit bound on the running entropy total, nats (0.1) */
  float stop_tau;       /* adaptive-stop threshold on the mean entropy, nats */
  int32_t max_steps;    /* step budget S of the canvas (48 on the pages) */
  int32_t stop_mode;    /* DG_STOP_* */
  /* 0: the full vocabulary.  1..8: top-k truncation ([mlqm] 九: truncating
   * the vocabulary to the top k raises throughput at high batch): the
   * distribution of a position is the softmax of its k largest logits (ties:
   * lower id) renormalised over them, all others 0; entropy, Gumbel-max
   * sample (over the k ids, each with its own draw of the Gumbel stream),
   * margin and the self-conditioning vector (sum over the k rows of E) use
   * it.  The LM head then keeps only each row's k best per vocabulary segment:
   * no exp(z - m) rows, no vocabulary-long softmax @ E product.  bf16 models
   * (any model in dg_sample_logits). */
  int32_t top_k;
} dg_sampler_params;

typedef struct dg_model dg_model;
typedef struct dg_state dg_state;
typedef struct ihipStream_t* dg_stream;   /* a hipStream_t; NULL = default stream */

/* Thread-local text of the last failure in this thread ("" if none). */
const char* dg_last_error(void);

/* Device views into a model's derived weights, for inspection:
 *   DG_MODEL_VIEW_EXPERT_GATEUP: layer `layer`'s packed gate/up expert weights
 *   DG_MODEL_VIEW_EXPERT_DOWN:   its packed down weights
 *     (FP8: codes P8GU[E][F/16][d/64][2][64][16], P8D[E][d/16][F/64][64][16],
 *     lane (c, g) of block (n/16, k/64) holding W[n][k0 + g*8 .. +8] then
 *     W[n][k0 + 32 + g*8 .. +8]; else the dtype's fragments
 *     [E][F/16][d/32][2][64][8] and [E][d/16][F/32][64][8])
 *   DG_MODEL_VIEW_EXPERT_SCALES_GATEUP: FP8 only, float [E][2][F] (gate, up)
 *   DG_MODEL_VIEW_EXPERT_SCALES_DOWN:   FP8 only, float [E][d]
 * DG_ERR_ARG if the model holds no such copy. */
#define DG_MODEL_VIEW_EXPERT_GATEUP 0
#define DG_MODEL_VIEW_EXPERT_DOWN 1
#define DG_MODEL_VIEW_EXPERT_SCALES_GATEUP 2
#define DG_MODEL_VIEW_EXPERT_SCALES_DOWN 3
/*   DG_MODEL_VIEW_HEAD_CODES:  FP8 LM head only (layer ignored): E4M3 codes
 *     of E in the order P8H[V/16][d/64][64][16], lane (c, g) of block
 *     (v/16, k/64) holding E[v][k0 + g*8 .. +8] then E[v][k0 + 32 + g*8 .. +8]
 *   DG_MODEL_VIEW_HEAD_SCALES: FP8 LM head only, float [V] */
#define DG_MODEL_VIEW_HEAD_CODES 4
#define DG_MODEL_VIEW_HEAD_SCALES 5
dg_status dg_model_view(const dg_model* model, int32_t which, int32_t layer, void** d_ptr, size_t* bytes);

/* Number of weight pointers dg_model_create expects for a config:
 * 2 + self_cond + 10 * n_layers. */
int32_t dg_weight_count(const dg_config* cfg);

/* Create a model over caller-owned device weights.
 * d_weights[i] point to tensors in this order ([out, in] layout for matrices,
 * row-major; type = cfg->dtype for matrices, float32 for norm gains):
 *   emb [V, d]; w_sc [d, d] (only if self_cond); final_norm [d];
 *   then per layer: attn_norm [d], wq [Hq*hd, d], wk [Hkv*hd, d], wv [Hkv*hd, d],
 *   wo [d, Hq*hd], ffn_norm [d], w_router [E, d], w_gate [E, F, d],
 *   w_up [E, F, d], w_down [E, d, F].
 * The weights are borrowed (must outlive the model; for the expert tensors see
 * the conventions above); the call synchronises the device once after building
 * the derived copies.  The LM head is tied to emb. */
dg_status dg_model_create(const dg_config* cfg, const void* const* d_weights, int32_t n_weights,
                          dg_model** out);
void dg_model_destroy(dg_model* model);

/* Device bytes needed by a state for `batch` requests and a KV capacity of
 * max_ctx positions per request (prompt + committed canvases + one canvas). */
dg_status dg_state_bytes(const dg_model* model, int32_t batch, int32_t max_ctx, size_t* bytes);

/* Build a state inside a caller-owned device buffer of at least dg_state_bytes.
 * Sets context length 0 and canvas index 0, and fills the RoPE table (enqueued
 * on the default stream, synchronised before return). */
dg_status dg_state_init(const dg_model* model, void* d_buf, size_t bytes, int32_t batch,
                        int32_t max_ctx, dg_state** out);
void dg_state_destroy(dg_state* state);

/* Largest context length N over the requests (positions held in the KV cache)
 * and largest canvas index.  Each request keeps its own N and canvas index in
 * device memory (DG_VIEW_CTX_LENS, DG_VIEW_CANVAS_INDEX); they differ once
 * dg_commit_canvas_to_kv has committed only some requests ([mlqm] 四: every
 * request stops on its own). */
int32_t dg_state_ctx_len(const dg_state* state);
int32_t dg_state_canvas_index(const dg_state* state);

/* Device views into the state buffer, for inspection and teacher forcing:
 *   DG_VIEW_K_CACHE: [L][B][Hkv][ctx_pad][hd], cfg dtype, ctx_pad = max_ctx rounded up to 64
 *   DG_VIEW_V_CACHE: [L][B][Hkv][hd][ctx_pad], cfg dtype (V transposed: each kv head's values
 *                    stored dimension-major, so attention reads V^T rows directly)
 *   DG_VIEW_SELF_COND: float [B][canvas_len][d], the vector s of the last step
 *   DG_VIEW_PREV_ARGMAX: int32 [B][canvas_len], argmax seen by the last commit
 *   DG_VIEW_ROUTE: int32 [L][B * canvas_len][top_k], expert ids chosen in each
 *     layer by the last pass (its first B * rows-per-request rows are valid)
 *   DG_VIEW_HIDDEN: float [rows][d], residual stream after the last layer of
 *     the last pass (before the final norm)
 *   DG_VIEW_ROUTER_LOGITS: float [L][B * canvas_len][n_experts], router logits
 *     of each layer of the last pass (same row convention)
 *   DG_VIEW_ATTN_OUT: [rows][n_q_heads * head_dim], cfg dtype, attention output
 *     (before the output projection) of the last layer of the last pass
 *   DG_VIEW_CTX_LENS: int32 [B], context length N of each request
 *   DG_VIEW_CANVAS_INDEX: int32 [B], canvas index of each request (Philox stream) */
#define DG_VIEW_K_CACHE 0
#define DG_VIEW_V_CACHE 1
#define DG_VIEW_SELF_COND 2
#define DG_VIEW_PREV_ARGMAX 3
#define DG_VIEW_ROUTE 4
#define DG_VIEW_HIDDEN 5
#define DG_VIEW_ROUTER_LOGITS 6
#define DG_VIEW_ATTN_OUT 7
#define DG_VIEW_CTX_LENS 8
#define DG_VIEW_CANVAS_INDEX 9
dg_status dg_state_view(dg_state* state, int32_t which, void** d_ptr, size_t* bytes);

/* Initial canvas: canvas_len uniformly random tokens per request ([mlqm] 一,
 * [chooseai]: the canvas is first filled with random placeholder tokens).
 * d_canvas: int32 [B, canvas_len] (written).  h_seeds: uint64 [B] per-request
 * Philox seeds.  Uses the state's current canvas index. */
dg_status dg_init_canvas(dg_state* state, int32_t* d_canvas, const uint64_t* h_seeds,
                         dg_stream stream);

/* Causal encode of a prompt ([mlqm] 二: causal attention over the user input;
 * [chooseai]: the encoder caches the prompt context).  d_ids: int32 [B, P] with
 * every id in [0, V) (an id outside is clamped to that range; token ids of a
 * canvas are treated the same way).  Appends P positions to each request's KV cache at
 * N..N+P-1 and sets N += P.  P = 0 is a no-op.  DG_ERR_CAPACITY if
 * N + P > max_ctx.  The prompt is encoded in chunks of canvas_len tokens. */
dg_status dg_encode_prompt(dg_state* state, const int32_t* d_ids, int32_t P, dg_stream stream);

/* One denoising round over the canvas ([mlqm] 一, 二, 四).
 * d_canvas: int32 [B, canvas_len] current tokens (read).  step: 0-based round t
 * of the current canvas (self-conditioning is off at t = 0; the temperature is
 * t_start + (t_end - t_start) * t / (max_steps - 1)).  h_seeds: uint64 [B].
 * d_active: uint8 [B] or NULL (= all active); an inactive request (0) takes
 * no part in the pass: its rows, tiles and attention blocks are skipped, it
 * routes no row to an expert, and none of its outputs nor its state (K/V
 * cache, self-conditioning vector) is written ([mlqm] 四: a request that has
 * stopped is done).
 * Outputs, all [B, canvas_len]: d_H float entropy (nats) of softmax(logits/T);
 * d_y int32 Gumbel-max sample of that distribution; d_argmax int32 argmax of
 * the logits; d_margin float best minus second-best Gumbel-perturbed score.
 * d_logits: float [B, canvas_len, V] or NULL; if given, the raw logits are
 * written there.  Updates the state's self-conditioning vector.  The canvas's
 * own keys and values occupy cache positions N..N+canvas_len-1 during the step
 * (DG_ERR_CAPACITY if N + canvas_len > max_ctx). */
dg_status dg_denoise_step(dg_state* state, const int32_t* d_canvas, int32_t step,
                          const dg_sampler_params* params, const uint64_t* h_seeds,
                          const uint8_t* d_active, float* d_H, int32_t* d_y, int32_t* d_argmax,
                          float* d_margin, float* d_logits, dg_stream stream);

/* The sampler stage of dg_denoise_step alone, on caller-supplied logits
 * ([mlqm] 四; [chooseai] llama.cpp paragraph: the entropy-bounded sampler runs
 * on the model's logits): per row the temperature softmax, its entropy, the
 * logit argmax, the Gumbel-max sample and the top-2 margin, exactly as
 * dg_denoise_step computes them after its LM head, and (self-conditioning
 * models) the next step's self-conditioning vector from the same
 * distribution.  d_logits: float [B, canvas_len, V] (read).  Other arguments
 * and outputs as for dg_denoise_step. */
dg_status dg_sample_logits(dg_state* state, const float* d_logits, int32_t step, const dg_sampler_params* params,
                           const uint64_t* h_seeds, const uint8_t* d_active, float* d_H, int32_t* d_y,
                           int32_t* d_argmax, float* d_margin, dg_stream stream);

/* For callers that cannot allocate device memory or hand over a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the statistics of dg_sample_logits -- entropy, Gumbel-max
 * sample, logit argmax, top-2 margin -- on caller-supplied logits, with no
 * state.  d_logits: float [rows, vocab], rows = requests x canvas_len; request
 * b = row / canvas_len draws with seed h_seeds[b] (host, uint64 [rows /
 * canvas_len]) at canvas index canvas_index and step `step` (temperature from
 * params).  Outputs d_H, d_y, d_argmax, d_margin: [rows], as dg_sample_logits
 * writes them (bitwise: the same kernels).  No self-conditioning output.
 * The per-(row, 128-id chunk) records live in a fixed 16 MiB device array of
 * the library, held on each GPU until the process ends, so the call allocates
 * nothing: rows x ceil(vocab / 128) x 32 bytes + 4 KiB must fit it, else
 * DG_ERR_CAPACITY (for example 256 rows at vocab 262144 fit; 512 do not).
 * Every call on one GPU shares that array and overwrites it: calls that
 * overlap on one GPU (two streams, two threads) race and must be ordered by
 * the caller.  Requests at most 128; params->top_k must be 0 (the full
 * vocabulary; DG_ERR_UNSUPPORTED otherwise). */
dg_status dg_sample_logits_static(const float* d_logits, int32_t rows, int32_t vocab, int32_t canvas_len,
                                  int32_t canvas_index, int32_t step, const dg_sampler_params* params,
                                  const uint64_t* h_seeds, float* d_H, int32_t* d_y, int32_t* d_argmax,
                                  float* d_margin, dg_stream stream);

/* Entropy-bounded commit / uniform re-noise / adaptive stop ([mlqm] 四, 一).
 * Per request b with d_done[b] == 0: sort positions by (H, position), commit the
 * longest prefix whose running fp64 entropy total stays <= entropy_bound; the
 * committed positions take d_y, the others a fresh uniform token.  If the stop
 * rule fires or step == max_steps-1, every position takes d_y and d_done[b] = 1.
 * d_canvas int32 [B, canvas_len] is updated in place; d_commit_mask uint8
 * [B, canvas_len] and d_n_committed int32 [B] are written (positions that took
 * y); requests already done are left untouched.  d_argmax is remembered for
 * DG_STOP_PAGES. */
dg_status dg_sample_commit(dg_state* state, const float* d_H, const int32_t* d_y,
                           const int32_t* d_argmax, int32_t* d_canvas, int32_t step,
                           const dg_sampler_params* params, const uint64_t* h_seeds,
                           uint8_t* d_commit_mask, int32_t* d_n_committed, uint8_t* d_done,
                           dg_stream stream);

/* Append the finished canvas to the KV cache by a causal encode at positions
 * N..N+canvas_len-1 ([bohu] 一, [chooseai]: block-autoregressive canvases);
 * N += canvas_len, canvas index += 1 -- for the requests d_which selects:
 * d_which uint8 [B] (nonzero = commit) or NULL (= every request).  The others
 * compute nothing and keep their N, canvas index and cache.  DG_ERR_CAPACITY
 * if the largest N + canvas_len > max_ctx. */
dg_status dg_commit_canvas_to_kv(dg_state* state, const int32_t* d_canvas, const uint8_t* d_which,
                                 dg_stream stream);

/* Device-driven canvas loop ([mlqm] 四: up to max_steps rounds with adaptive
 * stop; [mlqm] 五: the CPU-GPU exchange made asynchronous).  Runs steps
 * first_step .. first_step + n_steps - 1 of the current canvas, each one
 * dg_denoise_step over the requests not yet done followed by dg_sample_commit,
 * with the step index and temperature kept on the device: no host read of
 * device memory.  first_step == 0 starts a canvas: the initial canvas is drawn
 * (dg_init_canvas), d_done and the self-conditioning vector are cleared;
 * first_step > 0 must continue the canvas where the previous call stopped.
 * Outputs as for those calls (the last step's values); d_done uint8 [B]
 * holds every request's flag.
 * flags:
 *   DG_RUN_GRAPH      the step is captured once into a HIP graph (kept in the
 *                     state, re-captured when buffers, parameters, seeds or
 *                     the attention launch plan change) and replayed per step;
 *   DG_RUN_EARLY_EXIT the host stays at most two steps ahead of the device,
 *                     reading a progress record the device writes to mapped
 *                     host memory, and stops issuing steps once every request
 *                     is done (without it all n_steps steps are issued; steps
 *                     after the last request is done compute nothing);
 *   DG_RUN_COMMIT_KV  dg_commit_canvas_to_kv of every request once the canvas
 *                     is finished (its last step issued, or every request seen
 *                     done).
 * h_result (may be NULL) receives {steps issued, canvas finished}.  Results
 * are bitwise those of the explicit calls with the same inputs. */
#define DG_RUN_GRAPH 1u
#define DG_RUN_EARLY_EXIT 2u
#define DG_RUN_COMMIT_KV 4u
dg_status dg_run_canvas(dg_state* state, int32_t* d_canvas, const dg_sampler_params* params,
                        const uint64_t* h_seeds, float* d_H, int32_t* d_y, int32_t* d_argmax, float* d_margin,
                        uint8_t* d_commit_mask, int32_t* d_n_committed, uint8_t* d_done, int32_t first_step,
                        int32_t n_steps, uint32_t flags, int32_t* h_result, dg_stream stream);

/* Training-side forward pass ([mlqm] 一: in training a share of a sequence's
 * tokens, from 0% to 100%, is replaced by random vocabulary tokens and the
 * model learns to restore the original).  Per request b, every position of
 * the clean canvas d_clean (int32 [B, canvas_len], ids in [0, V); an id
 * outside is clamped to that range) is replaced independently
 * with probability h_rates[b] (host float [B], each in [0, 1]) by a uniform
 * vocabulary token: one Philox4x32-10 call per position under the request's
 * seed, counter (0, position, 0, 5 << 24 | canvas index), word 0 deciding
 * (u < rate in fp32, u as for every draw of this library) and word 1 giving
 * the token.  The corrupted canvas (d_corrupted, int32 [B, canvas_len],
 * written) goes through the model exactly as a denoising round's canvas does
 * (after the request's context, bidirectional attention over the canvas, no
 * self-conditioning term), and the cross-entropy of the clean token,
 * logsumexp(logits) - logits[clean] (temperature 1, nats), is written per
 * position (d_ce, float [B, canvas_len]) and as its mean per request (d_loss,
 * float [B]).  Like a denoising round it uses the cache positions
 * N..N+canvas_len-1 as scratch.  Forward only: no gradients. */
dg_status dg_corrupt_forward_loss(dg_state* state, const int32_t* d_clean, const float* h_rates,
                                  const uint64_t* h_seeds, int32_t* d_corrupted, float* d_ce, float* d_loss,
                                  dg_stream stream);

/* Stage timing ([mlqm] 五 splits a step's cost into MoE, sampling and
 * attention; these counters give the same split for this implementation).
 * When enabled, the step calls record a HIP event pair on their stream around
 * every launch of the stages in `stage_mask` (bit i = stage i below); events
 * come from a fixed pool created here (4096 pairs), so the step calls still
 * allocate nothing; recording stops silently once the pool is full.
 * dg_profile_read synchronises on the recorded events, adds each pair's
 * elapsed time to ms[stage] and 1 to launches[stage] (arrays of
 * DG_NUM_STAGES, overwritten), then empties the pool. */
#define DG_STAGE_EMBED 0       /* embedding gather, self-conditioning projection */
#define DG_STAGE_NORM 1        /* RMSNorm */
#define DG_STAGE_QKV 2         /* fused QKV projection + RoPE + cache write */
#define DG_STAGE_ATTN 3        /* attention (+ split merge) */
#define DG_STAGE_OPROJ 4       /* output projection + residual */
#define DG_STAGE_ROUTER 5      /* router logits, top-k, bucketing */
#define DG_STAGE_EXPERT_UP 6   /* grouped expert gate/up + SwiGLU */
#define DG_STAGE_EXPERT_DOWN 7 /* grouped expert down projection */
#define DG_STAGE_COMBINE 8     /* weighted combine of expert outputs */
#define DG_STAGE_LM_HEAD 9     /* tied LM head */
#define DG_STAGE_SAMPLER 10    /* temperature softmax, entropy, Gumbel-max (partial + merge) */
#define DG_STAGE_SELFCOND 11   /* softmax @ E contraction (+ chunk reduce) */
#define DG_STAGE_COMMIT 12     /* commit / re-noise / stop */
#define DG_NUM_STAGES 13
dg_status dg_profile_enable(dg_state* state, uint32_t stage_mask);
dg_status dg_profile_read(dg_state* state, double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* DG_H_ */
