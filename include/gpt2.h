/*
 * gpt2.h -- C-ABI of libgpt2hip.so: one GPT-2 training micro-step and
 * optimizer step on an AMD Instinct MI355X (gfx950).
 *
 * The calls mirror the training loop the pages print:
 *   optimizer.zero_grad(); for each micro-step { loss = model(x, y) / G;
 *   loss.backward(); } clip_grad_norm_(params, 1.0); optimizer.step()
 *   ("How I trained my own GPT-2 124M on FineWeb-Edu", sections 8.1 and 9;
 *    "Reproduce GPT-2 124M 复盘", training-optimisation list: clipping;
 *    "Making Training Fast on One GPU", "How the measurements were taken").
 *
 * Conventions shared by every entry point
 *  - Memory: every device buffer is allocated and owned by the caller.  The
 *    library allocates no device memory; it keeps the pointers it is given,
 *    which must stay valid until gpt2_destroy.  Sizes come from
 *    gpt2_query_sizes.  Pointers named d_* are device pointers.
 *  - Streams: `stream` arguments are hipStream_t values passed as void*
 *    (NULL = the default stream).  Every call is asynchronous on its stream,
 *    except the few whose comments say they synchronise: gpt2_get_status,
 *    gpt2_get_step, gpt2_graph_capture, gpt2_op_gemm_grouped,
 *    gpt2_profile_reset and gpt2_destroy.
 *  - Layouts: row-major.  Tokens and targets are int32 [B, T].  Linear
 *    weights are [out, in] (nn.Linear).  The parameter table (order, offsets,
 *    shapes) is given by gpt2_param_info.
 *  - Errors: host-checkable problems (null pointers, shapes, limits) are
 *    returned immediately as a negative gpt2_status and nothing is enqueued.
 *    Device-detected problems (an out-of-range token or target id, a
 *    non-finite gradient norm) set a flag in the context: kernels clamp the
 *    offending index so no access leaves its buffer, and the flag is
 *    reported (and cleared) by gpt2_get_status.
 *  - Threads: one context is used by one host thread at a time.
 */
#ifndef GPT2_HIP_H
#define GPT2_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT2_OK = 0,
  GPT2_WARN_NO_TARGETS = 1, /* a micro-batch had no valid target: loss is NaN, no gradient added */
  GPT2_ERR_ARG = -1,        /* null pointer, bad enum or out-of-range scalar */
  GPT2_ERR_SHAPE = -2,      /* B, T, M, N, K or config not supported */
  GPT2_ERR_HIP = -3,        /* a HIP runtime call failed */
  GPT2_ERR_UNBOUND = -4,    /* a required buffer was not given */
  GPT2_ERR_BAD_ID = -5,     /* a token id outside [0, V) or a target outside [0, V) and not -1 */
  GPT2_ERR_NONFINITE = -6   /* the global gradient norm was not finite: the update was skipped */
} gpt2_status;

enum { GPT2_PRECISION_FP32 = 0, GPT2_PRECISION_BF16 = 1 };
enum { GPT2_ARCH_GPT2 = 0, GPT2_ARCH_ROTARY = 1 };

/* Model and capacity.  GPT2Config of "How I trained my own GPT-2 124M on
 * FineWeb-Edu" section 2.1 plus the MLP width (section 2.6, 4 * n_embd for
 * GPT-2), the largest micro-batch the buffers are sized for, and the compute
 * precision:
 *   FP32: every tensor and every product in float32.
 *   BF16: bfloat16 operands for the matrix products and attention, with
 *         float32 accumulation, float32 master weights, gradients, optimizer
 *         state, residual streams, norm and softmax statistics and loss
 *         ("Making Training Fast on One GPU", Step 1, BF16 autocast).
 * Limits: n_embd % n_head == 0; head_dim = n_embd / n_head must be 64 in
 * BF16 mode and at most 64 in FP32 mode; in BF16 mode vocab_size, n_embd and
 * mlp_hidden must be multiples of 8 (the page pads the vocabulary to 50304
 * for the same alignment reason, section 8.3); max_batch * block_size (the
 * rows of one micro-step) at most 131,072 (the embedding backward sorts a
 * micro-step's rows by token so that every gradient row sums its rows in a
 * fixed order); vocab_size * n_embd below 2^31.
 * arch selects the model family:
 *   GPT2_ARCH_GPT2:   the GPT-2 model above (LayerNorm, learned positions,
 *                     GELU MLP of width mlp_hidden, biases).
 *   GPT2_ARCH_ROTARY: the modern variant of "Reproduce GPT-2 124M 复盘"
 *                     (its model listing and training improvements): no
 *                     position table, RMSNorm (weight only, eps = float32
 *                     machine epsilon) for the block norms and ln_f, rotary
 *                     embedding (base 10000, rotate_half form) on q and k,
 *                     a SwiGLU feed-forward silu(x W_gate^T) * (x W_up^T)
 *                     W_down^T of hidden width mlp_hidden, no biases, lm_head
 *                     tied to wte.  BF16 only; n_embd % 256 == 0, head_dim
 *                     64, mlp_hidden % 32 == 0.  Its table: wte, per layer
 *                     ln_1.weight, attn.c_attn.weight [3C, C],
 *                     attn.c_proj.weight, ln_2.weight, mlp.c_fc.weight
 *                     [2F, C] (rows 0..F-1 W_gate, F..2F-1 W_up),
 *                     mlp.c_proj.weight [C, F], then ln_f.weight.
 * n_kv_head (0 means n_head) selects grouped-query attention ("Making
 * Training Fast on One GPU", step 2, whose model shares each key/value head
 * among n_head / n_kv_head consecutive query heads): the rotary variant
 * accepts any divisor of n_head, c_attn.weight then being
 * [C + 2 n_kv_head head_dim, C] (q rows, then the k rows and the v rows of
 * the n_kv_head shared heads); the GPT-2 model requires n_kv_head == n_head
 * (or 0). */
typedef struct {
  int32_t vocab_size;
  int32_t block_size;
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;
  int32_t mlp_hidden;
  int32_t max_batch;
  int32_t precision;
  int32_t arch;
  int32_t n_kv_head;  /* key/value heads; 0 = n_head (see above) */
} gpt2_config;

/* Byte sizes of the caller-owned buffers. */
typedef struct {
  size_t n_params;          /* number of parameters (tied wte counted once) */
  size_t n_elems;           /* elements of the flat parameter buffer (with alignment padding) */
  int32_t n_tensors;        /* entries of the parameter table */
  int32_t n_decayed;        /* leading entries with weight decay (dim >= 2) */
  size_t params_bytes;      /* float32 [n_elems] master weights */
  size_t grads_bytes;       /* float32 [n_elems] gradients */
  size_t adam_m_bytes;      /* float32 [n_elems] first moment */
  size_t adam_v_bytes;      /* float32 [n_elems] second moment */
  size_t shadow_bytes;      /* bfloat16 [n_elems] copy of the weights (0 in FP32 mode) */
  size_t activations_bytes; /* activations kept for the backward, for max_batch x block_size */
  size_t scratch_bytes;     /* per-call temporaries */
} gpt2_sizes;

typedef struct {
  void *params, *grads, *adam_m, *adam_v, *shadow, *activations, *scratch;
} gpt2_buffers;

/* AdamW hyper-parameters ("How I trained my own GPT-2 124M on FineWeb-Edu"
 * section 6: betas (0.9, 0.95), eps 1e-8, decay only on dim >= 2;
 * clip max_norm 1.0 from "Reproduce GPT-2 124M 复盘"). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay, max_norm;
} gpt2_adamw;

/* One entry of the parameter table: HF-style name, element offset into the
 * flat buffers (params, grads, adam_m, adam_v, shadow share offsets), shape
 * ([out, in] for Linear weights), and whether AdamW decays it. */
typedef struct {
  char name[64];
  size_t offset;
  int32_t ndim;
  int32_t shape[2];
  int32_t decayed;
} gpt2_param_desc;

typedef struct gpt2_ctx gpt2_ctx;

/* ---------------------------------------------------------------- setup -- */

/* Validate cfg and report buffer sizes.  Host only; no GPU needed.
 * Returns GPT2_ERR_ARG / GPT2_ERR_SHAPE for an unsupported config. */
int gpt2_query_sizes(const gpt2_config* cfg, gpt2_sizes* out);

/* Entry idx (0 <= idx < n_tensors) of the parameter table: the GPT-2
 * parameters of the named_parameters listing in "How I trained my own GPT-2
 * 124M on FineWeb-Edu" section 2 (lm_head is wte, section 4), ordered with
 * the decayed 2-D tensors first.  Host only. */
int gpt2_param_info(const gpt2_config* cfg, int idx, gpt2_param_desc* out);

/* Bind the caller's buffers (sizes from gpt2_query_sizes; shadow may be NULL
 * in FP32 mode) and a stream.  *out receives the context.  The step counter
 * starts at 0 and the device error flag is cleared. */
int gpt2_create(const gpt2_config* cfg, const gpt2_buffers* bufs, void* stream, gpt2_ctx** out);
int gpt2_destroy(gpt2_ctx* ctx);
int gpt2_set_stream(gpt2_ctx* ctx, void* stream);

/* Packed windows under a document mask ("GPT" chapter of Zero to Frontier,
 * "Document boundaries, packing and masking": documents concatenated with an
 * end-of-text separator before each, attention block-diagonal over the
 * documents of a window, position ids restarted at each document).  With
 * eot in [0, vocab_size), every later gpt2_fwd_bwd treats each row of tokens
 * as such a window: a document begins at each token equal to eot (the
 * separator is its first token, at position 0) and the tokens before the
 * row's first eot form a document of their own.  Query t sees key s iff
 * start(t) <= s <= t, start(t) the last eot position <= t (0 if none); the
 * GPT-2 model adds wpe[t - start(t)]; the rotary variant applies only the
 * mask (with the mask in place, rotating by t or by t - start(t) gives the
 * same scores, as that section notes).  Targets are untouched (the last
 * token of a document still predicts the next eot).  eot == -1 restores the
 * plain causal model.  Changing the setting discards a captured graph
 * (gpt2_graph_capture).  eot outside [-1, vocab_size): GPT2_ERR_ARG. */
int gpt2_set_doc_mask(gpt2_ctx* ctx, int eot);

/* Initialise every parameter: Linear weights and both embeddings ~ N(0,
 * 0.02), the two residual projections (attn.c_proj, mlp.c_proj) ~ N(0, 0.02 /
 * sqrt(2 n_layer)), biases 0, LayerNorm weight 1 and bias 0 ("How I trained
 * my own GPT-2 124M on FineWeb-Edu" section 7).  Normals come from
 * Philox4x32-10 (Salmon et al., SC 2011) with the Box-Muller transform:
 * element j of table entry k under seed s uses counter (j/4 low, j/4 high,
 * k, 0x6770), key (s low, s high), and takes output pair j%4/2 of the four
 * words.  Also zeroes grads and both moments, refreshes the bf16 shadow and
 * sets the step counter to 0. */
int gpt2_init_params(gpt2_ctx* ctx, uint64_t seed);

/* Refresh the bf16 shadow from the float32 master weights (after the caller
 * wrote params directly).  No-op in FP32 mode. */
int gpt2_sync_shadow(gpt2_ctx* ctx);

/* ----------------------------------------------------------- train step -- */

/* grads <- 0 (optimizer.zero_grad with set_to_none=False, the form "Making
 * Training Fast on One GPU" found necessary under graph replay). */
int gpt2_zero_grad(gpt2_ctx* ctx);

/* One micro-step ("How I trained my own GPT-2 124M on FineWeb-Edu" sections
 * 2.10-2.13, 4, 5, 8.1): the forward pass of the B x T tokens, the mean
 * cross-entropy of the logits over all vocab_size columns against the
 * targets (targets equal to -1 are ignored; the mean divides by the number
 * of valid targets of this call: "Multi-GPU calculation of gradients for
 * accelerated training", "Cross-entropy averages within one micro-batch"),
 * and the backward pass, which ADDS d(loss_scale * loss)/d(theta) into
 * grads (loss_scale = 1 / grad_accum_steps reproduces loss / grad_accum_steps).
 *   d_tokens, d_targets: int32 [B, T] device arrays; tokens in [0, V),
 *     targets in [0, V) or -1.  Out-of-range ids set GPT2_ERR_BAD_ID in the
 *     context flag and are clamped.
 *   1 <= B <= max_batch, 1 <= T <= block_size.
 *   d_loss: device float, receives the UNSCALED mean loss of this micro-batch
 *     (NaN if no target is valid; then nothing is added to grads and the flag
 *     reports GPT2_WARN_NO_TARGETS).
 *   d_token_loss: optional device float [B, T], per-position loss (0 where
 *     the target is ignored).
 * The logits are never stored whole: the tied lm_head and the loss run over
 * chunks of 8192 rows (bf16 mode, as gpt2_lmhead_ce) or 4096 rows (FP32
 * mode), and each chunk's part of the backward runs before the next chunk.
 * The embedding gradients (wte rows of repeated tokens, and wpe rows of
 * restarted positions under the document mask) are summed in a fixed order,
 * so they are the same bit for bit when a call is repeated.
 * The first call on a context (any B, T) also copies the weight-gradient
 * launch's table to the scratch buffer, once, asynchronously on the stream;
 * the call does not synchronise. */
int gpt2_fwd_bwd(gpt2_ctx* ctx, const int32_t* d_tokens, const int32_t* d_targets, int B, int T,
                 float loss_scale, float* d_loss, float* d_token_loss);

/* Learning rate of optimizer step `step` (counted from 0) under the warmed-up
 * cosine schedule that "Reproduce GPT-2 124M 复盘" trains with (its
 * hyper-parameter listing: max_lr 1.5e-3, min_lr 0.1 max_lr, warmup 300,
 * max_steps 19,073; the page names the shape, not the formula):
 *   step < warmup:            max_lr (step + 1) / warmup
 *   warmup <= step <= max_steps: min_lr + (max_lr - min_lr) (1 + cos(pi r)) / 2,
 *                              r = (step - warmup) / (max_steps - warmup)
 *   step > max_steps:         min_lr
 * Host function (no device work).  NaN when warmup < 1, max_steps <= warmup
 * or step < 0. */
double gpt2_lr_at(int64_t step, double max_lr, double min_lr, int64_t warmup, int64_t max_steps);

/* HIP graph of one micro-step (the whole gpt2_fwd_bwd launch sequence),
 * for callers that replay it instead of issuing ~200 launches per
 * micro-step.  gpt2_graph_capture captures gpt2_fwd_bwd(ctx, d_tokens,
 * d_targets, B, T, loss_scale, d_loss, NULL) on an internal stream (after a
 * synchronisation of the context's stream) and keeps the instantiated graph
 * in the context, replacing any earlier one; nothing runs during capture.
 * gpt2_graph_launch replays it on the context's stream: each replay reads
 * whatever the token and target buffers hold at that time and adds its
 * gradients like gpt2_fwd_bwd.  Capture needs the profiler off and one
 * earlier gpt2_fwd_bwd on the context (any B and T: the weight-gradient
 * table is set up then); otherwise GPT2_ERR_ARG or GPT2_ERR_HIP.  gpt2_graph_launch
 * without a captured graph: GPT2_ERR_UNBOUND.  ("Build an LLM From Scratch:
 * Making Training Fast on One GPU", the compile modes: graphs of the step,
 * which there fail with gradient accumulation unless the gradients are
 * zeroed in place, as gpt2_zero_grad does.) */
int gpt2_graph_capture(gpt2_ctx* ctx, const int32_t* d_tokens, const int32_t* d_targets, int B, int T,
                       float loss_scale, float* d_loss);
int gpt2_graph_launch(gpt2_ctx* ctx);

/* Global-norm clipping then AdamW on every parameter, one fused pass
 * ("Reproduce GPT-2 124M 复盘": clip_grad_norm_(params, 1.0) and fused AdamW;
 * "How I trained my own GPT-2 124M on FineWeb-Edu" section 6: betas, eps, and
 * decay only on dim >= 2):
 *   norm = ||grads||_2 over every parameter;  if norm is finite:
 *   t = t + 1;  coef = min(1, max_norm / (norm + 1e-6))
 *   g = coef * grad;  p *= 1 - lr*wd (decayed tensors only)
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2
 *   p -= lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 * and refreshes the bf16 shadow.  grads are left as they were (unclipped).
 * d_grad_norm (optional device float) receives the pre-clip norm.  A
 * non-finite norm leaves params, m, v and the step counter t unchanged (a
 * skipped step, as an optimizer that skips on overflow leaves its count) and
 * sets GPT2_ERR_NONFINITE in the context flag.  The decision is taken on the
 * device: t lives in the scratch buffer. */
int gpt2_clip_adamw_step(gpt2_ctx* ctx, const gpt2_adamw* hp, float* d_grad_norm);

/* The step counter t (the number of updates applied since gpt2_init_params
 * or the last gpt2_set_step).  gpt2_get_step synchronises the context's
 * stream and reads it back; gpt2_set_step writes it asynchronously (t >= 0,
 * GPT2_ERR_ARG otherwise). */
int gpt2_get_step(gpt2_ctx* ctx, int64_t* t);
int gpt2_set_step(gpt2_ctx* ctx, int64_t t);

/* Synchronise the context's stream, then return (and clear) the device
 * flag: GPT2_OK, GPT2_WARN_NO_TARGETS, GPT2_ERR_BAD_ID or
 * GPT2_ERR_NONFINITE (the most severe seen since the last call), or
 * GPT2_ERR_HIP if the stream reported an error. */
int gpt2_get_status(gpt2_ctx* ctx);

const char* gpt2_strerror(int status);

/* --------------------------------------------- isolated lm_head + loss -- */

/* Bytes of scratch gpt2_lmhead_ce needs for M rows, width C, vocab V:
 * M * (C + 1) * 4 bytes plus one chunk of min(M, 8192) rows of bf16 logits
 * and their tile statistics (8192 * V * 2 + 8192 * ceil(V / 256) * 8). */
size_t gpt2_lmhead_ce_scratch_bytes(int M, int C, int V);

/* Tied lm_head and mean cross-entropy, forward and backward, for M rows
 * ("How I trained my own GPT-2 124M on FineWeb-Edu" section 4: logits =
 * hidden @ weight^T without bias, cross-entropy over every column; the mean
 * divides by the number of valid targets, "Multi-GPU calculation of
 * gradients for accelerated training", "Cross-entropy averages within one
 * micro-batch").
 *   d_hidden: bf16 [M, C]; d_weight: bf16 [V, C]; d_targets: int32 [M].
 *   ignore_index: rows whose target equals it are ignored (the library
 *     cross-entropy's argument of that name; the isolated lm_head workload
 *     uses -1).  Any other target must lie in [0, V).
 *   d_loss: device float, the mean loss (NaN if no target is valid).
 *   d_dhidden: bf16 [M, C], written: d(loss)/d(hidden).
 *   d_dweight: float32 [V, C], d(loss)/d(weight) is ADDED to it.
 *   d_scratch: gpt2_lmhead_ce_scratch_bytes(M, C, V) bytes.
 *   d_flag: optional device int32, receives GPT2_ERR_BAD_ID if a target
 *     other than ignore_index is outside [0, V) (that row is then ignored)
 *     or GPT2_WARN_NO_TARGETS if no target is valid (else left unchanged).
 * C and V must be multiples of 8, M >= 1, every pointer but d_targets,
 * d_loss and d_flag 16-byte aligned (GPT2_ERR_SHAPE / GPT2_ERR_ARG
 * otherwise).  Device-side only: asynchronous on `stream`.
 * The rows run in chunks of 8192: per chunk the logits product keeps, per
 * row and 256-column tile, the float32 maximum and sum of exponentials and
 * stores the chunk's logits in bf16 as offsets from that tile maximum; one
 * pass per row then forms the log-sum-exp, the loss (target logit
 * recomputed in float32) and the bf16 logit gradient in place, and one
 * launch runs both products of the backward on it (dHidden rows of the
 * chunk, and the chunk's share of dWeight) before the next chunk reuses the
 * buffer.  The logits of all M rows are never stored. */
int gpt2_lmhead_ce(void* stream, const void* d_hidden, const void* d_weight, const int32_t* d_targets,
                   int M, int C, int V, int ignore_index, float* d_loss, void* d_dhidden, float* d_dweight,
                   void* d_scratch, int32_t* d_flag);

/* ------------------------------------------------------- single kernels -- */
/* The building blocks of the step, exposed for kernel-level parity tests and
 * measurement.  All are asynchronous on `stream`. */

/* Matrix product C = alpha * op(A) op(B)^T with an epilogue.
 * op(A) is [M, K]: a_kmajor=1 means A is stored [M][lda] (K contiguous),
 *   a_kmajor=0 means A is stored [K][lda] (M contiguous).
 * op(B) is [N, K]: b_kmajor=1 means B is stored [N][ldb] (K contiguous),
 *   b_kmajor=0 means B is stored [K][ldb] (N contiguous).
 * dtype: GPT2_PRECISION_BF16 (A, B bf16, MFMA with float32 accumulation) or
 *   GPT2_PRECISION_FP32 (A, B float32).
 * epilogue, with v = alpha * acc + (bias ? bias[n] : 0):
 *   GPT2_EPI_STORE:      C[m][n] = v                        (C in out_bf16 ? bf16 : float32)
 *   GPT2_EPI_RESIDUAL:   C[m][n] = R[m][n] + v              (float32; R may equal C)
 *   GPT2_EPI_GELU:       C[m][n] = v, C2[m][n] = gelu_tanh(C[m][n])  (both out dtype)
 *   GPT2_EPI_DGELU:      C[m][n] = v * gelu_tanh'(U[m][n])   (U in out dtype)
 *   GPT2_EPI_ACCUMULATE: C[m][n] += v                       (float32)
 *   GPT2_EPI_GELU_GRAD:  u = v rounded to the out dtype; C[m][n] = gelu_tanh(u),
 *                        C2[m][n] = gelu_tanh'(u)            (both out dtype)
 *   GPT2_EPI_MUL:        C[m][n] = v * U[m][n]               (U in out dtype)
 * The rotary variant ("Reproduce GPT-2 124M": RoPE in the rotate_half form,
 * SwiGLU), bf16 only, A and B K-major unless noted, 256-wide block tiles:
 *   GPT2_EPI_ROPE:       C = v in bf16, except that in every 64-column head
 *                        below rope_cols, with t = m % rope_period and
 *                        (c, s) = rope[t][i]: C[m][h+i] = v[h+i] c - v[h+i+32] s,
 *                        C[m][h+i+32] = v[h+i+32] c + v[h+i] s (i < 32).
 *                        N and rope_cols multiples of 64.
 *   GPT2_EPI_SWIGLU:     B is the stacked [W_gate; W_up] ([2F][ldb], N = 2F,
 *                        F % 32 == 0, K % 64 == 0, no bias); with
 *                        g = bf16(v[m][f]), u = bf16(v[m][F+f]):
 *                        C[m][f] = bf16(silu(g) u) (ldc), C2[m][f] = g and
 *                        C2[m][F+f] = u (row pitch ld2 >= 2F).
 *   GPT2_EPI_SWIGLU_BWD: A K-major, B not (a Linear's input gradient); N = F,
 *                        U holds [gate | up] (row pitch ld2), v is d(act):
 *                        C[m][f] = v u silu'(g), C[m][F+f] = v silu(g)
 *                        (bf16, ldc >= 2F).  silu(g) = g sigmoid(g).
 * ("How I trained my own GPT-2 124M on FineWeb-Edu" 2.13 for the tanh GELU;
 * its derivative by the chain rule.)  GELU_GRAD feeds the MLP's second
 * product with gelu(u) and keeps gelu'(u) so that the backward's input
 * gradient is a MUL epilogue.
 * ldc is the row pitch of C, C2, R and U (but see ld2).  For bf16, M, N, K,
 * lda, ldb, ldc must be multiples of 8, every pointer 16-byte aligned, and
 * out_bf16 must be 1 for GELU, DGELU, GELU_GRAD, MUL, ROPE, SWIGLU and
 * SWIGLU_BWD and 0 for RESIDUAL and ACCUMULATE.  The three rotary-variant
 * epilogues exist in bf16 only. */
enum {
  GPT2_EPI_STORE = 0,
  GPT2_EPI_RESIDUAL = 1,
  GPT2_EPI_GELU = 2,
  GPT2_EPI_DGELU = 3,
  GPT2_EPI_ACCUMULATE = 4,
  GPT2_EPI_GELU_GRAD = 5,
  GPT2_EPI_MUL = 6,
  GPT2_EPI_ROPE = 7,
  GPT2_EPI_SWIGLU = 8,
  GPT2_EPI_SWIGLU_BWD = 9
};
typedef struct {
  int32_t M, N, K;
  int32_t dtype;
  int32_t a_kmajor, b_kmajor;
  int64_t lda, ldb, ldc;
  const void* A;
  const void* B;
  void* C;
  void* C2;
  const float* R;
  const void* U;
  const float* bias;
  float alpha;
  int32_t epilogue;
  int32_t out_bf16;
  /* GPT2_EPI_ROPE: (cos, sin) float32 pairs [rope_period][32] (see
   * gpt2_op_rope_table); row m is at position m % rope_period; columns
   * below rope_cols are rotated. */
  const void* rope;
  int32_t rope_period, rope_cols;
  /* GPT2_EPI_SWIGLU: row pitch of C2; GPT2_EPI_SWIGLU_BWD: row pitch of U. */
  int64_t ld2;
} gpt2_gemm_args;
int gpt2_op_gemm(void* stream, const gpt2_gemm_args* args);

/* Grouped weight-gradient products: the n products args[0..n) (each a
 * Linear's weight gradient dW += dY^T X summed over tokens, the backward of
 * "How I trained my own GPT-2 124M on FineWeb-Edu" section 2.3's Linear
 * layers) in ONE launch.  Every product must be bf16 with both operands
 * K-slow (a_kmajor = b_kmajor = 0), epilogue GPT2_EPI_ACCUMULATE, no bias,
 * and satisfy gpt2_op_gemm's rules; d_row_sums (a host array of n device
 * pointers, or NULL; entries may be NULL) receive row_sum_i[m] +=
 * alpha_i * sum_k A_i(m, k) (the bias gradient).  One block per 256x256
 * output tile; when the tiles leave a partial last round of blocks, the
 * products at the end of the list may be split in K into four (or two)
 * pieces that add their partial sums atomically, where a list-scheduling
 * estimate says that shortens the launch (pieces keep at least 16 K steps
 * of 64); every other tile is computed whole and added once.  The n outputs must not overlap.  d_workspace: device memory of
 * gpt2_gemm_grouped_workspace_bytes(args, n) bytes (16-byte aligned) that
 * receives the group table; the call copies it there synchronously (it
 * blocks until the copy is done), then launches on the stream.
 * GPT2_ERR_ARG for an invalid product or n < 1. */
size_t gpt2_gemm_grouped_workspace_bytes(const gpt2_gemm_args* args, int n);
int gpt2_op_gemm_grouped(void* stream, const gpt2_gemm_args* args, int n, float* const* d_row_sums,
                         void* d_workspace);

/* Column sums: db[n] += sum_m Y[m][n], Y [M][ld] in bf16 (y_bf16=1) or float32. */
int gpt2_op_colsum(void* stream, const void* d_y, int y_bf16, int M, int N, int64_t ld, float* d_db);

/* LayerNorm over rows of x [rows, C] float32 ("How I trained my own GPT-2
 * 124M on FineWeb-Edu" section 2.3, nn.LayerNorm defaults: eps 1e-5, biased
 * variance): y = (x - mean) * rstd * w + b, y in bf16 (y_bf16=1) or float32;
 * mean and rstd float32 [rows] are written for the backward. */
int gpt2_op_layernorm_fwd(void* stream, const float* d_x, const float* d_w, const float* d_b, void* d_y,
                          int y_bf16, float* d_mean, float* d_rstd, int rows, int C);
/* Backward of the above for dy [rows, C] (float32, or bf16 when dy_bf16):
 * dx is ADDED to the float32 d_dx; when d_dx_bf16 is not NULL it also
 * receives bf16 of the updated d_dx; sum over rows of dy * xhat and of dy
 * are ADDED to d_dw and d_db.  When C is a multiple of 256 every pointer
 * (and, with y_bf16, those of the forward) must be 16-byte aligned
 * (GPT2_ERR_ARG otherwise). */
int gpt2_op_layernorm_bwd(void* stream, const void* d_dy, int dy_bf16, const float* d_x, const float* d_mean,
                          const float* d_rstd, const float* d_w, float* d_dx, void* d_dx_bf16, float* d_dw,
                          float* d_db, int rows, int C);

/* RMSNorm of the rotary variant: y = x rstd w (bf16), rstd = (mean(x^2) +
 * eps)^-1/2 per row (float32), eps = 2^-23.  C % 256 == 0, C <= 1024,
 * pointers 16-byte aligned. */
int gpt2_op_rmsnorm_fwd(void* stream, const float* d_x, const float* d_w, void* d_y, float* d_rstd, int rows, int C);
/* Its backward for dy float32 or bf16 (dy_bf16): dx (float32) += rstd (g -
 * xhat mean(g xhat)) with g = dy w and xhat = x rstd; d_dx_bf16 (nullable)
 * receives bf16 of the updated dx; dw += sum over rows of dy xhat. */
int gpt2_op_rmsnorm_bwd(void* stream, const void* d_dy, int dy_bf16, const float* d_x, const float* d_rstd,
                        const float* d_w, float* d_dx, void* d_dx_bf16, float* d_dw, int rows, int C);

/* Rotary embedding, head dimension 64 ("Reproduce GPT-2 124M 复盘": x cos +
 * rotate_half(x) sin, dimension i paired with i + 32):
 * gpt2_op_rope_table writes (cos, sin) of t base^(-2i/64) as float32 pairs
 * [T][32] (angles in double precision); gpt2_op_rope_bwd applies, in place,
 * the transpose of the rotation to the first `cols` columns (q and k, heads
 * of 64) of the bf16 matrix d_dqkv [rows][ld], row r at position r % T:
 * z_i' = z_i c + z_{i+32} s, z_{i+32}' = z_{i+32} c - z_i s.
 * cols % 64 == 0, ld % 4 == 0, d_dqkv 8-byte aligned. */
int gpt2_op_rope_table(void* stream, int T, double base, float* d_table);
int gpt2_op_rope_bwd(void* stream, void* d_dqkv, int rows, int64_t ld, int cols, int T, const float* d_table);

/* Causal multi-head attention ("How I trained my own GPT-2 124M on
 * FineWeb-Edu" sections 2.12 and 5): qkv [B*T, (H + 2 Hkv) hd] holds the H
 * query heads, then the Hkv key heads, then the Hkv value heads (hd columns
 * each); query head h attends with key/value head h / (H / Hkv) (grouped-
 * query attention, "Making Training Fast on One GPU" step 2; Hkv == H is
 * plain multi-head attention, H % Hkv must be 0); y [B*T, H*hd] receives the
 * concatenated heads; lse float32 [B, H, T] the row log-sum-exp of the scaled
 * scores (natural log).  dtype selects bf16 or float32 tensors.
 * d_seg (nullable) int32 [B, T]: document starts of packed windows (as
 * gpt2_op_segment_starts writes them: 0 <= seg[t] <= t, non-decreasing
 * along a row); query t then sees only keys seg[t] .. t.  Starts that break
 * those rules give unspecified values (never an access outside the
 * tensors). */
int gpt2_op_attention_fwd(void* stream, int dtype, int B, int T, int H, int Hkv, int hd, const void* d_qkv,
                          void* d_y, float* d_lse, const int32_t* d_seg);
/* Backward: dqkv [B*T, (H + 2 Hkv) hd] is written (a shared key/value
 * head receives the sum over its query heads).  d_scratch needs
 * gpt2_attention_bwd_scratch_bytes(B, T, H) = 8 B H T bytes (two floats
 * per row, 4-byte aligned); d_seg as in the forward.
 * d_rope (nullable; bf16 only, 16-byte aligned): a [T][32] (cos, sin) table
 * as gpt2_op_rope_table writes it; dq and dk are then rotated back with the
 * transpose of the rotary embedding at their row's position before they
 * are written (what gpt2_op_rope_bwd does in a separate pass, here with one
 * bf16 rounding instead of two). */
size_t gpt2_attention_bwd_scratch_bytes(int B, int T, int H);
int gpt2_op_attention_bwd(void* stream, int dtype, int B, int T, int H, int Hkv, int hd, const void* d_qkv,
                          const void* d_y, const void* d_dy, const float* d_lse, void* d_dqkv,
                          void* d_scratch, const int32_t* d_seg, const float* d_rope);

/* The attention backward above without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels, with
 * their two floats per row (D = rowsum(dO o O) and the row's log-sum-exp in
 * log2 units) kept in a static device array of the library (one per GPU,
 * gpt2_noalloc_scratch_bytes() = 8 MiB, held until the process ends).
 * B * H * T must not exceed gpt2_noalloc_scratch_bytes() / 8 = 1,048,576
 * (GPT2_ERR_SHAPE otherwise; nothing is launched).  Allocates nothing: the
 * first call on a device looks up that device's copy of the array once.
 * Every call on one GPU shares the array; calls that overlap in time on one
 * GPU (two streams or threads) race on it and must be serialised by the
 * caller.  Arguments, layouts and results as gpt2_op_attention_bwd;
 * GPT2_ERR_HIP if the array's address cannot be obtained or the launch
 * fails. */
size_t gpt2_noalloc_scratch_bytes(void);
int gpt2_op_attention_bwd_noalloc(void* stream, int dtype, int B, int T, int H, int Hkv, int hd, const void* d_qkv,
                                  const void* d_y, const void* d_dy, const float* d_lse, void* d_dqkv,
                                  const int32_t* d_seg, const float* d_rope);

/* Embedding backward ("How I trained my own GPT-2 124M on FineWeb-Edu"
 * sections 2.2 and 2.10, x = wte[idx] + wpe[t]), the kernels gpt2_fwd_bwd
 * runs: for every row i = b T + t of d_dres [B*T, C] (float32, the gradient
 * of x), d_dwte[tokens[i]] += d_dres[i] and, when d_dwpe is not NULL,
 * d_dwpe[p(i)] += d_dres[i], with p(i) = t, or t - d_seg[i] under a
 * document mask (d_seg as gpt2_op_segment_starts writes it; nullable).
 * Both tables are float32 [V, C] and [T, C] and are accumulated into.  Every
 * gradient row adds its source rows in increasing i, so repeated calls give
 * the same bits.  Token ids outside [0, V) add to row 0 (the forward flags
 * them).  d_scratch: gpt2_embedding_bwd_scratch_bytes(B*T, C) bytes,
 * 256-byte aligned (GPT2_ERR_ARG otherwise).  GPT2_ERR_SHAPE unless
 * B*T <= 131,072, B*T*C < 2^31 and V*C < 2^31. */
size_t gpt2_embedding_bwd_scratch_bytes(int rows, int C);
int gpt2_op_embedding_bwd(void* stream, const int32_t* d_tokens, const float* d_dres, float* d_dwte, float* d_dwpe,
                          int B, int T, int C, int V, const int32_t* d_seg, void* d_scratch);

/* Document starts of packed rows ("GPT" chapter of Zero to Frontier,
 * "Document boundaries, packing and masking"): d_seg[b*T + t] = the last
 * position s <= t with d_tokens[b*T + s] == eot, 0 if there is none (int32,
 * device).  Any eot value is accepted (one that never occurs gives 0s). */
int gpt2_op_segment_starts(void* stream, const int32_t* d_tokens, int B, int T, int eot, int32_t* d_seg);

/* ---------------------------------------------------------- measurement -- */

/* When enabled, the context brackets every kernel launch it makes with HIP
 * events on its stream and accumulates, per launch site, the number of
 * launches and their summed duration.  Site names are stable strings such
 * as "gemm.fc_fwd" or "attn.fwd". */
int gpt2_profile_enable(gpt2_ctx* ctx, int on);
/* Restrict the timing to launches from one site (site == NULL: all sites),
 * so that a measurement of one kernel adds no events around the others. */
int gpt2_profile_only(gpt2_ctx* ctx, const char* site);
/* When on, every timed launch is preceded by one launch of an empty kernel
 * (g2::site_marker_kernel, 1 x 64 threads) on the context's stream, so that
 * a per-dispatch hardware-counter trace can attribute the dispatch that
 * follows each marker to the selected site.  Off by default; it adds one
 * tiny launch per timed launch. */
int gpt2_profile_mark(gpt2_ctx* ctx, int on);
/* One launch of the same empty marker kernel on `stream` (NULL: the null
 * stream), to delimit foreign work in such a trace. */
int gpt2_op_marker(void* stream);
int gpt2_profile_reset(gpt2_ctx* ctx);
int gpt2_profile_count(gpt2_ctx* ctx);
/* Entry i: site name (static storage), launches, summed milliseconds.  Call
 * after gpt2_get_status so the events have completed. */
int gpt2_profile_entry(gpt2_ctx* ctx, int i, const char** name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_HIP_H */
