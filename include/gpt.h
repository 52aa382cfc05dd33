/* gpt.h - C ABI of one GPT forward+backward training step on an MI355X (gfx950).
 *
 * The step computes, for one batch of token rows, the mean next-token
 * cross-entropy of a decoder-only transformer and the gradient of that loss
 * with respect to every weight.  The network is the one the nanochat pages
 * describe:
 *   - "Introducing nanochat" (github.com/karpathy/nanochat/discussions/1),
 *     pretraining log and the paragraph after it: untied embedding and
 *     lm_head, separate Q, K, V, O projections, a 4*d MLP, no biases and no
 *     norm gains;
 *   - nanochat User Guide, section 10 "How It Works", base model paragraph:
 *     rotary embeddings, QK-norm, ReLU^2 MLP, sliding-window pattern;
 *   - "supa beginna nanochat" (discussions/677), troubleshooting: mean
 *     cross-entropy over rows of T+1 tokens split into inputs and targets.
 * Per layer: a = N(h); q,k,v = a Wq^T, a Wk^T, a Wv^T; q^ = N_h(RoPE(q)),
 * k^ = N_h(RoPE(k)); o = softmax(q^ k^T / sqrt(Dh) | window mask) v, head by
 * head (with n_kv_head < n_head, groups of query heads share k and v);
 * h += o Wo^T; h += relu(N(h) W1^T)^2 W2^T.  Then loss = mean CE(N(h) U^T, y).
 * N is parameter-free RMSNorm with eps = norm_eps; RoPE rotates the pairs
 * (x[i], x[i+Dh/2]) by t * base^(-2i/Dh); a layer of window W lets query i
 * see keys j with 0 <= i - j <= W - 1.
 *
 * Conventions.  All tensors are row-major and contiguous.  Pointers are
 * device pointers unless marked "host".  No function throws, aborts or
 * exits; every failure is a negative return code, with details available
 * from gpt_last_error() on the calling thread.  A model handle is not
 * thread-safe: use one handle per stream.
 */
#ifndef GPT_MI355X_H
#define GPT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- codes */
#define GPT_OK 0
#define GPT_EINVAL (-1)      /* bad configuration or argument value            */
#define GPT_ENULL (-2)       /* a required pointer is NULL                     */
#define GPT_ETOKEN (-3)      /* a token id outside [0, vocab) (device check)   */
#define GPT_EHIP (-4)        /* a HIP runtime call failed                      */
#define GPT_ENONFINITE (-5)  /* the loss came out NaN or infinite              */
#define GPT_ESPACE (-6)      /* workspace smaller than gpt_workspace_bytes()   */
#define GPT_EALIGN (-7)      /* a pointer is not 256-byte aligned              */

typedef enum { GPT_FP32 = 0, GPT_BF16 = 1, GPT_FP8 = 2 } gpt_precision;

typedef struct gpt_config {
  int32_t depth;        /* L, number of blocks                                */
  int32_t d_model;      /* d = n_head * head_dim, multiple of 64              */
  int32_t n_head;       /* H                                                  */
  int32_t head_dim;     /* Dh: 32 or 64 (GPT_FP32); 64 or 128 (GPT_BF16, GPT_FP8) */
  int32_t mlp_hidden;   /* F, multiple of 64                                  */
  int32_t vocab;        /* V, multiple of 8, <= 65536                         */
  int32_t seq_len;      /* T >= 1                                             */
  int32_t batch;        /* B >= 1, with B*T <= 32768                          */
  int32_t window;       /* keys per 'S' layer incl. the query itself (>= 1)   */
  char window_pattern[8]; /* NUL-terminated, chars 'S'/'L', cycled over layers;
                             the last layer is always 'L' (full causal)       */
  float rope_base;      /* RoPE base (10000)                                  */
  float norm_eps;       /* RMSNorm epsilon for every norm (1e-6), > 0         */
  int32_t precision;    /* gpt_precision: storage/compute policy, see below   */
  const void* weights;  /* device, caller-owned parameter buffer: see layout  */
  void* workspace;      /* device, caller-owned, >= gpt_workspace_bytes()     */
  size_t workspace_bytes;
  void* stream;         /* hipStream_t on which all work is enqueued (NULL = default) */
  int32_t n_kv_head;    /* Hkv, key/value heads (grouped-query attention): a
                           divisor of n_head; 0 means n_head (plain multi-head
                           attention).  Query head h uses key/value head
                           h / (n_head / Hkv) (nanochat User Guide, section 10,
                           base model paragraph: Group-Query Attention). */
} gpt_config;
/* Precision policy.  GPT_FP32: weights, activations and every product in
 * fp32 (fp32 MFMA).  GPT_BF16: bf16 weights and activations, fp32
 * accumulation, fp32 residual stream, fp32 norm/softmax statistics.
 * GPT_FP8: as GPT_BF16, except that the four linear layers of every block
 * (QKV, O, W1, W2) multiply fp8 operands with fp32 accumulation: weights and
 * activations in OCP E4M3, gradients in OCP E5M2, each tensor quantised in
 * every step with its own current scale (see gpt_fp8_quantize); embedding,
 * attention, norms, lm_head and the loss stay bf16/fp32.  B*T must be a
 * multiple of 64.  The "FP8 matrix products" of the d24 speedrun ("supa
 * beginna nanochat" discussion) and the alpha-nanochat-d24 model card are the
 * prior art; the format split and scaling rule are this library's. */

/* Parameter layout.  One contiguous buffer, tensors in this order:
 *   E [V, d]; for l in 0..L-1: Wq [d, d], Wk, Wv [Hkv*Dh, d], Wo [d, d],
 *   W1 [F, d], W2 [d, F]; U [V, d].
 * Shapes are [out, in].  Each tensor starts at an element offset that is a
 * multiple of 128; Wq, Wk, Wv of a layer are adjacent (one
 * [d + 2*Hkv*Dh, d] block; [3d, d] without grouping).
 * The weight buffer holds elements of the parameter type (fp32 for GPT_FP32,
 * bf16 otherwise); the gradient buffer uses the same element offsets with
 * fp32 elements. */
typedef struct gpt_model gpt_model;  /* opaque handle ("params" of a step) */

typedef struct gpt_tensor_desc {
  char name[24];        /* "E", "L3.Wq", ..., "U"                             */
  int64_t offset;       /* element offset in the weight / gradient buffer     */
  int32_t rows, cols;
} gpt_tensor_desc;

/* Number of parameter tensors (2 + 6*depth) and total elements of the
 * buffer including alignment gaps.  Returns GPT_EINVAL for a bad config. */
int gpt_param_layout(const gpt_config* cfg, gpt_tensor_desc* out, int capacity, int* n_tensors,
                     int64_t* total_elems);

/* Bytes of device workspace gpt_create needs for this config. */
int gpt_workspace_bytes(const gpt_config* cfg, size_t* bytes);

/* Validate cfg, build the launch plan and write the RoPE table into the
 * workspace (one small host->device copy on cfg->stream).  The handle keeps
 * cfg->weights, cfg->workspace and cfg->stream; the caller keeps them alive
 * and unchanged until gpt_destroy.  No device memory is allocated. */
int gpt_create(const gpt_config* cfg, gpt_model** out_model);

/* One forward+backward step.
 *   tokens, targets: device int32 [B, T], ids in [0, V) (checked on device).
 *   grads: device fp32 buffer in the parameter layout; every element is
 *          overwritten with d(loss)/d(weight) (not accumulated).
 *   loss:  host float, receives the mean cross-entropy.
 * Enqueues on cfg->stream, then waits for the stream; buffers may be reused
 * as soon as it returns.  Returns GPT_ETOKEN (grads undefined) for an
 * out-of-range id and GPT_ENONFINITE for a NaN/inf loss. */
int gpt_step(gpt_model* model, const int32_t* tokens, const int32_t* targets, float* grads, float* loss);

/* Gradient accumulation over micro-batches: a batch too large for one step
 * is split into k micro-batches of B rows each, and the gradient of the
 * mean loss over the whole batch is the mean of the micro-batch gradients
 * (nanochat's training loop, gradient accumulation over micro-steps).
 * Same as gpt_step, except that
 *   grads <- grad_scale * g               (accumulate == 0)
 *   grads <- grads + grad_scale * g       (accumulate == 1)
 * where g is the gradient of this micro-batch's mean loss; *loss receives
 * that (unscaled) mean.  grad_scale = 1/k with accumulate = 0 for the first
 * micro-batch and 1 for the rest gives the full batch's gradient.  The scale
 * multiplies the logit gradient, so every gradient carries it exactly once;
 * each accumulated element is the fp32 sum, rounded once, of its previous
 * value and the value a non-accumulating call would have stored.
 * grad_scale must be finite (GPT_EINVAL otherwise); accumulate must be 0 or
 * 1.  On GPT_ETOKEN / GPT_ENONFINITE the contents of grads are undefined
 * (an accumulation in progress is lost).  gpt_step(...) is
 * gpt_step_accum(..., 1.0f, 0, loss). */
int gpt_step_accum(gpt_model* model, const int32_t* tokens, const int32_t* targets, float* grads,
                   float grad_scale, int accumulate, float* loss);

/* n_micro micro-batches in one call, replayed as one captured HIP graph:
 * tokens and targets are device int32 [n_micro, batch, seq_len] (all
 * resident), grads as in gpt_step_accum: the first micro-batch stores
 * (accumulate == 0) or adds (accumulate == 1), every later one adds, each
 * scaled by grad_scale.  losses: host float[n_micro], each micro-batch's mean
 * loss.  1 <= n_micro <= 1024.  The graph is captured on the first call and
 * again whenever a pointer or argument differs from the captured call's; it
 * runs on a stream of the handle ordered after cfg->stream by events, and
 * the call waits for it.  With profiling on, the steps run eagerly.
 * GPT_ETOKEN if any id is out of range, GPT_ENONFINITE if any loss is not
 * finite (grads undefined then). */
int gpt_step_micro(gpt_model* model, const int32_t* tokens, const int32_t* targets, int n_micro, float* grads,
                   float grad_scale, int accumulate, float* losses);

/* ------------------------------------------------------------ optimizer
 * One optimizer step over every parameter, after the gradients of the step
 * (or of accumulated micro-batches) are complete: Muon on the projection
 * matrices (Wq, Wk, Wv, Wo, W1, W2, each matrix on its own) and AdamW on the
 * embedding E and the lm_head U ("Introducing nanochat", the pretraining log
 * and the paragraph after it; learning rates, weight decay and the gradient
 * clip of its report card's base-model section).  The pages name Muon
 * without its algorithm; it follows the published description (K. Jordan et
 * al., 2024): Nesterov momentum, then the update is orthogonalised by the
 * quintic Newton-Schulz iteration X <- a X + (b A + c A^2) X, A = X X^T,
 * (a, b, c) = (3.4445, -4.7750, 2.0315), on the Frobenius-normalised update
 * in bf16, and scaled by sqrt(max(1, rows/cols)).  AdamW has bias-corrected
 * moments and decoupled weight decay.  Muon momentum is kept as
 *   buf <- mu buf + (1 - mu) g,   u = (1 - mu) g + mu buf   (nesterov)
 *   or u = buf,
 * which differs from mu buf + g only by a factor the normalisation removes.
 * Every gradient is first scaled by min(1, grad_clip / (||g|| + 1e-6)),
 * ||g|| the 2-norm over all parameters (grad_clip <= 0: no clipping). */
typedef struct {
  float matrix_lr;       /* Muon learning rate */
  float momentum;        /* Muon momentum mu, in [0, 1) */
  int32_t nesterov;      /* 1: Nesterov look-ahead, 0: plain momentum */
  int32_t ns_steps;      /* Newton-Schulz iterations, 1..32 (5) */
  float embedding_lr;    /* AdamW learning rate of E */
  float unembedding_lr;  /* AdamW learning rate of U */
  float beta1, beta2;    /* AdamW moment decays, in [0, 1) */
  float eps;             /* AdamW denominator epsilon, > 0 */
  float weight_decay;    /* decoupled: p <- p (1 - lr wd) for every parameter */
  float grad_clip;       /* global-norm clip; <= 0 disables */
  int32_t step;          /* AdamW step count t >= 1 (bias correction) */
} gpt_optim_params;

/* Bytes of device state the optimizer needs for this config: fp32 master
 * weights (bf16 parameters only), Muon momenta, AdamW moments, pass tables
 * and the Newton-Schulz work buffers. */
int gpt_optim_state_bytes(const gpt_config* cfg, size_t* bytes);

/* Prepare `state` (device, 256-byte aligned, at least gpt_optim_state_bytes)
 * for this model: master weights from the model's weight buffer, zero
 * moments.  Synchronises the model's stream.  The model remembers the state;
 * a later gpt_optim_init (any state) replaces it. */
int gpt_optim_init(gpt_model* model, void* state, size_t state_bytes);

/* One optimizer step with device fp32 gradients `grads` (parameter layout):
 * updates the master weights and moments in `state` and rewrites the
 * model's weight buffer (cfg->weights) with the new weights (bf16: rounded
 * to nearest even from the fp32 masters).  Enqueued on the model's stream;
 * returns without waiting unless grad_norm (host, optional) is given, which
 * then receives the gradient norm before clipping.  Errors: GPT_EINVAL for
 * a state not prepared for this model or out-of-range parameters (nothing
 * is enqueued then). */
int gpt_optim_step(gpt_model* model, void* state, const float* grads, const gpt_optim_params* hp,
                   float* grad_norm);

/* Device pointer to the fp32 master weights in the parameter layout (inside
 * the state gpt_optim_init prepared; for GPT_FP32 models, the weight buffer
 * itself), e.g. to checkpoint them. */
int gpt_optim_master(gpt_model* model, float** master);

/* ------------------------------------------------------------ inference
 * Forward-only generation with a KV cache ("Introducing nanochat": the
 * model is served by an inference engine with a KV cache, prefill then
 * token-by-token decoding).  Every row of the batch advances together: a
 * prompt of n tokens per row is prefilled, then one token per row is decoded
 * per call.  Runs on bf16 parameters (GPT_BF16; GPT_FP8 models decode with
 * their bf16 weights); batch <= 32, head_dim 64 or 128; positions up to
 * seq_len - 1 (the RoPE table's length).  The model's workspace is reused, so
 * these calls must not overlap gpt_step on the same handle.
 *
 * KV cache: caller-owned device memory of gpt_kv_cache_bytes, bf16, layer l
 * at K = base + 2l * S, V = base + (2l + 1) * S, each [batch][n_head]
 * [seq_len][head_dim] (S = batch * n_head * seq_len * head_dim elements);
 * it holds the QK-normalised, rotated keys and the raw values. */
int gpt_kv_cache_bytes(const gpt_config* cfg, size_t* bytes);

/* tokens: device int32 [batch, n_tokens] (row-major), 1 <= n_tokens <=
 * seq_len.  Runs the forward over positions 0..n_tokens-1, writes their keys
 * and values into the cache, and writes logits: device fp32 [batch, vocab],
 * the next-token logits after each row's last token.  Waits for the stream.
 * GPT_ETOKEN for an id outside [0, vocab). */
int gpt_prefill(gpt_model* model, const int32_t* tokens, int n_tokens, void* kv_cache, float* logits);

/* tokens: device int32 [batch], the token at position pos of each row,
 * 1 <= pos < seq_len, with positions 0..pos-1 already in the cache (from
 * gpt_prefill and earlier gpt_decode calls).  Appends its key and value at
 * pos and writes logits [batch, vocab] fp32 (device) for position pos + 1.
 * Waits for the stream.  GPT_ETOKEN for an id outside [0, vocab). */
int gpt_decode(gpt_model* model, const int32_t* tokens, int pos, void* kv_cache, float* logits);

/* The RoPE table the step uses, computed on the host (no GPU needed):
 * cos_out[t][i] = cos(t * theta_i), sin_out[t][i] = sin(t * theta_i) with
 * theta_i = rope_base^(-2i/head_dim), 0 <= t < seq_len, 0 <= i < head_dim/2
 * (nanochat User Guide, section 10, rotary embeddings; the half-split pair
 * convention is stated at the top of this header).  Evaluated in double and
 * rounded to fp32.  cos_out, sin_out: host float[seq_len * head_dim / 2],
 * caller-owned.  GPT_EINVAL for a bad config, GPT_ENULL for a NULL output. */
int gpt_rope_table(const gpt_config* cfg, float* cos_out, float* sin_out);

/* Overlap of the backward's weight-gradient products (on by default).  The
 * weight gradients feed nothing else in the step, so the handle runs them on
 * a second stream of its own (created by gpt_create, default priority),
 * concurrently with the chain of input gradients; events order them after
 * their inputs and before any reuse of those inputs' buffers, and the step
 * waits for them before it returns (or, in gpt_step_micro's graph, before
 * the graph ends).  on = 0 runs every product on cfg->stream in program
 * order (as profiling does).  The two modes plan the weight gradients
 * differently (in order: split along K where the output has too few tiles
 * to fill the GPU, with the partial sums added in split order; overlapped:
 * the fewest of those splits that give 96 work-groups, since the product
 * shares the GPU with the other stream), so each is bitwise reproducible
 * and they agree to fp32 summation-order rounding.  In GPT_FP8 models the
 * product reads the transposed gradient codes, which alternate between two
 * workspace buffers while the overlap is on. */
int gpt_overlap_enable(gpt_model* model, int on);

/* The rotary step and QK norm in the QKV product's epilogue (on by
 * default).  It applies to GPT_BF16 models with head_dim 128 and seq_len a
 * multiple of 64; there the product rotates the fp32 accumulators of each q
 * and k head (the pair (x[i], x[i+64]) by t * theta_i, "How It Works" in
 * the nanochat User Guide), RMS-normalises the head and stores q^, k^, v
 * with their transposed copies, instead of storing bf16 q, k, v for a
 * separate pass to read back.  on = 0 runs that separate pass (which
 * rotates the bf16-rounded product), as every other configuration does.
 * The two agree to bf16 rounding. */
int gpt_rope_epilogue_enable(gpt_model* model, int on);

/* Release the handle (host memory only). */
void gpt_destroy(gpt_model* model);

/* Inspect a saved intermediate of the last step (device pointer into the
 * workspace).  which: 0 residual h after the forward [B*T, d] fp32,
 * 1 normalised q/k + raw v of `layer` [B*T, 3d], 2 attention output of
 * `layer` [B*T, d], 3 per-row loss [B*T] fp32, 4 per-row logsumexp [B*T] fp32,
 * 5 u (MLP pre-activation) of `layer` [B*T, F] (fp32 in GPT_FP8 models).
 * Activation-typed buffers hold the parameter type.  *elem_bytes receives the
 * element size. */
int gpt_debug_tensor(gpt_model* model, int which, int layer, void** ptr, int64_t* rows, int64_t* cols,
                     int* elem_bytes);

/* A single product through the step's GEMM kernel, for testing and
 * measurement: C[M,N] = A B^T with A [M,K], B [N,K] (layout 0), A [M,K],
 * B [K,N] (layout 1) or A [K,M], B [K,N] (layout 2).  dtype 0 = fp32,
 * 1 = bf16 inputs; C is fp32 [M, N].  M, N, K multiples of 8.  splits >= 1
 * splits K (needs a workspace of splits*M*N floats, else pass splits = 1).
 * Enqueued on `stream`; does not synchronise. */
int gpt_gemm(int dtype, int layout, int M, int N, int K, const void* A, const void* B, float* C,
             float* workspace, int splits, int tile, void* stream);

/* gpt_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same product, kernels and argument rules as gpt_gemm, with the split-K
 * partial sums kept in a scratch array inside the library instead of a
 * caller workspace.  The array is GPT_NOALLOC_SCRATCH_BYTES (64 MiB) of
 * device memory per GPU, part of the library's code object, held until the
 * process ends; its device address is looked up once per device (on the
 * first call with that device current).  The call allocates nothing.
 * splits * M * N must not exceed GPT_NOALLOC_SCRATCH_BYTES / 4 partial sums
 * (splits counted after K is rounded to whole K steps): GPT_EINVAL
 * otherwise, before anything is enqueued.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads)
 * race on it, so order them.  Nothing in the array needs clearing between
 * calls (each split writes its whole block before it is summed).  Enqueued
 * on `stream`; does not synchronise. */
#define GPT_NOALLOC_SCRATCH_BYTES (64u << 20)
int gpt_gemm_noalloc(int dtype, int layout, int M, int N, int K, const void* A, const void* B, float* C,
                     int splits, int tile, void* stream);

/* Per-tensor fp8 quantisation, as used by GPT_FP8 (current scaling):
 *   s = fmax / max|x| (fmax 448 for E4M3, 57344 for E5M2; s = 1 if x is all
 *   zero; s capped at 2^64), computed in fp32;
 *   q[r][c] = OCP code of x[r][c] * s (fp32 product) rounded to nearest even
 *   with saturation to +-fmax.
 * fmt: 0 = E4M3, 1 = E5M2.  x: device bf16 [rows, cols], cols a multiple of
 * 64, 16-byte aligned.  amax: device uint32 scratch of 64 elements
 * (overwritten).  scale: device float, receives s.  q: device uint8
 * [rows, cols]; qT: NULL or device uint8 [cols, rows] receiving the
 * transposed codes.  Enqueued on `stream`; does not synchronise.
 * GPT_EALIGN for a misaligned x. */
int gpt_fp8_quantize(int fmt, const void* x, int rows, int cols, uint32_t* amax, float* scale, void* q, void* qT,
                     void* stream);

/* A single fp8 product through the step's fp8 GEMM kernel:
 *   C[M,N] = (A B^T) / (scale_a * scale_b), A [M,K] codes in E4M3 (fmt_a = 0)
 *   or E5M2 (fmt_a = 1), B [N,K] E4M3 codes, fp32 accumulation, C fp32.
 * scale_a, scale_b: device floats (as written by gpt_fp8_quantize).  M, N
 * multiples of 8, K a multiple of 16.  splits >= 1 splits K (workspace of
 * splits*M*N floats).  Enqueued on `stream`; does not synchronise. */
int gpt_gemm_fp8(int fmt_a, int M, int N, int K, const void* A, const void* B, const float* scale_a,
                 const float* scale_b, float* C, float* workspace, int splits, void* stream);

/* Per-launch-site timing, for measurement.  When enabled, every kernel
 * launch of gpt_step is bracketed by HIP events on the step's stream; after
 * each step the elapsed times are added to named sites ("gemm_qkv",
 * "attn_fwd_causal", "rmsnorm_fwd", ...).  gpt_profile_enable(m, 1) also
 * resets the counters; 0 turns timing off.  For each site, `work` is the
 * summed algorithmic work of its launches: FLOPs (work_kind 0: 2*M*N*K for a
 * product, 4*Dh per visible (query, key) pair for the attention forward) or
 * HBM bytes (work_kind 1: each input read once, each output written once). */
int gpt_profile_enable(gpt_model* model, int on);
int gpt_profile_sites(gpt_model* model, int* n_sites);
int gpt_profile_get(gpt_model* model, int index, char* name, int name_len, char* kernel, int kernel_len,
                    int64_t* launches, double* total_ms, double* work, int* work_kind);

/* Static description of a return code. */
const char* gpt_strerror(int code);
/* Details of the last failure on this thread ("" if none). */
const char* gpt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GPT_MI355X_H */
