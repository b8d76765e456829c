/*
 * ttt.h -- C ABI of the TTT-E2E inner-loop library for AMD MI355X (gfx950).
 *
 * The library runs the test-time-training inner loop of a sliding-window-
 * attention transformer on one GPU:
 *   - [P1] "TTT-E2E：端到端测试时训练的长上下文语言建模" (metaphor-xennon), section
 *     持续学习框架: the per-token next-token loss l_t is taken under the
 *     weights before step t, and W_t = W_{t-1} - alpha * grad l_t; section
 *     内层循环：测试时训练: the context is split into chunks of b tokens, one
 *     gradient step per chunk; section 关键设计参数: window k >= chunk b;
 *     section 架构设计 (sketch): only the last quarter of the blocks update;
 *     the lm_head is tied to the embedding.
 *   - [P2] "NVIDIA开源TTT-E2E：128K上下文快2.7倍" (longzhangge), sections 另辟蹊径
 *     and 学会如何“持续学习”: only MLP weights are updated (embeddings, norms
 *     and attention frozen); updated blocks carry a frozen static MLP beside
 *     the dynamic one.
 *   - [P3] "Rethinking Expressivity and Efficiency in Test-Time Training",
 *     section 方法细节, Proposition 3.1 and Algorithm 1: the E2-TTT chunk-end
 *     state (e2ttt_chunk_scan).
 *
 * Model read from those pages: pre-RMSNorm residual blocks (eps from the
 * config, no biases); attention with RoPE (base rope_theta, half-split
 * rotation, absolute positions), scale 1/sqrt(head_dim), causal window
 * (key t visible to query i iff i - window < t <= i), GQA by contiguous head
 * groups; SwiGLU MLPs  h + W3 (silu(W1 u) * (W2 u)); in the last n_dynamic
 * blocks a dynamic SwiGLU MLP sublayer follows the static one. Logits =
 * RMSNorm(h) lm_head^T; per-token loss l_i = logsumexp(z_i) - z_i[x_{i+1}].
 *
 * Conventions
 *   Pointers marked (device) are device memory owned by the caller; the
 *   library never frees them. Weight matrices use the nn.Linear layout
 *   [out, in], row-major, in the config's storage dtype (float32 for
 *   TTT_F32, bfloat16 for TTT_BF16); gain vectors [d] in the same dtype.
 *   ttt_init copies everything it needs into memory it owns and synchronises
 *   its stream before returning, so the caller may free its copies.
 *   Streams are hipStream_t values passed as void* (NULL = the null stream).
 *   Every other call only enqueues work on the given stream and returns;
 *   outputs are valid once that stream has been synchronised.
 *   Errors: calls return a ttt_status; nothing throws across the ABI.
 *   Argument errors are detected on the host before any device work.
 *   Device-detected conditions (token id outside [0, vocab), non-finite
 *   loss) raise a flag that ttt_sync reports. ttt_last_error gives text.
 *   A ttt_ctx is not thread-safe; distinct contexts are independent.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTT_OK = 0,
  TTT_ERR_INVALID_ARG = -1, /* null pointer, out-of-range size or value */
  TTT_ERR_UNSUPPORTED = -2, /* a shape the kernels do not implement */
  TTT_ERR_OOM = -3,         /* device allocation failed */
  TTT_ERR_HIP = -4,         /* a HIP runtime call failed */
  TTT_ERR_STATE = -5,       /* call not allowed in the context's state */
  TTT_ERR_TOKEN_RANGE = -6, /* (ttt_sync) a token id was outside [0, vocab) */
  TTT_ERR_NONFINITE = -7,   /* (ttt_sync) a loss was not finite */
  TTT_ERR_NO_DEVICE = -8    /* no usable gfx950 device */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;
typedef enum { TTT_LOSS_MEAN = 0, TTT_LOSS_SUM = 1 } ttt_reduction;

/* Model and inner-loop hyper-parameters. */
typedef struct {
  int32_t n_layers;       /* L >= 1 */
  int32_t d_model;        /* d, multiple of 16, at most 8192 */
  int32_t n_heads;        /* query heads H */
  int32_t n_kv_heads;     /* Hk, divides H */
  int32_t head_dim;       /* 16, 64 or 128 */
  int32_t ffn_hidden;     /* static SwiGLU hidden size, multiple of 32 */
  int32_t dyn_ffn_hidden; /* dynamic SwiGLU hidden size, multiple of 32 */
  int32_t vocab;          /* V, multiple of 8 */
  int32_t window;         /* k, >= minibatch */
  int32_t minibatch;      /* b >= 1: tokens per SGD step */
  int32_t n_dynamic;      /* updated blocks (the last n_dynamic); 0 => L - (3L)/4 */
  int32_t max_seq;        /* largest position + 1 ever used (prefill + decode); a
                           * window above max(max_seq, minibatch) is clamped to it
                           * (no query can see more keys) */
  float alpha;            /* SGD step size, finite, >= 0 */
  float rms_eps;          /* RMSNorm epsilon, > 0 */
  float rope_theta;       /* RoPE base, > 1 */
  int32_t dtype;          /* ttt_dtype of weights and activations */
  int32_t reduction;      /* ttt_reduction of each mini-batch's loss */
  int32_t prefix_slab;    /* positions per slab of the frozen prefix (the blocks
                           * that precede the first fast weight run once over
                           * the whole stream, slab by slab); 0 => min(max_seq,
                           * 16384); raised to minibatch, lowered to max_seq. The
                           * per-layer key/value ring holds cap = next power of
                           * two >= max(window + max(minibatch, slab), 128)
                           * positions (slot = position mod cap), so a small slab
                           * gives a small ring that is reused sooner; results do
                           * not depend on it. Negative => TTT_ERR_INVALID_ARG;
                           * a ring slice of one key head of 2^31 bytes or more
                           * => TTT_ERR_UNSUPPORTED. */
  int32_t n_seq;          /* B: independent sequences processed side by side by
                           * ttt_prefill, each with its own fast weights, window
                           * and losses (the same T for all); 0 => 1, at most 64.
                           * Rings, residual stream and fast weights are held
                           * per sequence; the loop's products with frozen
                           * weights run on B b rows. Decode needs n_seq 1. */
} ttt_config;

/* Weights (device pointers, storage dtype). Per-layer fields are host arrays
 * of n_layers device pointers; dyn_* are host arrays of n_dynamic device
 * pointers (block L - n_dynamic + i) holding the initial fast weights W0. */
typedef struct {
  const void* embed;      /* [V, d] */
  const void* lm_head;    /* [V, d]; may equal embed (tied) */
  const void* final_norm; /* [d] */
  const void* const* attn_norm; /* [d] */
  const void* const* wq;        /* [H*dh, d] */
  const void* const* wk;        /* [Hk*dh, d] */
  const void* const* wv;        /* [Hk*dh, d] */
  const void* const* wo;        /* [d, H*dh] */
  const void* const* mlp_norm;  /* [d] */
  const void* const* w1;        /* [F, d]  gate (silu) */
  const void* const* w2;        /* [F, d]  up */
  const void* const* w3;        /* [d, F]  down */
  const void* const* dyn_norm;  /* [d] */
  const void* const* dyn_w1;    /* [Fd, d] */
  const void* const* dyn_w2;    /* [Fd, d] */
  const void* const* dyn_w3;    /* [d, Fd] */
} ttt_weights;

typedef struct ttt_ctx ttt_ctx;

/* Validates cfg and weights, allocates the context (static weights, fp32
 * fast-weight master, W0 snapshot, key/value rings, activation buffers) and
 * uploads. Returns TTT_ERR_INVALID_ARG / TTT_ERR_UNSUPPORTED on a bad config
 * before touching the device, TTT_ERR_NO_DEVICE without a GPU, TTT_ERR_OOM
 * if memory runs out. On success *out owns everything; free with
 * ttt_destroy. */
ttt_status ttt_init(const ttt_config* cfg, const ttt_weights* w, void* stream, ttt_ctx** out);

/* The inner loop over tokens[0..T) (device int32). Requires position 0
 * (a fresh context or after ttt_reset), 2 <= T <= max_seq. Mini-batches
 * P_m = [m b, min((m+1) b, T)) are processed in order: forward under the
 * current fast weights, loss[i] = l_i for i in P_m, i <= T-2, then one SGD
 * step on the dynamic MLP weights from the MEAN (or SUM) of those losses;
 * a mini-batch with no target is forward only. loss (device float [T-1])
 * receives the prequential per-token losses. last_logits (device float [V]
 * or NULL) receives the logits at position T-1. Leaves the context at
 * position T with the adapted fast weights.
 * With n_seq = B > 1, tokens holds B rows of T ids ([B][T], row-major) and
 * each row is its own sequence: loss is [B][T-1] and last_logits [B][V];
 * sequence j's results equal those of a single-sequence context fed row j
 * (up to the order of floating-point sums, which the row count can change). */
ttt_status ttt_prefill(ttt_ctx* ctx, const int32_t* tokens, int64_t T, float* loss,
                       float* last_logits, void* stream);

/* Forward of one token (device int32 [1]) at the current position p under
 * the current fast weights, appending its keys/values to the window;
 * logits (device float [V]) are the prediction for position p + 1. No
 * update. Requires 1 <= p < max_seq (after a prefill). The token is read
 * from device memory so that the per-token launch sequence can be captured
 * once as a HIP graph and replayed. Cost independent of the context length
 * ([P1] 实验结果 -> 推理延迟: latency flat in the context). A context with
 * n_seq > 1 returns TTT_ERR_UNSUPPORTED. */
ttt_status ttt_decode_step(ttt_ctx* ctx, const int32_t* token, float* logits, void* stream);

/* Decode with test-time training continuing into generation ([P2]
 * "NVIDIA开源TTT-E2E：128K上下文快2.7倍", section 效果惊人: the model keeps
 * learning from what it reads after the context). The positions consumed
 * since the last update are trained in groups of minibatch b: a prefill of T
 * tokens leaves position T - 1 as the first without a target; when this
 * token completes the targets of the b positions [u, u + b) (u = that
 * first untrained position), the inner-loop step runs on them first --
 * forward under the current fast weights (their keys/values stored again),
 * next-token losses, backward, SGD step on the dynamic MLPs, exactly as for
 * a prefill mini-batch -- and then this token is decoded as by
 * ttt_decode_step, under the new weights. loss (device float [b] or NULL)
 * receives the b losses of such an update; *updated (host, may be NULL) is
 * set to 1 if one ran, else 0. After a prefill of T = m b + 1 tokens the
 * updates fall on the same mini-batches, with the same results, as a prefill
 * of the longer stream. Same requirements and errors as ttt_decode_step. */
ttt_status ttt_decode_step_update(ttt_ctx* ctx, const int32_t* token, float* logits, float* loss,
                                  int32_t* updated, void* stream);

/* Copies dynamic block dyn_idx's current fast weights (fp32 master) into
 * device float buffers w1 [Fd, d], w2 [Fd, d], w3 [d, Fd]: the compressed
 * context W_T ([P1] 持续学习框架: the sequence is learned into the weights).
 * With n_seq > 1 these are sequence 0's. */
ttt_status ttt_get_fast_weights(ttt_ctx* ctx, int32_t dyn_idx, float* w1, float* w2, float* w3,
                                void* stream);

/* The same for sequence seq of a multi-sequence context (0 <= seq < n_seq,
 * else TTT_ERR_INVALID_ARG). */
ttt_status ttt_get_fast_weights_seq(ttt_ctx* ctx, int32_t seq, int32_t dyn_idx, float* w1, float* w2,
                                    float* w3, void* stream);

/* Restores W0 and position 0 (the rings are overwritten before being read):
 * the per-sequence restart of the inner loop ([P1] 完整PyTorch实现: the
 * sketch snapshots the weights before the inner loop and restores them
 * after it). */
ttt_status ttt_reset(ttt_ctx* ctx, void* stream);

/* Synchronises the stream and reports device flags raised since the last
 * sync (TTT_ERR_TOKEN_RANGE, TTT_ERR_NONFINITE), clearing them. */
ttt_status ttt_sync(ttt_ctx* ctx, void* stream);

/* Current position (tokens consumed). */
int64_t ttt_position(const ttt_ctx* ctx);

/* Text of the last error recorded on ctx (never NULL). */
const char* ttt_last_error(const ttt_ctx* ctx);

void ttt_destroy(ttt_ctx* ctx);

/* Diagnostics: live per-kernel-class timing with HIP events recorded on the
 * launch stream around every launch of the selected classes. */
typedef enum {
  TTT_KC_GEMM_PREFIX = 0, /* projections and MLP GEMMs of the hoisted prefix */
  TTT_KC_ATTN_PREFIX = 1, /* SWA forward of the hoisted prefix */
  TTT_KC_GEMM_LOOP = 2,   /* loop forward GEMMs and backward dX / dHmid GEMMs */
  TTT_KC_ATTN_LOOP = 3,   /* SWA forward inside the loop */
  TTT_KC_LMHEAD = 4,      /* lm_head forward and its dX product */
  TTT_KC_CE = 5,          /* fused softmax-CE + logit gradient */
  TTT_KC_ATTN_BWD = 6,    /* SWA backward (dQ and dK/dV kernels) */
  TTT_KC_DW_SGD = 7,      /* dW = X^T dH with the fused fp32 SGD update */
  TTT_KC_OTHER = 8,       /* norms, RoPE, embedding, copies */
  TTT_KC_COUNT = 9
} ttt_kernel_class;

/* Starts timing the classes in class_mask (bit i = class i) and clears the
 * counters; 0 stops timing. */
ttt_status ttt_timing_enable(ttt_ctx* ctx, uint32_t class_mask);

/* Synchronises the device and returns, for one class, the summed kernel time
 * (ms), the number of launches and their algorithmic FLOPs and HBM bytes
 * (the minimal operand/result traffic each launch must move). Any pointer
 * may be NULL. */
ttt_status ttt_timing_read(ttt_ctx* ctx, int32_t kclass, double* total_ms, int64_t* launches,
                           double* flops, double* bytes);

/* E2-TTT chunk-end scan ([P3] 方法细节, Proposition 3.1; Algorithm 1 state
 * update). For every head h and chunk [r C, min((r+1) C, T)), with W0, M0 the
 * state at chunk start and G_t = (W0 k_t - v_t) k_t^T:
 *   M_C = beta~_0 M0 + sum_t eta_t beta~_t G_t
 *   W_C = gamma~_0 W0 + beta~_0 R_1 M0 + sum_t eta_t beta~_t R_t G_t
 * which equals the per-token recursion M_t = beta_t M_{t-1} + eta_t G_t,
 * W_t = gamma_t W_{t-1} + M_t at the chunk end. k, v: device bf16 [H, T, D];
 * eta, beta, gamma: device float [H, T], beta, gamma in (0, 1], eta >= 0;
 * W, M: device float [H, D, D], 16-byte aligned, updated in place to the
 * state after the last chunk. D must be 128 or 64; C a multiple of 64, at
 * most 2048; T >= 1. Errors: TTT_ERR_UNSUPPORTED for other D or C,
 * TTT_ERR_INVALID_ARG for null or misaligned pointers, TTT_ERR_OOM when its
 * work buffer cannot be had. Each call takes its own device work buffer on
 * `stream` from the device's default memory pool (stream-ordered
 * allocation) and gives it back on the same stream after its kernels, so
 * calls on different streams or host threads may overlap (on different
 * W, M). The pool keeps what is given back for later calls: its release
 * threshold is raised on the first call on a device. */
ttt_status e2ttt_chunk_scan(const void* k, const void* v, const float* eta, const float* beta,
                            const float* gamma, float* W, float* M, int32_t H, int64_t T,
                            int32_t D, int32_t C, void* stream);

/* Allocation-free variant of e2ttt_chunk_scan for callers that cannot
 * allocate device memory (work under HIP graph capture, tight serving loops,
 * hosts that forbid hipMalloc). Same arguments, result and errors. Its work
 * buffer is a fixed device array of e2ttt_chunk_scan_noalloc_max_bytes()
 * bytes (32 MiB), one copy per GPU, held until the process ends; a call
 * needs 8 H T + 16 H ceil(T / C) + 4 H D^2 + 512 bytes of it (16 heads x
 * 32768 tokens x D 128: 5.3 MB), and a larger problem returns
 * TTT_ERR_UNSUPPORTED before any device work. The call never allocates or
 * frees device memory; the first call on a device looks up that device's
 * copy. The array keeps the last call's contents (every value a call reads
 * is written by that call first). Calls on one GPU share its array, so
 * calls that overlap on one GPU (different streams or host threads) race. */
ttt_status e2ttt_chunk_scan_noalloc(const void* k, const void* v, const float* eta, const float* beta,
                                    const float* gamma, float* W, float* M, int32_t H, int64_t T,
                                    int32_t D, int32_t C, void* stream);

/* Size in bytes of the allocation-free variant's work buffer. */
int64_t e2ttt_chunk_scan_noalloc_max_bytes(void);

/* The chunk-wise baseline E2-TTT is compared with ([P3] 背景知识: LaCT's
 * large-chunk rule, whose momentum factor is the chunk's average of beta_t;
 * section 实验结果, the "chunk-averaged" ablation). For every head and chunk,
 * with W0, M0 the state at chunk start and G_t = (W0 k_t - v_t) k_t^T:
 *   M_C = mean_t(beta_t) M0 + sum_t eta_t G_t,   W_C = W0 + M_C
 * (one update direction per chunk, no decay). Arguments, layouts and errors
 * as for e2ttt_chunk_scan without gamma, with a work buffer of its own
 * taken in the same way. */
ttt_status lact_chunk_scan(const void* k, const void* v, const float* eta, const float* beta, float* W,
                           float* M, int32_t H, int64_t T, int32_t D, int32_t C, void* stream);

/* The E2-TTT token mixer's TTT path with a linear fast weight ([P3] 方法细节:
 * 混合模型架构设计 -- shared projections, SiLU and L2 normalisation of q and
 * k; 依赖于输入的动态参数化 -- eta_t = eta_base sigma(z_eta), beta_t =
 * sigma(z_beta)^(1/tau), gamma_t = 1 - eta_t alpha_base sigma(z_alpha);
 * Algorithm 1 -- outputs under the chunk-start state, then the chunk-end
 * state of e2ttt_chunk_scan with the page's G_t, the negative gradient
 * (v_t - W0 k_t) k_t^T). x: device bf16 [T, dm]; wqkv: device bf16
 * [3 H D + 3 H, dm], rows Wq (H D), Wk (H D), Wv (H D), then the eta, beta
 * and alpha logit rows (H each); bias: device float [3 H] added to the
 * logits. q, k, v are kept in bf16 and eta, beta, gamma in float between the
 * steps. out: device float [T, H D], o_t = W q_t with W the state at the
 * start of t's chunk; W, M: device float [H, D, D], updated in place. D 128
 * or 64, C a multiple of 64 up to 2048, dm a multiple of 8, pointers 16-byte
 * aligned. Its work buffer is taken per call on `stream` as for
 * e2ttt_chunk_scan. */
ttt_status e2ttt_mixer_forward(const void* x, const void* wqkv, const float* bias, float eta_base,
                               float alpha_base, float tau, float* W, float* M, float* out, int32_t H,
                               int64_t T, int32_t D, int32_t dm, int32_t C, void* stream);

/* The same token mixer with the SwiGLU fast-weight net ([P3] 方法细节,
 * 快速权重网络实例化): per head f_W(x) = x + LN(W3 (SiLU(W1 x) * (W2 x)))
 * with LN a layer normalisation over the D features without affine
 * parameters (eps 1e-5); the per-token loss 1/2 ||f_W0(k_t) - v_t||^2 at
 * the chunk-start W0 (Algorithm 1: its gradient g_t feeds both
 * aggregations), and Proposition 3.1 applied to each of W1, W2, W3 with its
 * own momentum and the shared eta_t, beta_t, gamma_t (descent). Outputs o_t =
 * f_W(q_t) under the chunk-start state. Products run on bf16 MFMA with
 * fp32 accumulation (weights rounded to bf16 for each chunk's products, the
 * state kept in fp32). W1, W2, M1, M2: device float [H, Dh, D]; W3, M3:
 * device float [H, D, Dh]; all updated in place. Other arguments as for
 * e2ttt_mixer_forward; Dh a multiple of 32 up to 4096 (else
 * TTT_ERR_UNSUPPORTED). Work buffer per call, as for e2ttt_chunk_scan. */
ttt_status e2ttt_mixer_swiglu_forward(const void* x, const void* wqkv, const float* bias, float eta_base,
                                      float alpha_base, float tau, float* W1, float* W2, float* W3, float* M1,
                                      float* M2, float* M3, float* out, int32_t H, int64_t T, int32_t D,
                                      int32_t Dh, int32_t dm, int32_t C, void* stream);

/* The same token mixer with the GELU fast-weight net ([P3] 方法细节,
 * 快速权重网络实例化): per head f_W(x) = x + LN(W2 GELU(W1 x)) with the
 * exact GELU (u Phi(u), Phi the standard normal distribution function) and
 * LN, loss, aggregations and outputs as for e2ttt_mixer_swiglu_forward.
 * W1, M1: device float [H, Dh, D]; W2, M2: device float [H, D, Dh]; all
 * updated in place. Other arguments, requirements and errors as for
 * e2ttt_mixer_swiglu_forward (work buffer per call). */
ttt_status e2ttt_mixer_gelu_forward(const void* x, const void* wqkv, const float* bias, float eta_base,
                                    float alpha_base, float tau, float* W1, float* W2, float* M1, float* M2,
                                    float* out, int32_t H, int64_t T, int32_t D, int32_t Dh, int32_t dm, int32_t C,
                                    void* stream);

/* The hybrid token-mixer block ([P3] 方法细节, 混合模型架构设计 and Figure 2):
 * sliding-window attention on the shared projections beside the TTT path,
 * interpolated element-wise by a data-dependent gate:
 *   out = g * o_SWA + (1 - g) * o_TTT,   g = sigmoid(x wgate^T + bgate).
 * The TTT path is e2ttt_mixer_forward (Dh = 0: W1 = W, M1 = M [H, D, D];
 * W2, W3, M2, M3 unused and may be NULL), e2ttt_mixer_swiglu_forward
 * (Dh > 0) or, with Dh > 0 and W3, M3 both NULL, e2ttt_mixer_gelu_forward
 * (W1, M1 [H, Dh, D]; W2, M2 [H, D, Dh]), with the same arguments and state
 * updates. The attention uses
 * the q, k, v columns of the same projection before the TTT path's SiLU and
 * L2 normalisation, rounded to bf16, with RoPE (half-split rotation, base
 * rope_theta > 1, positions 0 .. T-1) on q and k, scale 1/sqrt(D), causal
 * window `window` >= 1 (key t visible to query i iff i - window < t <= i),
 * one key head per query head. wgate: device bf16 [H D, dm] (16-byte
 * aligned); bgate: device float [H D]. out: device float [T, H D] (before
 * any output projection). Errors as for the mixer calls; a key/value store
 * slice of one head of 2^31 bytes or more (T above 2^23 for D 128) returns
 * TTT_ERR_UNSUPPORTED. Work buffer per call, as for e2ttt_chunk_scan. */
ttt_status e2ttt_hybrid_forward(const void* x, const void* wqkv, const float* bias, const void* wgate,
                                const float* bgate, float eta_base, float alpha_base, float tau, float rope_theta,
                                int32_t window, float* W1, float* W2, float* W3, float* M1, float* M2, float* M3,
                                int32_t Dh, float* out, int32_t H, int64_t T, int32_t D, int32_t dm, int32_t C,
                                void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H_ */
