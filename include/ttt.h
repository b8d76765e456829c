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
  int32_t max_seq;        /* largest position + 1 ever used (prefill + decode) */
  float alpha;            /* SGD step size, finite, >= 0 */
  float rms_eps;          /* RMSNorm epsilon, > 0 */
  float rope_theta;       /* RoPE base, > 1 */
  int32_t dtype;          /* ttt_dtype of weights and activations */
  int32_t reduction;      /* ttt_reduction of each mini-batch's loss */
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
 * position T with the adapted fast weights. */
ttt_status ttt_prefill(ttt_ctx* ctx, const int32_t* tokens, int64_t T, float* loss,
                       float* last_logits, void* stream);

/* Forward of one token (device int32 [1]) at the current position p under
 * the current fast weights, appending its keys/values to the window;
 * logits (device float [V]) are the prediction for position p + 1. No
 * update. Requires 1 <= p < max_seq (after a prefill). */
ttt_status ttt_decode_step(ttt_ctx* ctx, const int32_t* token, float* logits, void* stream);

/* Copies dynamic block dyn_idx's current fast weights (fp32 master) into
 * device float buffers w1 [Fd, d], w2 [Fd, d], w3 [d, Fd]. */
ttt_status ttt_get_fast_weights(ttt_ctx* ctx, int32_t dyn_idx, float* w1, float* w2, float* w3,
                                void* stream);

/* Restores W0 and position 0 (the rings are overwritten before being read). */
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
 * TTT_ERR_INVALID_ARG for null or misaligned pointers. The call keeps one
 * device work buffer per process (grown on demand; growing it waits for the
 * calling stream), so calls must not run concurrently on different streams
 * or host threads: a later call may only start once the earlier one's work
 * on its stream is ordered before it. */
ttt_status e2ttt_chunk_scan(const void* k, const void* v, const float* eta, const float* beta,
                            const float* gamma, float* W, float* M, int32_t H, int64_t T,
                            int32_t D, int32_t C, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H_ */
