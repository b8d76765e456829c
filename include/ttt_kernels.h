/*
 * ttt_kernels.h -- kernel-level entry points of the TTT-E2E library, for
 * testing single kernels against the oracle and measuring them in
 * isolation. They enqueue one kernel (family) on the given stream; all
 * pointers are device memory owned by the caller; shapes are checked on the
 * host before launch (TTT_ERR_INVALID_ARG / TTT_ERR_UNSUPPORTED).
 */
#ifndef TTT_KERNELS_H_
#define TTT_KERNELS_H_

#include <stdint.h>

#include "ttt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of tttk_gemm. */
typedef enum {
  TTTK_EPI_STORE = 0,      /* C (dtype) = scale * acc */
  TTTK_EPI_STORE_F32 = 1,  /* C (float) = acc */
  TTTK_EPI_ADD_F32 = 2,    /* C (float) += acc */
  TTTK_EPI_SWIGLU = 3,     /* N = 2F columns interleaved in blocks of 16 (gate, up):
                              C (dtype, may be NULL) = pre-activations,
                              C2 (dtype) [M, F] = silu(gate) * up */
  TTTK_EPI_SWIGLU_BWD = 4, /* acc = dHmid [M, N]; X (dtype) [M, 2N] pre-activations;
                              C (dtype) [M, 2N] = (d gate, d up) */
  TTTK_EPI_SGD = 5,        /* C (float master) -= scale * acc; C2 (dtype) = round(C);
                              C3 (dtype, may be NULL) = round(C - C2) */
  TTTK_EPI_PARTIAL = 6,    /* C (float) [splits][M][ldc] = partial sums over K chunks */
  TTTK_EPI_STORE_F32_LSE = 8 /* bf16, a_kmajor and b_kmajor: C (float) = acc, and for each
                                row and 64-column group g, C2 (float2 [M][ceil(N / 64)])
                                = (max, sum exp(acc - max)) over the group's columns < N */
} tttk_epi;

/* C[m, n] = sum_k A(m, k) B(n, k) on MFMA with fp32 accumulation, where
 * A(m, k) = A[m lda + k] if a_kmajor else A[k lda + m], and
 * B(n, k) = B[n ldb + k] if b_kmajor else B[k ldb + n];
 * B2 (optional, bf16, NT layout, SWIGLU/ADD_F32/PARTIAL only) is a second term
 * added to B. The contiguous dimension of A and B must be a multiple of 8
 * and the pointers 16-byte aligned. kchunk > 0 splits K into chunks (a
 * multiple of 64) for TTTK_EPI_PARTIAL. tile (bf16; fp32 always uses
 * 64x64): 0 = chosen from the shape, 1 = 128x128 (4 waves of 64x64),
 * 2 = 256x128 (4 of 128x64), 3 = 256x128 (8 of 64x64), 4 = 256x256 (4 of
 * 128x128), 5 = 256x256 (8 of 128x64), 6 = 128x256 (4 of 64x128); K steps
 * of 64. seed (TTTK_EPI_SGD, bf16, C2 a separate working copy, C3 NULL;
 * else 0): nonzero rounds C2 from the master stochastically -- up with
 * probability equal to the fraction of a bf16 ulp that rounding drops,
 * from 16 random bits hashed from (seed, element index) -- instead of to
 * nearest. */
ttt_status tttk_gemm(int32_t dtype, int32_t a_kmajor, int32_t b_kmajor, int32_t epi, const void* A,
                     int64_t lda, const void* B, int64_t ldb, const void* B2, int32_t M, int32_t N,
                     int32_t K, void* C, int64_t ldc, void* C2, void* C3, const void* X, float scale,
                     int32_t kchunk, int32_t tile, uint32_t seed, void* stream);

/* Sliding-window attention forward for n queries at positions pos0 .. pos0+n-1
 * (q: [n, H, dh]) over a key/value store k, v: [Hk][cap][dh] indexed by
 * position & (cap - 1) (cap a power of two >= 64; every key the queries see
 * must already be stored); vt (optional): the values transposed,
 * [Hk][dh][cap], slot s of the store at position (s & ~15) | (s & 3) |
 * ((s & 4) << 1) | ((s & 8) >> 1) (bits 2 and 3 swapped inside each block of
 * 16). o: [n, H, dh]; lse: float [H, n] or NULL. variant: 0 =
 * chosen from the shape, 1 = 16x16 MFMA kernel, 2 / 3 = 32x32 MFMA kernel
 * with 32 / 64 queries per wave, 4 = 32x32 MFMA kernel with 32 queries per
 * wave in 8-wave workgroups (2-4: bf16, dh 64/128, need vt; q, k, v, vt and
 * o 16-byte aligned, else TTT_ERR_INVALID_ARG). */
ttt_status tttk_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v, const void* vt,
                         void* o, float* lse, int32_t n, int32_t H, int32_t Hk, int32_t dh, int32_t cap,
                         int32_t window, int64_t pos0, int32_t variant, int32_t ksplit, void* work,
                         void* stream);

/* ksplit (32x32 kernels only): the key range of each query block is split
 * over that many workgroups (1..4; 0 = chosen from the shape) whose partial
 * results go to work (caller-owned device memory of
 * tttk_attn_fwd_workspace() bytes; may be NULL when that is 0) and are
 * merged by a combine pass. */
int64_t tttk_attn_fwd_workspace(int32_t n, int32_t H, int32_t dh, int32_t window, int32_t ksplit);

/* Its backward for the query side and for the keys of the call's own
 * positions (cached earlier keys are constants): given dO [n, H, dh] and
 * D = rowsum(dO * O) float [H, n], writes dq float [n, H, dh] and
 * dk, dv float [n, Hk, dh]. variant: 0 = chosen from the shape, 1 = 16x16
 * MFMA kernels, 2 = 32x32 MFMA kernels (bf16, dh 64/128), which produce
 * partial sums in work (device memory of tttk_attn_bwd_workspace() bytes,
 * owned by the caller; may be NULL when that is 0) and add them into dq, dk,
 * dv. */
ttt_status tttk_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v, const float* lse,
                         const void* dO, const float* D, float* dq, float* dk, float* dv, int32_t n,
                         int32_t H, int32_t Hk, int32_t dh, int32_t cap, int32_t window, int64_t pos0,
                         int32_t variant, void* work, void* stream);

/* Bytes of work tttk_attn_bwd needs for this shape and variant. */
int64_t tttk_attn_bwd_workspace(int32_t dtype, int32_t n, int32_t H, int32_t Hk, int32_t dh, int32_t window,
                                int32_t variant);

/* The same from the logits' per-64-column (max, sum exp) partials
 * (TTTK_EPI_STORE_F32_LSE): float2 [n][ceil(V / 64)]; reads the logits once.
 * bf16 dz only; V a multiple of 4. */
ttt_status tttk_ce_lse(const float* logits, const void* parts, int32_t n, int32_t nt, int32_t V,
                       const int32_t* labels, float scale, float* loss, void* dz, int* err, void* stream);

/* Fused softmax cross-entropy over V columns of fp32 logits [n, V] for the
 * first nt rows (labels int32 [nt]): loss float [nt], dz (dtype) [n, V] =
 * (softmax - onehot) * scale (zero rows past nt). err: device int flag. */
ttt_status tttk_ce(int32_t dtype, const float* logits, int32_t n, int32_t nt, int32_t V,
                   const int32_t* labels, float scale, float* loss, void* dz, int* err, void* stream);

/* One weight-gradient product with the fp32 SGD step fused in (bf16
 * operands; see tttk_dw_sgd). */
typedef struct {
  const void* A;  /* bf16, A(m, k) = A[k lda + m] (output gradients, token-major) */
  int64_t lda;
  const void* B;  /* bf16, B(n, k) = B[k ldb + n] (inputs, token-major) */
  int64_t ldb;
  float* W;       /* fp32 master [M][ldw], updated in place */
  void* Hi;       /* bf16 [M][ldw] = RNE(W) after the step */
  void* Lo;       /* bf16 [M][ldw] = RNE(W - Hi), or NULL */
  int64_t ldw;
  int32_t M, N;
} tttk_dw_problem;

/* W -= lr * sum_k A(m, k) B(n, k) for nprob (1 or 2) problems sharing K, in
 * one persistent launch of grid workgroups (0 = two per CU); the bf16
 * working copy and its low term are re-rounded from the new master. This is
 * the fused dW + SGD update of a dynamic SwiGLU block ([P1] section
 * 持续学习框架, the SGD step). M, N multiples of 16; lda, ldb multiples of 8,
 * ldw of 4, lda >= M, ldb >= N, ldw >= N; A, B, W 16-byte and Hi, Lo 8-byte
 * aligned; else TTT_ERR_UNSUPPORTED / TTT_ERR_INVALID_ARG. */
ttt_status tttk_dw_sgd(int32_t nprob, const tttk_dw_problem* probs, int32_t K, float lr, int32_t grid,
                       void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TTT_KERNELS_H_ */
