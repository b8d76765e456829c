// GEMM-family argument block and epilogues (included by kernels.hpp).
#pragma once
#include <stdint.h>

namespace ttt {

// ---------------------------------------------------------------- GEMM family
// C[m, n] = sum_k A(m, k) B(n, k).
//   A(m, k) = A[m * lda + k] if a_kmajor else A[k * lda + m]
//   B(n, k) = B[n * ldb + k] if b_kmajor else B[k * ldb + n]
// The contiguous dimension of each operand must be a multiple of 8 elements
// and its base 16-byte aligned; other dimensions are arbitrary (zero-filled).
enum class Epi : int {
  STORE = 0,    // C (storage type) = scale * acc
  STORE_F32,    // C (float) = acc
  ADD_F32,      // C (float) += acc            (residual stream)
  SWIGLU,       // columns interleaved by 16 (gate | up): C2 (T)[m, j] = silu(a) c,
                // optional C (T) = the pre-activations themselves
  SWIGLU_BWD,   // acc = dHmid[m, j]; X = pre-activations (ld = 2N):
                // C (T) [m, gate/up col] = (dA, dC)
  SGD,          // C (float master) -= scale * acc; C2 (T) = round(master),
                // C3 (T, optional) = round(master - C2); or, with seed != 0,
                // C2 = stochastic rounding of the master (no C3)
  PARTIAL,      // C (float) [split][M][ldc] = acc  (split-K)
  PARTIAL_BF16, // C (bf16) [split][M][ldc] = acc  (split-K gradient partials; bf16 NN only)
  STORE_F32_LSE,// C (float) = acc, and per 64-column group of each row its (max, sum of
                // exp(x - max)) into C2 (float2 [M][ceil(N / 64)]); bf16 NT only
};

struct GemmArgs {
  const void* A;
  const void* B;
  const void* B2;  // optional low part of B (B = B + B2, two bf16 terms of an fp32 value)
  int M, N, K;
  long lda, ldb;
  void* C;
  long ldc;
  void* C2;
  void* C3;        // SGD: low part of the re-rounded weight (bf16 split), or null
  const void* X;
  float scale;
  int kchunk;  // split-K chunk (multiple of gemm_k_granule); <= 0 means no split
  int tile;    // tile configuration (0 = chosen from the shape)
  // Batched products (batch > 1: grid.y = batch): product j reads and writes
  // A + j sA, B and B2 + j sB, C + j sC, C2 and C3 + j sC2, X + j sX
  // (strides in elements of each operand's type)
  int batch;
  long sA, sB, sC, sC2, sX;
  long split_ld;  // PARTIAL epilogues: elements between split-K slices (0: M ldc)
  // SGD with a bf16 working copy: 0 = C2 is the master rounded to nearest;
  // otherwise C2 is rounded stochastically (unbiased) with random bits from
  // this seed and the element's index, and C3 is not written
  uint32_t seed;
};

}  // namespace ttt
