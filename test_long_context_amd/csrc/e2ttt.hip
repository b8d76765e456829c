// E2-TTT chunk-end state on gfx950 ([P3] "Rethinking Expressivity and
// Efficiency in Test-Time Training", section 方法细节: Proposition 3.1 and the
// state-update lines of Algorithm 1).
//
// For a chunk of C tokens with start state (W0, M0) and G_t = (W0 k_t - v_t) k_t^T:
//   M_C = beta~_0 M0 + sum_t KM_t G_t,                    KM_t = eta_t beta~_t
//   W_C = gamma~_0 W0 + beta~_0 R_1 M0 + sum_t KW_t G_t,  KW_t = eta_t beta~_t R_t
// with beta~_t = prod_{i>t} beta_i, gamma~_t likewise, R_t = sum_{i>=t} gamma~_i / beta~_i.
// beta~_0 underflows fp32 at C = 2048, so the ratio form is never evaluated:
// A_t := beta~_t R_t obeys A_C = 1, A_t = gamma~_t + beta_{t+1} A_{t+1}, which
// gives KW_t = eta_t A_t and beta~_0 R_1 = beta_1 A_1 (scan in float64).
//
// The two aggregations share e_t = W0 k_t - v_t (one "backward"); each is a
// contraction over tokens, sum_t K_t e_t k_t^T, on bf16 MFMA. fp32 operands
// (W0 for e_t, then the scaled e_t) are split into bf16 hi + lo parts so that
// the products keep ~16 significant bits; k, v are bf16 inputs (exact).
//
// Kernels: e2_scalars (all chunks at once), then per chunk e2_partial (one
// workgroup per (128-token slice, head): partial sums of the two
// aggregations) and e2_combine (sum of slices + the W0/M0 terms, in place).
#include <math.h>

#include <algorithm>

#include "../../include/ttt.h"
#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

// ------------------------------------------------------------ scalar scan
// One workgroup of E2_ST threads per (head, chunk), 8 consecutive tokens per
// thread, all in float64. For token i of the chunk (0-based, n tokens):
//   Pb(i) = prod_{j>i} beta_j,  Pg(i) = prod_{j>i} gamma_j   (beta~, gamma~)
//   A(n-1) = 1,  A(i) = Pg(i) + beta_{i+1} A(i+1)
// The products are suffix scans; A is a suffix scan of the affine maps
// f_i(x) = Pg(i) + beta_{i+1} x (f_{n-1} = 1 + 0 x), composed as
// (c1, m1) o (c2, m2) = (c1 + m1 c2, m1 m2) -- no division anywhere.
// KW_i = eta_i A(i), KM_i = eta_i Pb(i); chunk coefficients gamma~_0 =
// prod gamma, beta_1 A_1 = beta_0 A(0) and beta~_0 = prod beta.
static constexpr int E2_ST = 256;
static constexpr int E2_TPT = 8;  // tokens per thread (C <= E2_ST * E2_TPT)

__global__ void __launch_bounds__(E2_ST) e2_scalar_kernel(const float* eta, const float* beta, const float* gamma,
                                                          int H, int64_t T, int C, float* KW, float* KM,
                                                          float* coef) {
  __shared__ double sb[E2_ST], sg[E2_ST], sc[E2_ST], sm[E2_ST];
  const int64_t nch = (T + C - 1) / C;
  const int h = blockIdx.x / (int)nch;
  const int64_t r = blockIdx.x % nch;
  const int64_t a = r * C;
  const int n = (int)min((int64_t)C, T - a);
  const int tid = threadIdx.x;
  const float* et = eta + h * T + a;
  const float* bt = beta + h * T + a;
  const float* gt = gamma + h * T + a;
  const int i0 = tid * E2_TPT;
  double b[E2_TPT], g[E2_TPT], bn[E2_TPT];
#pragma unroll
  for (int j = 0; j < E2_TPT; ++j) {
    const int i = i0 + j;
    b[j] = i < n ? (double)bt[i] : 1.0;
    g[j] = i < n ? (double)gt[i] : 1.0;
    bn[j] = (i + 1 < n) ? (double)bt[i + 1] : 0.0;  // beta_{i+1}; 0 ends the chain at n-1
  }
  // thread-local suffix products (exclusive) and the thread's totals
  double lb[E2_TPT], lg[E2_TPT];
  double pb = 1.0, pg = 1.0;
#pragma unroll
  for (int j = E2_TPT - 1; j >= 0; --j) {
    lb[j] = pb;
    lg[j] = pg;
    pb *= b[j];
    pg *= g[j];
  }
  // suffix scans over threads (inclusive), then shift to exclusive
  sb[tid] = pb;
  sg[tid] = pg;
  __syncthreads();
  for (int d = 1; d < E2_ST; d <<= 1) {
    const double xb = tid + d < E2_ST ? sb[tid + d] : 1.0;
    const double xg = tid + d < E2_ST ? sg[tid + d] : 1.0;
    __syncthreads();
    sb[tid] *= xb;
    sg[tid] *= xg;
    __syncthreads();
  }
  const double eb = tid + 1 < E2_ST ? sb[tid + 1] : 1.0;
  const double eg = tid + 1 < E2_ST ? sg[tid + 1] : 1.0;
  double Pb[E2_TPT], Pg[E2_TPT];
#pragma unroll
  for (int j = 0; j < E2_TPT; ++j) {
    Pb[j] = lb[j] * eb;
    Pg[j] = lg[j] * eg;
  }
  // affine maps f_i(x) = Pg(i) + bn_i x for tokens of the chunk; identity
  // (0 + 1 x) past its end; the thread's composition f_i0 o ... o f_i7
  double C_ = 0.0, M_ = 1.0;
#pragma unroll
  for (int j = E2_TPT - 1; j >= 0; --j) {
    const bool in = i0 + j < n;
    const double c = in ? Pg[j] : 0.0, m = in ? bn[j] : 1.0;
    C_ = c + m * C_;
    M_ = m * M_;
  }
  sc[tid] = C_;
  sm[tid] = M_;
  __syncthreads();
  for (int d = 1; d < E2_ST; d <<= 1) {
    const double c2 = tid + d < E2_ST ? sc[tid + d] : 0.0;
    const double m2 = tid + d < E2_ST ? sm[tid + d] : 1.0;
    __syncthreads();
    // (c1, m1) o (c2, m2): this thread's maps applied after the later ones
    sc[tid] = sc[tid] + sm[tid] * c2;
    sm[tid] = sm[tid] * m2;
    __syncthreads();
  }
  // value of the chain after this thread's tokens (its later threads'
  // composition evaluated anywhere: it ends in f_{n-1}, a constant)
  double v = tid + 1 < E2_ST ? sc[tid + 1] : 0.0;
  double A[E2_TPT];
#pragma unroll
  for (int j = E2_TPT - 1; j >= 0; --j) {
    if (i0 + j < n) v = Pg[j] + bn[j] * v;
    A[j] = v;
  }
  float* kw = KW + h * T + a;
  float* km = KM + h * T + a;
#pragma unroll
  for (int j = 0; j < E2_TPT; ++j) {
    const int i = i0 + j;
    if (i < n) {
      const double e = et[i];
      kw[i] = (float)(e * A[j]);
      km[i] = (float)(e * Pb[j]);
    }
  }
  if (tid == 0) {
    float* cf = coef + ((int64_t)h * nch + r) * 4;
    cf[0] = (float)(Pg[0] * g[0]);  // gamma~_0 = prod gamma
    cf[1] = (float)(b[0] * A[0]);   // beta~_0 R_1 = beta_1 A_1
    cf[2] = (float)(Pb[0] * b[0]);  // beta~_0 = prod beta
    cf[3] = 0.f;
  }
}

hipError_t e2_scalars(const float* eta, const float* beta, const float* gamma, int H, int64_t T, int C,
                      float* KW, float* KM, float* coef, hipStream_t st) {
  if (C > E2_ST * E2_TPT) return hipErrorInvalidValue;
  const int64_t nch = (T + C - 1) / C;
  hipLaunchKernelGGL(e2_scalar_kernel, dim3((unsigned)(nch * H)), dim3(E2_ST), 0, st, eta, beta, gamma, H, T, C,
                     KW, KM, coef);
  return hipGetLastError();
}

// ------------------------------------------------------- slice aggregation
static constexpr int SL = 128;  // tokens per slice

template <int D>
__global__ void __launch_bounds__(256) e2_partial_kernel(const bf16* __restrict__ K,
                                                         const bf16* __restrict__ Vv,
                                                         const float* __restrict__ KW,
                                                         const float* __restrict__ KM,
                                                         const float* __restrict__ W, int64_t T,
                                                         int64_t a0, int n, float* __restrict__ part,
                                                         int nslice, int H) {
  constexpr int P = SL + 8;     // row stride of token-contiguous tiles
  constexpr int PD = D + 8;     // row stride of feature-contiguous tiles
  // region X: W0 hi/lo [D][PD] during phase 1, then E hi/lo [D][P]
  __shared__ __attribute__((aligned(16))) bf16 X[2 * D * (P > PD ? P : PD)];
  __shared__ __attribute__((aligned(16))) bf16 Ks[SL * PD];  // [t][j]
  __shared__ __attribute__((aligned(16))) bf16 Kt[D * P];    // [j][t]
  __shared__ float ksc[2][SL];

  const int slice = blockIdx.x, h = blockIdx.y;
  const int t0 = slice * SL;
  const int nt = min(SL, n - t0);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const bf16* Kh = K + ((int64_t)h * T + a0 + t0) * D;
  const bf16* Vh = Vv + ((int64_t)h * T + a0 + t0) * D;
  const float* W0 = W + (int64_t)h * D * D;

  // W0 -> hi/lo (bf16) rows [i][j]
  bf16* Whi = X;
  bf16* Wlo = X + D * PD;
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    const float w = W0[e];
    const bf16 hi = (bf16)w;
    Whi[i * PD + j] = hi;
    Wlo[i * PD + j] = (bf16)(w - (float)hi);
  }
  // K slice [t][j] and its transpose [j][t]; rows past the chunk are zero
  for (int e = tid; e < SL * (D / 8); e += 256) {
    const int t = e / (D / 8), j8 = (e % (D / 8)) * 8;
    Frag8<bf16> f;
    if (t < nt) ld8(f, Kh + (int64_t)t * D + j8);
    else zero8(f);
    st8(Ks + t * PD + j8, f);
#pragma unroll
    for (int q = 0; q < 8; ++q) Kt[(j8 + q) * P + t] = f.v[q];
  }
  if (tid < SL) {
    ksc[0][tid] = tid < nt ? KW[h * T + a0 + t0 + tid] : 0.f;
    ksc[1][tid] = tid < nt ? KM[h * T + a0 + t0 + tid] : 0.f;
  }
  __syncthreads();

  // phase 1: E[t][i] = sum_j K[t][j] W0[i][j] - V[t][i]; wave owns 32 tokens.
  constexpr int FI = D / 16;
  floatx4 e[2][FI];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ni = 0; ni < FI; ++ni) e[mt][ni] = floatx4{0, 0, 0, 0};
#pragma unroll
  for (int kk = 0; kk < D; kk += 32) {
    Frag8<bf16> a[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) ld8(a[mt], Ks + (wid * 32 + mt * 16 + fr) * PD + kk + fg * 8);
#pragma unroll
    for (int ni = 0; ni < FI; ++ni) {
      Frag8<bf16> bh, bl;
      ld8(bh, Whi + (ni * 16 + fr) * PD + kk + fg * 8);
      ld8(bl, Wlo + (ni * 16 + fr) * PD + kk + fg * 8);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        mma16(e[mt][ni], a[mt], bh);
        mma16(e[mt][ni], a[mt], bl);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ni = 0; ni < FI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = wid * 32 + mt * 16 + fg * 4 + r;
        const int i = ni * 16 + fr;
        const float vv = t < nt ? (float)Vh[(int64_t)t * D + i] : 0.f;
        e[mt][ni][r] -= vv;
      }
  __syncthreads();  // W0 tiles no longer needed

  // phase 2: for each aggregation, write the scaled E^T split hi/lo as
  // [i][t] rows and contract over t with K^T rows [j][t].
  bf16* Ehi = X;
  bf16* Elo = X + D * P;
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ni = 0; ni < FI; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = wid * 32 + mt * 16 + fg * 4 + r;
          const int i = ni * 16 + fr;
          const float x = e[mt][ni][r] * ksc[which][t];
          const bf16 hi = (bf16)x;
          Ehi[i * P + t] = hi;
          Elo[i * P + t] = (bf16)(x - (float)hi);
        }
    __syncthreads();
    // output [i][j], wave owns rows i in [wid * D/4, +D/4)
    constexpr int FM = D / 64;  // 16-row tiles per wave
    floatx4 acc[FM][FI];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int nj = 0; nj < FI; ++nj) acc[mi][nj] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < SL; kk += 32) {
      Frag8<bf16> ah[FM], al[FM];
#pragma unroll
      for (int mi = 0; mi < FM; ++mi) {
        const int i = wid * (D / 4) + mi * 16 + fr;
        ld8(ah[mi], Ehi + i * P + kk + fg * 8);
        ld8(al[mi], Elo + i * P + kk + fg * 8);
      }
#pragma unroll
      for (int nj = 0; nj < FI; ++nj) {
        Frag8<bf16> bk;
        ld8(bk, Kt + (nj * 16 + fr) * P + kk + fg * 8);
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
          mma16(acc[mi][nj], ah[mi], bk);
          mma16(acc[mi][nj], al[mi], bk);
        }
      }
    }
    float* out = part + ((((int64_t)slice * H + h) * 2 + which) * D) * D;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int nj = 0; nj < FI; ++nj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = wid * (D / 4) + mi * 16 + fg * 4 + r;
          const int j = nj * 16 + fr;
          out[i * D + j] = acc[mi][nj][r];
        }
    __syncthreads();
  }
}

// W <- c0 W + c1 M + sum_s dW_s ;  M <- c2 M + sum_s dM_s   (per head)
__global__ void e2_combine_kernel(float* W, float* M, const float* part, const float* coef, int H,
                                  int D, int nslice, int64_t nch, int64_t r) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)D * D;
  if (e >= per * H) return;
  const int h = (int)(e / per);
  const int64_t o = e % per;
  const float* cf = coef + ((int64_t)h * nch + r) * 4;
  float dw = 0.f, dm = 0.f;
  for (int s = 0; s < nslice; ++s) {
    const float* p = part + (((int64_t)s * H + h) * 2) * per;
    dw += p[o];
    dm += p[per + o];
  }
  const float w0 = W[e], m0 = M[e];
  W[e] = cf[0] * w0 + cf[1] * m0 + dw;
  M[e] = cf[2] * m0 + dm;
}

}  // namespace ttt

// ==================================================================== C ABI
namespace {
struct E2Scratch {
  void* p = nullptr;
  size_t bytes = 0;
  int dev = -1;
};
E2Scratch g_e2;
}  // namespace

extern "C" ttt_status e2ttt_chunk_scan(const void* k, const void* v, const float* eta, const float* beta,
                                       const float* gamma, float* W, float* M, int32_t H, int64_t T,
                                       int32_t D, int32_t C, void* stream) {
  using namespace ttt;
  if (!k || !v || !eta || !beta || !gamma || !W || !M) return TTT_ERR_INVALID_ARG;
  if (H < 1 || T < 1 || C < 1) return TTT_ERR_INVALID_ARG;
  if (D != 128 && D != 64) return TTT_ERR_UNSUPPORTED;
  if (C % 64 || C > 2048) return TTT_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return TTT_ERR_NO_DEVICE;
  }
  hipStream_t st = (hipStream_t)stream;
  const int64_t nch = (T + C - 1) / C;
  const int nslice = (C + SL - 1) / SL;
  const size_t need = (size_t)2 * H * T * 4 + (size_t)H * nch * 4 * 4 +
                      (size_t)nslice * H * 2 * D * D * 4 + 256 * 4;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TTT_ERR_HIP;
  // Work buffer cached per process (grown on demand, reallocated on a device change).
  if (g_e2.bytes < need || g_e2.dev != dev) {
    if (g_e2.p) {
      (void)hipStreamSynchronize(st);
      (void)hipFree(g_e2.p);
    }
    g_e2.p = nullptr;
    g_e2.bytes = 0;
    if (hipMalloc(&g_e2.p, need) != hipSuccess) {
      (void)hipGetLastError();
      return TTT_ERR_OOM;
    }
    g_e2.bytes = need;
    g_e2.dev = dev;
  }
  float* KW = (float*)g_e2.p;
  float* KM = KW + (size_t)H * T;
  float* coef = KM + (size_t)H * T;
  float* part = coef + (size_t)H * nch * 4 + 64;
  if (e2_scalars(eta, beta, gamma, H, T, C, KW, KM, coef, st) != hipSuccess) return TTT_ERR_HIP;
  const int64_t per = (int64_t)H * D * D;
  for (int64_t r = 0; r < nch; ++r) {
    const int n = (int)std::min<int64_t>(C, T - r * C);
    const int ns = (n + SL - 1) / SL;
    if (D == 128)
      hipLaunchKernelGGL(e2_partial_kernel<128>, dim3(ns, H), dim3(256), 0, st, (const bf16*)k,
                         (const bf16*)v, KW, KM, W, T, r * C, n, part, ns, H);
    else
      hipLaunchKernelGGL(e2_partial_kernel<64>, dim3(ns, H), dim3(256), 0, st, (const bf16*)k,
                         (const bf16*)v, KW, KM, W, T, r * C, n, part, ns, H);
    hipLaunchKernelGGL(e2_combine_kernel, dim3((unsigned)((per + 255) / 256)), dim3(256), 0, st, W, M,
                       part, coef, H, D, ns, nch, r);
    if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  }
  return TTT_OK;
}
