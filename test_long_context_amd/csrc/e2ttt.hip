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
// Kernels: e2_scalars (all chunks at once), then one e2_chunk launch per
// chunk (the aggregations and the state update for that chunk).
#include <math.h>

#include <algorithm>
#include <mutex>

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
// ------------------------------------------------------------ chunk kernel
// One launch per chunk; workgroup (16-row block of the state, half of its
// columns, head) of 4 waves. Each wave takes 32-token blocks of the chunk
// (block b for b = wave, wave + 4, ...):
//   E [32 t x 16 i] = K W0^T - V  (A = K rows from LDS, B = W0 rows i as
//                                   bf16 hi + lo terms held in registers),
//   x = K_t E split into bf16 hi + lo -- the A operand of the aggregations,
//     straight from the accumulators: k-slot 8 g + e of lane group g is token
//     4 g + e (e < 4) or 16 + 4 g + (e - 4), the tokens the E tiles leave
//     there;
//   dW, dM [16 i x 16 j tiles] += x^T K with the B operand K^T (tokens in
//     that slot order) read from the wave's LDS copy of the K block by
//     transposing LDS reads (ds_read_b64_tr_b16, rows 4 g .. 4 g + 3 and
//     16 + 4 g .. 16 + 4 g + 3).
// The waves' sums meet in LDS and the workgroup writes
//   W_out = gamma~_0 W0 + beta~_0 R_1 M0 + dW,  M = beta~_0 M0 + dM.
// W is read whole-row (for E) by both column halves of a row block, so it
// ping-pongs between two buffers across chunks; M is read and written
// element by element by one workgroup and stays in place.
typedef short e2_shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) e2_shortx4* e2_lds_s4_t;

constexpr int E2_NW = 8;  // waves per chunk workgroup

template <int D>
__global__ void __launch_bounds__(E2_NW * 64) e2_chunk_kernel(const bf16* __restrict__ K, const bf16* __restrict__ Vv,
                                                       const float* __restrict__ KW, const float* __restrict__ KM,
                                                       const float* __restrict__ coef, const float* __restrict__ Win,
                                                       float* __restrict__ Wout, float* __restrict__ M, int64_t T,
                                                       int64_t a0, int n, int64_t nch, int64_t r) {
  constexpr int KS = D / 32;   // 32-wide steps over the feature dimension
  constexpr int JH = D / 2;    // state columns per workgroup
  constexpr int JT = JH / 16;  // their 16-column tiles
  constexpr int KP = D + 8;    // LDS row pitch of a K block (elements)
  constexpr int BT = 32;       // tokens per block
  constexpr int NV = BT * D / 8 / 64;  // 16-byte vectors of a K block per lane
  constexpr int NW = E2_NW;
  constexpr int RED = NW * 2 * 16 * JH;  // floats of the cross-wave sums
  static_assert(RED * 4 <= NW * BT * KP * 2, "the cross-wave sums reuse the K blocks' LDS");
  __shared__ __attribute__((aligned(16))) bf16 Kb[NW][BT * KP];
  // Workgroups are dealt to the 8 XCDs round-robin (XCD = id % 8). With
  // H % 8 == 0 the index is remapped so all 2 D / 16 workgroups of a head
  // run on one XCD (heads x, x + 8, ... on XCD x): each reads the head's
  // whole K block, which then comes from that XCD's L2 instead of once per
  // XCD from memory.
  constexpr int NB = 2 * (D / 16);  // workgroups per head
  const int H = gridDim.x / NB;
  int bid = blockIdx.x, h;
  if ((H & 7) == 0) {
    const int x = bid & 7, j = bid >> 3;
    h = x + 8 * (j / NB);
    bid = j % NB;
  } else {
    h = bid / NB;
    bid = bid % NB;
  }
  const int ib = bid >> 1, jh = bid & 1;
  const int i0 = ib * 16, j0 = jh * JH;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const bf16* Kh = K + ((int64_t)h * T + a0) * D;
  const bf16* Vh = Vv + ((int64_t)h * T + a0) * D;
  const float* KWh = KW + (int64_t)h * T + a0;
  const float* KMh = KM + (int64_t)h * T + a0;
  const float* W0 = Win + (int64_t)h * D * D;

  Frag8<bf16> wh[KS], wl[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const floatx4* src = (const floatx4*)(W0 + (i0 + c) * D + 32 * s + 8 * g);
    const floatx4 w4[2] = {src[0], src[1]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float w = w4[e >> 2][e & 3];
      const bf16 hi = (bf16)w;
      wh[s].v[e] = hi;
      wl[s].v[e] = (bf16)(w - (float)hi);
    }
  }
  floatx4 dw[JT], dm[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) dw[jt] = dm[jt] = floatx4{0.f, 0.f, 0.f, 0.f};

  bf16* Ks = Kb[wid];
  const int nb = (n + BT - 1) / BT;
  // a block's operands: its K rows (NV vectors per lane) and, for the tokens
  // of this lane's accumulator rows, v (column i0 + c), K^W and K^M
  // Loads are unconditional (token indices past the chunk clamp to its last
  // token) and raw, so nothing consumes them before the block is processed;
  // tokens past the chunk get K^W = K^M = 0 there, which zeroes their x and
  // hence their share of the products (the clamped rows are finite).
  struct Blk {
    bf16x8 k[NV];
    bf16 v[2][4];
    float kw[2][4], km[2][4];
  };
  auto load = [&](Blk& o, int blk) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int vi = lane + 64 * q, row = vi / (D / 8), col = (vi % (D / 8)) * 8;
      const int t = min(blk * BT + row, n - 1);
      o.k[q] = *(const bf16x8*)(Kh + (int64_t)t * D + col);
    }
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = min(blk * BT + 16 * tile + 4 * g + e, n - 1);
        o.v[tile][e] = Vh[(int64_t)t * D + i0 + c];
        o.kw[tile][e] = KWh[t];
        o.km[tile][e] = KMh[t];
      }
  };
  // operands run one block ahead of the products (two waves per SIMD hide
  // the rest)
  auto step = [&](Blk& cur, Blk& nxt, int blk) {
    // the previous block's LDS reads were consumed by its products, so the
    // wave's single buffer can be refilled (LDS operations of a wave are in order)
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int vi = lane + 64 * q, row = vi / (D / 8), col = (vi % (D / 8)) * 8;
      *(bf16x8*)(Ks + row * KP + col) = cur.k[q];
    }
    if (blk + NW < nb) load(nxt, blk + NW);

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    floatx4 et[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag8<bf16> a;
        ld8(a, Ks + (16 * tile + c) * KP + 32 * s + 8 * g);
        mma16(et[tile], a, wh[s]);
        mma16(et[tile], a, wl[s]);
      }
    Frag8<bf16> xwh, xwl, xmh, xml;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = blk * BT + 16 * tile + 4 * g + e < n;
        const float ee = et[tile][e] - (float)cur.v[tile][e];
        const float xw = ok ? cur.kw[tile][e] * ee : 0.f, xm = ok ? cur.km[tile][e] * ee : 0.f;
        const bf16 hw = (bf16)xw, hm = (bf16)xm;
        xwh.v[4 * tile + e] = hw;
        xwl.v[4 * tile + e] = (bf16)(xw - (float)hw);
        xmh.v[4 * tile + e] = hm;
        xml.v[4 * tile + e] = (bf16)(xm - (float)hm);
      }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const bf16* p = Ks + (4 * g + (c >> 2)) * KP + j0 + 16 * jt + 4 * (c & 3);
      const e2_shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((e2_lds_s4_t)p);
      const e2_shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((e2_lds_s4_t)(p + 16 * KP));
      typedef short e2_shortx8 __attribute__((ext_vector_type(8)));
      Frag8<bf16> bk;
      bk.v = __builtin_bit_cast(bf16x8, (e2_shortx8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      mma16(dw[jt], xwh, bk);
      mma16(dw[jt], xwl, bk);
      mma16(dm[jt], xmh, bk);
      mma16(dm[jt], xml, bk);
    }
  };
  Blk b0, b1;
  if (wid < nb) load(b0, wid);
  for (int blk = wid; blk < nb; blk += 2 * NW) {
    step(b0, b1, blk);
    if (blk + NW < nb) step(b1, b0, blk + NW);
  }
  // cross-wave sums: red[w][0 / 1][i][j]
  __syncthreads();
  float* red = (float*)&Kb[0][0];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * g + e, j = 16 * jt + c;
      red[((wid * 2 + 0) * 16 + i) * JH + j] = dw[jt][e];
      red[((wid * 2 + 1) * 16 + i) * JH + j] = dm[jt][e];
    }
  __syncthreads();
  const float* cf = coef + ((int64_t)h * nch + r) * 4;
  const float c0 = cf[0], c1 = cf[1], c2 = cf[2];
  float* Wo = Wout + (int64_t)h * D * D;
  float* Mh = M + (int64_t)h * D * D;
  for (int e = threadIdx.x; e < 16 * JH; e += NW * 64) {
    const int i = e / JH, j = e % JH;
    float sw = 0.f, sm = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sw += red[((w * 2 + 0) * 16 + i) * JH + j];
      sm += red[((w * 2 + 1) * 16 + i) * JH + j];
    }
    const int64_t idx = (int64_t)(i0 + i) * D + j0 + j;
    const float w0 = W0[idx], m0 = Mh[idx];
    Wo[idx] = c0 * w0 + c1 * m0 + sw;
    Mh[idx] = c2 * m0 + sm;
  }
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
std::mutex g_e2_mu;  // guards g_e2 on the host
}  // namespace

extern "C" ttt_status e2ttt_chunk_scan(const void* k, const void* v, const float* eta, const float* beta,
                                       const float* gamma, float* W, float* M, int32_t H, int64_t T,
                                       int32_t D, int32_t C, void* stream) {
  using namespace ttt;
  if (!k || !v || !eta || !beta || !gamma || !W || !M) return TTT_ERR_INVALID_ARG;
  if (H < 1 || T < 1 || C < 1) return TTT_ERR_INVALID_ARG;
  if (D != 128 && D != 64) return TTT_ERR_UNSUPPORTED;
  if (C % 64 || C > 2048) return TTT_ERR_UNSUPPORTED;
  if (((uintptr_t)W & 15) || ((uintptr_t)M & 15)) return TTT_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return TTT_ERR_NO_DEVICE;
  }
  hipStream_t st = (hipStream_t)stream;
  const int64_t nch = (T + C - 1) / C;
  const size_t need = (size_t)2 * H * T * 4 + (size_t)H * nch * 4 * 4 + (size_t)H * D * D * 4 + 512;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TTT_ERR_HIP;
  // Work buffer cached per process (grown on demand, reallocated on a device change).
  std::lock_guard<std::mutex> lock(g_e2_mu);
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
  // the other W buffer, 256-byte aligned (its rows are read as 16-byte vectors)
  float* W2 = (float*)(((uintptr_t)(coef + (size_t)H * nch * 4) + 255) & ~(uintptr_t)255);
  if (e2_scalars(eta, beta, gamma, H, T, C, KW, KM, coef, st) != hipSuccess) return TTT_ERR_HIP;
  const dim3 grid(2 * (D / 16) * H);
  for (int64_t r = 0; r < nch; ++r) {
    const int n = (int)std::min<int64_t>(C, T - r * C);
    const float* src = (r & 1) ? W2 : W;
    float* dst = (r & 1) ? W : W2;
    if (D == 128)
      hipLaunchKernelGGL(e2_chunk_kernel<128>, grid, dim3(E2_NW * 64), 0, st, (const bf16*)k, (const bf16*)v, KW, KM, coef,
                         src, dst, M, T, r * C, n, nch, r);
    else
      hipLaunchKernelGGL(e2_chunk_kernel<64>, grid, dim3(E2_NW * 64), 0, st, (const bf16*)k, (const bf16*)v, KW, KM, coef,
                         src, dst, M, T, r * C, n, nch, r);
    if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  }
  // an odd number of chunks leaves the state in the work buffer
  if (nch & 1) {
    if (hipMemcpyAsync(W, W2, (size_t)H * D * D * 4, hipMemcpyDeviceToDevice, st) != hipSuccess) return TTT_ERR_HIP;
  }
  return TTT_OK;
}
