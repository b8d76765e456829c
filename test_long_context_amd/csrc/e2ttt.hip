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

// LaCT's chunk coefficients ([P3] 背景知识): per (head, chunk) the mean of
// the chunk's beta_t (float64, fixed-order tree), coef = (1, mean, mean, 0):
// W_out = W0 + mean M0 + dM, M = mean M0 + dM with dM = sum_t eta_t G_t.
__global__ void __launch_bounds__(E2_ST) lact_scalar_kernel(const float* beta, int64_t T, int C, float* coef) {
  __shared__ double sb[E2_ST];
  const int64_t nch = (T + C - 1) / C;
  const int h = blockIdx.x / (int)nch;
  const int64_t r = blockIdx.x % nch;
  const int64_t a = r * C;
  const int n = (int)min((int64_t)C, T - a);
  const float* bt = beta + h * T + a;
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += E2_ST) s += (double)bt[i];
  sb[threadIdx.x] = s;
  __syncthreads();
  for (int d = E2_ST / 2; d > 0; d >>= 1) {
    if (threadIdx.x < d) sb[threadIdx.x] += sb[threadIdx.x + d];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float* cf = coef + ((int64_t)h * nch + r) * 4;
    const float mean = (float)(sb[0] / n);
    cf[0] = 1.f;
    cf[1] = mean;
    cf[2] = mean;
    cf[3] = 0.f;
  }
}

// ------------------------------------------------------ token-mixer inputs
// [P3] 混合模型架构设计 and 依赖于输入的动态参数化: from the projections
// P = x wqkv^T (float [T, 3 H D + 3 H]) of one token per workgroup: q, k =
// L2-normalised SiLU of their head slices, v as projected (all bf16 [H, T, D],
// the chunk kernel's layout), and per head eta = eta_base sigma(z_eta),
// beta = sigma(z_beta)^(1/tau), gamma = 1 - eta alpha_base sigma(z_alpha)
// (float [H, T]; z = scalar logit + bias; eta is stored negated, see
// below). A group of 16 lanes handles one head; each lane D / 16
// consecutive features.
template <int D>
__global__ void __launch_bounds__(256) mixer_prologue_kernel(const float* __restrict__ P, const float* __restrict__ bias,
                                                             int H, int64_t T, float eta_base, float alpha_base,
                                                             float inv_tau, bf16* __restrict__ q, bf16* __restrict__ k,
                                                             bf16* __restrict__ v, float* __restrict__ eta,
                                                             float* __restrict__ beta, float* __restrict__ gamma) {
  constexpr int E = D / 16;  // features per lane
  const int64_t t = blockIdx.x;
  const int grp = threadIdx.x >> 4, l = threadIdx.x & 15;
  const int64_t N = 3LL * H * D + 3LL * H;
  const float* row = P + t * N;
  for (int h = grp; h < H; h += 16) {
    const int f0 = h * D + l * E;
    // q and k: SiLU, then L2 normalisation over the head's D features
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      float x[E];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float z = row[(int64_t)which * H * D + f0 + e];
        x[e] = z / (1.f + __expf(-z));
        ss += x[e] * x[e];
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 16);
      const float rn = rsqrtf(ss);
      bf16* dst = (which == 0 ? q : k) + ((int64_t)h * T + t) * D + l * E;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = (bf16)(x[e] * rn);
    }
    bf16* dv = v + ((int64_t)h * T + t) * D + l * E;
#pragma unroll
    for (int e = 0; e < E; ++e) dv[e] = (bf16)row[2LL * H * D + f0 + e];
    if (l == 0) {
      const float* z = row + 3LL * H * D;
      const float se = 1.f / (1.f + __expf(-(z[h] + bias[h])));
      const float sb = 1.f / (1.f + __expf(-(z[H + h] + bias[H + h])));
      const float sa = 1.f / (1.f + __expf(-(z[2 * H + h] + bias[2 * H + h])));
      const float et = eta_base * se;
      // the page's G_t is the negative gradient (descent) while the chunk
      // kernels aggregate G_t = (W0 k - v) k^T: hand them -eta_t
      eta[(int64_t)h * T + t] = -et;
      beta[(int64_t)h * T + t] = powf(sb, inv_tau);
      gamma[(int64_t)h * T + t] = 1.f - et * (alpha_base * sa);
    }
  }
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
typedef __bf16 e2_bf16x2 __attribute__((ext_vector_type(2)));
typedef float e2_floatx2 __attribute__((ext_vector_type(2)));

// raw buffer resource over nbytes from p (loads beyond it return 0); p and
// nbytes are the same in every lane and are moved to scalar registers here
// (a descriptor the compiler takes for divergent costs a loop per load)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t e2_rsrc(const void* p, uint32_t nbytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* q = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)__builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
}

// x = hi + lo in bf16, both rounded to nearest even, two values per
// conversion: hi = RNE(x), lo = RNE(x - hi)
__device__ __forceinline__ void e2_split(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const e2_bf16x2 h = __builtin_convertvector((e2_floatx2){x[2 * p], x[2 * p + 1]}, e2_bf16x2);
    const uint32_t hu = __builtin_bit_cast(uint32_t, h);
    const float h0 = __builtin_bit_cast(float, hu << 16), h1 = __builtin_bit_cast(float, hu & 0xffff0000u);
    const e2_bf16x2 l = __builtin_convertvector((e2_floatx2){x[2 * p] - h0, x[2 * p + 1] - h1}, e2_bf16x2);
    hi[2 * p] = h[0];
    hi[2 * p + 1] = h[1];
    lo[2 * p] = l[0];
    lo[2 * p + 1] = l[1];
  }
}

// waves per chunk workgroup: 12 (three per SIMD) where the registers allow
// it (head size 128 without outputs), else 8
__host__ __device__ constexpr int e2_waves(int D, bool OUT) { return (D == 128 && !OUT) ? 12 : 8; }

// LACT: the chunk-wise baseline's single aggregation (K^W unused, dW taken
// as dM): W_out = coef0 W0 + coef1 M0 + dM, M = coef2 M0 + dM.
// OUT: also the outputs o_t = W0 q_t of the chunk's tokens (Q [H, T, D]
// bf16, out float [T, H D]): the two workgroups of a 16-row block take one
// 16-token tile of every 32-token block each, with the same W0 terms.
template <int D, bool LACT = false, bool OUT = false>
__global__ void __launch_bounds__(e2_waves(D, OUT) * 64) e2_chunk_kernel(const bf16* __restrict__ K, const bf16* __restrict__ Vv,
                                                       const float* __restrict__ KW, const float* __restrict__ KM,
                                                       const float* __restrict__ coef, const float* __restrict__ Win,
                                                       float* __restrict__ Wout, float* __restrict__ M, int64_t T,
                                                       int64_t a0, int n, int64_t nch, int64_t r,
                                                       const bf16* __restrict__ Q = nullptr, float* __restrict__ out = nullptr) {
  constexpr int KS = D / 32;   // 32-wide steps over the feature dimension
  constexpr int JH = D / 2;    // state columns per workgroup
  constexpr int JT = JH / 16;  // their 16-column tiles
  constexpr int KP = D + 8;    // LDS row pitch of a K block (elements)
  constexpr int BT = 32;       // tokens per block
  constexpr int NV = BT * D / 8 / 64;  // 16-byte vectors of a K block per lane
  constexpr int NW = e2_waves(D, OUT);
  constexpr int RED = NW * 2 * 16 * JH;  // floats of the cross-wave sums
  static_assert(RED * 4 <= NW * BT * KP * 2, "the cross-wave sums reuse the K blocks' LDS");
  __shared__ __attribute__((aligned(16))) bf16 Kb[NW][BT * KP];
  // per wave: the block's v columns i0 .. i0 + 15 ([32 tokens][16], read
  // back by transposing reads) and its K^W, K^M ([64]: K^W then K^M)
  __shared__ __attribute__((aligned(16))) bf16 Vb[NW][BT * 16];
  __shared__ __attribute__((aligned(16))) float Sb[NW][2 * BT];
  // with three waves per SIMD the W0 terms (the E product's B operand, the
  // same for every wave) live in LDS instead of each wave's registers
  constexpr bool W_LDS = NW > 8;
  constexpr int WP = D + 8;  // LDS row pitch of the W0 terms
  __shared__ __attribute__((aligned(16))) bf16 Wt[W_LDS ? 2 * 16 * WP : 8];
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
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const bf16* Kh = K + ((int64_t)h * T + a0) * D;
  const bf16* Vh = Vv + ((int64_t)h * T + a0) * D;
  const float* KWh = KW + (int64_t)h * T + a0;
  const float* KMh = KM + (int64_t)h * T + a0;
  const float* W0 = Win + (int64_t)h * D * D;
  // lane parts of the byte offsets within a block: a K block is BT whole
  // rows, so vector q of lane l is bytes 16 (l + 64 q) of it; lane l reads
  // v columns i0 + 8 (l % 2) .. + 7 of token l / 2, and K^W, K^M of token
  // l % 32 (one coalesced load each; the lanes that need them read them
  // back from LDS)
  const uint32_t ko = lane * 16, vo = ((lane >> 1) * D + i0 + 8 * (lane & 1)) * 2, so = (lane & 31) * 4;

  // W0 rows i0 + c (this lane's B operand of e_t), requested first; the
  // first block's operands and the state elements of the final update are
  // requested before the W0 terms are formed, so the latencies overlap
  floatx4 w4[KS][2];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const floatx4* src = (const floatx4*)(W0 + (i0 + c) * D + 32 * s + 8 * g);
    w4[s][0] = src[0];
    w4[s][1] = src[1];
  }
  Frag8<bf16> wh[KS], wl[KS];  // formed below, once the other loads are out
  floatx4 dw[JT], dm[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) dw[jt] = dm[jt] = floatx4{0.f, 0.f, 0.f, 0.f};

  bf16* Ks = Kb[wid];
  bf16* Vs = Vb[wid];
  float* Ss = Sb[wid];
  const int nb = (n + BT - 1) / BT;
  // a block's operands: its K rows (NV vectors per lane) and, for the tokens
  // of this lane's accumulator rows, v (column i0 + c), K^W and K^M
  // Loads are unconditional (token indices past the chunk clamp to its last
  // token) and raw, so nothing consumes them before the block is processed;
  // tokens past the chunk get K^W = K^M = 0 there, which zeroes their x and
  // hence their share of the products (the clamped rows are finite).
  struct Blk {
    bf16x8 k[NV];
    bf16x8 v;
    float kw, km;
  };
  // Each block is read through buffer resources that start at the block
  // and cover only its tokens inside the chunk (none for blocks past it), so
  // tokens past the chunk -- only the sequence's last chunk has them, and
  // they lie past T -- read as k = v = 0 and K^W = K^M = 0 without touching
  // memory: their x is exactly 0 and they add nothing to the products. The
  // loads are therefore unconditional (a skipped prefetch would make the
  // wait for the current block's operands cover the next block's loads).
  auto load = [&](Blk& o, int blk) {
    const int nt = max(0, min(BT, n - blk * BT));
    const int64_t t0 = (int64_t)blk * BT;
    const __amdgpu_buffer_rsrc_t rk = e2_rsrc(Kh + t0 * D, (uint32_t)nt * D * 2);
    const __amdgpu_buffer_rsrc_t rv = e2_rsrc(Vh + t0 * D, (uint32_t)nt * D * 2);
    const __amdgpu_buffer_rsrc_t rkw = e2_rsrc(KWh + t0, (uint32_t)nt * 4);
    const __amdgpu_buffer_rsrc_t rkm = e2_rsrc(KMh + t0, (uint32_t)nt * 4);
#pragma unroll
    for (int q = 0; q < NV; ++q)
      o.k[q] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 1024 * q, 0, 0));
    o.v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, 0));
    o.kw = LACT ? 0.f : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkw, so, 0, 0));
    o.km = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkm, so, 0, 0));
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
    *(bf16x8*)(Vs + (lane >> 1) * 16 + 8 * (lane & 1)) = cur.v;
    Ss[lane] = lane < 32 ? cur.kw : cur.km;
    load(nxt, blk + NW);

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    floatx4 et[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (W_LDS) {
      // (per tile the same order of products as below)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag8<bf16> bh, bl;
        ld8(bh, Wt + c * WP + 32 * s + 8 * g);
        ld8(bl, Wt + (16 + c) * WP + 32 * s + 8 * g);
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          Frag8<bf16> a;
          ld8(a, Ks + (16 * tile + c) * KP + 32 * s + 8 * g);
          mma16(et[tile], a, bh);
          mma16(et[tile], a, bl);
        }
      }
    } else {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          Frag8<bf16> a;
          ld8(a, Ks + (16 * tile + c) * KP + 32 * s + 8 * g);
          mma16(et[tile], a, wh[s]);
          mma16(et[tile], a, wl[s]);
        }
    }
    if constexpr (OUT) {
      // this workgroup's output tile of the block: o = Q W0^T for rows i0 .. i0 + 15
      const int tile = jh;
      floatx4 ot = floatx4{0.f, 0.f, 0.f, 0.f};
      const int tq = min(blk * BT + 16 * tile + c, n - 1);
      const bf16* Qh = Q + ((int64_t)h * T + a0 + tq) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag8<bf16> aq;
        aq.v = *(const bf16x8*)(Qh + 32 * s + 8 * g);
        mma16(ot, aq, wh[s]);
        mma16(ot, aq, wl[s]);
      }
      const int HD = (gridDim.x / (2 * (D / 16))) * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = blk * BT + 16 * tile + 4 * g + e;
        if (tok < n) out[(a0 + tok) * HD + (int64_t)h * D + i0 + c] = ot[e];
      }
    }
    // v of tokens 16 tile + 4 g + e, column i0 + c (transposing reads of
    // the wave's v slice, as for the aggregations' K^T operand), and their
    // K^W, K^M (the same four values across each 16-lane group)
    float xw[8], xm[8];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const e2_shortx4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (e2_lds_s4_t)(Vs + (16 * tile + 4 * g + (c >> 2)) * 16 + 4 * (c & 3)));
      const floatx4 kw4 = *(const floatx4*)(Ss + 16 * tile + 4 * g);
      const floatx4 km4 = *(const floatx4*)(Ss + BT + 16 * tile + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ee = et[tile][e] - __builtin_bit_cast(float, (uint32_t)(unsigned short)vt[e] << 16);
        xw[4 * tile + e] = kw4[e] * ee;
        xm[4 * tile + e] = km4[e] * ee;
      }
    }
    Frag8<bf16> xwh, xwl, xmh, xml;
    e2_split(xw, xwh.v, xwl.v);
    e2_split(xm, xmh.v, xml.v);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const bf16* p = Ks + (4 * g + (c >> 2)) * KP + j0 + 16 * jt + 4 * (c & 3);
      const e2_shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((e2_lds_s4_t)p);
      const e2_shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((e2_lds_s4_t)(p + 16 * KP));
      typedef short e2_shortx8 __attribute__((ext_vector_type(8)));
      Frag8<bf16> bk;
      bk.v = __builtin_bit_cast(bf16x8, (e2_shortx8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (!LACT) {
        mma16(dw[jt], xwh, bk);
        mma16(dw[jt], xwl, bk);
      }
      mma16(dm[jt], xmh, bk);
      mma16(dm[jt], xml, bk);
    }
  };
  Blk b0, b1;
  load(b0, wid);
  // the state elements this thread updates at the end: (i, j) = (e / JH, e % JH)
  constexpr int NEL = 16 * JH, EPT = (NEL + NW * 64 - 1) / (NW * 64);
  float* Wo = Wout + (int64_t)h * D * D;
  float* Mh = M + (int64_t)h * D * D;
  float w0e[EPT], m0e[EPT];
  auto load_state = [&]() {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = min((int)threadIdx.x + k * NW * 64, NEL - 1);
      const int64_t idx = (int64_t)(i0 + e / JH) * D + j0 + e % JH;
      w0e[k] = W0[idx];
      m0e[k] = Mh[idx];
    }
  };
  // (with outputs or three waves per SIMD there are no registers to hold
  // them through the loop: they are read at the end)
  constexpr bool LATE_STATE = OUT || NW > 8;
  if constexpr (!LATE_STATE) load_state();
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float w = w4[s][e >> 2][e & 3];
      const bf16 hi = (bf16)w;
      wh[s].v[e] = hi;
      wl[s].v[e] = (bf16)(w - (float)hi);
    }
  if constexpr (W_LDS) {
    // every wave formed the same terms: wave 0 stores them (rows c, columns
    // 32 s + 8 g .. + 7 of each lane), then all waves read them from LDS
    if (wid == 0)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        *(bf16x8*)(Wt + c * WP + 32 * s + 8 * g) = wh[s].v;
        *(bf16x8*)(Wt + (16 + c) * WP + 32 * s + 8 * g) = wl[s].v;
      }
    __syncthreads();
  }
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
      red[((wid * 2 + 0) * 16 + i) * JH + j] = LACT ? dm[jt][e] : dw[jt][e];
      red[((wid * 2 + 1) * 16 + i) * JH + j] = dm[jt][e];
    }
  __syncthreads();
  const float* cf = coef + ((int64_t)h * nch + r) * 4;
  const float c0 = cf[0], c1 = cf[1], c2 = cf[2];
  if constexpr (LATE_STATE) load_state();
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = threadIdx.x + k * NW * 64;
    if (e >= NEL) break;
    const int i = e / JH, j = e % JH;
    float sw = 0.f, sm = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sw += red[((w * 2 + 0) * 16 + i) * JH + j];
      sm += red[((w * 2 + 1) * 16 + i) * JH + j];
    }
    const int64_t idx = (int64_t)(i0 + i) * D + j0 + j;
    Wo[idx] = c0 * w0e[k] + c1 * m0e[k] + sw;
    Mh[idx] = c2 * m0e[k] + sm;
  }
}


}  // namespace ttt

// ==================================================================== C ABI
namespace {
// Device work buffer of one call: taken on the call's stream from the
// device's default memory pool and given back on the same stream after the
// call's kernels (stream order), so calls on different streams or host
// threads never share one. The pool keeps what is given back for later calls
// (its release threshold is raised once per device), so repeated calls do not
// reach the driver.
constexpr int E2_POOL_MAX_DEV = 64;
bool g_pool_ready[E2_POOL_MAX_DEV] = {};
std::mutex g_pool_mu;  // guards g_pool_ready

class CallWork {
 public:
  CallWork() = default;
  CallWork(const CallWork&) = delete;
  CallWork& operator=(const CallWork&) = delete;
  ~CallWork() {
    if (p_) (void)hipFreeAsync(p_, st_);
  }
  ttt_status alloc(size_t bytes, hipStream_t st) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= E2_POOL_MAX_DEV) return TTT_ERR_HIP;
    {
      std::lock_guard<std::mutex> lock(g_pool_mu);
      if (!g_pool_ready[dev]) {
        hipMemPool_t pool = nullptr;
        if (hipDeviceGetDefaultMemPool(&pool, dev) != hipSuccess) return TTT_ERR_HIP;
        uint64_t keep = UINT64_MAX;
        if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) return TTT_ERR_HIP;
        g_pool_ready[dev] = true;
      }
    }
    if (hipMallocAsync(&p_, bytes, st) != hipSuccess) {
      (void)hipGetLastError();
      p_ = nullptr;
      return TTT_ERR_OOM;
    }
    st_ = st;
    return TTT_OK;
  }
  void* get() const { return p_; }

 private:
  void* p_ = nullptr;
  hipStream_t st_ = nullptr;
};

// Work buffer of the allocation-free entry point: a fixed device array, one
// copy per GPU, alive until the process ends. Host code never passes the
// symbol itself to a kernel (on the host it is only a stand-in): its device
// address is looked up once per device and kept in g_scr_ptr.
constexpr size_t E2_SCRATCH_BYTES = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[E2_SCRATCH_BYTES];
constexpr int E2_MAX_DEV = 64;
void* g_scr_ptr[E2_MAX_DEV] = {};
std::mutex g_scr_mu;  // guards g_scr_ptr

ttt_status e2_check(const void* k, const void* v, const float* eta, const float* beta, const float* gamma,
                    const float* W, const float* M, int32_t H, int64_t T, int32_t D, int32_t C) {
  if (!k || !v || !eta || !beta || !gamma || !W || !M) return TTT_ERR_INVALID_ARG;
  if (H < 1 || T < 1 || C < 1) return TTT_ERR_INVALID_ARG;
  if (D != 128 && D != 64) return TTT_ERR_UNSUPPORTED;
  if (C % 64 || C > 2048) return TTT_ERR_UNSUPPORTED;
  if (((uintptr_t)W & 15) || ((uintptr_t)M & 15)) return TTT_ERR_INVALID_ARG;
  return TTT_OK;
}

// Bytes of work buffer a call needs: the per-token coefficients KW, KM
// [H, T], the per-chunk coefficients [H, chunks, 4] and the second W buffer
// [H, D, D] at a 256-byte boundary.
size_t e2_work_bytes(int32_t H, int64_t T, int32_t D, int32_t C) {
  const int64_t nch = (T + C - 1) / C;
  return (size_t)2 * H * T * 4 + (size_t)H * nch * 4 * 4 + (size_t)H * D * D * 4 + 512;
}

// Enqueues the scan on st with the given work buffer (at least
// e2_work_bytes, 256-byte aligned).
ttt_status e2_run(const void* k, const void* v, const float* eta, const float* beta, const float* gamma, float* W,
                  float* M, int32_t H, int64_t T, int32_t D, int32_t C, void* work, hipStream_t st) {
  using namespace ttt;
  const int64_t nch = (T + C - 1) / C;
  float* KW = (float*)work;
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
      hipLaunchKernelGGL(e2_chunk_kernel<128>, grid, dim3(e2_waves(128, false) * 64), 0, st, (const bf16*)k, (const bf16*)v, KW, KM, coef,
                         src, dst, M, T, r * C, n, nch, r);
    else
      hipLaunchKernelGGL(e2_chunk_kernel<64>, grid, dim3(e2_waves(64, false) * 64), 0, st, (const bf16*)k, (const bf16*)v, KW, KM, coef,
                         src, dst, M, T, r * C, n, nch, r);
    if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  }
  // an odd number of chunks leaves the state in the work buffer
  if (nch & 1) {
    if (hipMemcpyAsync(W, W2, (size_t)H * D * D * 4, hipMemcpyDeviceToDevice, st) != hipSuccess) return TTT_ERR_HIP;
  }
  return TTT_OK;
}
}  // namespace

extern "C" ttt_status e2ttt_chunk_scan(const void* k, const void* v, const float* eta, const float* beta,
                                       const float* gamma, float* W, float* M, int32_t H, int64_t T,
                                       int32_t D, int32_t C, void* stream) {
  const ttt_status cs = e2_check(k, v, eta, beta, gamma, W, M, H, T, D, C);
  if (cs != TTT_OK) return cs;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return TTT_ERR_NO_DEVICE;
  }
  hipStream_t st = (hipStream_t)stream;
  CallWork w;
  const ttt_status ws = w.alloc(e2_work_bytes(H, T, D, C), st);
  if (ws != TTT_OK) return ws;
  return e2_run(k, v, eta, beta, gamma, W, M, H, T, D, C, w.get(), st);
}

extern "C" int64_t e2ttt_chunk_scan_noalloc_max_bytes(void) { return (int64_t)E2_SCRATCH_BYTES; }

extern "C" ttt_status e2ttt_chunk_scan_noalloc(const void* k, const void* v, const float* eta, const float* beta,
                                               const float* gamma, float* W, float* M, int32_t H, int64_t T,
                                               int32_t D, int32_t C, void* stream) {
  const ttt_status cs = e2_check(k, v, eta, beta, gamma, W, M, H, T, D, C);
  if (cs != TTT_OK) return cs;
  if (e2_work_bytes(H, T, D, C) > E2_SCRATCH_BYTES) return TTT_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return TTT_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TTT_ERR_HIP;
  if (dev < 0 || dev >= E2_MAX_DEV) return TTT_ERR_UNSUPPORTED;
  void* work = nullptr;
  {
    // first call on this device (it is current): look up its copy's address
    std::lock_guard<std::mutex> lock(g_scr_mu);
    if (!g_scr_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return TTT_ERR_HIP;
      }
      g_scr_ptr[dev] = p;
    }
    work = g_scr_ptr[dev];
  }
  return e2_run(k, v, eta, beta, gamma, W, M, H, T, D, C, work, (hipStream_t)stream);
}

namespace {
// Work buffer of the LaCT scan: the per-chunk coefficients [H, chunks, 4] and
// the second W buffer [H, D, D] at a 256-byte boundary.
size_t lact_work_bytes(int32_t H, int64_t T, int32_t D, int32_t C) {
  const int64_t nch = (T + C - 1) / C;
  return (size_t)H * nch * 4 * 4 + (size_t)H * D * D * 4 + 512;
}

ttt_status lact_run(const void* k, const void* v, const float* eta, const float* beta, float* W, float* M, int32_t H,
                    int64_t T, int32_t D, int32_t C, void* work, hipStream_t st) {
  using namespace ttt;
  const int64_t nch = (T + C - 1) / C;
  float* coef = (float*)work;
  float* W2 = (float*)(((uintptr_t)(coef + (size_t)H * nch * 4) + 255) & ~(uintptr_t)255);
  hipLaunchKernelGGL(lact_scalar_kernel, dim3((unsigned)(nch * H)), dim3(E2_ST), 0, st, beta, T, C, coef);
  if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  const dim3 grid(2 * (D / 16) * H);
  for (int64_t r = 0; r < nch; ++r) {
    const int n = (int)std::min<int64_t>(C, T - r * C);
    const float* src = (r & 1) ? W2 : W;
    float* dst = (r & 1) ? W : W2;
    // per-token weights eta_t; the K^W argument is not read by this rule
    if (D == 128)
      hipLaunchKernelGGL((e2_chunk_kernel<128, true>), grid, dim3(e2_waves(128, false) * 64), 0, st, (const bf16*)k, (const bf16*)v,
                         eta, eta, coef, src, dst, M, T, r * C, n, nch, r);
    else
      hipLaunchKernelGGL((e2_chunk_kernel<64, true>), grid, dim3(e2_waves(64, false) * 64), 0, st, (const bf16*)k, (const bf16*)v,
                         eta, eta, coef, src, dst, M, T, r * C, n, nch, r);
    if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  }
  if (nch & 1) {
    if (hipMemcpyAsync(W, W2, (size_t)H * D * D * 4, hipMemcpyDeviceToDevice, st) != hipSuccess) return TTT_ERR_HIP;
  }
  return TTT_OK;
}
}  // namespace

extern "C" ttt_status lact_chunk_scan(const void* k, const void* v, const float* eta, const float* beta, float* W,
                                      float* M, int32_t H, int64_t T, int32_t D, int32_t C, void* stream) {
  const ttt_status cs = e2_check(k, v, eta, beta, beta, W, M, H, T, D, C);
  if (cs != TTT_OK) return cs;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return TTT_ERR_NO_DEVICE;
  }
  hipStream_t st = (hipStream_t)stream;
  CallWork w;
  const ttt_status ws = w.alloc(lact_work_bytes(H, T, D, C), st);
  if (ws != TTT_OK) return ws;
  return lact_run(k, v, eta, beta, W, M, H, T, D, C, w.get(), st);
}

namespace {
// 256-byte aligned carve-out of the mixer's work buffer
struct Carve {
  uintptr_t p;
  template <typename X>
  X* take(size_t bytes) {
    X* r = (X*)p;
    p = (p + bytes + 255) & ~(uintptr_t)255;
    return r;
  }
};

size_t mixer_work_bytes(int32_t H, int64_t T, int32_t D, int32_t C) {
  const int64_t N = 3LL * H * D + 3LL * H, nch = (T + C - 1) / C;
  const size_t al = 256;
  return (size_t)T * N * 4 + al + 3 * ((size_t)H * T * D * 2 + al) + 5 * ((size_t)H * T * 4 + al) +
         (size_t)H * nch * 16 + al + (size_t)H * D * D * 4 + al + 256;
}
}  // namespace

namespace {
ttt_status device_present() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return TTT_ERR_NO_DEVICE;
  }
  return TTT_OK;
}

ttt_status mixer_check(const void* x, const void* wqkv, const float* bias, float eta_base, float alpha_base,
                       float tau, const float* out, int32_t H, int64_t T, int32_t D, int32_t dm, int32_t C) {
  if (!x || !wqkv || !bias || !out) return TTT_ERR_INVALID_ARG;
  if (H < 1 || T < 1 || C < 1 || dm < 1 || !(tau > 0.f) || !(eta_base >= 0.f) || !(alpha_base >= 0.f))
    return TTT_ERR_INVALID_ARG;
  if (D != 128 && D != 64) return TTT_ERR_UNSUPPORTED;
  if (C % 64 || C > 2048 || dm % 8) return TTT_ERR_UNSUPPORTED;
  if (((uintptr_t)x & 15) || ((uintptr_t)wqkv & 15) || ((uintptr_t)out & 15)) return TTT_ERR_INVALID_ARG;
  return TTT_OK;
}

// The linear-fast-weight mixer on a work buffer of mixer_work_bytes().
ttt_status mixer_linear_run(const void* x, const void* wqkv, const float* bias, float eta_base, float alpha_base,
                            float tau, float* W, float* M, float* out, int32_t H, int64_t T, int32_t D, int32_t dm,
                            int32_t C, void* work, void* stream) {
  using namespace ttt;
  hipStream_t st = (hipStream_t)stream;
  const int64_t N = 3LL * H * D + 3LL * H, nch = (T + C - 1) / C;
  Carve cv{((uintptr_t)work + 255) & ~(uintptr_t)255};
  float* P = cv.take<float>((size_t)T * N * 4);
  bf16* q = cv.take<bf16>((size_t)H * T * D * 2);
  bf16* k = cv.take<bf16>((size_t)H * T * D * 2);
  bf16* v = cv.take<bf16>((size_t)H * T * D * 2);
  float* eta = cv.take<float>((size_t)H * T * 4);
  float* beta = cv.take<float>((size_t)H * T * 4);
  float* gamma = cv.take<float>((size_t)H * T * 4);
  float* KW = cv.take<float>((size_t)H * T * 4);
  float* KM = cv.take<float>((size_t)H * T * 4);
  float* coef = cv.take<float>((size_t)H * nch * 16);
  float* W2 = cv.take<float>((size_t)H * D * D * 4);
  // projections: P = x wqkv^T (bf16 operands, fp32 accumulation and result)
  GemmArgs g{};
  g.A = x;
  g.B = wqkv;
  g.M = (int)T;
  g.N = (int)N;
  g.K = dm;
  g.lda = dm;
  g.ldb = dm;
  g.C = P;
  g.ldc = N;
  g.scale = 1.f;
  if (gemm(DT::BF16, true, true, Epi::STORE_F32, g, st) != hipSuccess) return TTT_ERR_HIP;
  if (D == 128)
    hipLaunchKernelGGL(mixer_prologue_kernel<128>, dim3((unsigned)T), dim3(256), 0, st, P, bias, H, T, eta_base,
                       alpha_base, 1.f / tau, q, k, v, eta, beta, gamma);
  else
    hipLaunchKernelGGL(mixer_prologue_kernel<64>, dim3((unsigned)T), dim3(256), 0, st, P, bias, H, T, eta_base,
                       alpha_base, 1.f / tau, q, k, v, eta, beta, gamma);
  if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  if (e2_scalars(eta, beta, gamma, H, T, C, KW, KM, coef, st) != hipSuccess) return TTT_ERR_HIP;
  const dim3 grid(2 * (D / 16) * H);
  for (int64_t r = 0; r < nch; ++r) {
    const int n = (int)std::min<int64_t>(C, T - r * C);
    const float* src = (r & 1) ? W2 : W;
    float* dst = (r & 1) ? W : W2;
    if (D == 128)
      hipLaunchKernelGGL((e2_chunk_kernel<128, false, true>), grid, dim3(e2_waves(128, true) * 64), 0, st, k, v, KW, KM, coef, src,
                         dst, M, T, r * C, n, nch, r, q, out);
    else
      hipLaunchKernelGGL((e2_chunk_kernel<64, false, true>), grid, dim3(e2_waves(64, true) * 64), 0, st, k, v, KW, KM, coef, src,
                         dst, M, T, r * C, n, nch, r, q, out);
    if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  }
  if (nch & 1) {
    if (hipMemcpyAsync(W, W2, (size_t)H * D * D * 4, hipMemcpyDeviceToDevice, st) != hipSuccess) return TTT_ERR_HIP;
  }
  return TTT_OK;
}
}  // namespace

extern "C" ttt_status e2ttt_mixer_forward(const void* x, const void* wqkv, const float* bias, float eta_base,
                                          float alpha_base, float tau, float* W, float* M, float* out, int32_t H,
                                          int64_t T, int32_t D, int32_t dm, int32_t C, void* stream) {
  ttt_status r = mixer_check(x, wqkv, bias, eta_base, alpha_base, tau, out, H, T, D, dm, C);
  if (r != TTT_OK) return r;
  if (!W || !M || ((uintptr_t)W & 15) || ((uintptr_t)M & 15)) return TTT_ERR_INVALID_ARG;
  if ((r = device_present()) != TTT_OK) return r;
  CallWork w;
  if ((r = w.alloc(mixer_work_bytes(H, T, D, C), (hipStream_t)stream)) != TTT_OK) return r;
  return mixer_linear_run(x, wqkv, bias, eta_base, alpha_base, tau, W, M, out, H, T, D, dm, C, w.get(), stream);
}

// ============================================ SwiGLU fast-weight token mixer
// [P3] 方法细节, 快速权重网络实例化: per head the fast weight is the net
//   f_W(x) = x + LN(W3 (silu(W1 x) * (W2 x)))   (LN without affine, eps 1e-5)
// with the per-token loss 1/2 ||f_W0(k_t) - v_t||^2 at the chunk-start W0 and
// Proposition 3.1 applied to each of W1, W2, W3 (own momentum, shared
// scalars). Per chunk, every step runs for all heads in one launch (grid.y =
// head):
//   A12 = K W12^T (SwiGLU epilogue: pre-activations A12 and H = silu * up),
//   Y = H W3^T (fp32), the same two products for the queries;
//   rows: LN(Y), g = k + LN(Y_k) - v, dY = LN^T g, scaled by K^W_t and K^M_t
//         (bf16), outputs o_t = q_t + LN(Y_q);
//   dA12 = (K dY) W3 with the SwiGLU backward in the epilogue (twice);
//   aggregations (tokens contracted): K dY^T H -> [D, Dh], dA12^T K -> [2 Dh, D]
//   (twice), then W = c0 W + c1 M + aggW, M = c2 M + aggM element-wise,
//   with the bf16 copy of W for the next chunk's products.
// W1 | W2 live 16-row interleaved (gate rows 32 j + w, up rows 32 j + 16 + w)
// in one [2 Dh, D] matrix per head, the layout of the SwiGLU epilogues.
namespace {
using ttt::bf16;
using ttt::bf16x4;
using ttt::floatx4;
constexpr float E2MLP_EPS = 1e-5f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One wave per (token, head); blockIdx.z = 0: keys (dY), 1: queries (outputs).
template <int D>
__global__ void __launch_bounds__(256) e2mlp_rows_kernel(const float* __restrict__ Yk, const float* __restrict__ Yq,
                                                         const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                         const bf16* __restrict__ v, const float* __restrict__ KW,
                                                         const float* __restrict__ KM, int64_t T, int64_t a, int n,
                                                         int Cmax, int H, bf16* __restrict__ dYw,
                                                         bf16* __restrict__ dYm, float* __restrict__ out) {
  constexpr int E = D / 64;
  const int h = blockIdx.y;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const bool keys = blockIdx.z == 0;
  const int64_t row = ((int64_t)h * Cmax + i) * D + lane * E;
  const float* y = (keys ? Yk : Yq) + row;
  float yv[E], z[E];
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    yv[e] = y[e];
    s += yv[e];
  }
  const float mu = wave_sum(s) * (1.f / D);
  float s2 = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) s2 += (yv[e] - mu) * (yv[e] - mu);
  const float r = rsqrtf(wave_sum(s2) * (1.f / D) + E2MLP_EPS);
#pragma unroll
  for (int e = 0; e < E; ++e) z[e] = (yv[e] - mu) * r;
  const int64_t t = a + i;
  const int64_t src = ((int64_t)h * T + t) * D + lane * E;
  if (keys) {
    float g[E];
    float sg = 0.f, sgz = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      g[e] = (float)k[src + e] + z[e] - (float)v[src + e];
      sg += g[e];
      sgz += g[e] * z[e];
    }
    const float mg = wave_sum(sg) * (1.f / D), mgz = wave_sum(sgz) * (1.f / D);
    const float kw = KW[(int64_t)h * T + t], km = KM[(int64_t)h * T + t];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float dy = r * (g[e] - mg - z[e] * mgz);
      dYw[row + e] = (bf16)(kw * dy);
      dYm[row + e] = (bf16)(km * dy);
    }
  } else {
    float* o = out + (t * H + h) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = (float)q[src + e] + z[e];
  }
}

// W = c0 W + c1 M + aw, M = c2 M + am, Wb = bf16(W) over H heads of `per`
// elements (a multiple of 4); c = coef[(h nch + r) * 4 + 0..2].
__global__ void __launch_bounds__(256) e2mlp_state_kernel(float* __restrict__ W, float* __restrict__ M,
                                                          const float* __restrict__ aw, const float* __restrict__ am,
                                                          bf16* __restrict__ Wb, const float* __restrict__ coef,
                                                          int64_t per, int H, int64_t nch, int64_t r) {
  const int64_t n4 = (int64_t)H * per / 4;
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < n4; j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = 4 * j;
    const int h = (int)(i / per);
    const float* c = coef + ((int64_t)h * nch + r) * 4;
    const float c0 = c[0], c1 = c[1], c2 = c[2];
    const floatx4 w = *(const floatx4*)(W + i), m = *(const floatx4*)(M + i);
    const floatx4 x = *(const floatx4*)(aw + i), y = *(const floatx4*)(am + i);
    const floatx4 wn = c0 * w + c1 * m + x;
    *(floatx4*)(W + i) = wn;
    *(floatx4*)(M + i) = c2 * m + y;
    bf16x4 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = (bf16)wn[e];
    *(bf16x4*)(Wb + i) = b;
  }
}

__global__ void __launch_bounds__(256) e2mlp_cast_kernel(const float* __restrict__ src, bf16* __restrict__ dst,
                                                         int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = (bf16)src[i];
}

// rows of [R, cols] fp32 <-> the 16-row interleaved pair layout ([2 R, cols])
hipError_t il_rows(float* dst, const float* src, int64_t R, int cols, int which, bool to_pair, hipStream_t st) {
  const size_t blk = (size_t)16 * cols * 4;
  if (to_pair)
    return hipMemcpy2DAsync((char*)dst + which * blk, 2 * blk, src, blk, blk, R / 16, hipMemcpyDeviceToDevice, st);
  return hipMemcpy2DAsync(dst, blk, (const char*)src + which * blk, 2 * blk, blk, R / 16, hipMemcpyDeviceToDevice,
                          st);
}

size_t mlp_mixer_work_bytes(int32_t H, int64_t T, int32_t D, int32_t Dh, int32_t C) {
  const size_t al = 256, h = H, c = C, d = D, f = Dh;
  return mixer_work_bytes(H, T, D, C) + 2 * (h * 2 * f * d * 4 + al) + h * 2 * f * d * 2 + al +
         h * d * f * 2 + al + 2 * (h * c * 2 * f * 2 + al) + 2 * (h * c * f * 2 + al) + 2 * (h * c * d * 4 + al) +
         2 * (h * c * d * 2 + al) + 2 * (h * c * 2 * f * 2 + al) + 2 * (h * 2 * f * d * 4 + al) +
         2 * (h * d * f * 4 + al) + 256;
}

// batched (over heads) bf16 product for the SwiGLU mixer
ttt::GemmArgs hg(const void* A, long lda, long sA, const void* B, long ldb, long sB, int M, int N, int K, void* C,
                 long ldc, long sC, int H) {
  ttt::GemmArgs g{};
  g.A = A;
  g.B = B;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.scale = 1.f;
  g.batch = H;
  g.sA = sA;
  g.sB = sB;
  g.sC = sC;
  return g;
}
}  // namespace

namespace {
ttt_status swiglu_check(const float* W1, const float* W2, const float* W3, const float* M1, const float* M2,
                        const float* M3, int32_t Dh) {
  if (!W1 || !W2 || !W3 || !M1 || !M2 || !M3 || Dh < 1) return TTT_ERR_INVALID_ARG;
  if (Dh % 32 || Dh > 4096) return TTT_ERR_UNSUPPORTED;
  for (const void* p : {(const void*)W1, (const void*)W2, (const void*)W3, (const void*)M1, (const void*)M2,
                        (const void*)M3})
    if ((uintptr_t)p & 15) return TTT_ERR_INVALID_ARG;
  return TTT_OK;
}

// The SwiGLU-fast-weight mixer on a work buffer of mlp_mixer_work_bytes().
ttt_status mixer_swiglu_run(const void* x, const void* wqkv, const float* bias, float eta_base, float alpha_base,
                            float tau, float* W1, float* W2, float* W3, float* M1, float* M2, float* M3, float* out,
                            int32_t H, int64_t T, int32_t D, int32_t Dh, int32_t dm, int32_t C, void* work,
                            void* stream) {
  using namespace ttt;
  hipStream_t st = (hipStream_t)stream;
  const int64_t N = 3LL * H * D + 3LL * H, nch = (T + C - 1) / C;
  const size_t h = H, c = C, d = D, f = Dh;
  Carve cv{((uintptr_t)work + 255) & ~(uintptr_t)255};
  float* P = cv.take<float>((size_t)T * N * 4);
  bf16* q = cv.take<bf16>(h * T * d * 2);
  bf16* k = cv.take<bf16>(h * T * d * 2);
  bf16* v = cv.take<bf16>(h * T * d * 2);
  float* eta = cv.take<float>(h * T * 4);
  float* beta = cv.take<float>(h * T * 4);
  float* gamma = cv.take<float>(h * T * 4);
  float* KW = cv.take<float>(h * T * 4);
  float* KM = cv.take<float>(h * T * 4);
  float* coef = cv.take<float>(h * nch * 16);
  (void)cv.take<float>(h * d * d * 4);  // (the linear mixer's second state buffer; unused here)
  float* W12 = cv.take<float>(h * 2 * f * d * 4);
  float* M12 = cv.take<float>(h * 2 * f * d * 4);
  bf16* W12b = cv.take<bf16>(h * 2 * f * d * 2);
  bf16* W3b = cv.take<bf16>(h * d * f * 2);
  bf16* A12k = cv.take<bf16>(h * c * 2 * f * 2);
  bf16* A12q = cv.take<bf16>(h * c * 2 * f * 2);
  bf16* Hk = cv.take<bf16>(h * c * f * 2);
  bf16* Hq = cv.take<bf16>(h * c * f * 2);
  float* Yk = cv.take<float>(h * c * d * 4);
  float* Yq = cv.take<float>(h * c * d * 4);
  bf16* dYw = cv.take<bf16>(h * c * d * 2);
  bf16* dYm = cv.take<bf16>(h * c * d * 2);
  bf16* dAw = cv.take<bf16>(h * c * 2 * f * 2);
  bf16* dAm = cv.take<bf16>(h * c * 2 * f * 2);
  float* a12w = cv.take<float>(h * 2 * f * d * 4);
  float* a12m = cv.take<float>(h * 2 * f * d * 4);
  float* a3w = cv.take<float>(h * d * f * 4);
  float* a3m = cv.take<float>(h * d * f * 4);
  (void)A12q;
#define E2CHK(call)                          \
  do {                                       \
    if ((call) != hipSuccess) {              \
      (void)hipGetLastError();               \
      return TTT_ERR_HIP;                    \
    }                                        \
  } while (0)
  // inputs: projections, then q, k, v and the scalars (as the linear mixer)
  {
    GemmArgs g{};
    g.A = x;
    g.B = wqkv;
    g.M = (int)T;
    g.N = (int)N;
    g.K = dm;
    g.lda = dm;
    g.ldb = dm;
    g.C = P;
    g.ldc = N;
    g.scale = 1.f;
    E2CHK(gemm(DT::BF16, true, true, Epi::STORE_F32, g, st));
  }
  if (D == 128)
    hipLaunchKernelGGL(mixer_prologue_kernel<128>, dim3((unsigned)T), dim3(256), 0, st, P, bias, H, T, eta_base,
                       alpha_base, 1.f / tau, q, k, v, eta, beta, gamma);
  else
    hipLaunchKernelGGL(mixer_prologue_kernel<64>, dim3((unsigned)T), dim3(256), 0, st, P, bias, H, T, eta_base,
                       alpha_base, 1.f / tau, q, k, v, eta, beta, gamma);
  E2CHK(hipGetLastError());
  E2CHK(e2_scalars(eta, beta, gamma, H, T, C, KW, KM, coef, st));
  // state: W1 | W2 and their momenta into the interleaved pair layout
  const int64_t R = (int64_t)H * Dh;
  E2CHK(il_rows(W12, W1, R, D, 0, true, st));
  E2CHK(il_rows(W12, W2, R, D, 1, true, st));
  E2CHK(il_rows(M12, M1, R, D, 0, true, st));
  E2CHK(il_rows(M12, M2, R, D, 1, true, st));
  hipLaunchKernelGGL(e2mlp_cast_kernel, dim3(1024), dim3(256), 0, st, W12, W12b, (int64_t)(h * 2 * f * d));
  hipLaunchKernelGGL(e2mlp_cast_kernel, dim3(1024), dim3(256), 0, st, W3, W3b, (int64_t)(h * d * f));
  E2CHK(hipGetLastError());
  const long sT = (long)T * D, s12 = 2L * Dh * D, s3 = (long)D * Dh;
  for (int64_t r = 0; r < nch; ++r) {
    const int n = (int)std::min<int64_t>(C, T - r * C);
    const size_t off = (size_t)r * C * D;
    // forward of keys and queries under the chunk-start weights
    for (int which = 0; which < 2; ++which) {
      const bf16* in = (which == 0 ? k : q) + off;
      bf16* Hx = which == 0 ? Hk : Hq;
      GemmArgs g = hg(in, D, sT, W12b, D, s12, n, 2 * Dh, D, which == 0 ? (void*)A12k : nullptr, 2 * Dh,
                      (long)C * 2 * Dh, H);
      g.C2 = Hx;
      g.sC2 = (long)C * Dh;
      E2CHK(gemm(DT::BF16, true, true, Epi::SWIGLU, g, st));
      GemmArgs g2 = hg(Hx, Dh, (long)C * Dh, W3b, Dh, s3, n, D, Dh, which == 0 ? Yk : Yq, D, (long)C * D, H);
      E2CHK(gemm(DT::BF16, true, true, Epi::STORE_F32, g2, st));
    }
    const dim3 rg((unsigned)((n + 3) / 4), (unsigned)H, 2);
    if (D == 128)
      hipLaunchKernelGGL(e2mlp_rows_kernel<128>, rg, dim3(256), 0, st, Yk, Yq, q, k, v, KW, KM, T, r * C, n, C, H,
                         dYw, dYm, out);
    else
      hipLaunchKernelGGL(e2mlp_rows_kernel<64>, rg, dim3(256), 0, st, Yk, Yq, q, k, v, KW, KM, T, r * C, n, C, H,
                         dYw, dYm, out);
    E2CHK(hipGetLastError());
    // backward through the net, once per scalar kernel, and the aggregations
    for (int which = 0; which < 2; ++which) {
      const bf16* dY = which == 0 ? dYw : dYm;
      bf16* dA = which == 0 ? dAw : dAm;
      GemmArgs gb = hg(dY, D, (long)C * D, W3b, Dh, s3, n, Dh, D, dA, 2 * Dh, (long)C * 2 * Dh, H);
      gb.X = A12k;
      gb.sX = (long)C * 2 * Dh;
      E2CHK(gemm(DT::BF16, true, false, Epi::SWIGLU_BWD, gb, st));
      GemmArgs g3 = hg(dY, D, (long)C * D, Hk, Dh, (long)C * Dh, D, Dh, n, which == 0 ? a3w : a3m, Dh, s3, H);
      E2CHK(gemm(DT::BF16, false, false, Epi::STORE_F32, g3, st));
      GemmArgs g12 = hg(dA, 2 * Dh, (long)C * 2 * Dh, k + off, D, sT, 2 * Dh, D, n, which == 0 ? a12w : a12m, D,
                        s12, H);
      E2CHK(gemm(DT::BF16, false, false, Epi::STORE_F32, g12, st));
    }
    hipLaunchKernelGGL(e2mlp_state_kernel, dim3(1024), dim3(256), 0, st, W12, M12, a12w, a12m, W12b, coef, s12, H,
                       nch, r);
    hipLaunchKernelGGL(e2mlp_state_kernel, dim3(1024), dim3(256), 0, st, W3, M3, a3w, a3m, W3b, coef, s3, H, nch,
                       r);
    E2CHK(hipGetLastError());
  }
  E2CHK(il_rows(W1, W12, R, D, 0, false, st));
  E2CHK(il_rows(W2, W12, R, D, 1, false, st));
  E2CHK(il_rows(M1, M12, R, D, 0, false, st));
  E2CHK(il_rows(M2, M12, R, D, 1, false, st));
#undef E2CHK
  return TTT_OK;
}
}  // namespace

namespace {
// ------------------------------------------------ GELU fast-weight net
// [P3] 方法细节, 快速权重网络实例化: f_W(x) = x + LN(W2 GELU(W1 x)) with the
// exact GELU, u Phi(u). Same per-chunk schedule as the SwiGLU net, with a
// plain bf16 store of the pre-activations U = x W1^T and two element-wise
// passes: A = GELU(U) before the W2 product, dU = dA GELU'(U) after the
// backward product dA = dY W2.
__device__ __forceinline__ float gelu_f(float u) { return 0.5f * u * (1.f + erff(u * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_grad_f(float u) {
  return 0.5f * (1.f + erff(u * 0.70710678118654752f)) + u * __expf(-0.5f * u * u) * 0.39894228040143268f;
}

// rows i < n of the H blocks [Cmax, Dh] (bf16): out = GELU(U), or, with dA,
// out = dA GELU'(U); Dh a multiple of 4
__global__ void __launch_bounds__(256) e2gelu_kernel(const bf16* __restrict__ U, const bf16* __restrict__ dA,
                                                     bf16* __restrict__ out, int n, int Cmax, int Dh, int H) {
  const int64_t per = (int64_t)n * Dh / 4, total = per * H;
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < total; j += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(j / per);
    const int64_t i = ((int64_t)h * Cmax * Dh) + 4 * (j - h * per);
    const bf16x4 u = *(const bf16x4*)(U + i);
    bf16x4 r;
    if (dA) {
      const bf16x4 g = *(const bf16x4*)(dA + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (bf16)((float)g[e] * gelu_grad_f((float)u[e]));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (bf16)gelu_f((float)u[e]);
    }
    *(bf16x4*)(out + i) = r;
  }
}

size_t gelu_mixer_work_bytes(int32_t H, int64_t T, int32_t D, int32_t Dh, int32_t C) {
  const size_t al = 256, h = H, c = C, d = D, f = Dh;
  return mixer_work_bytes(H, T, D, C) + 2 * (h * f * d * 2 + al) + 4 * (h * c * f * 2 + al) + 2 * (h * c * d * 4 + al) +
         2 * (h * c * d * 2 + al) + 2 * (h * c * f * 2 + al) + 4 * (h * f * d * 4 + al) + 256;
}

ttt_status gelu_check(const float* W1, const float* W2, const float* M1, const float* M2, int32_t Dh) {
  if (!W1 || !W2 || !M1 || !M2 || Dh < 1) return TTT_ERR_INVALID_ARG;
  if (Dh % 32 || Dh > 4096) return TTT_ERR_UNSUPPORTED;
  for (const void* p : {(const void*)W1, (const void*)W2, (const void*)M1, (const void*)M2})
    if ((uintptr_t)p & 15) return TTT_ERR_INVALID_ARG;
  return TTT_OK;
}

// The GELU-fast-weight mixer on a work buffer of gelu_mixer_work_bytes().
ttt_status mixer_gelu_run(const void* x, const void* wqkv, const float* bias, float eta_base, float alpha_base,
                          float tau, float* W1, float* W2, float* M1, float* M2, float* out, int32_t H, int64_t T,
                          int32_t D, int32_t Dh, int32_t dm, int32_t C, void* work, void* stream) {
  using namespace ttt;
  hipStream_t st = (hipStream_t)stream;
  const int64_t N = 3LL * H * D + 3LL * H, nch = (T + C - 1) / C;
  const size_t h = H, c = C, d = D, f = Dh;
  Carve cv{((uintptr_t)work + 255) & ~(uintptr_t)255};
  float* P = cv.take<float>((size_t)T * N * 4);
  bf16* q = cv.take<bf16>(h * T * d * 2);
  bf16* k = cv.take<bf16>(h * T * d * 2);
  bf16* v = cv.take<bf16>(h * T * d * 2);
  float* eta = cv.take<float>(h * T * 4);
  float* beta = cv.take<float>(h * T * 4);
  float* gamma = cv.take<float>(h * T * 4);
  float* KW = cv.take<float>(h * T * 4);
  float* KM = cv.take<float>(h * T * 4);
  float* coef = cv.take<float>(h * nch * 16);
  (void)cv.take<float>(h * d * d * 4);  // (the linear mixer's second state buffer; unused here)
  bf16* W1b = cv.take<bf16>(h * f * d * 2);
  bf16* W2b = cv.take<bf16>(h * d * f * 2);
  bf16* Uk = cv.take<bf16>(h * c * f * 2);
  bf16* Uq = cv.take<bf16>(h * c * f * 2);
  bf16* Hk = cv.take<bf16>(h * c * f * 2);
  bf16* Hq = cv.take<bf16>(h * c * f * 2);
  float* Yk = cv.take<float>(h * c * d * 4);
  float* Yq = cv.take<float>(h * c * d * 4);
  bf16* dYw = cv.take<bf16>(h * c * d * 2);
  bf16* dYm = cv.take<bf16>(h * c * d * 2);
  bf16* dA = cv.take<bf16>(h * c * f * 2);
  bf16* dU = cv.take<bf16>(h * c * f * 2);
  float* a1w = cv.take<float>(h * f * d * 4);
  float* a1m = cv.take<float>(h * f * d * 4);
  float* a2w = cv.take<float>(h * d * f * 4);
  float* a2m = cv.take<float>(h * d * f * 4);
#define E2CHK(call)                          \
  do {                                       \
    if ((call) != hipSuccess) {              \
      (void)hipGetLastError();               \
      return TTT_ERR_HIP;                    \
    }                                        \
  } while (0)
  // inputs: projections, then q, k, v and the scalars (as the linear mixer)
  {
    GemmArgs g{};
    g.A = x;
    g.B = wqkv;
    g.M = (int)T;
    g.N = (int)N;
    g.K = dm;
    g.lda = dm;
    g.ldb = dm;
    g.C = P;
    g.ldc = N;
    g.scale = 1.f;
    E2CHK(gemm(DT::BF16, true, true, Epi::STORE_F32, g, st));
  }
  if (D == 128)
    hipLaunchKernelGGL(mixer_prologue_kernel<128>, dim3((unsigned)T), dim3(256), 0, st, P, bias, H, T, eta_base,
                       alpha_base, 1.f / tau, q, k, v, eta, beta, gamma);
  else
    hipLaunchKernelGGL(mixer_prologue_kernel<64>, dim3((unsigned)T), dim3(256), 0, st, P, bias, H, T, eta_base,
                       alpha_base, 1.f / tau, q, k, v, eta, beta, gamma);
  E2CHK(hipGetLastError());
  E2CHK(e2_scalars(eta, beta, gamma, H, T, C, KW, KM, coef, st));
  hipLaunchKernelGGL(e2mlp_cast_kernel, dim3(1024), dim3(256), 0, st, W1, W1b, (int64_t)(h * f * d));
  hipLaunchKernelGGL(e2mlp_cast_kernel, dim3(1024), dim3(256), 0, st, W2, W2b, (int64_t)(h * d * f));
  E2CHK(hipGetLastError());
  const long sT = (long)T * D, s1 = (long)Dh * D, s2 = (long)D * Dh;
  for (int64_t r = 0; r < nch; ++r) {
    const int n = (int)std::min<int64_t>(C, T - r * C);
    const size_t off = (size_t)r * C * D;
    const unsigned eg = (unsigned)std::min<int64_t>(2048, ((int64_t)H * n * Dh / 4 + 255) / 256);
    // forward of keys and queries under the chunk-start weights
    for (int which = 0; which < 2; ++which) {
      const bf16* in = (which == 0 ? k : q) + off;
      bf16* Ux = which == 0 ? Uk : Uq;
      bf16* Hx = which == 0 ? Hk : Hq;
      GemmArgs g = hg(in, D, sT, W1b, D, s1, n, Dh, D, Ux, Dh, (long)C * Dh, H);
      E2CHK(gemm(DT::BF16, true, true, Epi::STORE, g, st));
      hipLaunchKernelGGL(e2gelu_kernel, dim3(eg), dim3(256), 0, st, Ux, (const bf16*)nullptr, Hx, n, C, Dh, H);
      E2CHK(hipGetLastError());
      GemmArgs g2 = hg(Hx, Dh, (long)C * Dh, W2b, Dh, s2, n, D, Dh, which == 0 ? Yk : Yq, D, (long)C * D, H);
      E2CHK(gemm(DT::BF16, true, true, Epi::STORE_F32, g2, st));
    }
    const dim3 rg((unsigned)((n + 3) / 4), (unsigned)H, 2);
    if (D == 128)
      hipLaunchKernelGGL(e2mlp_rows_kernel<128>, rg, dim3(256), 0, st, Yk, Yq, q, k, v, KW, KM, T, r * C, n, C, H,
                         dYw, dYm, out);
    else
      hipLaunchKernelGGL(e2mlp_rows_kernel<64>, rg, dim3(256), 0, st, Yk, Yq, q, k, v, KW, KM, T, r * C, n, C, H,
                         dYw, dYm, out);
    E2CHK(hipGetLastError());
    // backward through the net, once per scalar kernel, and the aggregations
    for (int which = 0; which < 2; ++which) {
      const bf16* dY = which == 0 ? dYw : dYm;
      GemmArgs gb = hg(dY, D, (long)C * D, W2b, Dh, s2, n, Dh, D, dA, Dh, (long)C * Dh, H);
      E2CHK(gemm(DT::BF16, true, false, Epi::STORE, gb, st));
      hipLaunchKernelGGL(e2gelu_kernel, dim3(eg), dim3(256), 0, st, (const bf16*)Uk, (const bf16*)dA, dU, n, C, Dh, H);
      E2CHK(hipGetLastError());
      GemmArgs g2 = hg(dY, D, (long)C * D, Hk, Dh, (long)C * Dh, D, Dh, n, which == 0 ? a2w : a2m, Dh, s2, H);
      E2CHK(gemm(DT::BF16, false, false, Epi::STORE_F32, g2, st));
      GemmArgs g1 = hg(dU, Dh, (long)C * Dh, k + off, D, sT, Dh, D, n, which == 0 ? a1w : a1m, D, s1, H);
      E2CHK(gemm(DT::BF16, false, false, Epi::STORE_F32, g1, st));
    }
    hipLaunchKernelGGL(e2mlp_state_kernel, dim3(1024), dim3(256), 0, st, W1, M1, a1w, a1m, W1b, coef, s1, H, nch, r);
    hipLaunchKernelGGL(e2mlp_state_kernel, dim3(1024), dim3(256), 0, st, W2, M2, a2w, a2m, W2b, coef, s2, H, nch, r);
    E2CHK(hipGetLastError());
  }
#undef E2CHK
  return TTT_OK;
}
}  // namespace

extern "C" ttt_status e2ttt_mixer_gelu_forward(const void* x, const void* wqkv, const float* bias, float eta_base,
                                               float alpha_base, float tau, float* W1, float* W2, float* M1,
                                               float* M2, float* out, int32_t H, int64_t T, int32_t D, int32_t Dh,
                                               int32_t dm, int32_t C, void* stream) {
  ttt_status r = mixer_check(x, wqkv, bias, eta_base, alpha_base, tau, out, H, T, D, dm, C);
  if (r != TTT_OK) return r;
  if ((r = gelu_check(W1, W2, M1, M2, Dh)) != TTT_OK) return r;
  if ((r = device_present()) != TTT_OK) return r;
  CallWork w;
  if ((r = w.alloc(gelu_mixer_work_bytes(H, T, D, Dh, C), (hipStream_t)stream)) != TTT_OK) return r;
  return mixer_gelu_run(x, wqkv, bias, eta_base, alpha_base, tau, W1, W2, M1, M2, out, H, T, D, Dh, dm, C, w.get(),
                        stream);
}

extern "C" ttt_status e2ttt_mixer_swiglu_forward(const void* x, const void* wqkv, const float* bias, float eta_base,
                                                 float alpha_base, float tau, float* W1, float* W2, float* W3,
                                                 float* M1, float* M2, float* M3, float* out, int32_t H, int64_t T,
                                                 int32_t D, int32_t Dh, int32_t dm, int32_t C, void* stream) {
  ttt_status r = mixer_check(x, wqkv, bias, eta_base, alpha_base, tau, out, H, T, D, dm, C);
  if (r != TTT_OK) return r;
  if ((r = swiglu_check(W1, W2, W3, M1, M2, M3, Dh)) != TTT_OK) return r;
  if ((r = device_present()) != TTT_OK) return r;
  CallWork w;
  if ((r = w.alloc(mlp_mixer_work_bytes(H, T, D, Dh, C), (hipStream_t)stream)) != TTT_OK) return r;
  return mixer_swiglu_run(x, wqkv, bias, eta_base, alpha_base, tau, W1, W2, W3, M1, M2, M3, out, H, T, D, Dh, dm,
                          C, w.get(), stream);
}

// ================================================== hybrid token-mixer block
// [P3] 方法细节, 混合模型架构设计 and Figure 2: sliding-window attention on the
// shared projections (RoPE on q and k, before the TTT path's SiLU and L2
// normalisation) beside the TTT path, mixed element-wise by a data-dependent
// gate: out = g o_SWA + (1 - g) o_TTT, g = sigmoid(x Wg^T + bg). The TTT
// path writes o_TTT into out; the attention reuses the engine's RoPE scatter
// into key/value stores of the whole stream and its second-generation
// window-attention kernel; one element-wise pass applies the gate.
namespace {
// bf16 [T, 3 H D] copy of the projections' q, k, v columns (row stride N)
__global__ void __launch_bounds__(256) raw_qkv_kernel(const float* __restrict__ P, int64_t N, int64_t T, int W,
                                                      bf16* __restrict__ out) {
  const int64_t n = T * W;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / W;
    out[i] = (bf16)P[t * N + (i - t * W)];
  }
}

// RoPE table [T][D / 2] of (cos, sin)(p theta^(-2 j / D)), angles in float64
__global__ void __launch_bounds__(256) rope_table_kernel(float2* __restrict__ tab, int64_t T, int half, double theta) {
  const int64_t n = T * half;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = i / half;
    const int j = (int)(i - p * half);
    const double inv = 1.0 / pow(theta, 2.0 * j / (2.0 * half));
    const double a = (double)p * inv;
    tab[i] = make_float2((float)cos(a), (float)sin(a));
  }
}

// out = s o_swa + (1 - s) out with s = sigmoid(G + bg) (G [T, HD] float)
__global__ void __launch_bounds__(256) gate_mix_kernel(const float* __restrict__ G, const float* __restrict__ bg,
                                                       const bf16* __restrict__ oswa, float* __restrict__ out,
                                                       int64_t T, int HD) {
  const int64_t n = T * HD;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(i % HD);
    const float s = 1.f / (1.f + __expf(-(G[i] + bg[j])));
    out[i] = s * (float)oswa[i] + (1.f - s) * out[i];
  }
}

int64_t hybrid_cap(int64_t T) {
  int64_t c = 64;
  while (c < T) c <<= 1;
  return c;
}

size_t hybrid_extra_bytes(int32_t H, int64_t T, int32_t D) {
  const size_t al = 256, HD = (size_t)H * D, cap = (size_t)hybrid_cap(T);
  return (size_t)T * 3 * HD * 2 + al + (size_t)T * HD * 2 + al + 3 * ((size_t)H * cap * D * 2 + al) +
         (size_t)T * HD * 2 + al + (size_t)T * HD * 4 + al + (size_t)T * (D / 2) * 8 + al + 256;
}
}  // namespace

extern "C" ttt_status e2ttt_hybrid_forward(const void* x, const void* wqkv, const float* bias, const void* wgate,
                                           const float* bgate, float eta_base, float alpha_base, float tau,
                                           float rope_theta, int32_t window, float* W1, float* W2, float* W3,
                                           float* M1, float* M2, float* M3, int32_t Dh, float* out, int32_t H,
                                           int64_t T, int32_t D, int32_t dm, int32_t C, void* stream) {
  using namespace ttt;
  ttt_status r = mixer_check(x, wqkv, bias, eta_base, alpha_base, tau, out, H, T, D, dm, C);
  if (r != TTT_OK) return r;
  if (!wgate || !bgate || ((uintptr_t)wgate & 15) || window < 1 || !(rope_theta > 1.f) || Dh < 0)
    return TTT_ERR_INVALID_ARG;
  // Dh > 0 with W3 and M3 both null: the GELU net (W1 [H, Dh, D], W2 [H, D, Dh])
  const bool gelu = Dh > 0 && !W3 && !M3;
  if (Dh > 0) {
    if ((r = gelu ? gelu_check(W1, W2, M1, M2, Dh) : swiglu_check(W1, W2, W3, M1, M2, M3, Dh)) != TTT_OK) return r;
  } else if (!W1 || !M1 || ((uintptr_t)W1 & 15) || ((uintptr_t)M1 & 15)) {
    return TTT_ERR_INVALID_ARG;
  }
  // one head's slice of a key/value store is addressed with 32-bit offsets
  if ((int64_t)hybrid_cap(T) * D * 2 >= (int64_t(1) << 31)) return TTT_ERR_UNSUPPORTED;
  if ((r = device_present()) != TTT_OK) return r;
  hipStream_t st = (hipStream_t)stream;
  const size_t base = Dh > 0 ? (gelu ? gelu_mixer_work_bytes(H, T, D, Dh, C) : mlp_mixer_work_bytes(H, T, D, Dh, C))
                             : mixer_work_bytes(H, T, D, C);
  CallWork w;
  if ((r = w.alloc(base + hybrid_extra_bytes(H, T, D), st)) != TTT_OK) return r;
  // TTT path: o_TTT into out; its projections P stay at the buffer's start
  if (gelu)
    r = mixer_gelu_run(x, wqkv, bias, eta_base, alpha_base, tau, W1, W2, M1, M2, out, H, T, D, Dh, dm, C, w.get(),
                       stream);
  else if (Dh > 0)
    r = mixer_swiglu_run(x, wqkv, bias, eta_base, alpha_base, tau, W1, W2, W3, M1, M2, M3, out, H, T, D, Dh, dm, C,
                         w.get(), stream);
  else
    r = mixer_linear_run(x, wqkv, bias, eta_base, alpha_base, tau, W1, M1, out, H, T, D, dm, C, w.get(), stream);
  if (r != TTT_OK) return r;
  const int64_t N = 3LL * H * D + 3LL * H, HD = (int64_t)H * D, cap = hybrid_cap(T);
  const float* P = (const float*)(((uintptr_t)w.get() + 255) & ~(uintptr_t)255);
  Carve cv{(((uintptr_t)w.get() + base) + 255) & ~(uintptr_t)255};
  bf16* qkv = cv.take<bf16>((size_t)T * 3 * HD * 2);
  bf16* qr = cv.take<bf16>((size_t)T * HD * 2);
  bf16* ks = cv.take<bf16>((size_t)H * cap * D * 2);
  bf16* vs = cv.take<bf16>((size_t)H * cap * D * 2);
  bf16* vts = cv.take<bf16>((size_t)H * cap * D * 2);
  bf16* oswa = cv.take<bf16>((size_t)T * HD * 2);
  float* G = cv.take<float>((size_t)T * HD * 4);
  float2* tab = cv.take<float2>((size_t)T * (D / 2) * 8);
  hipLaunchKernelGGL(raw_qkv_kernel, dim3(2048), dim3(256), 0, st, P, N, T, (int)(3 * HD), qkv);
  hipLaunchKernelGGL(rope_table_kernel, dim3(1024), dim3(256), 0, st, tab, T, D / 2, (double)rope_theta);
  if (hipGetLastError() != hipSuccess) return TTT_ERR_HIP;
  // the attention reads whole key tiles, so slots the stream never writes
  // (past T - 1, before 0) are read as masked keys: they must hold finite
  // values (0 x NaN is NaN), so the stores start zeroed
  for (bf16* p : {ks, vs, vts})
    if (fill_zero_bytes(p, (size_t)H * cap * D * 2, st) != hipSuccess) return TTT_ERR_HIP;
  if (rope_scatter(DT::BF16, qkv, (int)T, H, H, D, 0, tab, qr, ks, vs, vts, (int)cap, 0, st) != hipSuccess)
    return TTT_ERR_HIP;
  AttnArgs a{};
  a.q = qr;
  a.k = ks;
  a.v = vs;
  a.vt = vts;
  a.o = oswa;
  a.lse = nullptr;
  a.n = (int)T;
  a.H = H;
  a.Hk = H;
  a.dh = D;
  a.cap = (int)cap;
  a.window = (int)std::min<int64_t>(window, T);
  a.pos0 = 0;
  a.scale = 1.f / sqrtf((float)D);
  if (!attn_fwd2_supported(DT::BF16, a)) return TTT_ERR_UNSUPPORTED;
  if (attn_fwd2(DT::BF16, a, st) != hipSuccess) return TTT_ERR_HIP;
  GemmArgs g{};
  g.A = x;
  g.B = wgate;
  g.M = (int)T;
  g.N = (int)HD;
  g.K = dm;
  g.lda = dm;
  g.ldb = dm;
  g.C = G;
  g.ldc = HD;
  g.scale = 1.f;
  if (gemm(DT::BF16, true, true, Epi::STORE_F32, g, st) != hipSuccess) return TTT_ERR_HIP;
  hipLaunchKernelGGL(gate_mix_kernel, dim3(2048), dim3(256), 0, st, G, bgate, oswa, out, T, (int)HD);
  return hipGetLastError() == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}
