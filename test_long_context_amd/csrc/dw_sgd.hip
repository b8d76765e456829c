// Fused fast-weight update of one dynamic SwiGLU block on gfx950: the two
// weight-gradient contractions over the mini-batch's tokens,
//   dW[m, n] = sum_k A[k, m] B[k, n]   (A: output gradients, B: inputs, both
//                                       stored token-major, so neither is
//                                       K-contiguous),
// and the SGD step on the fp32 master W -= lr dW ([P1] "TTT-E2E：端到端测试时
// 训练的长上下文语言建模", section 持续学习框架: W_t = W_{t-1} - alpha grad),
// with the bf16 working copy hi = RNE(W) and low term lo = RNE(W - hi)
// re-derived from the new master, in ONE persistent launch for both products
// of the block (W12 = [gate | up] and W3).
//
// Why a dedicated kernel: with K = b = 1024 the products are short and the
// update moves 12 bytes per parameter, as much time on HBM as the products
// take on the matrix cores. A workgroup that finishes a tile and then runs
// its read-modify-write leaves the matrix cores idle meanwhile, and a wave
// that mixes the update's HBM loads into its K loop waits for HBM latency at
// every K step (one counter tracks all its memory operations). So the
// workgroup's waves are specialised: four MFMA waves compute a 128 x 128
// tile of dW (operands staged through LDS, as in the GEMM family) and hand
// the finished accumulators to an LDS staging tile; four update waves, one
// tile behind, apply the SGD step to the staged tile in 16 row slices, one
// per K step of the MFMA waves' current tile. The update waves request a
// tile's master values a whole tile ahead, so their HBM latency never
// stalls a barrier, and their stores never enter the MFMA waves' counters.
//
// Accumulator layout: the MFMA is fed (inputs, gradients) instead of
// (gradients, inputs), so it produces dW^T blocks; lane l of a 16 x 16 block
// then holds dW row (l % 16), columns 4 (l / 16) .. + 3 -- one 16-byte LDS
// store per block into the row-major staging tile.
#include <algorithm>

#include "gemm_impl.hpp"

namespace ttt {

namespace {

constexpr int DW_BM = 128, DW_BN = 128, DW_BK = 64;  // tile (rows of dW x columns), K step
constexpr int DW_NW = 4;                              // waves: 2 x 2 of 64 x 64

struct DwProblem {
  const bf16* A;  // A[k * lda + m]
  const bf16* B;  // B[k * ldb + n]
  float* W;       // fp32 master [M][ldw]
  bf16* Hi;       // [M][ldw]
  bf16* Lo;       // [M][ldw] or null
  int M, N;
  long lda, ldb, ldw;
  int tm_n, tn_n, tiles;
};

struct DwArgs {
  DwProblem p[2];
  int np, K, total;
  float lr;
};

// Logical tile -> (problem, row tile, column tile): problems back to back,
// inside each a grouped order (8 row tiles share their column panels).
__device__ __forceinline__ void dw_tile(const DwArgs& g, int t, int& q, int& m0, int& n0) {
  q = (g.np > 1 && t >= g.p[0].tiles) ? 1 : 0;
  if (q) t -= g.p[0].tiles;
  const DwProblem& P = g.p[q];
  constexpr int GM = 8;
  const int group = GM * P.tn_n;
  const int gid = t / group;
  const int first = gid * GM;
  const int gsz = min(P.tm_n - first, GM);
  const int in = t - gid * group;
  m0 = (first + in % gsz) * DW_BM;
  n0 = (in / gsz) * DW_BN;
}

// Workgroup w of G (G a multiple of 8) runs on XCD w % 8; each XCD walks a
// contiguous eighth of the tile list, so the workgroups that share an L2 work
// on neighbouring tiles. Returns the logical tile of the i-th visit, or -1.
__device__ __forceinline__ int dw_sched(int total, int w, int G, int i) {
  const int x = w & 7, j = w >> 3, per_xcd = G >> 3;
  const int span = (total + 7) >> 3;
  const int t = x * span + j + i * per_xcd;
  return (j + i * per_xcd < span && t < total) ? t : -1;
}

// buffer resource over an operand (loads past nbytes, capped at the 32-bit
// range, return zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dw_rsrc(const void* p, long nbytes) {
  return make_rsrc(p, nbytes < (long)OOB ? (uint32_t)nbytes : OOB);
}

struct DwEpi {
  float lr;
  // one 16 x 16 block of dW (accumulators a) at master row m, columns n .. n+3
  __device__ __forceinline__ void apply(const DwProblem& P, int m, int n, floatx4 a, floatx4 pre) const {
    const long idx = (long)m * P.ldw + n;
    const floatx4 w = pre - lr * a;
    *(floatx4*)(P.W + idx) = w;
    const bf16x4 hi = cvt4(w);
    *(bf16x4*)(P.Hi + idx) = hi;
    if (P.Lo) *(bf16x4*)(P.Lo + idx) = cvt4(w - upc4(hi));
  }
};

constexpr int DW_SP = DW_BN + 4;  // staging row pitch (floats): row r starts at bank 4 r

__global__ void __launch_bounds__(2 * DW_NW * 64, 2) dw_sgd_kernel(DwArgs g) {
  __shared__ __attribute__((aligned(1024))) bf16 As[2][DW_BM * DW_BK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs[2][DW_BN * DW_BK];
  __shared__ __attribute__((aligned(16))) float S[DW_BM * DW_SP];  // finished tile, row-major
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const bool mw = wid < DW_NW;  // MFMA wave (else update wave)
  const DwEpi epi{g.lr};
  const int nk = (g.K + DW_BK - 1) / DW_BK;

  // MFMA waves: 2 x 2 of 64 x 64
  const int wm = ((wid & 3) >> 1) * 64, wn = (wid & 1) * 64;
  const int fr = lane & 15, fg = lane >> 4;
  // update waves: slice e is rows 8 e .. 8 e + 7; wave u takes rows 8 e + 2 u,
  // + 1 (one per half-wave), 4 columns per lane
  const int u = wid - DW_NW;
  const int urow = 2 * u + (lane >> 5), ucol = 4 * (lane & 31);

  // Both roles walk the same tiles and run the same barrier sequence per
  // tile: B0, one per K step, X, H.
  if (mw) {
    TrDmaLoader<DW_BM, DW_NW> la;
    TrDmaLoader<DW_BN, DW_NW> lb;
    for (int i = 0;; ++i) {
      const int t = dw_sched(g.total, blockIdx.x, gridDim.x, i);
      if (t < 0) break;
      int q, m0, n0;
      dw_tile(g, t, q, m0, n0);
      const DwProblem& P = g.p[q];
      const __amdgpu_buffer_rsrc_t ra = dw_rsrc(P.A, (long)g.K * P.lda * 2);
      const __amdgpu_buffer_rsrc_t rb = dw_rsrc(P.B, (long)g.K * P.ldb * 2);
      if (nk > 0) {
        la.issue(ra, P.lda, m0, P.M, 0, g.K, As[0], wid, lane);
        lb.issue(rb, P.ldb, n0, P.N, 0, g.K, Bs[0], wid, lane);
      }
      floatx4 acc[4][4];  // [column block j][row block x]
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[j][x] = floatx4{0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // B0: stage 0 landed
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        Frag8<bf16> fa[2][4], fb[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            fb[s][x].v = ld_tr8<DW_BN>(Bs[cur], wn + 16 * x, s * 32, lane);
            fa[s][x].v = ld_tr8<DW_BM>(As[cur], wm + 16 * x, s * 32, lane);
          }
        if (kt + 1 < nk) {
          la.issue(ra, P.lda, m0, P.M, (kt + 1) * DW_BK, g.K, As[cur ^ 1], wid, lane);
          lb.issue(rb, P.ldb, n0, P.N, (kt + 1) * DW_BK, g.K, Bs[cur ^ 1], wid, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int x = 0; x < 4; ++x) mma16(acc[j][x], fb[s][j], fa[s][x]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // K step kt
      }
      __syncthreads();  // X: the update waves are done reading the staged tile
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int x = 0; x < 4; ++x)
          *(floatx4*)(S + (wm + 16 * x + fr) * DW_SP + wn + 16 * j + 4 * fg) = acc[j][x];
      __syncthreads();  // H: this tile staged
    }
  } else {
    floatx4 ma[16], mb[16];          // masters of the staged tile / of the tile in flight
    int pq = -1, pm0 = 0, pn0 = 0;   // the staged tile
    // update of slice e of the staged tile with master values v
    auto slice = [&](int e, floatx4 v) {
      const DwProblem& P = g.p[pq];
      const int r = 8 * e + urow;
      const int m = pm0 + r, n = pn0 + ucol;
      if (m < P.M && n < P.N) epi.apply(P, m, n, *(const floatx4*)(S + r * DW_SP + ucol), v);
    };
    auto slice_sw = [&](int e) {
      switch (e) {
#define DW_CASE(E) \
  case E:          \
    slice(E, ma[E]); \
    break;
        DW_CASE(0) DW_CASE(1) DW_CASE(2) DW_CASE(3) DW_CASE(4) DW_CASE(5) DW_CASE(6) DW_CASE(7)
        DW_CASE(8) DW_CASE(9) DW_CASE(10) DW_CASE(11) DW_CASE(12) DW_CASE(13) DW_CASE(14) DW_CASE(15)
#undef DW_CASE
        default: break;
      }
    };
    for (int i = 0;; ++i) {
      const int t = dw_sched(g.total, blockIdx.x, gridDim.x, i);
      if (t < 0) break;
      int q, m0, n0;
      dw_tile(g, t, q, m0, n0);
      const DwProblem& P = g.p[q];
      // masters of the tile staged last time were requested a tile ago
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int e = 0; e < 16; ++e) ma[e] = mb[e];
      // request this tile's masters (used once it is staged, a tile from now)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 8 * e + urow, n = n0 + ucol;
        if (m < P.M && n < P.N) mb[e] = *(const floatx4*)(P.W + (long)m * P.ldw + n);
      }
      __syncthreads();  // B0
      for (int kt = 0; kt < nk; ++kt) {
        if (pq >= 0 && kt < 16) slice_sw(kt);
        __syncthreads();  // K step kt
      }
      if (pq >= 0)
        for (int e = nk; e < 16; ++e) slice_sw(e);
      __syncthreads();  // X
      __syncthreads();  // H
      pq = q;
      pm0 = m0;
      pn0 = n0;
    }
    // the last staged tile
    if (pq >= 0) {
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int e = 0; e < 16; ++e) slice(e, mb[e]);
    }
  }
}

DwProblem dw_problem(const DwUpdate& u) {
  DwProblem p{};
  p.A = (const bf16*)u.A;
  p.B = (const bf16*)u.B;
  p.W = u.W;
  p.Hi = (bf16*)u.Hi;
  p.Lo = (bf16*)u.Lo;
  p.M = u.M;
  p.N = u.N;
  p.lda = u.lda;
  p.ldb = u.ldb;
  p.ldw = u.ldw;
  p.tm_n = (u.M + DW_BM - 1) / DW_BM;
  p.tn_n = (u.N + DW_BN - 1) / DW_BN;
  p.tiles = p.tm_n * p.tn_n;
  return p;
}

int cu_count() {
  static thread_local int dev = -1, cus = 0;
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) return 256;
  if (d != dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || n <= 0) n = 256;
    dev = d;
    cus = n;
  }
  return cus;
}

}  // namespace

bool dw_sgd_supported(const DwUpdate& u) {
  return u.M > 0 && u.N > 0 && u.M % 16 == 0 && u.N % 16 == 0 && u.lda % 8 == 0 && u.ldb % 8 == 0 &&
         u.ldw % 4 == 0 && u.ldw >= u.N && u.lda >= u.M && u.ldb >= u.N && ((uintptr_t)u.A & 15) == 0 &&
         ((uintptr_t)u.B & 15) == 0 && ((uintptr_t)u.W & 15) == 0 && ((uintptr_t)u.Hi & 7) == 0 &&
         ((uintptr_t)u.Lo & 7) == 0 && u.Hi != nullptr;
}

hipError_t dw_sgd(const DwUpdate* u, int n, int K, float lr, int grid, hipStream_t st) {
  if (n < 1 || n > 2 || K < 0) return hipErrorInvalidValue;
  DwArgs g{};
  g.np = n;
  g.K = K;
  g.lr = lr;
  g.total = 0;
  for (int i = 0; i < n; ++i) {
    if (!dw_sgd_supported(u[i])) return hipErrorInvalidValue;
    g.p[i] = dw_problem(u[i]);
    g.total += g.p[i].tiles;
  }
  if (g.total == 0) return hipSuccess;
  // one workgroup per CU (132 KB of LDS), a multiple of 8 (one share per XCD)
  int G = grid > 0 ? grid : cu_count();
  G = std::max(8, std::min(G, (g.total + 7) / 8 * 8));
  G = (G + 7) / 8 * 8;
  hipLaunchKernelGGL(dw_sgd_kernel, dim3(G), dim3(2 * DW_NW * 64), 0, st, g);
  return hipGetLastError();
}

}  // namespace ttt
