// GEMM family on gfx950 MFMA: the projections, SwiGLU MLP forward/backward,
// lm_head, the dX products of the backward and the dW = X^T dH contractions
// with the fused fp32 fast-weight SGD update in their epilogue.
//
// Structure: a workgroup owns a BM x BN output tile, split into waves of
// WM x WN; the K loop stages BK-wide slices of A and B through LDS in a
// K-contiguous layout (rows of BK + 8 elements, double-buffered), so that
// every lane reads its 8-element MFMA fragment with one 16-byte LDS load.
// Operands whose K dimension is not contiguous in HBM (the token-major
// operands of dW, the weight operand of dX) are loaded as 8 x 8 blocks and
// transposed in registers on the way into LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

template <typename T>
struct V8 {
  Frag8<T> r[8];
};

// Grouped, XCD-aware tile order: consecutive hardware workgroup ids are
// dealt round-robin over the 8 XCDs; remap so that each XCD receives a
// contiguous range of logical tiles, then walk tiles in groups of GM tile
// rows so that co-resident workgroups share A and B panels in L2.
__device__ __forceinline__ void tile_coords(int bid, int tm_n, int tn_n, int& tm, int& tn) {
  const int nt = tm_n * tn_n;
  if ((nt & 7) == 0) bid = (bid & 7) * (nt >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int group = GM * tn_n;
  const int gid = bid / group;
  const int first = gid * GM;
  const int gsz = min(tm_n - first, GM);
  const int in = bid - gid * group;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <typename T, int ROWS, int BK, int NT, bool KMAJ>
struct TileLoader {
  // K-major: ROWS x BK tile as 8-element vectors.
  // Row-major-in-K (not KMAJ): (BK / 8) x (ROWS / 8) blocks of 8 x 8.
  static constexpr int NV = KMAJ ? (ROWS * BK / 8) : ((BK / 8) * (ROWS / 8));
  static constexpr int PER = (NV + NT - 1) / NT;
  static constexpr int REGS = KMAJ ? PER : PER * 8;
  Frag8<T> r[REGS];

  __device__ __forceinline__ void load(const T* __restrict__ P, long ld, int row0, int nrows,
                                       int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * NT;
      if (KMAJ) {
        const int row = v / (BK / 8), kv = v % (BK / 8);
        const int gr = row0 + row, gk = k0 + kv * 8;
        if (v < NV && gr < nrows && gk < kend) ld8(r[i], P + (long)gr * ld + gk);
        else zero8(r[i]);
      } else {
        const int kb = v / (ROWS / 8), rb = v % (ROWS / 8);
        const int gr = row0 + rb * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gk = k0 + kb * 8 + j;
          if (v < NV && gr < nrows && gk < kend) ld8(r[i * 8 + j], P + (long)gk * ld + gr);
          else zero8(r[i * 8 + j]);
        }
      }
    }
  }

  template <int LDS>
  __device__ __forceinline__ void store(T* __restrict__ S, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * NT;
      if (v >= NV) break;
      if (KMAJ) {
        const int row = v / (BK / 8), kv = v % (BK / 8);
        st8(S + row * LDS + kv * 8, r[i]);
      } else {
        const int kb = v / (ROWS / 8), rb = v % (ROWS / 8);
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) {
          Frag8<T> t;
#pragma unroll
          for (int j = 0; j < 8; ++j) eset<T>(t, j, eget<T>(r[i * 8 + j], mm));
          st8(S + (rb * 8 + mm) * LDS + kb * 8, t);
        }
      }
    }
  }
};

template <typename T, int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(GemmArgs g) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int LDS = BK + 8;
  constexpr int FM = WM / 16, FN = WN / 16;
  __shared__ __attribute__((aligned(16))) T As[2][BM * LDS];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDS];
  // low part of B for the two-term split (one byte when unused)
  __shared__ __attribute__((aligned(16))) T Bs2[SPLITB ? 2 : 1][SPLITB ? BN * LDS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm0 = (wid / NWN) * WM;
  const int wn0 = (wid % NWN) * WN;

  const int tm_n = (g.M + BM - 1) / BM, tn_n = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tm_n, tn_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  int kbeg = 0, kend = g.K;
  if (g.kchunk > 0) {
    kbeg = blockIdx.z * g.kchunk;
    kend = min(g.K, kbeg + g.kchunk);
  }
  const T* __restrict__ A = (const T*)g.A;
  const T* __restrict__ B = (const T*)g.B;

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0, 0, 0, 0};

  TileLoader<T, BM, BK, NT, AK> la;
  TileLoader<T, BN, BK, NT, BKM> lb;
  TileLoader<T, SPLITB ? BN : 8, BK, NT, BKM> lb2;
  const T* __restrict__ B2 = (const T*)g.B2;
  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    la.load(A, g.lda, m0, g.M, kbeg, kend, tid);
    lb.load(B, g.ldb, n0, g.N, kbeg, kend, tid);
    if constexpr (SPLITB) lb2.load(B2, g.ldb, n0, g.N, kbeg, kend, tid);
    la.template store<LDS>(As[0], tid);
    lb.template store<LDS>(Bs[0], tid);
    if constexpr (SPLITB) lb2.template store<LDS>(Bs2[0], tid);
  }
  __syncthreads();

  const int fr = lane & 15;
  const int fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      const int k0 = kbeg + (kt + 1) * BK;
      la.load(A, g.lda, m0, g.M, k0, kend, tid);
      lb.load(B, g.ldb, n0, g.N, k0, kend, tid);
      if constexpr (SPLITB) lb2.load(B2, g.ldb, n0, g.N, k0, kend, tid);
    }
    const T* as = As[cur];
    const T* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      Frag8<T> af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) ld8(af[i], as + (wm0 + i * 16 + fr) * LDS + kk + fk);
#pragma unroll
      for (int j = 0; j < FN; ++j) ld8(bfr[j], bs + (wn0 + j * 16 + fr) * LDS + kk + fk);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma16(acc[i][j], af[i], bfr[j]);
      if constexpr (SPLITB) {
#pragma unroll
        for (int j = 0; j < FN; ++j) ld8(bfr[j], Bs2[cur] + (wn0 + j * 16 + fr) * LDS + kk + fk);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mma16(acc[i][j], af[i], bfr[j]);
      }
    }
    if (kt + 1 < nk) {
      la.template store<LDS>(As[cur ^ 1], tid);
      lb.template store<LDS>(Bs[cur ^ 1], tid);
      if constexpr (SPLITB) lb2.template store<LDS>(Bs2[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------- epilogue
  const int er = (lane >> 4) * 4;
  if constexpr (EPI == (int)Epi::SWIGLU) {
    static_assert(FN % 2 == 0, "SWIGLU needs gate/up tile pairs");
    T* H12 = (T*)g.C;
    T* Hm = (T*)g.C2;
    const long ldm = g.N / 2;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; j += 2) {
        const int na = n0 + wn0 + j * 16 + fr;
        const int jh = (n0 + wn0 + j * 16) / 2 + fr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm0 + i * 16 + er + r;
          if (m < g.M && na < g.N) {
            const float a = acc[i][j][r], c = acc[i][j + 1][r];
            if (H12) {
              H12[(long)m * g.ldc + na] = from_f<T>(a);
              H12[(long)m * g.ldc + na + 16] = from_f<T>(c);
            }
            Hm[(long)m * ldm + jh] = from_f<T>(silu_f(a) * c);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn0 + j * 16 + fr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm0 + i * 16 + er + r;
          if (m >= g.M || n >= g.N) continue;
          const float a = acc[i][j][r];
          const long idx = (long)m * g.ldc + n;
          if constexpr (EPI == (int)Epi::STORE) {
            ((T*)g.C)[idx] = from_f<T>(a * g.scale);
          } else if constexpr (EPI == (int)Epi::STORE_F32) {
            ((float*)g.C)[idx] = a;
          } else if constexpr (EPI == (int)Epi::ADD_F32) {
            ((float*)g.C)[idx] += a;
          } else if constexpr (EPI == (int)Epi::PARTIAL) {
            ((float*)g.C)[(long)blockIdx.z * g.M * g.ldc + idx] = a;
          } else if constexpr (EPI == (int)Epi::SGD) {
            float* W = (float*)g.C;
            const float w = W[idx] - g.scale * a;
            W[idx] = w;
            if (g.C2 != g.C) {
              const T hi = from_f<T>(w);
              ((T*)g.C2)[idx] = hi;
              if (g.C3) ((T*)g.C3)[idx] = from_f<T>(w - to_f(hi));
            }
          } else if constexpr (EPI == (int)Epi::SWIGLU_BWD) {
            // n indexes the hidden unit j; its gate/up columns in the
            // 16-interleaved layout are (j / 16) * 32 + j % 16 and + 16.
            const T* X = (const T*)g.X;
            T* D = (T*)g.C;
            const long ca = (long)m * g.ldc + (n >> 4) * 32 + (n & 15);
            const float av = to_f(X[ca]), cv = to_f(X[ca + 16]);
            const float sg = sigm_f(av);
            D[ca] = from_f<T>(a * cv * sg * (1.0f + av * (1.0f - sg)));
            D[ca + 16] = from_f<T>(a * av * sg);
          }
        }
      }
  }
}

// ------------------------------------------------------------------ dispatch
template <typename T, int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
static hipError_t launch(const GemmArgs& g, hipStream_t st) {
  const int tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  int splits = 1;
  if (g.kchunk > 0) splits = (g.K + g.kchunk - 1) / g.kchunk;
  dim3 grid(tm * tn, 1, splits);
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, AK, BKM, EPI, SPLITB>), grid, dim3(NT), 0, st, g);
  return hipGetLastError();
}

template <typename T, bool AK, bool BKM, int EPI, bool SPLITB = false>
static hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    return launch<T, 128, 128, 32, 64, 64, AK, BKM, EPI, SPLITB>(g, st);
  } else {
    return launch<T, 64, 64, 32, 32, 32, AK, BKM, EPI, SPLITB>(g, st);
  }
}

template <typename T, bool AK, bool BKM>
static hipError_t by_epi(Epi e, const GemmArgs& g, hipStream_t st) {
  switch (e) {
    case Epi::STORE: return launch_cfg<T, AK, BKM, (int)Epi::STORE>(g, st);
    case Epi::STORE_F32: return launch_cfg<T, AK, BKM, (int)Epi::STORE_F32>(g, st);
    case Epi::ADD_F32: return launch_cfg<T, AK, BKM, (int)Epi::ADD_F32>(g, st);
    case Epi::SWIGLU: return launch_cfg<T, AK, BKM, (int)Epi::SWIGLU>(g, st);
    case Epi::SWIGLU_BWD: return launch_cfg<T, AK, BKM, (int)Epi::SWIGLU_BWD>(g, st);
    case Epi::SGD: return launch_cfg<T, AK, BKM, (int)Epi::SGD>(g, st);
    case Epi::PARTIAL: return launch_cfg<T, AK, BKM, (int)Epi::PARTIAL>(g, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t by_layout(bool ak, bool bk, Epi e, const GemmArgs& g, hipStream_t st) {
  if (ak && bk) return by_epi<T, true, true>(e, g, st);
  if (ak && !bk) return by_epi<T, true, false>(e, g, st);
  if (!ak && !bk) return by_epi<T, false, false>(e, g, st);
  return by_epi<T, false, true>(e, g, st);
}

int gemm_k_granule(DT) { return 32; }

hipError_t gemm(DT dt, bool a_kmajor, bool b_kmajor, Epi epi, const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.B2) {
    // two-term split of B: forward products with the fast weights (bf16, NT)
    if (dt != DT::BF16 || !a_kmajor || !b_kmajor) return hipErrorInvalidValue;
    if (epi == Epi::SWIGLU) return launch_cfg<bf16, true, true, (int)Epi::SWIGLU, true>(g, st);
    if (epi == Epi::ADD_F32) return launch_cfg<bf16, true, true, (int)Epi::ADD_F32, true>(g, st);
    return hipErrorInvalidValue;
  }
  if (dt == DT::BF16) return by_layout<bf16>(a_kmajor, b_kmajor, epi, g, st);
  return by_layout<float>(a_kmajor, b_kmajor, epi, g, st);
}

}  // namespace ttt
