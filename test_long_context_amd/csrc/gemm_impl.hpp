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
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

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

// Buffer resource over a whole operand: loads at byte offsets >= nbytes
// return zero (hardware range check), so tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes, 0x00020000);
}
static constexpr uint32_t OOB = 0xFFFFFFF0u;

template <typename T>
__device__ __forceinline__ void bld8(Frag8<T>& f, __amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ void bld8<bf16>(Frag8<bf16>& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  f.v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <>
__device__ __forceinline__ void bld8<float>(Frag8<float>& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int i4 __attribute__((ext_vector_type(4)));
  const uint32_t o2 = off == OOB ? OOB : off + 16;
  f.lo = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  f.hi = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, o2, 0, 0));
}

template <typename T, int ROWS, int BK, int NT, bool KMAJ>
struct TileLoader {
  // K-major: ROWS x BK tile as 8-element vectors.
  // Row-major-in-K (not KMAJ): (BK / 8) x (ROWS / 8) blocks of 8 x 8,
  // transposed in registers on the way into LDS.
  static constexpr int NV = KMAJ ? (ROWS * BK / 8) : ((BK / 8) * (ROWS / 8));
  static constexpr int PER = (NV + NT - 1) / NT;
  static constexpr int REGS = KMAJ ? PER : PER * 8;
  Frag8<T> r[REGS];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, long ld, int row0, int nrows, int k0,
                                       int kend, int tid) {
    constexpr int ES = sizeof(T);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * NT;
      if (KMAJ) {
        const int row = v / (BK / 8), kv = v % (BK / 8);
        const int gr = row0 + row, gk = k0 + kv * 8;
        const bool ok = (NV % NT == 0 || v < NV) && gr < nrows && gk < kend;
        bld8<T>(r[i], rs, ok ? (uint32_t)(((long)gr * ld + gk) * ES) : OOB);
      } else {
        const int kb = v / (ROWS / 8), rb = v % (ROWS / 8);
        const int gr = row0 + rb * 8;
        const bool okr = (NV % NT == 0 || v < NV) && gr < nrows;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gk = k0 + kb * 8 + j;
          const bool ok = okr && gk < kend;
          bld8<T>(r[i * 8 + j], rs, ok ? (uint32_t)(((long)gk * ld + gr) * ES) : OOB);
        }
      }
    }
  }

  template <int LDS>
  __device__ __forceinline__ void store(T* __restrict__ S, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * NT;
      if (NV % NT != 0 && v >= NV) break;
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

// Writes a wave's FM x FN accumulator tiles (origin (mw, nw)) per EPI.
template <typename T, int FM, int FN, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, floatx4 (&acc)[FM][FN], int mw, int nw,
                                              int lane) {
  const int fr = lane & 15;
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
        const int na = nw + j * 16 + fr;
        const int jh = (nw + j * 16) / 2 + fr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mw + i * 16 + er + r;
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
        const int n = nw + j * 16 + fr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mw + i * 16 + er + r;
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

template <typename T, int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(GemmArgs g) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int LDS = BK + 8;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int KS = BK / 32;  // MFMA k-steps per LDS tile
  __shared__ __attribute__((aligned(16))) T As[2][BM * LDS];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDS];
  // low part of B for the two-term split (one element when unused)
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
  constexpr int ES = sizeof(T);
  // operand extents in bytes (rows x leading dimension)
  const long a_rows = AK ? g.M : g.K, b_rows = BKM ? g.N : g.K;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)min((long)OOB, a_rows * g.lda * ES));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)min((long)OOB, b_rows * g.ldb * ES));
  const __amdgpu_buffer_rsrc_t rb2 =
      make_rsrc(SPLITB ? g.B2 : g.B, (uint32_t)min((long)OOB, b_rows * g.ldb * ES));

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0, 0, 0, 0};

  TileLoader<T, BM, BK, NT, AK> la;
  TileLoader<T, BN, BK, NT, BKM> lb;
  TileLoader<T, SPLITB ? BN : 8, BK, NT, BKM> lb2;
  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    la.load(ra, g.lda, m0, g.M, kbeg, kend, tid);
    lb.load(rb, g.ldb, n0, g.N, kbeg, kend, tid);
    if constexpr (SPLITB) lb2.load(rb2, g.ldb, n0, g.N, kbeg, kend, tid);
    la.template store<LDS>(As[0], tid);
    lb.template store<LDS>(Bs[0], tid);
    if constexpr (SPLITB) lb2.template store<LDS>(Bs2[0], tid);
  }
  __syncthreads();

  const int fr = lane & 15;
  const int fk = (lane >> 4) * 8;
  // fragments double-buffered across k-steps
  Frag8<T> af[2][FM], bfr[2][FN], bf2[SPLITB ? 2 : 1][SPLITB ? FN : 1];
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      const int k0 = kbeg + (kt + 1) * BK;
      la.load(ra, g.lda, m0, g.M, k0, kend, tid);
      lb.load(rb, g.ldb, n0, g.N, k0, kend, tid);
      if constexpr (SPLITB) lb2.load(rb2, g.ldb, n0, g.N, k0, kend, tid);
    }
    const T* as = As[cur];
    const T* bs = Bs[cur];
#pragma unroll
    for (int i = 0; i < FM; ++i) ld8(af[0][i], as + (wm0 + i * 16 + fr) * LDS + fk);
#pragma unroll
    for (int j = 0; j < FN; ++j) ld8(bfr[0][j], bs + (wn0 + j * 16 + fr) * LDS + fk);
    if constexpr (SPLITB) {
#pragma unroll
      for (int j = 0; j < FN; ++j) ld8(bf2[0][j], Bs2[cur] + (wn0 + j * 16 + fr) * LDS + fk);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int p = s & 1;
      if (s + 1 < KS) {
        const int kk = (s + 1) * 32 + fk;
#pragma unroll
        for (int i = 0; i < FM; ++i) ld8(af[p ^ 1][i], as + (wm0 + i * 16 + fr) * LDS + kk);
#pragma unroll
        for (int j = 0; j < FN; ++j) ld8(bfr[p ^ 1][j], bs + (wn0 + j * 16 + fr) * LDS + kk);
        if constexpr (SPLITB) {
#pragma unroll
          for (int j = 0; j < FN; ++j) ld8(bf2[p ^ 1][j], Bs2[cur] + (wn0 + j * 16 + fr) * LDS + kk);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma16(acc[i][j], af[p][i], bfr[p][j]);
      if constexpr (SPLITB) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mma16(acc[i][j], af[p][i], bf2[p][j]);
      }
    }
    if (kt + 1 < nk) {
      la.template store<LDS>(As[cur ^ 1], tid);
      lb.template store<LDS>(Bs[cur ^ 1], tid);
      if constexpr (SPLITB) lb2.template store<LDS>(Bs2[cur ^ 1], tid);
    }
    __syncthreads();
  }

  gemm_epilogue<T, FM, FN, EPI>(g, acc, m0 + wm0, n0 + wn0, lane);
}

// =================================================================== bf16
// bf16 kernel: K tile of 64, LDS rows of 64 elements without padding whose
// logical 16-byte vector v is stored at physical slot v ^ (row & 7) (XOR
// swizzle; conflict-free for the 16-row fragment reads). K-major operands go
// global -> LDS by buffer_load ... lds (no VGPR staging; the hardware puts
// lane l's 16 bytes at base + 16 l, so each lane fetches the global vector
// that belongs in its swizzled slot); operands with the other orientation
// are staged through registers and transposed in 8 x 8 blocks.
__device__ __forceinline__ int swz64(int r, int v) { return r * 64 + ((v ^ (r & 7)) << 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int ROWS, int NW>
struct DmaLoader {
  static constexpr int NI = ROWS / 8;  // wave instructions per tile (8 rows each)
  static constexpr int PER = (NI + NW - 1) / NW;
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, long ld, int row0, int nrows, int k0,
                                        int kend, bf16* tile, int wid, int lane) const {
    const int rl = lane >> 3, p = lane & 7;
    const int kv = p ^ rl;  // instruction rows are 8-aligned, so row & 7 == rl
    const int gk = k0 + kv * 8;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = wid + i * NW;
      if (NI % NW != 0 && j >= NI) break;
      const int gr = row0 + j * 8 + rl;
      const uint32_t off = (gr < nrows && gk < kend) ? (uint32_t)(((long)gr * ld + gk) * 2) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(tile + j * 8 * 64), 16, off, 0, 0, 0);
    }
  }
};

template <int ROWS, int NT>
struct StageLoader {  // operand element (row m, k) at P[k * ld + m]
  static constexpr int NB = 8 * (ROWS / 8);  // 8 x 8 blocks per 64-wide K tile
  static constexpr int PER = (NB + NT - 1) / NT;
  Frag8<bf16> r[PER * 8];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, long ld, int row0, int nrows, int k0,
                                       int kend, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = tid + i * NT;
      const int kb = b / (ROWS / 8), rb = b % (ROWS / 8);
      const int gr = row0 + rb * 8;
      const bool okr = (NB % NT == 0 || b < NB) && gr < nrows;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        bld8<bf16>(r[i * 8 + j], rs, (okr && gk < kend) ? (uint32_t)(((long)gk * ld + gr) * 2) : OOB);
      }
    }
  }
  __device__ __forceinline__ void store(bf16* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = tid + i * NT;
      if (NB % NT != 0 && b >= NB) break;
      const int kb = b / (ROWS / 8), rb = b % (ROWS / 8);
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) {
        Frag8<bf16> t;
#pragma unroll
        for (int j = 0; j < 8; ++j) t.v[j] = r[i * 8 + j].v[mm];
        const int row = rb * 8 + mm;
        st8(tile + swz64(row, kb), t);
      }
    }
  }
};

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_bf16_kernel(GemmArgs g) {
  constexpr int NWN = BN / WN;
  constexpr int NW = (BM / WM) * NWN;
  constexpr int NT = NW * 64;
  constexpr int BK = 64;
  constexpr int FM = WM / 16, FN = WN / 16;
  __shared__ __attribute__((aligned(1024))) bf16 As[2][BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs[2][BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 Cs[SPLITB ? 2 : 1][SPLITB ? BN * BK : 8];

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
  const long a_rows = AK ? g.M : g.K, b_rows = BKM ? g.N : g.K;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, (uint32_t)min((long)OOB, a_rows * g.lda * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, (uint32_t)min((long)OOB, b_rows * g.ldb * 2));
  const __amdgpu_buffer_rsrc_t rb2 = make_rsrc(SPLITB ? g.B2 : g.B, (uint32_t)min((long)OOB, b_rows * g.ldb * 2));

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0, 0, 0, 0};

  DmaLoader<BM, NW> da;
  DmaLoader<BN, NW> db;
  StageLoader<AK ? 8 : BM, NT> sa;
  StageLoader<BKM ? 8 : BN, NT> sb;
  const int nk = (kend - kbeg + BK - 1) / BK;
  auto issue = [&](int kt, int buf) {
    const int k0 = kbeg + kt * BK;
    if constexpr (AK) da.issue(ra, g.lda, m0, g.M, k0, kend, As[buf], wid, lane);
    else sa.load(ra, g.lda, m0, g.M, k0, kend, tid);
    if constexpr (BKM) {
      db.issue(rb, g.ldb, n0, g.N, k0, kend, Bs[buf], wid, lane);
      if constexpr (SPLITB) db.issue(rb2, g.ldb, n0, g.N, k0, kend, Cs[buf], wid, lane);
    } else {
      sb.load(rb, g.ldb, n0, g.N, k0, kend, tid);
    }
  };
  auto stage_store = [&](int buf) {
    if constexpr (!AK) sa.store(As[buf], tid);
    if constexpr (!BKM) sb.store(Bs[buf], tid);
  };
  if (nk > 0) {
    issue(0, 0);
    stage_store(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int fr = lane & 15;
  const int fv = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // 1. every fragment of this K tile (both 32-wide steps) ...
    Frag8<bf16> af[2][FM], bfr[2][FN], bf2[SPLITB ? 2 : 1][SPLITB ? FN : 1];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int v = s * 4 + fv;
#pragma unroll
      for (int i = 0; i < FM; ++i) ld8(af[s][i], As[cur] + swz64(wm0 + i * 16 + fr, v));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        ld8(bfr[s][j], Bs[cur] + swz64(wn0 + j * 16 + fr, v));
        if constexpr (SPLITB) ld8(bf2[s][j], Cs[cur] + swz64(wn0 + j * 16 + fr, v));
      }
    }
    // 2. ... then the next tile's loads into the other stage (no LDS read of
    //    this iteration follows them, so nothing waits on them before the MFMAs)
    if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
    // 3. the products
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma16(acc[i][j], af[s][i], bfr[s][j]);
      if constexpr (SPLITB) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mma16(acc[i][j], af[s][i], bf2[s][j]);
      }
    }
    if (kt + 1 < nk) stage_store(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  gemm_epilogue<bf16, FM, FN, EPI>(g, acc, m0 + wm0, n0 + wn0, lane);
}

// ------------------------------------------------------------------ launch
template <typename T, int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
static hipError_t gemm_launch(const GemmArgs& g, hipStream_t st) {
  const int tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  int splits = 1;
  if (g.kchunk > 0) splits = (g.K + g.kchunk - 1) / g.kchunk;
  dim3 grid(tm * tn, 1, splits);
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, AK, BKM, EPI, SPLITB>), grid, dim3(NT), 0, st, g);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
static hipError_t gemm_bf16_launch(const GemmArgs& g, hipStream_t st) {
  const int tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  int splits = 1;
  if (g.kchunk > 0) splits = (g.K + g.kchunk - 1) / g.kchunk;
  dim3 grid(tm * tn, 1, splits);
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, AK, BKM, EPI, SPLITB>), grid, dim3(NT), 0, st, g);
  return hipGetLastError();
}

// Tile configurations (bf16): 1 = 128x128 (4 waves of 64x64), 2 = 256x128
// (4 waves of 128x64), 3 = 256x128 (8 waves of 64x64), 4 = 256x256 (4 waves
// of 128x128), 5 = 256x256 (8 waves of 128x64), 6 = 128x256 (4 waves of
// 64x128); K tile 64. fp32 always uses 64x64x32 (waves of 32x32).
template <typename T, bool AK, bool BKM, int EPI, bool SPLITB>
static hipError_t gemm_cfg(int cfg, const GemmArgs& g, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    switch (cfg) {
      case 1: return gemm_bf16_launch<128, 128, 64, 64, AK, BKM, EPI, SPLITB>(g, st);
      case 2: return gemm_bf16_launch<256, 128, 128, 64, AK, BKM, EPI, SPLITB>(g, st);
      case 3: return gemm_bf16_launch<256, 128, 64, 64, AK, BKM, EPI, SPLITB>(g, st);
      // (the two-term split needs a third LDS tile: 256 x 256 does not fit)
      case 4:
        if constexpr (SPLITB) return gemm_bf16_launch<256, 128, 128, 64, AK, BKM, EPI, SPLITB>(g, st);
        else return gemm_bf16_launch<256, 256, 128, 128, AK, BKM, EPI, SPLITB>(g, st);
      case 5:
        if constexpr (SPLITB) return gemm_bf16_launch<256, 128, 64, 64, AK, BKM, EPI, SPLITB>(g, st);
        else return gemm_bf16_launch<256, 256, 128, 64, AK, BKM, EPI, SPLITB>(g, st);
      case 6: return gemm_bf16_launch<128, 256, 64, 128, AK, BKM, EPI, SPLITB>(g, st);
    }
    return hipErrorInvalidValue;
  } else {
    return gemm_launch<T, 64, 64, 32, 32, 32, AK, BKM, EPI, SPLITB>(g, st);
  }
}

template <typename T, bool AK, bool BKM>
static hipError_t gemm_by_epi(Epi e, int cfg, const GemmArgs& g, hipStream_t st) {
  switch (e) {
    case Epi::STORE: return gemm_cfg<T, AK, BKM, (int)Epi::STORE, false>(cfg, g, st);
    case Epi::STORE_F32: return gemm_cfg<T, AK, BKM, (int)Epi::STORE_F32, false>(cfg, g, st);
    case Epi::ADD_F32: return gemm_cfg<T, AK, BKM, (int)Epi::ADD_F32, false>(cfg, g, st);
    case Epi::SWIGLU: return gemm_cfg<T, AK, BKM, (int)Epi::SWIGLU, false>(cfg, g, st);
    case Epi::SWIGLU_BWD: return gemm_cfg<T, AK, BKM, (int)Epi::SWIGLU_BWD, false>(cfg, g, st);
    case Epi::SGD: return gemm_cfg<T, AK, BKM, (int)Epi::SGD, false>(cfg, g, st);
    case Epi::PARTIAL: return gemm_cfg<T, AK, BKM, (int)Epi::PARTIAL, false>(cfg, g, st);
  }
  return hipErrorInvalidValue;
}

// per-layout entry points (one translation unit each)
hipError_t gemm_nt(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);
hipError_t gemm_nn(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);
hipError_t gemm_tn(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);
hipError_t gemm_tt(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);

}  // namespace ttt
