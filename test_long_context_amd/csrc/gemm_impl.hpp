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
// transposed in registers on the way into LDS by the fp32 kernel; the bf16
// kernel keeps them in their HBM orientation in LDS and transposes on the
// fragment reads instead.
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

// Batched launches (grid.y = batch): the view of product blockIdx.y, each
// operand pointer advanced by its stride times the element size it has
// under this epilogue (A, B, B2, C3 and X are T; C and C2 per epilogue).
template <typename T, int EPI>
__device__ __forceinline__ GemmArgs batch_view(const GemmArgs& g0) {
  constexpr long TS = sizeof(T);
  constexpr long CS = (EPI == (int)Epi::STORE || EPI == (int)Epi::SWIGLU || EPI == (int)Epi::SWIGLU_BWD) ? TS
                      : EPI == (int)Epi::PARTIAL_BF16                                                 ? 2
                                                                                                      : 4;
  constexpr long C2S = EPI == (int)Epi::STORE_F32_LSE ? 8 : TS;
  GemmArgs g = g0;
  if (g0.batch > 1) {
    const long j = blockIdx.y;
    auto off = [j](const void* p, long s, long es) -> void* {
      return p ? (void*)((const char*)p + j * s * es) : nullptr;
    };
    g.A = off(g0.A, g0.sA, TS);
    g.B = off(g0.B, g0.sB, TS);
    g.B2 = off(g0.B2, g0.sB, TS);
    g.C = off(g0.C, g0.sC, CS);
    g.C2 = off(g0.C2, g0.sC2, C2S);
    g.C3 = off(g0.C3, g0.sC2, TS);
    g.X = off(g0.X, g0.sX, TS);
  }
  return g;
}

// Elements between the split-K slices of a PARTIAL epilogue's output.
__device__ __forceinline__ long split_offset(const GemmArgs& g) {
  return (long)blockIdx.z * (g.split_ld > 0 ? g.split_ld : (long)g.M * g.ldc);
}

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
            ((float*)g.C)[split_offset(g) + idx] = a;
          } else if constexpr (EPI == (int)Epi::PARTIAL_BF16) {
            ((bf16*)g.C)[split_offset(g) + idx] = (bf16)a;
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
gemm_kernel(GemmArgs g0) {
  const GemmArgs g = batch_view<T, EPI>(g0);
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
// swizzle; conflict-free for the 16-row fragment reads). Operands go
// global -> LDS by buffer_load ... lds (no VGPR staging; the hardware puts
// lane l's 16 bytes at base + 16 l, so each lane fetches the global vector
// that belongs in its swizzled slot).
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

// Operands whose K dimension is not contiguous (element (row r, k) at
// P[k * ld + r]) keep that orientation in LDS: a [64 k][ROWS] tile, filled by
// the same direct-to-LDS loads, whose 16-byte vector v of k-row kr sits at
// slot v ^ trx(kr). Fragments come out through the CDNA4 transposing LDS
// read (ds_read_b64_tr_b16): inside each group of 16 lanes, result lane i,
// element e is element i % 4 of the 4 that source lane 4 e + i / 4 points
// at. Pointing lane j of the group at (k-row kb + j / 4, column r0 + 4 (j % 4))
// therefore hands lane i column r0 + i at k-rows kb .. kb + 3 -- four
// consecutive K elements of its MFMA fragment; two reads make the eight.
// Swizzle: the half-wave a pass serves reads 32 contiguous bytes (an even
// slot pair) from each of 8 k-rows (kb + 8 h + j / 4, h = 0, 1, or the same
// + 16); XOR-ing the slot with 2 (kr & 3) + (kr & 8) sends those 8 rows to 8
// different slot pairs, i.e. all 64 banks once. k-row kr + 4 shares kr's
// swizzle (kb is a multiple of 32).
__device__ __forceinline__ int trx(int kr) { return ((kr & 3) << 1) | (kr & 8); }

template <int ROWS, int NW>
struct TrDmaLoader {
  static_assert(ROWS >= 128, "the swizzle needs 16 vectors per k-row");
  static constexpr int VPR = ROWS / 8;  // 16-byte vectors per k-row
  static constexpr int NI = VPR;        // wave instructions per 64-deep tile (1 KB each)
  static constexpr int PER = (NI + NW - 1) / NW;
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, long ld, int row0, int nrows, int k0,
                                        int kend, bf16* tile, int wid, int lane) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = wid + i * NW;
      if (NI % NW != 0 && q >= NI) break;
      const int idx = q * 64 + lane;
      const int kr = idx / VPR, slot = idx % VPR;
      const int v = slot ^ trx(kr);
      const int gk = k0 + kr, gr = row0 + v * 8;
      const uint32_t off = (gk < kend && gr < nrows) ? (uint32_t)(((long)gk * ld + gr) * 2) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(tile + q * 512), 16, off, 0, 0, 0);
    }
  }
};

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4* lds_s4_t;

// MFMA fragment (rows r0 .. r0 + 15, K elements kb + 8 (lane / 16) .. + 7)
// from a [64 k][ROWS] tile.
template <int ROWS>
__device__ __forceinline__ bf16x8 ld_tr8(const bf16* tile, int r0, int kb, int lane) {
  const int j = lane & 15;
  const int kr = kb + 8 * (lane >> 4) + (j >> 2), r = r0 + 4 * (j & 3);
  const bf16* p = tile + kr * ROWS + (((r >> 3) ^ trx(kr)) << 3) + (r & 7);
  // k-row kr + 4 has the same swizzle (kb is a multiple of 8)
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t)p);
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t)(p + 4 * ROWS));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}


// bf16-kernel epilogue, staged through LDS: each wave writes one 16-row block
// of its accumulator tile into a private LDS strip, then reads it back as
// row-contiguous 4-column chunks, so every global access of the epilogue is
// a 16-byte (fp32) or 8-byte (bf16) vector over consecutive columns -- the
// fp32 read-modify-write of the SGD and ADD epilogues otherwise dominates
// the short-K dW products. Chunks that cross N, or calls whose ldc / pointers
// do not allow vectors, take the element-wise path.
__device__ __forceinline__ bf16x4 cvt4(floatx4 v) {
  bf16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (bf16)v[e];
  return r;
}
__device__ __forceinline__ floatx4 upc4(bf16x4 v) {
  floatx4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (float)v[e];
  return r;
}

// Stochastic rounding of the bf16 working copy: a 32-bit integer mixing
// function of (seed, element index) -- the xor-shift-multiply "lowbias32"
// hash -- supplies 16 random bits that are added to the bits bf16 drops,
// then the value is truncated: it rounds up with probability equal to the
// dropped fraction, so E[bf16(w)] = w and no update is lost coherently.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ bf16 sr_bf16(float w, uint32_t seed, long idx) {
  const uint32_t r = mix32((uint32_t)idx * 0x9E3779B1u + mix32(seed ^ (uint32_t)(idx >> 32)));
  const uint32_t u = __builtin_bit_cast(uint32_t, w) + (r & 0xFFFFu);
  return __builtin_bit_cast(bf16, (uint16_t)(u >> 16));
}

// pre: for ADD_F32 / SGD, the chunk's fp32 C values loaded ahead (used
// when the chunk is a whole vector)
template <int EPI>
__device__ __forceinline__ void epi_chunk(const GemmArgs& g, int m, int n, floatx4 v, bool vec,
                                          floatx4 pre = floatx4{0.f, 0.f, 0.f, 0.f}) {
  const long idx = (long)m * g.ldc + n;
  const int ne = min(4, g.N - n);
  vec = vec && ne == 4;
  if constexpr (EPI == (int)Epi::STORE) {
    bf16* C = (bf16*)g.C + idx;
    const floatx4 w = v * g.scale;
    if (vec) *(bf16x4*)C = cvt4(w);
    else for (int e = 0; e < ne; ++e) C[e] = (bf16)w[e];
  } else if constexpr (EPI == (int)Epi::STORE_F32 || EPI == (int)Epi::PARTIAL) {
    float* C = (float*)g.C + idx + (EPI == (int)Epi::PARTIAL ? split_offset(g) : 0);
    if (vec) *(floatx4*)C = v;
    else for (int e = 0; e < ne; ++e) C[e] = v[e];
  } else if constexpr (EPI == (int)Epi::PARTIAL_BF16) {
    bf16* C = (bf16*)g.C + idx + split_offset(g);
    if (vec) *(bf16x4*)C = cvt4(v);
    else for (int e = 0; e < ne; ++e) C[e] = (bf16)v[e];
  } else if constexpr (EPI == (int)Epi::ADD_F32) {
    float* C = (float*)g.C + idx;
    if (vec) *(floatx4*)C = pre + v;
    else for (int e = 0; e < ne; ++e) C[e] += v[e];
  } else if constexpr (EPI == (int)Epi::SGD) {
    float* W = (float*)g.C + idx;
    const bool two = g.C2 != g.C;
    bf16* H = (bf16*)g.C2 + idx;
    bf16* L = g.C3 ? (bf16*)g.C3 + idx : nullptr;
    // (the same bits for every product of a batch: a sequence's rounding
    // does not depend on its place in the batch)
    const uint32_t sd = g.seed;
    if (vec) {
      const floatx4 w = pre - g.scale * v;
      __builtin_nontemporal_store(w, (floatx4*)W);
      if (two) {
        if (g.seed) {
          bf16x4 hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) hi[e] = sr_bf16(w[e], sd, idx + e);
          __builtin_nontemporal_store(hi, (bf16x4*)H);
        } else {
          const bf16x4 hi = cvt4(w);
          *(bf16x4*)H = hi;
          if (L) *(bf16x4*)L = cvt4(w - upc4(hi));
        }
      }
    } else {
      for (int e = 0; e < ne; ++e) {
        const float w = W[e] - g.scale * v[e];
        W[e] = w;
        if (two) {
          if (g.seed) {
            H[e] = sr_bf16(w, sd, idx + e);
          } else {
            const bf16 hi = (bf16)w;
            H[e] = hi;
            if (L) L[e] = (bf16)(w - (float)hi);
          }
        }
      }
    }
  } else if constexpr (EPI == (int)Epi::SWIGLU_BWD) {
    // n indexes hidden units n .. n+3 (inside one 16-block); their gate/up
    // columns in the 16-interleaved layout are (n / 16) * 32 + n % 16 and + 16
    const long ca = (long)m * g.ldc + (n >> 4) * 32 + (n & 15);
    const bf16* X = (const bf16*)g.X + ca;
    bf16* D = (bf16*)g.C + ca;
    floatx4 av, cv;
    if (vec) {
      av = upc4(*(const bf16x4*)X);
      cv = upc4(*(const bf16x4*)(X + 16));
    } else {
      for (int e = 0; e < 4; ++e) {
        av[e] = e < ne ? (float)X[e] : 0.f;
        cv[e] = e < ne ? (float)X[e + 16] : 0.f;
      }
    }
    floatx4 da, dc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sg = sigm_f(av[e]);
      da[e] = v[e] * cv[e] * sg * (1.0f + av[e] * (1.0f - sg));
      dc[e] = v[e] * av[e] * sg;
    }
    if (vec) {
      *(bf16x4*)D = cvt4(da);
      *(bf16x4*)(D + 16) = cvt4(dc);
    } else {
      for (int e = 0; e < ne; ++e) {
        D[e] = (bf16)da[e];
        D[e + 16] = (bf16)dc[e];
      }
    }
  }
}

// SWIGLU: gate columns n .. n+3 with values a, up columns n+16 .. n+19 with c.
__device__ __forceinline__ void epi_swiglu_chunk(const GemmArgs& g, int m, int n, floatx4 a, floatx4 c,
                                                 bool vec) {
  bf16* H12 = (bf16*)g.C;
  const long ldm = g.N / 2;
  const int jh = (n >> 5) * 16 + (n & 15);
  floatx4 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = silu_f(a[e]) * c[e];
  if (vec) {
    if (H12) {
      *(bf16x4*)(H12 + (long)m * g.ldc + n) = cvt4(a);
      *(bf16x4*)(H12 + (long)m * g.ldc + n + 16) = cvt4(c);
    }
    *(bf16x4*)((bf16*)g.C2 + (long)m * ldm + jh) = cvt4(h);
  } else {
    for (int e = 0; e < 4; ++e) {
      if (H12) {
        H12[(long)m * g.ldc + n + e] = (bf16)a[e];
        H12[(long)m * g.ldc + n + 16 + e] = (bf16)c[e];
      }
      ((bf16*)g.C2)[(long)m * ldm + jh + e] = (bf16)h[e];
    }
  }
}

template <int FM, int FN, int EPI>
__device__ __forceinline__ void gemm_epilogue_staged(const GemmArgs& g, floatx4 (&acc)[FM][FN], int mw, int nw,
                                                     int lane, float* strip) {
  constexpr int WN = FN * 16;
  constexpr int SP = WN + 4;  // strip row pitch in floats
  const int fr = lane & 15, fg = lane >> 4;
  auto al = [](const void* p, int a) { return p == nullptr || ((uintptr_t)p & (a - 1)) == 0; };
  bool vec = (g.ldc % 4) == 0;
  if constexpr (EPI == (int)Epi::STORE_F32 || EPI == (int)Epi::PARTIAL || EPI == (int)Epi::ADD_F32 ||
                EPI == (int)Epi::SGD || EPI == (int)Epi::STORE_F32_LSE)
    vec = vec && al(g.C, 16);
  else
    vec = vec && al(g.C, 8);
  if constexpr (EPI == (int)Epi::SGD) vec = vec && al(g.C2, 8) && al(g.C3, 8);
  if constexpr (EPI == (int)Epi::SWIGLU) vec = vec && al(g.C2, 8) && (g.N / 2) % 4 == 0;
  if constexpr (EPI == (int)Epi::SWIGLU_BWD) vec = vec && al(g.X, 8);
  constexpr bool RMW = EPI == (int)Epi::ADD_F32 || EPI == (int)Epi::SGD;
  constexpr int CPR = WN / 4;              // 4-column chunks per strip row
  constexpr int NCH = RMW ? 16 * CPR / 64 : 1;  // chunks per lane per row block
  static_assert(!RMW || (16 * CPR) % 64 == 0, "whole chunk rounds per lane");
  if constexpr (RMW) vec = vec && g.N >= 4;
  // C values of row block i, loaded unconditionally from a clamped (valid)
  // address so no lane branches around a load; out-of-range chunks drop them
  floatx4 cur[NCH], nxt[NCH];
  auto rmw_load = [&](int i, floatx4 (&dst)[NCH]) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = lane + 64 * k;
      const int row = c / CPR, col = (c % CPR) * 4;
      const int m = min(mw + 16 * i + row, g.M - 1), n = min(nw + col, g.N - 4);
      const floatx4* src = (const floatx4*)((const float*)g.C + (long)m * g.ldc + n);
      // the SGD master is read and written once per update: streamed past
      // the caches, which then keep the other streams' operands
      if constexpr (EPI == (int)Epi::SGD) dst[k] = __builtin_nontemporal_load(src);
      else dst[k] = *src;
    }
  };
  if constexpr (RMW) {
    if (vec) rmw_load(0, cur);  // wave-uniform
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) strip[(4 * fg + r) * SP + j * 16 + fr] = acc[i][j][r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if constexpr (EPI == (int)Epi::SWIGLU) {
      static_assert(WN % 32 == 0, "SWIGLU needs whole gate/up block pairs");
      constexpr int CPR = WN / 8;  // gate chunks per row
#pragma unroll
      for (int c = lane; c < 16 * CPR; c += 64) {
        const int row = c / CPR, q = c % CPR;
        const int col = (q >> 2) * 32 + (q & 3) * 4;
        const floatx4 a = *(const floatx4*)(strip + row * SP + col);
        const floatx4 cc = *(const floatx4*)(strip + row * SP + col + 16);
        const int m = mw + 16 * i + row, n = nw + col;
        if (m < g.M && n < g.N) epi_swiglu_chunk(g, m, n, a, cc, vec);
      }
    } else if constexpr (RMW) {
      // the next row block's C values are requested before this block's
      // stores, so no chunk waits on a store's completion (the counter
      // that tracks loads also tracks stores)
      if (vec && i + 1 < FM) rmw_load(i + 1, nxt);
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c = lane + 64 * k;
        const int row = c / CPR, col = (c % CPR) * 4;
        const floatx4 v = *(const floatx4*)(strip + row * SP + col);
        const int m = mw + 16 * i + row, n = nw + col;
        if (m < g.M && n < g.N) epi_chunk<EPI>(g, m, n, v, vec, cur[k]);
      }
#pragma unroll
      for (int k = 0; k < NCH; ++k) cur[k] = nxt[k];
    } else if constexpr (EPI == (int)Epi::STORE_F32_LSE) {
      // the 16 lanes that hold one row's chunks of a 64-column group (CPR is
      // a multiple of 16) also reduce that group's (max, sum exp)
      static_assert(CPR % 16 == 0, "64-column groups inside the wave strip");
      const int np = (g.N + 63) / 64;
#pragma unroll
      for (int c = lane; c < 16 * CPR; c += 64) {
        const int row = c / CPR, col = (c % CPR) * 4;
        const floatx4 v = *(const floatx4*)(strip + row * SP + col);
        const int m = mw + 16 * i + row, n = nw + col;
        const bool in = m < g.M && n < g.N;
        if (in) epi_chunk<(int)Epi::STORE_F32>(g, m, n, v, vec);
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (in && n + e < g.N) mx = fmaxf(mx, v[e]);
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
        float sm = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (in && n + e < g.N) sm += __expf(v[e] - mx);
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) sm += __shfl_xor(sm, o, 16);
        const int ng = nw + ((c % CPR) & ~15) * 4;  // first column of the group
        if ((lane & 15) == 0 && m < g.M && ng < g.N)
          ((float2*)g.C2)[(long)m * np + ng / 64] = make_float2(mx, sm);
      }
    } else {
#pragma unroll
      for (int c = lane; c < 16 * CPR; c += 64) {
        const int row = c / CPR, col = (c % CPR) * 4;
        const floatx4 v = *(const floatx4*)(strip + row * SP + col);
        const int m = mw + 16 * i + row, n = nw + col;
        if (m < g.M && n < g.N) epi_chunk<EPI>(g, m, n, v, vec);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_bf16_kernel(GemmArgs g0) {
  const GemmArgs g = batch_view<bf16, EPI>(g0);
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
  TrDmaLoader<BM, NW> ta;
  TrDmaLoader<BN, NW> tb;
  const int nk = (kend - kbeg + BK - 1) / BK;
  auto issue = [&](int kt, int buf) {
    const int k0 = kbeg + kt * BK;
    if constexpr (AK) da.issue(ra, g.lda, m0, g.M, k0, kend, As[buf], wid, lane);
    else ta.issue(ra, g.lda, m0, g.M, k0, kend, As[buf], wid, lane);
    if constexpr (BKM) {
      db.issue(rb, g.ldb, n0, g.N, k0, kend, Bs[buf], wid, lane);
      if constexpr (SPLITB) db.issue(rb2, g.ldb, n0, g.N, k0, kend, Cs[buf], wid, lane);
    } else {
      tb.issue(rb, g.ldb, n0, g.N, k0, kend, Bs[buf], wid, lane);
    }
  };
  if (nk > 0) issue(0, 0);
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
      for (int i = 0; i < FM; ++i) {
        if constexpr (AK) ld8(af[s][i], As[cur] + swz64(wm0 + i * 16 + fr, v));
        else af[s][i].v = ld_tr8<BM>(As[cur], wm0 + i * 16, s * 32, lane);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BKM) ld8(bfr[s][j], Bs[cur] + swz64(wn0 + j * 16 + fr, v));
        else bfr[s][j].v = ld_tr8<BN>(Bs[cur], wn0 + j * 16, s * 32, lane);
        if constexpr (SPLITB) ld8(bf2[s][j], Cs[cur] + swz64(wn0 + j * 16 + fr, v));
      }
    }
    // 2. ... then the next tile's loads into the other stage (no LDS read of
    //    this iteration follows them, so nothing waits on them before the MFMAs)
    if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
    // 3. the products, at raised wave priority (the SIMD's other wave, in
    //    its fragment reads, then yields issue to these; measured 0.5% on
    //    the prefix products)
    __builtin_amdgcn_s_setprio(1);
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
    // keep every MFMA of this tile issued before the wait for the next
    // tile's loads: left to itself the scheduler hoists the wait (and the
    // barrier) above most of them, exposing the whole load latency
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // the loop ended on a barrier with every load landed: the operand tiles
  // are free to hold the epilogue strips
  constexpr int STRIP = 16 * (WN + 4);
  static_assert(NW * STRIP * 4 <= (BM >= BN ? BM : BN) * BK * 2 * 2, "epilogue strips exceed the tile area");
  float* strips = BM >= BN ? (float*)&As[0][0] : (float*)&Bs[0][0];
  gemm_epilogue_staged<FM, FN, EPI>(g, acc, m0 + wm0, n0 + wn0, lane, strips + wid * STRIP);
}

// ------------------------------------------------------------------ launch
template <typename T, int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
static hipError_t gemm_launch(const GemmArgs& g, hipStream_t st) {
  const int tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  int splits = 1;
  if (g.kchunk > 0) splits = (g.K + g.kchunk - 1) / g.kchunk;
  dim3 grid(tm * tn, g.batch > 1 ? g.batch : 1, splits);
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, AK, BKM, EPI, SPLITB>), grid, dim3(NT), 0, st, g);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, int EPI, bool SPLITB>
static hipError_t gemm_bf16_launch(const GemmArgs& g, hipStream_t st) {
  const int tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  int splits = 1;
  if (g.kchunk > 0) splits = (g.K + g.kchunk - 1) / g.kchunk;
  dim3 grid(tm * tn, g.batch > 1 ? g.batch : 1, splits);
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
    default: break;  // PARTIAL_BF16: bf16 NN only (gemm_nn)
  }
  return hipErrorInvalidValue;
}

// per-layout entry points (one translation unit each)
hipError_t gemm_nt(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);
hipError_t gemm_nn(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);
hipError_t gemm_tn(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);
hipError_t gemm_tt(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st);

}  // namespace ttt
