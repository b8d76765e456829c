// Sliding-window attention backward, second generation (bf16, head_dim
// 64/128) on v_mfma_f32_32x32x16_bf16.
//
// The query-side gradient over the whole window (cached keys are constants)
// and the key/value gradients of the call's own positions, as in attn.hip:
//   P = exp(scale q.k - lse),  dP = dO . v,  dS = P (dP - D),  D = rowsum(dO O)
//   dq_i = scale sum_t dS[i, t] k_t;  dk_t = scale sum_i dS[i, t] q_i;  dv_t = sum_i P[i, t] dO_i.
//
// dQ: a workgroup holds 128 consecutive queries of one head (32 per wave,
// kept in registers with their dO rows as MFMA B operands); key tiles of 64
// stream through a double-buffered, XOR-swizzled LDS area by direct-to-LDS
// loads. S^T = K Q^T and dP^T = V dO^T come out with one query per lane
// column, so the softmax terms are lane-local; dQ^T = K^T dS^T takes dS^T
// straight from those registers and K^T from the same K tile through the
// CDNA4 transposing LDS read (no transposed key store needed). The key range
// of a query block can be split over several workgroups (grid z), each
// writing its own partial dq; the consumer adds the parts in a fixed order.
//
// dK, dV: a workgroup holds 128 keys of one key head (32 per wave, K and V
// rows in registers) and walks a run of that key block's (query head, query
// tile) pairs; query tiles of 64 (Q and dO rows, plus their lse and D) stream
// through LDS. S = Q K^T and dP = dO V^T have one key per lane column;
// dV^T = dO^T P and dK^T = Q^T dS read dO^T and Q^T through the transposing
// LDS read. The first key block of a call is seen by every later query, the
// last by its own few, so each block's pairs are cut into runs of about equal
// length (at most one run length for the whole call, chosen so that all runs
// fit on the CUs at once); each run writes its own partial dk, dv.
//
// Contraction slots of the P / dS operands follow the accumulator layout:
// slot 8 g + e of lane group g (= lane / 32) is row 16 u + 4 g + e (e < 4) or
// 16 u + 8 + 4 g + (e - 4) of the 32-row block, for the 16-row step u.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

namespace {
constexpr int BT = 64;  // key tile (dQ) / query tile (dK, dV)
constexpr float LOG2E_B = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void* ldsv_t;
typedef short shortx4b __attribute__((ext_vector_type(4)));
typedef short shortx8b __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4b* lds4_t;

// [rows][DH] bf16 tile: 16-byte vector v of row r at slot v ^ rsw(r). Two
// access patterns must be conflict-free: plain 16-byte reads of one vector
// from 16 consecutive rows (a pass), and transposing reads of 64 bytes (an
// aligned group of 4 slots) from each of 4 consecutive rows. DH = 128 (rows
// of 256 bytes, all starting at bank 0): rsw = 4 (r & 3) + ((r >> 2) & 3) is
// a bijection on r % 16 and gives the 4 rows different slot groups. DH = 64
// (rows of 128 bytes: even and odd rows in different bank halves):
// rsw = 4 ((r >> 1) & 1) + ((r >> 2) & 3), a bijection on (r >> 1) % 8 that
// separates rows r and r + 2.
template <int DH>
__device__ __forceinline__ int rsw(int r) {
  if constexpr (DH == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int DH>
__device__ __forceinline__ int rswz(int r, int v) {
  return r * DH + ((v ^ rsw<DH>(r)) << 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(const void* p, uint64_t nbytes) {
  const uint32_t n = nbytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)nbytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// MFMA operand of the transposed tile: lane l takes column c0 + l % 32 and
// the permuted contraction rows rb + 4 (l / 32) + e and rb + 8 + 4 (l / 32) + e.
// ds_read_b64_tr_b16: inside a group of 16 lanes, result lane i element e is
// element i % 4 of what source lane 4 e + i / 4 addressed; source lane j
// addresses (row base + j / 4, column c + 4 (j % 4)).
template <int DH>
__device__ __forceinline__ bf16x8 ld_tr_op(const bf16* tile, int rb, int c0, int lane) {
  const int hgrp = lane >> 4, j = lane & 15;
  const int row = rb + 4 * (hgrp >> 1) + (j >> 2);
  const int col = c0 + 16 * (hgrp & 1) + 4 * (j & 3);
  const bf16* p0 = tile + rswz<DH>(row, col >> 3) + (col & 7);
  const bf16* p1 = tile + rswz<DH>(row + 8, col >> 3) + (col & 7);
  const shortx4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4_t)p0);
  const shortx4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4_t)p1);
  const shortx8b w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ void pack_slots(bf16x8 (&f)[2], const floatx16& x) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) f[u][e] = (bf16)x[8 * u + e];
}
}  // namespace

// ------------------------------------------------------------------- dQ
template <int DH>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq2_kernel(AttnArgs a, int ksplit) {
  constexpr int KS = DH / 16, DB = DH / 32, KV = DH / 8;
  constexpr int NI = BT * DH * 2 / 1024;  // DMA wave-instructions per tile
  __shared__ __attribute__((aligned(1024))) bf16 Ks0[BT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Ks1[BT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Vs0[BT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Vs1[BT * DH];

  // XCD-aware order (see attn2.hip): each XCD takes a contiguous range of
  // logical blocks ordered key head, key split, query block, query head
  int h, z, qblk;
  {
    const int nqb = gridDim.x, nz = gridDim.z, grp = a.H / a.Hk;
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    int id = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
    const int per_kh = grp * nqb * nz;
    const int khb = id / per_kh;
    int rem = id % per_kh;
    z = rem / (grp * nqb);
    rem %= grp * nqb;
    qblk = rem / grp;
    h = khb * grp + rem % grp;
  }
  const int kh = h / (a.H / a.Hk);
  const int q0 = qblk * 128;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const bf16* Q = (const bf16*)a.q;
  const bf16* dO = (const bf16*)a.dO;
  const __amdgpu_buffer_rsrc_t rk = rsrc_b((const bf16*)a.k + (long)kh * a.cap * DH, (uint64_t)a.cap * DH * 2);
  const __amdgpu_buffer_rsrc_t rv = rsrc_b((const bf16*)a.v + (long)kh * a.cap * DH, (uint64_t)a.cap * DH * 2);
  const int qw = q0 + wid * 32;
  const int row = qw + lr;

  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (row < a.n) {
      qf[ks] = *(const bf16x8*)(Q + ((long)row * a.H + h) * DH + ks * 16 + lg * 8);
      df[ks] = *(const bf16x8*)(dO + ((long)row * a.H + h) * DH + ks * 16 + lg * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf[ks][e] = (bf16)0.f;
        df[ks][e] = (bf16)0.f;
      }
    }
  }
  const float lse2 = row < a.n ? a.lse[(long)h * a.n + row] * LOG2E_B : 0.f;
  const float Dq = row < a.n ? a.D[(long)h * a.n + row] : 0.f;
  floatx16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;

  // positions relative to pos0 fit in 32 bits
  const int qr_hi = min(q0 + 128, a.n) - 1;
  const int k_lo = (int)((max((int64_t)0, a.pos0 + q0 - a.window + 1) & ~(int64_t)(BT - 1)) - a.pos0);
  const int ntile = (qr_hi - k_lo) / BT + 1;
  const int per = (ntile + ksplit - 1) / ksplit;
  const int t_beg = z * per, t_end = min(ntile, t_beg + per);
  const int cmask = a.cap - 1;
  const float sc2 = a.scale * LOG2E_B;
  const int wq_lo = qw, wq_hi = min(qw + 32, a.n) - 1;

  auto dma_tile = [&](int kt, bf16* kdst, bf16* vdst) {
    const int slot = (int)((a.pos0 + kt) & cmask);
#pragma unroll
    for (int i = 0; i < NI / 4; ++i) {
      const int jj = wid + 4 * i;
      const int key = jj * (1024 / (DH * 2)) + lane / KV, p = lane % KV;
      const int v = p ^ rsw<DH>(key);
      const uint32_t off = (uint32_t)(((slot + key) * DH + v * 8) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (ldsv_t)(kdst + jj * 512), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (ldsv_t)(vdst + jj * 512), 16, off, 0, 0, 0);
    }
  };

  auto tile = [&](int t, const bf16* ks_, const bf16* vs_, bf16* kn, bf16* vn) {
    const int kt = k_lo + t * BT;
    if (t + 1 < t_end) dma_tile(kt + BT, kn, vn);
    const bool any = wq_lo < a.n && (kt <= wq_hi) && (kt + BT - 1 > wq_lo - a.window);
    const bool full = (kt + BT - 1 <= wq_lo) && (kt > wq_hi - a.window);
    if (any) {
      // one 32-key half of the tile at a time, end to end (scores, softmax
      // terms, dQ update): fewer live registers, two waves per SIMD
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        floatx16 sv, dpv;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          sv[j] = 0.f;
          dpv[j] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int o = rswz<DH>(kb * 32 + lr, ks * 2 + lg);
          const bf16x8 kf = *(const bf16x8*)(ks_ + o);
          const bf16x8 vf = *(const bf16x8*)(vs_ + o);
          mma32(sv, kf, qf[ks]);
          mma32(dpv, vf, df[ks]);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kp = kt + kb * 32 + 8 * (j >> 2) + 4 * lg + (j & 3);
          // one select per element, after an unconditional exponential, with
          // the tile-uniform `full` ORed in without short-circuit: written as
          // a test inside `if (!full)`, the compiler gave every element an
          // exec-mask region, also on tiles that need no mask
          const bool keep = full | ((kp <= row) & (kp > row - a.window));
          const float e = __builtin_amdgcn_exp2f(sv[j] * sc2 - lse2);
          sv[j] = (keep ? e : 0.f) * (dpv[j] - Dq);
        }
        bf16x8 dsf[2];
        pack_slots(dsf, sv);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < DB; ++db) mma32(acc[db], ld_tr_op<DH>(ks_, kb * 32 + 16 * u, db * 32, lane), dsf[u]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (t_beg < t_end) dma_tile(k_lo + t_beg * BT, Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = t_beg; t < t_end; t += 2) {
    tile(t, Ks0, Vs0, Ks1, Vs1);
    if (t + 1 >= t_end) break;
    tile(t + 1, Ks1, Vs1, Ks0, Vs0);
  }

  if (row < a.n) {
    const long off = (long)z * a.n * a.H * DH + ((long)row * a.H + h) * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * jg + e] * a.scale;
        const long o = off + db * 32 + 8 * jg + 4 * lg;
        if (a.parts_bf16) *(bf16x4*)((bf16*)a.dq + o) = __builtin_convertvector(w, bf16x4);
        else *(floatx4*)(a.dq + o) = w;
      }
  }
}

// --------------------------------------------------------------- dK, dV
namespace {
struct KvSched {
  int run;    // longest run of (query head, query tile) pairs per workgroup
  int parts;  // partial sums per key
  int jobs;   // workgroups per key head
};
constexpr int KV_SLOTS = 256;  // one dK/dV workgroup per CU (448 registers per lane)

KvSched kv_sched(const AttnArgs& a) {
  const int grp = a.H / a.Hk, nkb = (a.n + 127) / 128;
  int maxt = 0;
  for (int kb = 0; kb < nkb; ++kb) maxt = max(maxt, grp * attn_bwd2_kv_block_tiles(a.n, a.window, kb));
  auto jobs_for = [&](int run, int* parts) {
    int j = 0, p = 1;
    for (int kb = 0; kb < nkb; ++kb) {
      const int c = (grp * attn_bwd2_kv_block_tiles(a.n, a.window, kb) + run - 1) / run;
      j += c;
      p = max(p, c);
    }
    *parts = p;
    return j;
  };
  KvSched s{maxt, 1, nkb};
  if ((long)nkb * a.Hk >= KV_SLOTS) {
    // the key blocks alone fill the CUs: one run per query head
    s.run = (maxt + grp - 1) / grp;
    s.jobs = jobs_for(s.run, &s.parts);
    return s;
  }
  // shortest run whose workgroups all fit at once, with at most
  // max(H / Hk, ATTN_BWD2_MAX_KV_PARTS) runs per key block (one run per
  // query head of the group is always among the candidates)
  const int maxp = max(grp, ATTN_BWD2_MAX_KV_PARTS);
  for (int run = max(1, (maxt + maxp - 1) / maxp); run <= maxt; ++run) {
    int parts = 1;
    const int j = jobs_for(run, &parts);
    if ((long)j * a.Hk <= KV_SLOTS || run == maxt) {
      s.run = run;
      s.parts = parts;
      s.jobs = j;
      break;
    }
  }
  return s;
}
}  // namespace

template <int DH>
__global__ void __launch_bounds__(256) attn_bwd_dkdv2_kernel(AttnArgs a, int run, int parts) {
  constexpr int KS = DH / 16, DB = DH / 32, KV = DH / 8;
  constexpr int NI = BT * DH * 2 / 1024;
  __shared__ __attribute__((aligned(1024))) bf16 Qs0[BT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Qs1[BT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Os0[BT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Os1[BT * DH];
  __shared__ float ls0[BT], ls1[BT], Ds0[BT], Ds1[BT];

  const int grp = a.H / a.Hk;
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin; remap so
  // that each XCD takes a contiguous range of logical blocks ordered key head,
  // key block, run. The runs of a key head then read that head's query and
  // output-gradient rows through one L2.
  int kh, kb, ch, nch, tasks;
  {
    const int nwg = gridDim.x;
    int id = blockIdx.x;
    if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
    const int jobs = nwg / a.Hk;
    kh = id / jobs;
    int job = id % jobs;
    const int nkb = (a.n + 127) / 128;
    kb = 0;
    nch = 1;
    tasks = grp;
    for (; kb < nkb; ++kb) {
      tasks = grp * attn_bwd2_kv_block_tiles(a.n, a.window, kb);
      nch = (tasks + run - 1) / run;
      if (job < nch) break;
      job -= nch;
    }
    ch = job;
  }
  const int ntile = tasks / grp;  // query tiles per head of this key block
  const int t_beg = (int)((long)ch * tasks / nch), t_end = (int)((long)(ch + 1) * tasks / nch);
  const int k0 = kb * 128;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int kw = k0 + wid * 32;
  const int key = kw + lr;  // local index of this lane's key
  const int cmask = a.cap - 1;
  const bf16* Kst = (const bf16*)a.k + (long)kh * a.cap * DH;
  const bf16* Vst = (const bf16*)a.v + (long)kh * a.cap * DH;

  bf16x8 kf[KS], vf[KS];
  {
    const long slot = (long)((a.pos0 + key) & cmask);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (key < a.n) {
        kf[ks] = *(const bf16x8*)(Kst + slot * DH + ks * 16 + lg * 8);
        vf[ks] = *(const bf16x8*)(Vst + slot * DH + ks * 16 + lg * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kf[ks][e] = (bf16)0.f;
          vf[ks][e] = (bf16)0.f;
        }
      }
    }
  }
  floatx16 accK[DB], accV[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      accK[db][j] = 0.f;
      accV[db][j] = 0.f;
    }

  const __amdgpu_buffer_rsrc_t rq = rsrc_b(a.q, (uint64_t)a.n * a.H * DH * 2);
  const __amdgpu_buffer_rsrc_t ro = rsrc_b(a.dO, (uint64_t)a.n * a.H * DH * 2);
  const float sc2 = a.scale * LOG2E_B;
  const int wk_lo = kw, wk_hi = min(kw + 32, a.n) - 1;

  // pair t of the run: query head t / ntile of the group, query tile
  // k0 + 64 (t % ntile)
  auto dma_tile = [&](int t, bf16* qdst, bf16* odst, float* lsd, float* Dd) {
    const int h = kh * grp + t / ntile, qt = k0 + BT * (t % ntile);
#pragma unroll
    for (int i = 0; i < NI / 4; ++i) {
      const int jj = wid + 4 * i;
      const int r = jj * (1024 / (DH * 2)) + lane / KV, p = lane % KV;
      const int v = p ^ rsw<DH>(r);
      const int qrow = qt + r;
      const uint32_t off = qrow < a.n ? (uint32_t)((((long)qrow * a.H + h) * DH + v * 8) * 2) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (ldsv_t)(qdst + jj * 512), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (ldsv_t)(odst + jj * 512), 16, off, 0, 0, 0);
    }
    if (tid < BT) {
      const int qrow = qt + tid;
      lsd[tid] = qrow < a.n ? a.lse[(long)h * a.n + qrow] * LOG2E_B : 0.f;
      Dd[tid] = qrow < a.n ? a.D[(long)h * a.n + qrow] : 0.f;
    }
  };

  auto tile = [&](int t, const bf16* qs_, const bf16* os_, const float* lsc, const float* Dc, bf16* qn, bf16* on,
                  float* lsn, float* Dn) {
    if (t + 1 < t_end) dma_tile(t + 1, qn, on, lsn, Dn);
    const int qt = k0 + BT * (t % ntile);
    // key t sees query i iff t <= i < t + window
    const bool any = wk_lo < a.n && (qt + BT - 1 >= wk_lo) && (qt <= wk_hi + a.window - 1);
    const bool full = (qt >= wk_hi) && (qt + BT - 1 <= wk_lo + a.window - 1) && (qt + BT <= a.n);
    if (any) {
      floatx16 s[2], dp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          s[qb][j] = 0.f;
          dp[qb][j] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int o = rswz<DH>(qb * 32 + lr, ks * 2 + lg);
          mma32(s[qb], *(const bf16x8*)(qs_ + o), kf[ks]);
          mma32(dp[qb], *(const bf16x8*)(os_ + o), vf[ks]);
        }
      }
      bf16x8 pb[2][2], sb[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        floatx16 ds;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int ql = qb * 32 + 8 * (j >> 2) + 4 * lg + (j & 3);
          const int qi = qt + ql;
          // one select per element, as in the dQ kernel
          const bool keep = full | ((qi >= key) & (qi < key + a.window) & (qi < a.n) & (key < a.n));
          const float e = __builtin_amdgcn_exp2f(s[qb][j] * sc2 - lsc[ql]);
          const float p = keep ? e : 0.f;
          s[qb][j] = p;
          ds[j] = p * (dp[qb][j] - Dc[ql]);
        }
        pack_slots(pb[qb], s[qb]);
        pack_slots(sb[qb], ds);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            mma32(accV[db], ld_tr_op<DH>(os_, qb * 32 + 16 * u, db * 32, lane), pb[qb][u]);
            mma32(accK[db], ld_tr_op<DH>(qs_, qb * 32 + 16 * u, db * 32, lane), sb[qb][u]);
          }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (t_beg < t_end) dma_tile(t_beg, Qs0, Os0, ls0, Ds0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = t_beg; t < t_end; t += 2) {
    tile(t, Qs0, Os0, ls0, Ds0, Qs1, Os1, ls1, Ds1);
    if (t + 1 >= t_end) break;
    tile(t + 1, Qs1, Os1, ls1, Ds1, Qs0, Os0, ls0, Ds0);
  }

  if (key < a.n) {
    const long kstride = (long)a.n * a.Hk * DH;
    const long base = (long)ch * kstride + ((long)key * a.Hk + kh) * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = accK[db][4 * jg + e] * a.scale;
          wv[e] = accV[db][4 * jg + e];
        }
        const long o = base + db * 32 + 8 * jg + 4 * lg;
        if (a.parts_bf16) {
          *(bf16x4*)((bf16*)a.dk + o) = __builtin_convertvector(wk, bf16x4);
          *(bf16x4*)((bf16*)a.dv + o) = __builtin_convertvector(wv, bf16x4);
        } else {
          *(floatx4*)(a.dk + o) = wk;
          *(floatx4*)(a.dv + o) = wv;
        }
      }
    // the block's first run clears the parts no run of this block writes
    // (for consumers that add all parts of every key)
    if (a.kv_fill && ch == 0)
      for (int p = nch; p < parts; ++p)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const long o = (long)p * kstride + ((long)key * a.Hk + kh) * DH + db * 32 + 8 * jg + 4 * lg;
            if (a.parts_bf16) {
              const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
              *(bf16x4*)((bf16*)a.dk + o) = z;
              *(bf16x4*)((bf16*)a.dv + o) = z;
            } else {
              *(floatx4*)(a.dk + o) = floatx4{0.f, 0.f, 0.f, 0.f};
              *(floatx4*)(a.dv + o) = floatx4{0.f, 0.f, 0.f, 0.f};
            }
          }
  }
}

// ------------------------------------------------------------------ launch
bool attn_bwd2_supported(DT dt, const AttnArgs& a) {
  return dt == DT::BF16 && (a.dh == 128 || a.dh == 64);
}

int attn_bwd2_dq_parts(const AttnArgs& a) {
  // key-range parts (1..ATTN_BWD2_MAX_DQ_PARTS, at least 8 key tiles each)
  // minimising the load per workgroup slot, ceil(base s / 512) / s (two
  // workgroups fit on each of the 256 CUs), with a small charge per part for
  // the partial sums (as for the forward's key splits)
  const long base = (long)((a.n + 127) / 128) * a.H;
  const long tiles = (a.window + 128 + BT - 1) / BT + 1;
  int best = 1;
  double best_cost = 1e30;
  for (int s = 1; s <= ATTN_BWD2_MAX_DQ_PARTS && (s == 1 || s <= tiles / 8); ++s) {
    const double cost = (double)((base * s + 511) / 512) / s + 0.02 * s;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

int attn_bwd2_kv_parts(const AttnArgs& a) { return a.n > 0 ? kv_sched(a).parts : 1; }
int attn_bwd2_kv_run(const AttnArgs& a) { return a.n > 0 ? kv_sched(a).run : 1; }

hipError_t attn_bwd_dq2(DT dt, const AttnArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  if (!attn_bwd2_supported(dt, a)) return hipErrorInvalidValue;
  const int parts = attn_bwd2_dq_parts(a);
  const dim3 grid((a.n + 127) / 128, a.H, parts);
  if (a.dh == 128) hipLaunchKernelGGL(attn_bwd_dq2_kernel<128>, grid, dim3(256), 0, st, a, parts);
  else hipLaunchKernelGGL(attn_bwd_dq2_kernel<64>, grid, dim3(256), 0, st, a, parts);
  return hipGetLastError();
}

hipError_t attn_bwd_dkdv2(DT dt, const AttnArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  if (!attn_bwd2_supported(dt, a)) return hipErrorInvalidValue;
  const KvSched s = kv_sched(a);
  const dim3 grid((unsigned)(s.jobs * a.Hk));
  if (a.dh == 128) hipLaunchKernelGGL(attn_bwd_dkdv2_kernel<128>, grid, dim3(256), 0, st, a, s.run, s.parts);
  else hipLaunchKernelGGL(attn_bwd_dkdv2_kernel<64>, grid, dim3(256), 0, st, a, s.run, s.parts);
  return hipGetLastError();
}

}  // namespace ttt
