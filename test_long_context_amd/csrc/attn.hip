// Causal sliding-window attention on gfx950 MFMA: forward, dQ and (dK, dV).
//
// Window: key t is visible to query i iff i - window < t <= i ([P1]
// "TTT-E2E：端到端测试时训练的长上下文语言建模", 关键设计参数: window k >= chunk b,
// read causally). Keys and values live in a store [Hk][cap][dh] indexed by
// position & (cap - 1); tiles of 64 positions are aligned, so a tile never
// straddles the wrap (cap is a power of two >= 64).
//
// Lane layout: every product is arranged so that the softmax statistics of a
// query stay in one lane. Scores are formed transposed, S^T = K Q^T (MFMA A =
// keys from LDS, B = the wave's queries held in registers), so lane l holds
// query l % 16 and keys 4 (l / 16) + r of a 16-key block. The P V product is
// formed as O^T = V^T P^T with P^T taken straight from those registers: the
// 32-element contraction slot 8 g + j of lane group g maps to key 4 g + j of
// the first 16-key block (j < 4) and of the second (j >= 4); the V^T operand
// is read from LDS with the same key permutation. GQA: query head h reads key
// head h / (H / Hk).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

static constexpr int BKV = 64;

// Copy ROWS x DH rows (row r from src + r * sstride) into LDS dst[r * DP + c];
// rows with !valid(r) are zero-filled.
template <typename T, int ROWS, int DH, int DP, int NT>
__device__ __forceinline__ void lds_rows(T* dst, const T* src, long sstride, int nvalid_lo,
                                         int nvalid_hi, int tid) {
  constexpr int VPR = DH / 8;
  for (int v = tid; v < ROWS * VPR; v += NT) {
    const int r = v / VPR, c = (v % VPR) * 8;
    Frag8<T> f;
    if (r >= nvalid_lo && r < nvalid_hi) ld8(f, src + (long)r * sstride + c);
    else zero8(f);
    st8(dst + r * DP + c, f);
  }
}

// Same rows, stored transposed: dst[c * RP + r].
template <typename T, int ROWS, int DH, int RP, int NT>
__device__ __forceinline__ void lds_rows_t(T* dst, const T* src, long sstride, int nvalid_lo,
                                           int nvalid_hi, int tid) {
  constexpr int NB = (ROWS / 8) * (DH / 8);
  for (int b = tid; b < NB; b += NT) {
    const int rb = b % (ROWS / 8), cb = b / (ROWS / 8);
    Frag8<T> in[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = rb * 8 + j;
      if (r >= nvalid_lo && r < nvalid_hi) ld8(in[j], src + (long)r * sstride + cb * 8);
      else zero8(in[j]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      Frag8<T> o;
#pragma unroll
      for (int j = 0; j < 8; ++j) eset<T>(o, j, eget<T>(in[j], c));
      st8(dst + (cb * 8 + c) * RP + rb * 8, o);
    }
  }
}

// A fragment of a transposed tile X^T[row][key] (row stride RP) for the
// permuted 32-key contraction block kk: slots 8 g + j -> key kk + 4 g + j
// (j < 4) and kk + 16 + 4 g + (j - 4).
template <typename T>
__device__ __forceinline__ void ld_perm(Frag8<T>& f, const T* rowp, int kk, int g) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    eset<T>(f, j, rowp[kk + 4 * g + j]);
    eset<T>(f, j + 4, rowp[kk + 16 + 4 * g + j]);
  }
}

// B fragment from two 16-row accumulator blocks (rows 4 g + r of each).
template <typename T>
__device__ __forceinline__ void pack_perm(Frag8<T>& f, const floatx4& lo, const floatx4& hi) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    set8(f, j, lo[j]);
    set8(f, j + 4, hi[j]);
  }
}

__device__ __forceinline__ bool visible(int64_t kp, int64_t qp, int window) {
  return kp <= qp && kp > qp - window;
}

// ------------------------------------------------------------------ forward
template <typename T, int DH, int QF>
__global__ void __launch_bounds__(256) attn_fwd_kernel(AttnArgs a) {
  constexpr int NT = 256;
  constexpr int BQ = 4 * 16 * QF;
  constexpr int KP = DH + 8, VP = BKV + 8;
  constexpr int KC = (DH + 31) / 32, DB = DH / 16;
  __shared__ __attribute__((aligned(16))) T Ks[BKV * KP];
  __shared__ __attribute__((aligned(16))) T Vt[DH * VP];

  const int h = blockIdx.y, kh = h / (a.H / a.Hk);
  const int q0 = blockIdx.x * BQ;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const T* Q = (const T*)a.q;
  const T* Kst = (const T*)a.k + (long)kh * a.cap * DH;
  const T* Vst = (const T*)a.v + (long)kh * a.cap * DH;
  const int qw = q0 + wid * 16 * QF;

  Frag8<T> qf[QF][KC];
#pragma unroll
  for (int qi = 0; qi < QF; ++qi)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int row = qw + qi * 16 + fr, ko = kc * 32 + fg * 8;
      if (row < a.n && ko < DH) ld8(qf[qi][kc], Q + ((long)row * a.H + h) * DH + ko);
      else zero8(qf[qi][kc]);
    }
  float m_run[QF], l_run[QF];
  floatx4 ot[DB][QF];
#pragma unroll
  for (int qi = 0; qi < QF; ++qi) {
    m_run[qi] = -INFINITY;
    l_run[qi] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) ot[db][qi] = floatx4{0, 0, 0, 0};
  }

  const int64_t qp_lo = a.pos0 + q0;
  const int64_t qp_hi = a.pos0 + min(q0 + BQ, a.n) - 1;
  const int64_t k_lo = (max((int64_t)0, qp_lo - a.window + 1)) & ~(int64_t)(BKV - 1);
  const int cmask = a.cap - 1;
  const float scale = a.scale;

  for (int64_t kt = k_lo; kt <= qp_hi; kt += BKV) {
    __syncthreads();
    const int slot = (int)(kt & cmask);
    const int hi = (int)min((int64_t)BKV, qp_hi - kt + 1);
    lds_rows<T, BKV, DH, KP, NT>(Ks, Kst + (long)slot * DH, DH, 0, hi, tid);
    lds_rows_t<T, BKV, DH, VP, NT>(Vt, Vst + (long)slot * DH, DH, 0, hi, tid);
    __syncthreads();

    floatx4 s[4][QF];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag8<T> af[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int ko = kc * 32 + fg * 8;
        if (ko < DH) ld8(af[kc], Ks + (kb * 16 + fr) * KP + ko);
        else zero8(af[kc]);
      }
#pragma unroll
      for (int qi = 0; qi < QF; ++qi) {
        s[kb][qi] = floatx4{0, 0, 0, 0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma16(s[kb][qi], af[kc], qf[qi][kc]);
      }
    }
#pragma unroll
    for (int qi = 0; qi < QF; ++qi) {
      const int64_t qp = a.pos0 + qw + qi * 16 + fr;
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t kp = kt + kb * 16 + fg * 4 + r;
          const float v = visible(kp, qp, a.window) ? s[kb][qi][r] * scale : -INFINITY;
          s[kb][qi][r] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(m_run[qi], tmax);
      const float mu = (mnew == -INFINITY) ? 0.f : mnew;
      const float corr = __expf(m_run[qi] - mu);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __expf(s[kb][qi][r] - mu);
          s[kb][qi][r] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run[qi] = l_run[qi] * corr + rs;
      m_run[qi] = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) ot[db][qi] *= corr;
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      Frag8<T> pb[QF];
#pragma unroll
      for (int qi = 0; qi < QF; ++qi) pack_perm(pb[qi], s[2 * k2][qi], s[2 * k2 + 1][qi]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        Frag8<T> vf;
        ld_perm(vf, Vt + (db * 16 + fr) * VP, 32 * k2, fg);
#pragma unroll
        for (int qi = 0; qi < QF; ++qi) mma16(ot[db][qi], vf, pb[qi]);
      }
    }
  }

  T* O = (T*)a.o;
#pragma unroll
  for (int qi = 0; qi < QF; ++qi) {
    const int row = qw + qi * 16 + fr;
    if (row >= a.n) continue;
    const float inv = l_run[qi] > 0.f ? 1.f / l_run[qi] : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        O[((long)row * a.H + h) * DH + db * 16 + fg * 4 + r] = from_f<T>(ot[db][qi][r] * inv);
    if (fg == 0 && a.lse) a.lse[(long)h * a.n + row] = m_run[qi] + __logf(l_run[qi]);
  }
}

// ------------------------------------------------------------- backward: dQ
// dq[i] = scale * sum_t dS[i, t] k_t over the window, with
// dS = P (dP - D), P = exp(scale q.k - lse), dP = dO . v; cached keys are
// constants here, so this is the whole query-side gradient.
template <typename T, int DH, int QF>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(AttnArgs a) {
  constexpr int NT = 256;
  constexpr int BQ = 4 * 16 * QF;
  constexpr int KP = DH + 8, VP = BKV + 8;
  constexpr int KC = (DH + 31) / 32, DB = DH / 16;
  __shared__ __attribute__((aligned(16))) T Ks[BKV * KP];
  __shared__ __attribute__((aligned(16))) T Vs[BKV * KP];
  __shared__ __attribute__((aligned(16))) T Kt[DH * VP];

  const int h = blockIdx.y, kh = h / (a.H / a.Hk);
  const int q0 = blockIdx.x * BQ;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const T* Q = (const T*)a.q;
  const T* dO = (const T*)a.dO;
  const T* Kst = (const T*)a.k + (long)kh * a.cap * DH;
  const T* Vst = (const T*)a.v + (long)kh * a.cap * DH;
  const int qw = q0 + wid * 16 * QF;

  Frag8<T> qf[QF][KC], df[QF][KC];
  float lse[QF], Dq[QF];
#pragma unroll
  for (int qi = 0; qi < QF; ++qi) {
    const int row = qw + qi * 16 + fr;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int ko = kc * 32 + fg * 8;
      if (row < a.n && ko < DH) {
        ld8(qf[qi][kc], Q + ((long)row * a.H + h) * DH + ko);
        ld8(df[qi][kc], dO + ((long)row * a.H + h) * DH + ko);
      } else {
        zero8(qf[qi][kc]);
        zero8(df[qi][kc]);
      }
    }
    lse[qi] = row < a.n ? a.lse[(long)h * a.n + row] : 0.f;
    Dq[qi] = row < a.n ? a.D[(long)h * a.n + row] : 0.f;
  }
  floatx4 dqt[DB][QF];
#pragma unroll
  for (int qi = 0; qi < QF; ++qi)
#pragma unroll
    for (int db = 0; db < DB; ++db) dqt[db][qi] = floatx4{0, 0, 0, 0};

  const int64_t qp_lo = a.pos0 + q0;
  const int64_t qp_hi = a.pos0 + min(q0 + BQ, a.n) - 1;
  const int64_t k_lo = (max((int64_t)0, qp_lo - a.window + 1)) & ~(int64_t)(BKV - 1);
  const int cmask = a.cap - 1;
  const float scale = a.scale;

  for (int64_t kt = k_lo; kt <= qp_hi; kt += BKV) {
    __syncthreads();
    const int slot = (int)(kt & cmask);
    const int hi = (int)min((int64_t)BKV, qp_hi - kt + 1);
    lds_rows<T, BKV, DH, KP, NT>(Ks, Kst + (long)slot * DH, DH, 0, hi, tid);
    lds_rows<T, BKV, DH, KP, NT>(Vs, Vst + (long)slot * DH, DH, 0, hi, tid);
    lds_rows_t<T, BKV, DH, VP, NT>(Kt, Kst + (long)slot * DH, DH, 0, hi, tid);
    __syncthreads();

    floatx4 s[4][QF], dp[4][QF];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag8<T> kf[KC], vf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int ko = kc * 32 + fg * 8;
        if (ko < DH) {
          ld8(kf[kc], Ks + (kb * 16 + fr) * KP + ko);
          ld8(vf[kc], Vs + (kb * 16 + fr) * KP + ko);
        } else {
          zero8(kf[kc]);
          zero8(vf[kc]);
        }
      }
#pragma unroll
      for (int qi = 0; qi < QF; ++qi) {
        s[kb][qi] = floatx4{0, 0, 0, 0};
        dp[kb][qi] = floatx4{0, 0, 0, 0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          mma16(s[kb][qi], kf[kc], qf[qi][kc]);
          mma16(dp[kb][qi], vf[kc], df[qi][kc]);
        }
      }
    }
#pragma unroll
    for (int qi = 0; qi < QF; ++qi) {
      const int64_t qp = a.pos0 + qw + qi * 16 + fr;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t kp = kt + kb * 16 + fg * 4 + r;
          const float p = visible(kp, qp, a.window) ? __expf(s[kb][qi][r] * scale - lse[qi]) : 0.f;
          s[kb][qi][r] = p * (dp[kb][qi][r] - Dq[qi]);
        }
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      Frag8<T> sb[QF];
#pragma unroll
      for (int qi = 0; qi < QF; ++qi) pack_perm(sb[qi], s[2 * k2][qi], s[2 * k2 + 1][qi]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        Frag8<T> kf;
        ld_perm(kf, Kt + (db * 16 + fr) * VP, 32 * k2, fg);
#pragma unroll
        for (int qi = 0; qi < QF; ++qi) mma16(dqt[db][qi], kf, sb[qi]);
      }
    }
  }

#pragma unroll
  for (int qi = 0; qi < QF; ++qi) {
    const int row = qw + qi * 16 + fr;
    if (row >= a.n) continue;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.dq[((long)row * a.H + h) * DH + db * 16 + fg * 4 + r] = dqt[db][qi][r] * scale;
  }
}

// --------------------------------------------------------- backward: dK, dV
// For the keys of this call's own positions (the current mini-batch): dk_t =
// scale sum_i dS[i, t] q_i and dv_t = sum_i P[i, t] dO_i over the queries of
// this call that see t, summed over the query heads of the key head's group.
// Here the roles flip: lane l holds key l % 16 of the wave's 16 keys, and
// queries form the contraction.
template <typename T, int DH>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_kernel(AttnArgs a) {
  constexpr int NT = 256;
  constexpr int BQT = 64;  // query tile
  constexpr int KP = DH + 8, VP = BQT + 8;
  constexpr int KC = (DH + 31) / 32, DB = DH / 16;
  __shared__ __attribute__((aligned(16))) T Qs[BQT * KP];
  __shared__ __attribute__((aligned(16))) T dOs[BQT * KP];
  __shared__ __attribute__((aligned(16))) T Qt[DH * VP];
  __shared__ __attribute__((aligned(16))) T dOt[DH * VP];
  __shared__ float lse_s[BQT], D_s[BQT];

  const int kh = blockIdx.y;
  const int grp = a.H / a.Hk;
  const int k0 = blockIdx.x * BKV;  // local index of the first key of the tile
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int kl = k0 + wid * 16 + fr;  // this lane's key (local index)
  const T* Kst = (const T*)a.k + (long)kh * a.cap * DH;
  const T* Vst = (const T*)a.v + (long)kh * a.cap * DH;
  const int cmask = a.cap - 1;
  const float scale = a.scale;

  Frag8<T> kf[KC], vf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int ko = kc * 32 + fg * 8;
    if (kl < a.n && ko < DH) {
      const long slot = (long)((a.pos0 + kl) & cmask);
      ld8(kf[kc], Kst + slot * DH + ko);
      ld8(vf[kc], Vst + slot * DH + ko);
    } else {
      zero8(kf[kc]);
      zero8(vf[kc]);
    }
  }
  floatx4 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkt[db] = floatx4{0, 0, 0, 0};
    dvt[db] = floatx4{0, 0, 0, 0};
  }
  const int64_t kp = a.pos0 + kl;
  const int qend = (int)min((int64_t)a.n, (int64_t)k0 + BKV - 1 + a.window);
  const T* Q = (const T*)a.q;
  const T* dO = (const T*)a.dO;

  for (int hq = 0; hq < grp; ++hq) {
    const int h = kh * grp + hq;
    for (int qt = k0; qt < qend; qt += BQT) {
      __syncthreads();
      const int nq = min(BQT, a.n - qt);
      const T* qsrc = Q + ((long)qt * a.H + h) * DH;
      const T* dsrc = dO + ((long)qt * a.H + h) * DH;
      lds_rows<T, BQT, DH, KP, NT>(Qs, qsrc, (long)a.H * DH, 0, nq, tid);
      lds_rows<T, BQT, DH, KP, NT>(dOs, dsrc, (long)a.H * DH, 0, nq, tid);
      lds_rows_t<T, BQT, DH, VP, NT>(Qt, qsrc, (long)a.H * DH, 0, nq, tid);
      lds_rows_t<T, BQT, DH, VP, NT>(dOt, dsrc, (long)a.H * DH, 0, nq, tid);
      if (tid < BQT) {
        lse_s[tid] = tid < nq ? a.lse[(long)h * a.n + qt + tid] : 0.f;
        D_s[tid] = tid < nq ? a.D[(long)h * a.n + qt + tid] : 0.f;
      }
      __syncthreads();

      floatx4 p[4], ds[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        Frag8<T> qa[KC], da[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const int ko = kc * 32 + fg * 8;
          if (ko < DH) {
            ld8(qa[kc], Qs + (qb * 16 + fr) * KP + ko);
            ld8(da[kc], dOs + (qb * 16 + fr) * KP + ko);
          } else {
            zero8(qa[kc]);
            zero8(da[kc]);
          }
        }
        floatx4 sv = floatx4{0, 0, 0, 0}, dpv = floatx4{0, 0, 0, 0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          mma16(sv, qa[kc], kf[kc]);
          mma16(dpv, da[kc], vf[kc]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = qb * 16 + fg * 4 + r;
          const int64_t qp = a.pos0 + qt + ql;
          const bool ok = (qt + ql < a.n) && (kl < a.n) && visible(kp, qp, a.window);
          const float pv = ok ? __expf(sv[r] * scale - lse_s[ql]) : 0.f;
          p[qb][r] = pv;
          ds[qb][r] = pv * (dpv[r] - D_s[ql]);
        }
      }
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        Frag8<T> pb, sb;
        pack_perm(pb, p[2 * q2], p[2 * q2 + 1]);
        pack_perm(sb, ds[2 * q2], ds[2 * q2 + 1]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          Frag8<T> oa, qa;
          ld_perm(oa, dOt + (db * 16 + fr) * VP, 32 * q2, fg);
          ld_perm(qa, Qt + (db * 16 + fr) * VP, 32 * q2, fg);
          mma16(dvt[db], oa, pb);
          mma16(dkt[db], qa, sb);
        }
      }
    }
  }
  if (kl < a.n) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long o = ((long)kl * a.Hk + kh) * DH + db * 16 + fg * 4 + r;
        a.dk[o] = dkt[db][r] * scale;
        a.dv[o] = dvt[db][r];
      }
  }
}

// ------------------------------------------------------------------ launch
template <typename T, int DH>
static hipError_t fwd_dh(const AttnArgs& a, hipStream_t st) {
  constexpr int QF = 1;
  dim3 grid((a.n + 64 * QF - 1) / (64 * QF), a.H);
  hipLaunchKernelGGL((attn_fwd_kernel<T, DH, QF>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename T, int DH>
static hipError_t dq_dh(const AttnArgs& a, hipStream_t st) {
  constexpr int QF = 1;
  dim3 grid((a.n + 64 * QF - 1) / (64 * QF), a.H);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DH, QF>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename T, int DH>
static hipError_t dkdv_dh(const AttnArgs& a, hipStream_t st) {
  dim3 grid((a.n + BKV - 1) / BKV, a.Hk);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DH>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

#define TTT_ATTN_DISPATCH(FN)                                          \
  if (a.n <= 0) return hipSuccess;                                     \
  if (dt == DT::BF16) {                                                \
    switch (a.dh) {                                                    \
      case 64: return FN<bf16, 64>(a, st);                             \
      case 128: return FN<bf16, 128>(a, st);                           \
      case 16: return FN<bf16, 16>(a, st);                             \
    }                                                                  \
  } else {                                                             \
    switch (a.dh) {                                                    \
      case 16: return FN<float, 16>(a, st);                            \
      case 64: return FN<float, 64>(a, st);                            \
      case 128: return FN<float, 128>(a, st);                          \
    }                                                                  \
  }                                                                    \
  return hipErrorInvalidValue;

hipError_t attn_fwd(DT dt, const AttnArgs& a, hipStream_t st) { TTT_ATTN_DISPATCH(fwd_dh) }
hipError_t attn_bwd_dq(DT dt, const AttnArgs& a, hipStream_t st) { TTT_ATTN_DISPATCH(dq_dh) }
hipError_t attn_bwd_dkdv(DT dt, const AttnArgs& a, hipStream_t st) { TTT_ATTN_DISPATCH(dkdv_dh) }

}  // namespace ttt
