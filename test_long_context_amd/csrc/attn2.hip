// Sliding-window attention forward, second generation (bf16, head_dim 64/128)
// on v_mfma_f32_32x32x16_bf16.
//
// Same window and GQA as attn.hip. A workgroup holds 128 * QB consecutive
// queries of one head; each wave owns 32 * QB of them, kept in registers as
// MFMA B operands for the whole key sweep. Keys advance in tiles of 64: the
// next tile's K ([key][dh]) and V^T ([dh][key], from the transposed value
// ring) are loaded into registers while the current tile is consumed, then
// stored into the other half of a double-buffered, XOR-swizzled LDS area.
// Scores are formed transposed, S^T = K Q^T, so lane l holds 16 keys of
// query l % 32 and the softmax statistics stay lane-local (one exchange with
// lane l ^ 32). The P V product is O^T = V^T P^T with P^T read from the
// score registers; its contraction slot 8 g + j maps to key 4 g + j
// (j < 4) or 8 + 4 g + (j - 4) of each 16-key group, and the transposed
// value store keeps each 16-key group in that order (vt_slot), so a V^T
// fragment is one 16-byte LDS read. Softmax runs in base 2 (scale folded with log2 e);
// masks are evaluated only on tiles the window or the diagonal cuts.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

namespace {
constexpr int BKV2 = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int DH>
__device__ __forceinline__ int kswz(int key, int v) {  // K tile [64][DH], 16-byte vectors
  return key * DH + ((v ^ (key & (DH / 8 - 1))) << 3);
}
__device__ __forceinline__ int vswz(int row, int v) {  // V^T tile [DH][64], rows of 128 bytes
  // consecutive rows alternate bank halves; row pairs take different slots
  return row * 64 + ((v ^ ((row >> 1) & 7)) << 3);
}
}  // namespace

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup order: the hardware deals consecutive workgroup ids round-robin
// over the 8 XCDs (each with its own L2). Remap so that each XCD gets a
// contiguous range of logical blocks, ordered key head first, then query
// block, then the query heads of the group -- workgroups that run together
// on an XCD read the same key/value tiles. Grid: (query blocks, H, key
// splits); logical order key head, key split, query block, query head.
__device__ __forceinline__ void attn_block_order(const AttnArgs& a, int& qblk, int& h, int& z) {
  const int nqb = gridDim.x, nz = gridDim.z, nwg = gridDim.x * gridDim.y * gridDim.z;
  int id = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int grp = a.H / a.Hk;
  const int per_kh = grp * nqb * nz;
  const int kh = id / per_kh;
  int rem = id % per_kh;
  z = rem / (grp * nqb);
  rem %= grp * nqb;
  qblk = rem / grp;
  h = kh * grp + rem % grp;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes, 0x00020000);
}

// max / sum of a lane's value and that of lane ^ 32 without LDS: the
// half-swap of gfx950 (v_permlane32_swap) hands every lane both values, and
// the operation is commutative, so the result equals op(v, shfl_xor(v, 32))
// bit for bit whichever way round the halves are swapped
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float xor32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

template <int DH, int QB, int NWV = 4>
__global__ void __launch_bounds__(NWV * 64, (QB == 1 && NWV == 4) ? 2 : 1) attn_fwd2_kernel(AttnArgs a) {
  constexpr int BQ = NWV * 32 * QB;
  constexpr int KS = DH / 16;   // contraction steps over dh for S^T
  constexpr int DB = DH / 32;   // 32-row dh blocks of O^T
  constexpr int KV = DH / 8;    // 16-byte vectors per K row
  constexpr int NIK = BKV2 * DH * 2 / 1024;  // DMA wave-instructions per K tile
  constexpr int NIV = DH * BKV2 * 2 / 1024;  // ... per V^T tile
  constexpr float RESCALE = 8.f;  // log2 headroom before O is rescaled
  // two stages as distinct objects: the compiler then knows that the DMA
  // into one stage never aliases reads of the other
  __shared__ __attribute__((aligned(1024))) bf16 Ks0[BKV2 * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Ks1[BKV2 * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Vs0[DH * BKV2];
  __shared__ __attribute__((aligned(1024))) bf16 Vs1[DH * BKV2];

  int qblk, h, z;
  attn_block_order(a, qblk, h, z);
  const int kh = h / (a.H / a.Hk);
  const int q0 = qblk * BQ;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const bf16* Q = (const bf16*)a.q;
  const __amdgpu_buffer_rsrc_t rk = rsrc((const bf16*)a.k + (long)kh * a.cap * DH, (uint32_t)a.cap * DH * 2);
  const __amdgpu_buffer_rsrc_t rv = rsrc((const bf16*)a.vt + (long)kh * DH * a.cap, (uint32_t)a.cap * DH * 2);
  const int qw = q0 + wid * 32 * QB;

  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + qb * 32 + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row < a.n) qf[qb][ks] = *(const bf16x8*)(Q + ((long)row * a.H + h) * DH + ks * 16 + lg * 8);
      else
        for (int e = 0; e < 8; ++e) qf[qb][ks][e] = (bf16)0.f;
    }
  }
  floatx16 o[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[qb][db][j] = 0.f;
  }

  // positions relative to pos0 fit in 32 bits
  const int qr_lo = q0, qr_hi = min(q0 + BQ, a.n) - 1;
  const int k_lo = (int)((max((int64_t)0, a.pos0 + qr_lo - a.window + 1) & ~(int64_t)(BKV2 - 1)) - a.pos0);
  const int cmask = a.cap - 1;
  const float sc2 = a.scale * LOG2E;
  const int wq_lo = qw, wq_hi = min(qw + 32 * QB, a.n) - 1;
  // key tiles [k_lo, qr_hi], split over gridDim.z workgroups
  const int ntile = (qr_hi - k_lo) / BKV2 + 1;
  const int per = (ntile + gridDim.z - 1) / gridDim.z;
  const int t_beg = z * per, t_end = min(ntile, t_beg + per);

  // DMA of key tile kt (relative position): lane l writes the swizzled slot
  // base + 16 l, so it fetches the logical vector belonging to that slot
  auto dma_tile = [&](int kt, bf16* kdst, bf16* vdst) {
    const int slot = (int)((a.pos0 + kt) & cmask);
    static_assert(NIK % NWV == 0 && NIV % NWV == 0, "tile loads must split evenly over the waves");
#pragma unroll
    for (int i = 0; i < NIK / NWV; ++i) {
      const int j = wid + NWV * i;
      const int key = j * (1024 / (DH * 2)) + lane / KV, p = lane % KV;
      const int v = p ^ (key & (KV - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(kdst + j * 512), 16,
                                               (uint32_t)(((slot + key) * DH + v * 8) * 2), 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NIV / NWV; ++i) {
      const int j = wid + NWV * i;
      const int row = j * 8 + lane / 8, p = lane % 8;
      const int v = p ^ ((row >> 1) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(vdst + j * 512), 16,
                                               (uint32_t)((row * a.cap + slot + v * 8) * 2), 0, 0, 0);
    }
  };

  auto tile = [&](int t, const bf16* ks_, const bf16* vs_, bf16* kn, bf16* vn) {
    const int kt = k_lo + t * BKV2;
    if (t + 1 < t_end) dma_tile(kt + BKV2, kn, vn);  // overlaps this whole tile
    const bool any = (kt <= wq_hi) && (kt + BKV2 - 1 > wq_lo - a.window);
    const bool full = (kt + BKV2 - 1 <= wq_lo) && (kt > wq_hi - a.window);
    if (any) {
      floatx16 s[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int j = 0; j < 16; ++j) s[kb][qb][j] = 0.f;
#pragma unroll
        for (int ksi = 0; ksi < KS; ++ksi) {
          const bf16x8 kf = *(const bf16x8*)(ks_ + kswz<DH>(kb * 32 + lr, ksi * 2 + lg));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mma32(s[kb][qb], kf, qf[qb][ksi]);
        }
      }
      bf16x8 pf[2][2][QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qp = qw + qb * 32 + lr;
        // the maximum is taken on raw scores and the scale folded into the
        // exponent below (exp2(s sc2 - m) as one fma), sc2 > 0
        float tmax = -INFINITY;
        // the tile-uniform mask decision as its own branch around two
        // versions of the loop (folded into the element test, it costs every
        // element of every tile a save / mask / branch of the lane mask)
        if (full) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, s[kb][qb][j]);
        } else {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int kp = kt + kb * 32 + 8 * (j >> 2) + 4 * lg + (j & 3);
              const float v = (kp <= qp && kp > qp - a.window) ? s[kb][qb][j] : -INFINITY;
              s[kb][qb][j] = v;
              tmax = fmaxf(tmax, v);
            }
        }
        tmax = xor32_max(tmax) * sc2;
        // lazy rescale: keep the reference max unless this tile exceeds it by
        // more than RESCALE (then p <= 2^RESCALE); wave-uniform branch
        const bool need = tmax > m_run[qb] + RESCALE;
        if (__any(need)) {
          const float mnew = need ? tmax : m_run[qb];
          const float corr = (m_run[qb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - mnew);
          l_run[qb] *= corr;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[qb][db] *= corr;
          m_run[qb] = mnew;
        }
        const float nmu = (m_run[qb] == -INFINITY) ? 0.f : -m_run[qb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][j], sc2, nmu));
            s[kb][qb][j] = p;
            rs += p;
          }
        rs = xor32_add(rs);
        l_run[qb] += rs;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[kb][u][qb][e] = (bf16)s[kb][qb][8 * u + e];
      }
      // O^T += V^T P^T over the 64 keys (4 MFMAs of 16 keys each)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int row = db * 32 + lr;
            // keys of this lane's contraction slots are positions
            // 16 u + 8 lg .. + 7 of the tile (vt_slot order): one vector
            const bf16x8 vf = *(const bf16x8*)(vs_ + vswz(row, 4 * kb + 2 * u + lg));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) mma32(o[qb][db], vf, pf[kb][u][qb]);
          }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (t_beg < t_end) dma_tile(k_lo + t_beg * BKV2, Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = t_beg; t < t_end; t += 2) {
    tile(t, Ks0, Vs0, Ks1, Vs1);
    if (t + 1 >= t_end) break;
    tile(t + 1, Ks1, Vs1, Ks0, Vs0);
  }

  if (gridDim.z > 1) {
    // partial: unnormalised output and (max, sum) of this key range
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = qw + qb * 32 + lr;
      if (row >= a.n) continue;
      float* op = a.opart + (long)z * a.n * a.H * DH + ((long)row * a.H + h) * DH;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          floatx4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = o[qb][db][4 * jg + e];
          *(floatx4*)(op + db * 32 + 8 * jg + 4 * lg) = w;
        }
      if (lg == 0) {
        float* ml = a.mlpart + (long)z * 2 * a.H * a.n;
        ml[(long)h * a.n + row] = m_run[qb];
        ml[(long)a.H * a.n + (long)h * a.n + row] = l_run[qb];
      }
    }
    return;
  }

  bf16* O = (bf16*)a.o;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + qb * 32 + lr;
    if (row >= a.n) continue;
    const float inv = l_run[qb] > 0.f ? 1.f / l_run[qb] : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        bf16x4v w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[qb][db][4 * jg + e] * inv);
        *(bf16x4v*)(O + ((long)row * a.H + h) * DH + db * 32 + 8 * jg + 4 * lg) = w;
      }
    if (lg == 0 && a.lse) a.lse[(long)h * a.n + row] = (m_run[qb] + __log2f(l_run[qb])) * LN2;
  }
}

// o = sum_z o_z 2^(m_z - M) / sum_z l_z 2^(m_z - M), lse = (M + log2 L) ln 2;
// one workgroup per query row: the first H threads turn each head's ks
// (m, l) pairs into weights in LDS, then the row's H * DH outputs are
// combined four at a time.
__global__ void __launch_bounds__(256) attn_fwd_combine_kernel(const float* opart, const float* ml, int ks, int n,
                                                               int H, int DH, bf16* o, float* lse) {
  extern __shared__ float cw[];  // [ks][H]
  const int row = blockIdx.x;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float M = -INFINITY;
    for (int z = 0; z < ks; ++z) M = fmaxf(M, ml[(long)z * 2 * H * n + (long)h * n + row]);
    float L = 0.f;
    for (int z = 0; z < ks; ++z) {
      const float mz = ml[(long)z * 2 * H * n + (long)h * n + row];
      const float w = mz == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mz - M);
      L += ml[(long)z * 2 * H * n + (long)H * n + (long)h * n + row] * w;
      cw[z * H + h] = w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int z = 0; z < ks; ++z) cw[z * H + h] *= inv;
    if (lse) lse[(long)h * n + row] = (M + __log2f(L)) * LN2;
  }
  __syncthreads();
  const int W4 = H * DH / 4;  // DH is a multiple of 4
  for (int i = threadIdx.x; i < W4; i += blockDim.x) {
    const int h = i * 4 / DH;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < ks; ++z)
      acc += *(const floatx4*)(opart + (long)z * n * H * DH + (long)row * H * DH + 4 * i) * cw[z * H + h];
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (bf16)acc[e];
    *(bf16x4*)(o + (long)row * H * DH + 4 * i) = r;
  }
}

hipError_t attn_fwd2_combine(const AttnArgs& a, hipStream_t st) {
  const int ks = (a.ksplit > 1 && a.opart && a.mlpart) ? a.ksplit : 1;
  if (ks <= 1 || a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_combine_kernel, dim3(a.n), dim3(256), (size_t)ks * a.H * sizeof(float), st, a.opart,
                     a.mlpart, ks, a.n, a.H, a.dh, (bf16*)a.o, a.lse);
  return hipGetLastError();
}

// Key-range splits for a launch of few query blocks: the split count s
// (1..4, at least 4 key tiles per part) that minimises the per-CU load,
// ceil(base s / 256) parts of 1/s of the keys each, plus a small charge per
// split for the combine pass (measured at 1024 queries x 24 heads: s = 4
// fills 256 CUs evenly and beats s = 3 by a sixth).
int attn_fwd2_splits(const AttnArgs& a) {
  if (a.n <= 0) return 1;
  const long base = (long)((a.n + 127) / 128) * a.H;  // 32 queries per wave
  if (base >= 512) return 1;
  const long tiles = (a.window + 128 + BKV2 - 1) / BKV2;
  int best = 1;
  double best_cost = 1e30;
  for (int s = 1; s <= 4 && (s == 1 || s <= tiles / 4); ++s) {
    const double cost = (double)((base * s + 255) / 256) / s + 0.02 * s;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

bool attn_fwd2_supported(DT dt, const AttnArgs& a) {
  return dt == DT::BF16 && (a.dh == 128 || a.dh == 64) && a.vt != nullptr;
}

static int ks_of(const AttnArgs& a) { return (a.ksplit > 1 && a.opart && a.mlpart) ? a.ksplit : 1; }

hipError_t attn_fwd2(DT dt, const AttnArgs& a, hipStream_t st, int qb) {
  if (a.n <= 0) return hipSuccess;
  if (!attn_fwd2_supported(dt, a)) return hipErrorInvalidValue;
  // qb: 0 = chosen from the shape, 1 = 32 queries per wave (4 waves),
  // 2 = 64 queries per wave, 3 = 32 queries per wave in 8-wave workgroups
  // (one K/V^T tile per CU instead of two). dh 128 with 64 queries per wave
  // runs out of registers (spills) and is no faster even on long prefixes,
  // so it is only taken on request.
  const bool big = qb == 2 || (qb == 0 && a.dh == 64 && (long)((a.n + 255) / 256) * a.H >= 512);
  // 8-wave workgroups are faster on isolated long launches (3-9% at 16384
  // queries x 24 heads) but not inside the prefill step, so only on request
  const bool wide = qb == 3;
  const int ks = ks_of(a);
  const int bq = (big || wide) ? 256 : 128;
  const dim3 grid((a.n + bq - 1) / bq, a.H, ks);
  if (a.dh == 128) {
    if (wide) hipLaunchKernelGGL((attn_fwd2_kernel<128, 1, 8>), grid, dim3(512), 0, st, a);
    else if (big) hipLaunchKernelGGL((attn_fwd2_kernel<128, 2>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_fwd2_kernel<128, 1>), grid, dim3(256), 0, st, a);
  } else {
    if (wide) hipLaunchKernelGGL((attn_fwd2_kernel<64, 1, 8>), grid, dim3(512), 0, st, a);
    else if (big) hipLaunchKernelGGL((attn_fwd2_kernel<64, 2>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_fwd2_kernel<64, 1>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace ttt
