// Decode: the forward of one new token at position p (read from a device
// counter, so the per-token launch sequence can be captured once in a HIP
// graph and replayed) through every block, with the window's keys/values
// from the rings and the dynamic MLPs under the current fp32 fast-weight
// masters ([P1] "TTT-E2E：端到端测试时训练的长上下文语言建模", 推理: decoding
// with a constant-size window cache; [P2] 另辟蹊径: per-token cost does not
// grow with the context). Activations are fp32; every product reads its
// weights once, so the step is bound by HBM bandwidth.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

namespace {
constexpr int GV_THREADS = 256;
constexpr int GV_ROWS = 4;   // rows per wave (two pairs)

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  __syncthreads();
  return s;
}
}  // namespace

// Destinations of the ROPE epilogue: the query row (fp32 [H dh]) and the
// key / value rings ([Hk][cap][dh], values also transposed [Hk][dh][cap] at
// vt_slot()) of the decode step at position *pos.
struct GvRope {
  const int64_t* pos;
  const float2* tab;  // cos / sin per (position, frequency)
  float* q;
  void* ks;
  void* vs;
  void* vts;  // may be null
  int H, Hk, dh, cap;
};

// Rows (r0, r1) that pair p of a GEMV produces together: adjacent rows,
// the (gate, up) rows of the 16-interleaved SwiGLU layout, or the two rows
// (j, j + dh / 2) of one head that RoPE rotates together.
template <int EPI>
__device__ __forceinline__ void gv_pair_rows(int p, int N, int half, int& r0, int& r1) {
  if constexpr (EPI == (int)GvEpi::SWIGLU) {
    r0 = (p >> 4) * 32 + (p & 15);
    r1 = r0 + 16;
  } else if constexpr (EPI == (int)GvEpi::ROPE) {
    const int hh = p / half, j = p - hh * half;
    r0 = hh * 2 * half + j;
    r1 = r0 + half;
  } else {
    r0 = 2 * p;
    r1 = min(2 * p + 1, N - 1);
  }
}

template <int EPI>
__host__ __device__ __forceinline__ int gv_npairs(int N) {
  return EPI == (int)GvEpi::SWIGLU || EPI == (int)GvEpi::ROPE ? N / 2 : (N + 1) / 2;
}

// Writes the results (a, c) of rows (r0, r1) of pair p.
template <typename TW, int EPI>
__device__ __forceinline__ void gv_store_pair(int p, float a, float c, int N, float* y, const GvRope& rp) {
  if constexpr (EPI == (int)GvEpi::SWIGLU) {
    y[p] = silu_f(a) * c;
  } else if constexpr (EPI == (int)GvEpi::ROPE) {
    const int half = rp.dh / 2;
    const int hh = p / half, j = p - hh * half;
    const int64_t pos = *rp.pos;
    const long slot = pos & (rp.cap - 1);
    if (hh < rp.H + rp.Hk) {
      const float2 cs = rp.tab[pos * half + j];
      const float ra = a * cs.x - c * cs.y, rb = c * cs.x + a * cs.y;
      if (hh < rp.H) {
        rp.q[hh * rp.dh + j] = ra;
        rp.q[hh * rp.dh + j + half] = rb;
      } else {
        TW* ks = (TW*)rp.ks + ((long)(hh - rp.H) * rp.cap + slot) * rp.dh;
        ks[j] = from_f<TW>(ra);
        ks[j + half] = from_f<TW>(rb);
      }
    } else {
      const int kh = hh - rp.H - rp.Hk;
      const TW va = from_f<TW>(a), vc = from_f<TW>(c);
      TW* vs = (TW*)rp.vs + ((long)kh * rp.cap + slot) * rp.dh;
      vs[j] = va;
      vs[j + half] = vc;
      if (rp.vts) {
        TW* vt = (TW*)rp.vts + (long)kh * rp.dh * rp.cap + vt_slot(slot);
        vt[(long)j * rp.cap] = va;
        vt[(long)(j + half) * rp.cap] = vc;
      }
    }
  } else {
    const int n = 2 * p;
    if constexpr (EPI == (int)GvEpi::ADD_F32) {
      y[n] += a;
      if (n + 1 < N) y[n + 1] += c;
    } else {
      y[n] = a;
      if (n + 1 < N) y[n + 1] = c;
    }
  }
}

// 16 bytes of weights -> floats (bf16 widens by a shift).
__device__ __forceinline__ void gv_unpack(const uint4& u, float (&o)[8]) {
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void gv_unpack(const uint4& u, float (&o)[4]) {
  o[0] = __uint_as_float(u.x);
  o[1] = __uint_as_float(u.y);
  o[2] = __uint_as_float(u.z);
  o[3] = __uint_as_float(u.w);
}

// The GEMVs below compute y = W x for one row x (fp32 [K]); W [N][K]
// row-major (nn.Linear layout), fp32 or bf16. NORM: x is RMS-normalised
// with gain g first; since RMSNorm(x) g = r (x g) with the scalar
// r = 1 / rms(x), the products use x g and the sums are scaled by r at the
// end, r coming from the same pass over x. EPI: STORE y[n] = acc; ADD_F32
// y[n] += acc; SWIGLU: rows are the 16-interleaved (gate, up) layout and
// y[j] = silu(gate_j) * up_j; ROPE: the fused q/k/v projection, stored
// rotated into q and the rings (gv_store_pair). Rows come in pairs, GV_ROWS
// (two pairs) per wave. Every load a lane needs for a sweep is issued
// before any is used (out-of-range lanes load a clamped, valid address and
// drop the value), so a sweep costs one memory latency, not one per vector;
// lane l reads vectors l, l + 64, ... of its range, so a wave instruction
// reads 1 KB of a row.

// Few rows: the four waves of a workgroup share its GV_ROWS rows and take
// a quarter of K each; each lane loads the x (and g) elements that match
// its weight vectors straight from global memory (no staging, no barrier
// before the products), and the partial sums (and the sum of squares of x)
// meet in LDS.
template <typename TW, int EPI, bool NORM, int NVL>
__global__ void __launch_bounds__(GV_THREADS) gemv_split_kernel(const TW* __restrict__ W, const float* __restrict__ x,
                                                                const float* __restrict__ g, float eps, int N, int K,
                                                                float* __restrict__ y, GvRope rp) {
  __shared__ float part[GV_THREADS / 64][GV_ROWS + 1];
  constexpr int VE = 16 / sizeof(TW);
  constexpr int NWV = GV_THREADS / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int npairs = gv_npairs<EPI>(N);
  const int p0 = blockIdx.x * (GV_ROWS / 2);
  const int nv = K / VE;
  const uint4* Wr[GV_ROWS];
#pragma unroll
  for (int i = 0; i < GV_ROWS / 2; ++i) {
    int r0, r1;
    gv_pair_rows<EPI>(min(p0 + i, npairs - 1), N, rp.dh / 2, r0, r1);
    Wr[2 * i] = (const uint4*)W + (long)r0 * nv;
    Wr[2 * i + 1] = (const uint4*)W + (long)r1 * nv;
  }
  const int q = (nv + NWV - 1) / NWV;
  const int kb = min(nv, wid * q), ke = min(nv, kb + q);
  floatx4 xr[NVL][VE / 4], gr[NVL][VE / 4];
  uint4 wr[NVL][GV_ROWS];
#pragma unroll
  for (int v = 0; v < NVL; ++v)
    if (kb + 64 * v < ke) {  // wave-uniform
      const int vi = min(kb + 64 * v + lane, nv - 1);
#pragma unroll
      for (int u = 0; u < VE / 4; ++u) {
        xr[v][u] = ((const floatx4*)x)[vi * (VE / 4) + u];
        if constexpr (NORM) gr[v][u] = ((const floatx4*)g)[vi * (VE / 4) + u];
      }
    }
#pragma unroll
  for (int v = 0; v < NVL; ++v)
    if (kb + 64 * v < ke) {
      const int vi = min(kb + 64 * v + lane, nv - 1);
#pragma unroll
      for (int r = 0; r < GV_ROWS; ++r) wr[v][r] = Wr[r][vi];
    }
  float acc[GV_ROWS], ss = 0.f;
#pragma unroll
  for (int r = 0; r < GV_ROWS; ++r) acc[r] = 0.f;
#pragma unroll
  for (int v = 0; v < NVL; ++v)
    if (kb + 64 * v < ke && kb + 64 * v + lane < ke) {
      float xv[VE];
#pragma unroll
      for (int u = 0; u < VE / 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = xr[v][u][e];
          if constexpr (NORM) {
            ss = fmaf(t, t, ss);
            xv[4 * u + e] = t * gr[v][u][e];
          } else {
            xv[4 * u + e] = t;
          }
        }
#pragma unroll
      for (int r = 0; r < GV_ROWS; ++r) {
        float wv[VE];
        gv_unpack(wr[v][r], wv);
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[r] = fmaf(wv[e], xv[e], acc[r]);
      }
    }
#pragma unroll
  for (int r = 0; r < GV_ROWS; ++r) acc[r] = wave_sum(acc[r]);
  if constexpr (NORM) ss = wave_sum(ss);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r) part[wid][r] = acc[r];
    part[wid][GV_ROWS] = ss;
  }
  __syncthreads();
  if (threadIdx.x < GV_ROWS / 2) {
    const int i = threadIdx.x;
    if (p0 + i < npairs) {
      float a = 0.f, c = 0.f, sq = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        a += part[w][2 * i];
        c += part[w][2 * i + 1];
        sq += part[w][GV_ROWS];
      }
      if constexpr (NORM) {
        const float rn = rsqrtf(sq / K + eps);
        a *= rn;
        c *= rn;
      }
      gv_store_pair<TW, EPI>(p0 + i, a, c, N, y, rp);
    }
  }
}

// Many rows: a persistent grid; each workgroup stages x g (float4 loads)
// in LDS once, and each wave then sweeps its own groups of GV_ROWS rows
// over all of K, group after group (the first group's weights requested
// before the staging). K is read in chunks of 64 NVL vectors.
template <typename TW, int EPI, bool NORM, int NVL>
__global__ void __launch_bounds__(GV_THREADS) gemv_rows_kernel(const TW* __restrict__ W, const float* __restrict__ x,
                                                               const float* __restrict__ g, float eps, int N, int K,
                                                               float* __restrict__ y, GvRope rp) {
  extern __shared__ float xs[];
  __shared__ float red[GV_THREADS / 64];
  constexpr int VE = 16 / sizeof(TW);
  constexpr int NWV = GV_THREADS / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int npairs = gv_npairs<EPI>(N);
  const int ngroups = (npairs + GV_ROWS / 2 - 1) / (GV_ROWS / 2);
  const int nv = K / VE;
  const int gstride = gridDim.x * NWV;
  int grp = blockIdx.x * NWV + wid;
  const uint4* Wr[GV_ROWS];
  auto set_rows = [&](int gi) {
#pragma unroll
    for (int i = 0; i < GV_ROWS / 2; ++i) {
      int r0, r1;
      gv_pair_rows<EPI>(max(0, min(gi * (GV_ROWS / 2) + i, npairs - 1)), N, rp.dh / 2, r0, r1);
      Wr[2 * i] = (const uint4*)W + (long)r0 * nv;
      Wr[2 * i + 1] = (const uint4*)W + (long)r1 * nv;
    }
  };
  uint4 wr[NVL][GV_ROWS];
  auto load = [&](int c0) {
#pragma unroll
    for (int v = 0; v < NVL; ++v)
      if (c0 + 64 * v < nv) {  // wave-uniform
        const int vi = min(c0 + 64 * v + lane, nv - 1);
#pragma unroll
        for (int r = 0; r < GV_ROWS; ++r) wr[v][r] = Wr[r][vi];
      }
  };
  set_rows(grp);
  if (grp < ngroups) load(0);
  // stage x g; sum of squares of x for the norm
  float ss = 0.f;
  const int K4 = K / 4;
  for (int b = 0; b < K4; b += 4 * GV_THREADS) {
    floatx4 xv[4], gv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = b + u * GV_THREADS + threadIdx.x;
      if (i < K4) {
        xv[u] = ((const floatx4*)x)[i];
        if constexpr (NORM) gv[u] = ((const floatx4*)g)[i];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = b + u * GV_THREADS + threadIdx.x;
      if (i < K4) {
        floatx4 t = xv[u];
        if constexpr (NORM) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ss = fmaf(t[e], t[e], ss);
            t[e] *= gv[u][e];
          }
        }
        ((floatx4*)xs)[i] = t;
      }
    }
  }
  float rn = 1.f;
  if constexpr (NORM) rn = rsqrtf(block_sum(ss, red) / K + eps);
  else __syncthreads();
  for (; grp < ngroups; grp += gstride) {
    float acc[GV_ROWS];
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r) acc[r] = 0.f;
    for (int c0 = 0; c0 < nv; c0 += 64 * NVL) {
      if (c0 != 0) load(c0);
#pragma unroll
      for (int v = 0; v < NVL; ++v) {
        const int vi = c0 + 64 * v + lane;
        if (c0 + 64 * v < nv && vi < nv) {
          float xv[VE];
          const floatx4* xp = (const floatx4*)(xs + vi * VE);
#pragma unroll
          for (int u = 0; u < VE / 4; ++u) {
            const floatx4 t = xp[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[4 * u + e] = t[e];
          }
#pragma unroll
          for (int r = 0; r < GV_ROWS; ++r) {
            float wv[VE];
            gv_unpack(wr[v][r], wv);
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[r] = fmaf(wv[e], xv[e], acc[r]);
          }
        }
      }
    }
    const int p0 = grp * (GV_ROWS / 2);
    // the next group's first chunk is requested before this one's sums
    // are reduced and stored
    set_rows(grp + gstride);
    if (grp + gstride < ngroups) load(0);
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r) acc[r] = wave_sum(acc[r]) * rn;
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < GV_ROWS / 2; ++i)
        if (p0 + i < npairs) gv_store_pair<TW, EPI>(p0 + i, acc[2 * i], acc[2 * i + 1], N, y, rp);
  }
}

template <typename TW, int EPI, bool NORM, int NVL>
static int gemv_rows_grid(size_t lds) {
  // workgroups that fit on the current device at once, kept per host thread
  // for the last (device, LDS size) asked for
  static thread_local size_t last_lds = 0;
  static thread_local int last_dev = -1;
  static thread_local int n = 0;
  int cur = 0;
  (void)hipGetDevice(&cur);
  if (lds != last_lds || cur != last_dev) {
    int cus = 0, per = 0;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, cur);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, gemv_rows_kernel<TW, EPI, NORM, NVL>, GV_THREADS, lds);
    n = std::max(1, cus) * std::max(1, per);
    last_lds = lds;
    last_dev = cur;
  }
  return n;
}

template <typename TW, int EPI, bool NORM, int NVL>
static void gemv_rows_launch(int groups, size_t lds, hipStream_t st, const TW* W, const float* x, const float* g,
                             float eps, int N, int K, float* y, const GvRope& rp) {
  const int need = (groups + GV_THREADS / 64 - 1) / (GV_THREADS / 64);
  const int blocks = std::min(need, gemv_rows_grid<TW, EPI, NORM, NVL>(lds));
  hipLaunchKernelGGL((gemv_rows_kernel<TW, EPI, NORM, NVL>), dim3(blocks), dim3(GV_THREADS), lds, st, W, x, g, eps, N,
                     K, y, rp);
}

template <typename TW, int EPI, bool NORM>
static void gemv_dispatch(const TW* W, const float* x, const float* g, float eps, int N, int K, float* y,
                          const GvRope& rp, hipStream_t st) {
  const int npairs = gv_npairs<EPI>(N);
  const int nv = K / (16 / (int)sizeof(TW));
  // many rows: a wave per GV_ROWS rows keeps enough loads in flight; few
  // rows: split K over the waves of a workgroup to occupy more of the chip
  const int groups = (npairs + GV_ROWS / 2 - 1) / (GV_ROWS / 2);
  if (groups >= 2048) {
    const size_t lds = (size_t)K * sizeof(float);
    const int nvl = (nv + 63) / 64;
    if (nvl <= 4) gemv_rows_launch<TW, EPI, NORM, 4>(groups, lds, st, W, x, g, eps, N, K, y, rp);
    else if (nvl <= 6) gemv_rows_launch<TW, EPI, NORM, 6>(groups, lds, st, W, x, g, eps, N, K, y, rp);
    else gemv_rows_launch<TW, EPI, NORM, 8>(groups, lds, st, W, x, g, eps, N, K, y, rp);
    return;
  }
  const int nvl = ((nv + 3) / 4 + 63) / 64;
  if (nvl <= 2)
    hipLaunchKernelGGL((gemv_split_kernel<TW, EPI, NORM, 2>), dim3(groups), dim3(GV_THREADS), 0, st, W, x, g, eps, N, K, y, rp);
  else if (nvl <= 4)
    hipLaunchKernelGGL((gemv_split_kernel<TW, EPI, NORM, 4>), dim3(groups), dim3(GV_THREADS), 0, st, W, x, g, eps, N, K, y, rp);
  else
    hipLaunchKernelGGL((gemv_split_kernel<TW, EPI, NORM, 8>), dim3(groups), dim3(GV_THREADS), 0, st, W, x, g, eps, N, K, y, rp);
}

template <typename TW, int EPI>
static hipError_t gemv_t(const TW* W, const float* x, const float* g, float eps, int N, int K, float* y,
                         const GvRope& rp, hipStream_t st) {
  if (g) gemv_dispatch<TW, EPI, true>(W, x, g, eps, N, K, y, rp, st);
  else gemv_dispatch<TW, EPI, false>(W, x, g, eps, N, K, y, rp, st);
  return hipGetLastError();
}

hipError_t gemv(DT wdt, const void* W, const float* x, const float* g, float eps, int N, int K, GvEpi epi,
                float* y, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if ((K * 4) > 64 * 1024 || K % 8) return hipErrorInvalidValue;
  const GvRope rp{};
  if (wdt == DT::BF16) {
    switch (epi) {
      case GvEpi::STORE: return gemv_t<bf16, (int)GvEpi::STORE>((const bf16*)W, x, g, eps, N, K, y, rp, st);
      case GvEpi::ADD_F32: return gemv_t<bf16, (int)GvEpi::ADD_F32>((const bf16*)W, x, g, eps, N, K, y, rp, st);
      case GvEpi::SWIGLU: return gemv_t<bf16, (int)GvEpi::SWIGLU>((const bf16*)W, x, g, eps, N, K, y, rp, st);
      default: break;
    }
  } else {
    switch (epi) {
      case GvEpi::STORE: return gemv_t<float, (int)GvEpi::STORE>((const float*)W, x, g, eps, N, K, y, rp, st);
      case GvEpi::ADD_F32: return gemv_t<float, (int)GvEpi::ADD_F32>((const float*)W, x, g, eps, N, K, y, rp, st);
      case GvEpi::SWIGLU: return gemv_t<float, (int)GvEpi::SWIGLU>((const float*)W, x, g, eps, N, K, y, rp, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t gemv_qkv_rope(DT dt, const void* W, const float* x, const float* g, float eps, int H, int Hk, int dh,
                         int K, const int64_t* pos, const float2* rope_tab, float* q, void* kstore, void* vstore,
                         void* vtstore, int cap, hipStream_t st) {
  if ((K * 4) > 64 * 1024 || K % 8 || dh % 2) return hipErrorInvalidValue;
  const int N = (H + 2 * Hk) * dh;
  const GvRope rp{pos, rope_tab, q, kstore, vstore, vtstore, H, Hk, dh, cap};
  if (dt == DT::BF16)
    return gemv_t<bf16, (int)GvEpi::ROPE>((const bf16*)W, x, g, eps, N, K, nullptr, rp, st);
  return gemv_t<float, (int)GvEpi::ROPE>((const float*)W, x, g, eps, N, K, nullptr, rp, st);
}

// ------------------------------------------------------------- embedding
template <typename T>
__global__ void embed_row_kernel(const int32_t* tok, const T* E, int d, int V, float* h, int* err) {
  int t = *tok;
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    t = 0;
  }
  for (int i = threadIdx.x; i < d; i += blockDim.x) h[i] = to_f(E[(long)t * d + i]);
}

hipError_t embed_row(DT dt, const int32_t* tok, const void* embed, int d, int V, float* h, int* err,
                     hipStream_t st) {
  if (dt == DT::BF16)
    hipLaunchKernelGGL(embed_row_kernel<bf16>, dim3(1), dim3(256), 0, st, tok, (const bf16*)embed, d, V, h, err);
  else
    hipLaunchKernelGGL(embed_row_kernel<float>, dim3(1), dim3(256), 0, st, tok, (const float*)embed, d, V, h, err);
  return hipGetLastError();
}

// ------------------------------------------------------- window attention
// One query per head at position p over keys (p - window, p]. Workgroup
// (kv head, split) takes a contiguous chunk of the window for the query
// heads of that key head; LPR lanes cover one key row in 16-byte vectors,
// so a wave instruction reads 64 / LPR whole rows. Each lane group keeps an
// online softmax (max, sum, output slice); the groups and waves are merged
// through LDS into one partial (m, l, o) per (head, split).
template <typename T, int DH, int GMAX>
__global__ void __launch_bounds__(256) decode_attn_kernel(const float* q, const T* kst, const T* vst, int H, int Hk,
                                                          int cap, int window, const int64_t* pos, float scale,
                                                          int nsplit, float* part) {
  constexpr int EV = 16 / sizeof(T);     // elements per 16-byte vector
  constexpr int LPR = DH / EV;           // lanes per key row
  constexpr int KPW = 64 / LPR;          // keys per wave instruction
  // GMAX = query heads per key head (the group)
  __shared__ float sm[4 * KPW][GMAX], sl[4 * KPW][GMAX];
  __shared__ float so[4 * KPW][DH];
  const int kh = blockIdx.x, split = blockIdx.y;
  const int grp = H / Hk;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane % LPR, kg = lane / LPR;  // vector within the row, key slot of the wave
  const int slotid = wid * KPW + kg;            // 0 .. 4 KPW - 1
  const int64_t p = *pos;
  const int64_t lo = p - window + 1 > 0 ? p - window + 1 : 0;
  const int64_t count = p - lo + 1;
  const int64_t chunk = ((count + nsplit - 1) / nsplit + 4 * KPW - 1) / (4 * KPW) * (4 * KPW);  // whole key groups
  const int64_t c0 = lo + (int64_t)split * chunk, c1 = min(p + 1, c0 + chunk);

  float qv[GMAX][EV];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int e = 0; e < EV; ++e) qv[g][e] = g < grp ? q[(kh * grp + g) * DH + sub * EV + e] * scale : 0.f;
  float m[GMAX], l[GMAX], o[GMAX][EV];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) o[g][e] = 0.f;
  }
  const T* kb = kst + (long)kh * cap * DH;
  const T* vb = vst + (long)kh * cap * DH;
  constexpr int UNR = 4;  // key groups whose loads are in flight together
  for (int64_t t0 = c0; t0 < c1; t0 += 4 * KPW * UNR) {
    float kv[UNR][EV], vv[UNR][EV];
    bool okv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t t = t0 + u * 4 * KPW + slotid;
      okv[u] = t < c1;  // uniform over the LPR lanes of a key row
      const long slot = (long)(t & (cap - 1));
#pragma unroll
      for (int e = 0; e < EV; ++e) kv[u][e] = vv[u][e] = 0.f;
      if (okv[u]) {
        if constexpr (sizeof(T) == 2) {
          const bf16x8 a = *(const bf16x8*)(kb + slot * DH + sub * EV);
          const bf16x8 b = *(const bf16x8*)(vb + slot * DH + sub * EV);
#pragma unroll
          for (int e = 0; e < EV; ++e) {
            kv[u][e] = (float)a[e];
            vv[u][e] = (float)b[e];
          }
        } else {
          const floatx4 a = *(const floatx4*)(kb + slot * DH + sub * EV);
          const floatx4 b = *(const floatx4*)(vb + slot * DH + sub * EV);
#pragma unroll
          for (int e = 0; e < EV; ++e) {
            kv[u][e] = a[e];
            vv[u][e] = b[e];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g >= grp) break;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) s += qv[g][e] * kv[u][e];
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        if (okv[u]) {
          const float mn = fmaxf(m[g], s);
          const float c = __expf(m[g] - mn), pe = __expf(s - mn);
          l[g] = l[g] * c + pe;
#pragma unroll
          for (int e = 0; e < EV; ++e) o[g][e] = o[g][e] * c + pe * vv[u][e];
          m[g] = mn;
        }
      }
    }
  }
  // merge the 4 KPW lane groups of the workgroup, one query head at a time
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= grp) break;
    if (sub == 0) {
      sm[slotid][g] = m[g];
      sl[slotid][g] = l[g];
    }
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= grp) break;
    float M = -INFINITY;
    for (int i = 0; i < 4 * KPW; ++i) M = fmaxf(M, sm[i][g]);
    const float w = (m[g] == -INFINITY) ? 0.f : __expf(m[g] - M);
#pragma unroll
    for (int e = 0; e < EV; ++e) so[slotid][sub * EV + e] = o[g][e] * w;
    __syncthreads();
    float* dst = part + ((long)(kh * grp + g) * nsplit + split) * (DH + 2);
    for (int dd = threadIdx.x; dd < DH; dd += blockDim.x) {
      float acc = 0.f;
      for (int i = 0; i < 4 * KPW; ++i) acc += so[i][dd];
      dst[dd] = acc;
    }
    if (threadIdx.x == 0) {
      float L = 0.f;
      for (int i = 0; i < 4 * KPW; ++i)
        if (sm[i][g] != -INFINITY) L += sl[i][g] * __expf(sm[i][g] - M);
      dst[DH] = M;
      dst[DH + 1] = L;
    }
    __syncthreads();
  }
}

// o[h] = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}: the split weights
// are formed once per head in LDS; then thread t sums the splits
// s = t / dh (mod 256 / dh) of column t % dh, eight loads in flight, and
// the column's partial sums meet in LDS.
__global__ void __launch_bounds__(256) decode_attn_combine_kernel(const float* part, int nsplit, int dh, float* o) {
  __shared__ float wsh[256];
  __shared__ float csum[256];
  __shared__ float Lsh;
  const int h = blockIdx.x;
  const float* ph = part + (long)h * nsplit * (dh + 2);
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float mloc = -INFINITY;
    for (int s = lane; s < nsplit; s += 64) mloc = fmaxf(mloc, ph[s * (dh + 2) + dh]);
    const float M = wave_max(mloc);
    float lsum = 0.f;
    for (int s = lane; s < nsplit; s += 64) {
      const float ms = ph[s * (dh + 2) + dh];
      const float w = ms == -INFINITY ? 0.f : __expf(ms - M);
      wsh[s] = w;
      lsum += ph[s * (dh + 2) + dh + 1] * w;
    }
    const float L = wave_sum(lsum);
    if (lane == 0) Lsh = L;
  }
  __syncthreads();
  const int nsub = blockDim.x / dh;
  const int dd = threadIdx.x % dh, sub = threadIdx.x / dh;
  float acc = 0.f;
  if (sub < nsub) {
#pragma unroll 8
    for (int s = sub; s < nsplit; s += nsub) acc += ph[s * (dh + 2) + dd] * wsh[s];
  }
  csum[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < dh) {
    float t = 0.f;
    for (int u = 0; u < nsub; ++u) t += csum[u * dh + threadIdx.x];
    o[h * dh + threadIdx.x] = t / Lsh;
  }
}

// Window attention of one token on MFMA (bf16 stores, dh 64 / 128, up to 16
// query heads per key head). Workgroup (key head, split) of 4 waves; wave w
// of split s takes the key blocks of 32 positions (aligned to 32, so a block
// never wraps the ring) blk = b0 + 4 s + w + i * 4 nsplit. Per block:
//   S^T [32 keys x 16 queries] = K Q^T as two 16x16x32 tiles per 32 of dh,
//   masked to the window, exponentiated (base 2, scale folded into q) after
//   the running maximum is raised to the block's;
//   O^T [dh x 16] += V^T P^T with V^T read from the transposed store.
// The PV product's k-slot 8 g + e (lane group g) is key 4 g + e for e < 4 and
// 16 + 4 g + (e - 4) otherwise: exactly the keys the S^T tiles leave in lane
// group g, so P goes from the accumulators to the B operand without a lane
// exchange; under the store's slot permutation (bits 2 and 3 swapped) those
// four keys sit at four consecutive slots of each 16-slot group. The waves
// merge through LDS into one (o, max, sum) partial per (query head, split),
// max in natural-log units for the combine kernel.
constexpr float LN2F = 0.6931471805599453f;

template <int DH>
__global__ void __launch_bounds__(256) decode_attn_mfma_kernel(const float* q, const bf16* kst, const bf16* vts,
                                                               int H, int Hk, int cap, int window,
                                                               const int64_t* pos, float scale2, int nsplit,
                                                               float* part) {
  constexpr int KS = DH / 32;  // 32-wide steps of the QK product
  constexpr int MT = DH / 16;  // 16-row tiles of O^T
  __shared__ float sm[4][16], sl[4][16];
  __shared__ float so[4][DH][17];
  const int kh = blockIdx.x, split = blockIdx.y;
  const int G = H / Hk;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t p = *pos;
  const int64_t lo = p - window + 1 > 0 ? p - window + 1 : 0;
  const int64_t b0 = lo >> 5, b1 = p >> 5;

  // query rows as 16-byte loads from a valid row (lanes past the group read
  // its last row and zero it), all issued before any is used: a load under
  // the lane condition becomes a branch with its own wait per element
  Frag8<bf16> qf[KS];
  {
    const floatx4* qr = (const floatx4*)(q + (long)(kh * G + min(c, G - 1)) * DH + 8 * g);
    floatx4 qv[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qv[s][0] = qr[8 * s];
      qv[s][1] = qr[8 * s + 1];
    }
    const float qs = c < G ? scale2 : 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s].v[e] = (bf16)(qv[s][e >> 2][e & 3] * qs);
  }
  float m = -INFINITY, l = 0.f;
  floatx4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const bf16* kb = kst + (long)kh * cap * DH;
  const bf16* vb = vts + (long)kh * DH * cap;
  const int vo = 8 * (g & 1) + 4 * (g >> 1);
  for (int64_t blk = b0 + 4 * split + wid; blk <= b1; blk += 4 * (int64_t)nsplit) {
    const long base = (long)((blk << 5) & (cap - 1));
    Frag8<bf16> kf[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s) ld8(kf[t][s], kb + (base + 16 * t + c) * DH + 32 * s + 8 * g);
    Frag8<bf16> vf[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16* row = vb + (long)(16 * mt + c) * cap + base + vo;
      const bf16x4 a = *(const bf16x4*)row;
      const bf16x4 bq = *(const bf16x4*)(row + 16);
      vf[mt].v = __builtin_shufflevector(a, bq, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    floatx4 st[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s) mma16(st[t], kf[t][s], qf[s]);
    float sv[8];
    float bm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t pk = (blk << 5) + 16 * t + 4 * g + j;
        const float x = (pk >= lo && pk <= p) ? st[t][j] : -INFINITY;
        sv[4 * t + j] = x;
        bm = fmaxf(bm, x);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = fmaxf(m, bm);
    if (mn == -INFINITY) continue;  // no key of the window so far (the same for every lane)
    const float cr = __builtin_amdgcn_exp2f(m - mn);
    float ps = 0.f;
    Frag8<bf16> pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(sv[e] - mn);
      ps += pe;
      pf.v[e] = (bf16)pe;
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = l * cr + ps;
    m = mn;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      o[mt] *= cr;
      mma16(o[mt], vf[mt], pf);
    }
  }
  if (g == 0) {
    sm[wid][c] = m;
    sl[wid][c] = l;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) so[wid][16 * mt + 4 * g + j][c] = o[mt][j];
  __syncthreads();
  for (int e = threadIdx.x; e < G * DH; e += blockDim.x) {
    const int qc = e / DH, dd = e % DH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][qc]);
    float acc = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float ww = __builtin_amdgcn_exp2f(sm[w][qc] - M);
        acc += ww * so[w][dd][qc];
        L += ww * sl[w][qc];
      }
    }
    float* dst = part + ((long)(kh * G + qc) * nsplit + split) * (DH + 2);
    dst[dd] = acc;
    if (dd == 0) {
      dst[DH] = M == -INFINITY ? -INFINITY : M * LN2F;
      dst[DH + 1] = L;
    }
  }
}

template <typename T, int DH>
static hipError_t decode_attn_t(const float* q, const void* ks, const void* vs, int H, int Hk, int cap,
                                int window, const int64_t* pos, float* part, float* o, int nsplit,
                                hipStream_t st) {
  const dim3 grid(Hk, nsplit);
  const float sc = 1.f / sqrtf((float)DH);
  switch (H / Hk) {
    case 1: hipLaunchKernelGGL((decode_attn_kernel<T, DH, 1>), grid, dim3(256), 0, st, q, (const T*)ks, (const T*)vs, H, Hk, cap, window, pos, sc, nsplit, part); break;
    case 2: hipLaunchKernelGGL((decode_attn_kernel<T, DH, 2>), grid, dim3(256), 0, st, q, (const T*)ks, (const T*)vs, H, Hk, cap, window, pos, sc, nsplit, part); break;
    case 3: hipLaunchKernelGGL((decode_attn_kernel<T, DH, 3>), grid, dim3(256), 0, st, q, (const T*)ks, (const T*)vs, H, Hk, cap, window, pos, sc, nsplit, part); break;
    case 4: hipLaunchKernelGGL((decode_attn_kernel<T, DH, 4>), grid, dim3(256), 0, st, q, (const T*)ks, (const T*)vs, H, Hk, cap, window, pos, sc, nsplit, part); break;
    case 8: hipLaunchKernelGGL((decode_attn_kernel<T, DH, 8>), grid, dim3(256), 0, st, q, (const T*)ks, (const T*)vs, H, Hk, cap, window, pos, sc, nsplit, part); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(decode_attn_combine_kernel, dim3(H), dim3(256), 0, st, part, nsplit, DH, o);
  return hipGetLastError();
}

static bool decode_mfma_ok(DT dt, int H, int Hk, int dh, bool has_vt) {
  return dt == DT::BF16 && has_vt && (dh == 64 || dh == 128) && H / Hk <= 16;
}

int decode_attn_splits(DT dt, int H, int Hk, int dh, int window, bool has_vt) {
  if (!decode_mfma_ok(dt, H, Hk, dh, has_vt)) return 64;
  // one 32-key block per wave: the window touches at most window / 32 + 1 blocks
  const long blocks = (long)window / 32 + 1;
  const long s = (blocks + 3) / 4;
  return (int)std::min<long>(std::max<long>(s, 1), 256);
}

hipError_t decode_attn(DT dt, const float* q, const void* kstore, const void* vstore, const void* vtstore, int H,
                       int Hk, int dh, int cap, int window, const int64_t* pos, float* part, float* o,
                       hipStream_t st) {
  const int nsplit = decode_attn_splits(dt, H, Hk, dh, window, vtstore != nullptr);
  if (decode_mfma_ok(dt, H, Hk, dh, vtstore != nullptr)) {
    if ((uintptr_t)q & 15) return hipErrorInvalidValue;  // query rows are read as 16-byte vectors
    const dim3 grid(Hk, nsplit);
    const float sc2 = 1.f / sqrtf((float)dh) * 1.4426950408889634f;
    if (dh == 128)
      hipLaunchKernelGGL(decode_attn_mfma_kernel<128>, grid, dim3(256), 0, st, q, (const bf16*)kstore,
                         (const bf16*)vtstore, H, Hk, cap, window, pos, sc2, nsplit, part);
    else
      hipLaunchKernelGGL(decode_attn_mfma_kernel<64>, grid, dim3(256), 0, st, q, (const bf16*)kstore,
                         (const bf16*)vtstore, H, Hk, cap, window, pos, sc2, nsplit, part);
    hipLaunchKernelGGL(decode_attn_combine_kernel, dim3(H), dim3(256), 0, st, part, nsplit, dh, o);
    return hipGetLastError();
  }
  if (dt == DT::BF16) {
    if (dh == 128) return decode_attn_t<bf16, 128>(q, kstore, vstore, H, Hk, cap, window, pos, part, o, nsplit, st);
    if (dh == 64) return decode_attn_t<bf16, 64>(q, kstore, vstore, H, Hk, cap, window, pos, part, o, nsplit, st);
    if (dh == 16) return decode_attn_t<bf16, 16>(q, kstore, vstore, H, Hk, cap, window, pos, part, o, nsplit, st);
  } else {
    if (dh == 128) return decode_attn_t<float, 128>(q, kstore, vstore, H, Hk, cap, window, pos, part, o, nsplit, st);
    if (dh == 64) return decode_attn_t<float, 64>(q, kstore, vstore, H, Hk, cap, window, pos, part, o, nsplit, st);
    if (dh == 16) return decode_attn_t<float, 16>(q, kstore, vstore, H, Hk, cap, window, pos, part, o, nsplit, st);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------- position
__global__ void pos_kernel(int64_t* pos, int64_t value, int add) {
  if (threadIdx.x == 0) *pos = add ? *pos + 1 : value;
}

hipError_t bump_pos(int64_t* pos, hipStream_t st) {
  hipLaunchKernelGGL(pos_kernel, dim3(1), dim3(64), 0, st, pos, (int64_t)0, 1);
  return hipGetLastError();
}

hipError_t set_pos(int64_t* pos, int64_t value, hipStream_t st) {
  hipLaunchKernelGGL(pos_kernel, dim3(1), dim3(64), 0, st, pos, value, 0);
  return hipGetLastError();
}

}  // namespace ttt
