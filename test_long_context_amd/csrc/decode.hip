// Decode: the forward of one new token at position p (read from a device
// counter, so the per-token launch sequence can be captured once in a HIP
// graph and replayed) through every block, with the window's keys/values
// from the rings and the dynamic MLPs under the current fp32 fast-weight
// masters ([P1] "TTT-E2E：端到端测试时训练的长上下文语言建模", 推理: decoding
// with a constant-size window cache; [P2] 另辟蹊径: per-token cost does not
// grow with the context). Activations are fp32; every product reads its
// weights once, so the step is bound by HBM bandwidth.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ttt {

namespace {
constexpr int GV_THREADS = 256;
constexpr int GV_ROWS = 4;   // split-K kernel: rows per workgroup (two pairs)
constexpr int GV_RPW = 4;   // row kernel: rows per wave (two pairs)

template <typename TW> struct WVec;  // 16 bytes of weights -> floats
template <> struct WVec<bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const bf16* p, float (&o)[8]) {
    const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
  }
};
template <> struct WVec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float (&o)[4]) {
    const floatx4 v = *(const floatx4*)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[e];
  }
};

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

// y = W x for one row x (fp32 [K]); W [N][K] row-major (nn.Linear layout).
// NORM: x = RMSNorm(h) * g computed by every workgroup while staging x in
// LDS. EPI: STORE y[n] = acc; ADD_F32 y[n] += acc; SWIGLU: rows are the
// 16-interleaved (gate, up) layout and y[j] = silu(gate_j) * up_j.
// Large N: a wave takes GV_RPW rows (two pairs) over the whole K; lanes
// stride the row in 16-byte vectors, so each row is one coalesced sweep.
template <typename TW, int EPI, bool NORM>
__global__ void __launch_bounds__(GV_THREADS) gemv_rows_kernel(const TW* __restrict__ W, const float* __restrict__ x,
                                                          const float* __restrict__ g, float eps, int N, int K,
                                                          float* __restrict__ y) {
  extern __shared__ float xs[];
  __shared__ float red[GV_THREADS / 64];
  constexpr int VE = WVec<TW>::N;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (GV_THREADS / 64) + (threadIdx.x >> 6);
  const int npairs = EPI == (int)GvEpi::SWIGLU ? N / 2 : (N + 1) / 2;
  const int p0 = wave * (GV_RPW / 2);
  const bool active = p0 < npairs;  // waves past the last row still help stage x
  int rows[GV_RPW];
#pragma unroll
  for (int i = 0; i < GV_RPW / 2; ++i) {
    const int p = max(0, min(p0 + i, npairs - 1));
    if constexpr (EPI == (int)GvEpi::SWIGLU) {
      rows[2 * i] = (p >> 4) * 32 + (p & 15);
      rows[2 * i + 1] = rows[2 * i] + 16;
    } else {
      rows[2 * i] = 2 * p;
      rows[2 * i + 1] = min(2 * p + 1, N - 1);
    }
  }
  const int nv = K / VE;
  // the first sweep's weights are requested before x is staged, so their
  // latency overlaps the normalisation
  float w0[GV_RPW][VE];
  const bool first = active && lane < nv;
  if (first)
#pragma unroll
    for (int r = 0; r < GV_RPW; ++r) WVec<TW>::load(W + (long)rows[r] * K + lane * VE, w0[r]);
  if constexpr (NORM) {
    float ss = 0.f;
    for (int k = threadIdx.x; k < K; k += GV_THREADS) ss += x[k] * x[k];
    const float r = rsqrtf(block_sum(ss, red) / K + eps);
    for (int k = threadIdx.x; k < K; k += GV_THREADS) xs[k] = x[k] * r * g[k];
  } else {
    for (int k = threadIdx.x; k < K; k += GV_THREADS) xs[k] = x[k];
  }
  __syncthreads();
  if (!active) return;
  float acc[GV_RPW];
#pragma unroll
  for (int r = 0; r < GV_RPW; ++r) acc[r] = 0.f;
  if (first) {
    float xv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) xv[e] = xs[lane * VE + e];
#pragma unroll
    for (int r = 0; r < GV_RPW; ++r)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[r] += w0[r][e] * xv[e];
  }
  for (int v = lane + 64; v < nv; v += 64) {
    float xv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) xv[e] = xs[v * VE + e];
#pragma unroll
    for (int r = 0; r < GV_RPW; ++r) {
      float wv[VE];
      WVec<TW>::load(W + (long)rows[r] * K + v * VE, wv);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[r] += wv[e] * xv[e];
    }
  }
#pragma unroll
  for (int r = 0; r < GV_RPW; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < GV_RPW / 2; ++i) {
      const int p = p0 + i;
      if (p >= npairs) break;
      if constexpr (EPI == (int)GvEpi::SWIGLU) {
        const float a = acc[2 * i], c = acc[2 * i + 1];
        y[p] = silu_f(a) * c;
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int n = 2 * p + u;
          if (n >= N) break;
          if constexpr (EPI == (int)GvEpi::ADD_F32) y[n] += acc[2 * i + u];
          else y[n] = acc[2 * i + u];
        }
      }
    }
  }
}

// y = W x for one row x (fp32 [K]); W [N][K] row-major (nn.Linear layout).
// NORM: x = RMSNorm(h) * g computed by every workgroup while staging x in
// LDS. EPI: STORE y[n] = acc; ADD_F32 y[n] += acc; SWIGLU: rows are the
// 16-interleaved (gate, up) layout and y[j] = silu(gate_j) * up_j.
// A workgroup takes GV_ROWS rows (GV_ROWS / 2 pairs) and splits K over its
// waves; lanes stride each row's quarter in 16-byte vectors, so every row
// is read once, coalesced, with many loads in flight per lane; the partial
// dot products meet in LDS.
template <typename TW, int EPI, bool NORM>
__global__ void __launch_bounds__(GV_THREADS) gemv_kernel(const TW* __restrict__ W, const float* __restrict__ x,
                                                          const float* __restrict__ g, float eps, int N, int K,
                                                          float* __restrict__ y) {
  extern __shared__ float xs[];
  __shared__ float red[GV_THREADS / 64];
  __shared__ float part[GV_THREADS / 64][GV_ROWS];
  constexpr int VE = WVec<TW>::N;
  constexpr int NWV = GV_THREADS / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int npairs = EPI == (int)GvEpi::SWIGLU ? N / 2 : (N + 1) / 2;
  const int p0 = blockIdx.x * (GV_ROWS / 2);
  int rows[GV_ROWS];
#pragma unroll
  for (int i = 0; i < GV_ROWS / 2; ++i) {
    const int p = min(p0 + i, npairs - 1);
    if constexpr (EPI == (int)GvEpi::SWIGLU) {
      rows[2 * i] = (p >> 4) * 32 + (p & 15);
      rows[2 * i + 1] = rows[2 * i] + 16;
    } else {
      rows[2 * i] = 2 * p;
      rows[2 * i + 1] = min(2 * p + 1, N - 1);
    }
  }
  const int nv = K / VE;
  const int q = (nv + NWV - 1) / NWV;  // vectors per wave
  const int v0 = wid * q, v1 = min(nv, v0 + q);
  // the first sweep's weights are requested before x is staged, so their
  // latency overlaps the normalisation
  float w0[GV_ROWS][VE];
  const bool first = v0 + lane < v1;
  if (first)
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r) WVec<TW>::load(W + (long)rows[r] * K + (v0 + lane) * VE, w0[r]);
  if constexpr (NORM) {
    float ss = 0.f;
    for (int k = threadIdx.x; k < K; k += GV_THREADS) ss += x[k] * x[k];
    const float r = rsqrtf(block_sum(ss, red) / K + eps);
    for (int k = threadIdx.x; k < K; k += GV_THREADS) xs[k] = x[k] * r * g[k];
  } else {
    for (int k = threadIdx.x; k < K; k += GV_THREADS) xs[k] = x[k];
  }
  __syncthreads();
  float acc[GV_ROWS];
#pragma unroll
  for (int r = 0; r < GV_ROWS; ++r) acc[r] = 0.f;
  if (first) {
    float xv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) xv[e] = xs[(v0 + lane) * VE + e];
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[r] += w0[r][e] * xv[e];
  }
  for (int v = v0 + lane + 64; v < v1; v += 64) {
    float xv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) xv[e] = xs[v * VE + e];
    float wv[GV_ROWS][VE];
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r) WVec<TW>::load(W + (long)rows[r] * K + v * VE, wv[r]);
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[r] += wv[r][e] * xv[e];
  }
#pragma unroll
  for (int r = 0; r < GV_ROWS; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r) part[wid][r] = acc[r];
  __syncthreads();
  if (threadIdx.x < GV_ROWS / 2) {
    const int i = threadIdx.x;
    const int p = p0 + i;
    if (p < npairs) {
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        a += part[w][2 * i];
        c += part[w][2 * i + 1];
      }
      if constexpr (EPI == (int)GvEpi::SWIGLU) {
        y[p] = silu_f(a) * c;
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
  }
}

template <typename TW, int EPI>
static hipError_t gemv_t(const TW* W, const float* x, const float* g, float eps, int N, int K, float* y,
                         hipStream_t st) {
  const int npairs = EPI == (int)GvEpi::SWIGLU ? N / 2 : (N + 1) / 2;
  const size_t lds = (size_t)K * sizeof(float);
  // many rows: a wave per GV_RPW rows keeps enough loads in flight; few
  // rows: split K over the waves of a workgroup to occupy more of the chip
  const int waves_rows = (npairs + GV_RPW / 2 - 1) / (GV_RPW / 2);
  if (waves_rows >= 2048) {
    const int blocks = (waves_rows + GV_THREADS / 64 - 1) / (GV_THREADS / 64);
    if (g) hipLaunchKernelGGL((gemv_rows_kernel<TW, EPI, true>), dim3(blocks), dim3(GV_THREADS), lds, st, W, x, g, eps, N, K, y);
    else hipLaunchKernelGGL((gemv_rows_kernel<TW, EPI, false>), dim3(blocks), dim3(GV_THREADS), lds, st, W, x, g, eps, N, K, y);
    return hipGetLastError();
  }
  const int blocks = (npairs + GV_ROWS / 2 - 1) / (GV_ROWS / 2);
  if (g) hipLaunchKernelGGL((gemv_kernel<TW, EPI, true>), dim3(blocks), dim3(GV_THREADS), lds, st, W, x, g, eps, N, K, y);
  else hipLaunchKernelGGL((gemv_kernel<TW, EPI, false>), dim3(blocks), dim3(GV_THREADS), lds, st, W, x, g, eps, N, K, y);
  return hipGetLastError();
}

hipError_t gemv(DT wdt, const void* W, const float* x, const float* g, float eps, int N, int K, GvEpi epi,
                float* y, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if ((K * 4) > 64 * 1024 || K % 8) return hipErrorInvalidValue;
  if (wdt == DT::BF16) {
    switch (epi) {
      case GvEpi::STORE: return gemv_t<bf16, (int)GvEpi::STORE>((const bf16*)W, x, g, eps, N, K, y, st);
      case GvEpi::ADD_F32: return gemv_t<bf16, (int)GvEpi::ADD_F32>((const bf16*)W, x, g, eps, N, K, y, st);
      case GvEpi::SWIGLU: return gemv_t<bf16, (int)GvEpi::SWIGLU>((const bf16*)W, x, g, eps, N, K, y, st);
    }
  } else {
    switch (epi) {
      case GvEpi::STORE: return gemv_t<float, (int)GvEpi::STORE>((const float*)W, x, g, eps, N, K, y, st);
      case GvEpi::ADD_F32: return gemv_t<float, (int)GvEpi::ADD_F32>((const float*)W, x, g, eps, N, K, y, st);
      case GvEpi::SWIGLU: return gemv_t<float, (int)GvEpi::SWIGLU>((const float*)W, x, g, eps, N, K, y, st);
    }
  }
  return hipErrorInvalidValue;
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

// ------------------------------------------------------ RoPE + ring store
// Rotates q and k of position p (half-split pairs (j, j + dh/2) by the
// angle table) and stores k, v (and v transposed when vts is given) at ring
// slot p & (cap - 1).
template <typename T>
__global__ void decode_rope_store_kernel(const float* qkv, int H, int Hk, int dh, const int64_t* pos,
                                         const float2* tab, float* q, T* ks, T* vs, T* vts, int cap) {
  // workgroup hh < H: query head; H <= hh < H + Hk: key head; then value heads
  const int64_t p = *pos;
  const int half = dh / 2;
  const long slot = p & (cap - 1);
  const int hh = blockIdx.x;
  if (hh < H + Hk) {
    const float2* tb = tab + p * half;
    for (int j = threadIdx.x; j < half; j += blockDim.x) {
      const float2 cs = tb[j];
      const float a = qkv[hh * dh + j], b = qkv[hh * dh + j + half];
      const float ra = a * cs.x - b * cs.y, rb = b * cs.x + a * cs.y;
      if (hh < H) {
        q[hh * dh + j] = ra;
        q[hh * dh + j + half] = rb;
      } else {
        const int kh = hh - H;
        ks[((long)kh * cap + slot) * dh + j] = from_f<T>(ra);
        ks[((long)kh * cap + slot) * dh + j + half] = from_f<T>(rb);
      }
    }
  } else {
    const int kh = hh - H - Hk;
    for (int j = threadIdx.x; j < dh; j += blockDim.x) {
      const T v = from_f<T>(qkv[(H + Hk) * dh + kh * dh + j]);
      vs[((long)kh * cap + slot) * dh + j] = v;
      if (vts) vts[((long)kh * dh + j) * cap + vt_slot(slot)] = v;
    }
  }
}

hipError_t decode_rope_store(DT dt, const float* qkv, int H, int Hk, int dh, const int64_t* pos,
                             const float2* rope_tab, float* q, void* kstore, void* vstore, void* vtstore, int cap,
                             hipStream_t st) {
  const dim3 grid(H + 2 * Hk);
  if (dt == DT::BF16)
    hipLaunchKernelGGL(decode_rope_store_kernel<bf16>, grid, dim3(64), 0, st, qkv, H, Hk, dh, pos, rope_tab, q,
                       (bf16*)kstore, (bf16*)vstore, (bf16*)vtstore, cap);
  else
    hipLaunchKernelGGL(decode_rope_store_kernel<float>, grid, dim3(64), 0, st, qkv, H, Hk, dh, pos, rope_tab, q,
                       (float*)kstore, (float*)vstore, (float*)vtstore, cap);
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
// are formed once per head in LDS, then each thread sums one output column.
__global__ void __launch_bounds__(128) decode_attn_combine_kernel(const float* part, int nsplit, int dh, float* o) {
  __shared__ float wsh[256];
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
  const float inv = 1.f / Lsh;
  for (int dd = threadIdx.x; dd < dh; dd += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) acc += ph[s * (dh + 2) + dd] * wsh[s];
    o[h * dh + dd] = acc * inv;
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

  Frag8<bf16> qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      qf[s].v[e] = (bf16)(c < G ? q[(long)(kh * G + c) * DH + 32 * s + 8 * g + e] * scale2 : 0.f);
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
  hipLaunchKernelGGL(decode_attn_combine_kernel, dim3(H), dim3(128), 0, st, part, nsplit, DH, o);
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
    const dim3 grid(Hk, nsplit);
    const float sc2 = 1.f / sqrtf((float)dh) * 1.4426950408889634f;
    if (dh == 128)
      hipLaunchKernelGGL(decode_attn_mfma_kernel<128>, grid, dim3(256), 0, st, q, (const bf16*)kstore,
                         (const bf16*)vtstore, H, Hk, cap, window, pos, sc2, nsplit, part);
    else
      hipLaunchKernelGGL(decode_attn_mfma_kernel<64>, grid, dim3(256), 0, st, q, (const bf16*)kstore,
                         (const bf16*)vtstore, H, Hk, cap, window, pos, sc2, nsplit, part);
    hipLaunchKernelGGL(decode_attn_combine_kernel, dim3(H), dim3(128), 0, st, part, nsplit, dh, o);
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
